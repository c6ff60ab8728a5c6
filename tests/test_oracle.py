"""Pins of the CPU float64 oracle against facts fixed by the pages and by mathematics.

Nothing here compares the oracle with itself: every check is a hand-solved case,
a closed form, an invariant the definition implies, a finite difference of the
forward, or an independent library routine.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _val(x):
    """Parse golden values: numbers, 'lnN', 'a/b', and '*' products of those."""
    if isinstance(x, (int, float)):
        return float(x)
    out = 1.0
    for f in x.split("*"):
        f = f.strip()
        if f.startswith("ln"):
            out *= math.log(float(f[2:]))
        elif "/" in f:
            a, b = f.split("/")
            out *= float(a) / float(b)
        else:
            out *= float(f)
    return out


def _arr(x):
    return np.vectorize(_val, otypes=[float])(np.array(x, dtype=object))


def _load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def _one_head(x):
    return np.asarray(x, dtype=np.float64)[None, None]


# --------------------------------------------------------------------------- hand cases

@pytest.mark.parametrize("kind", ["dense", "causal"])
def test_hand_n2(kind):
    g = _load("hand_n2.json")
    inp = g["inputs"]
    q, k, v, do = (_one_head(_arr(inp[n])) for n in ("q", "k", "v", "do"))
    causal = kind == "causal"
    O, LSE = oracle.forward(q, k, v, _val(inp["scale"]), causal=causal)
    dQ, dK, dV = oracle.backward(q, k, v, do, _val(inp["scale"]), causal=causal)
    exp = g[kind]
    np.testing.assert_allclose(O[0, 0], _arr(exp["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(LSE[0, 0], _arr(exp["lse"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dQ[0, 0], _arr(exp["dq"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dK[0, 0], _arr(exp["dk"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dV[0, 0], _arr(exp["dv"]), rtol=0, atol=1e-14)
    ok = oracle.allowed_matrix(2, causal)
    _, _, _, dsum = oracle.head_backward(q[0, 0], k[0, 0], v[0, 0], do[0, 0], _val(inp["scale"]), ok)
    np.testing.assert_allclose(dsum, _arr(exp["D"]), rtol=0, atol=1e-14)


@pytest.mark.parametrize("kind", ["dense", "causal", "key_len_2", "block_identity_bs2"])
def test_hand_n4(kind):
    g = _load("hand_n4.json")
    inp = g["inputs"]
    q, k, v = (_one_head(_arr(inp[n])) for n in ("q", "k", "v"))
    exp = g[kind]
    kw = {}
    if kind == "causal":
        kw["causal"] = True
    if "key_len" in exp:
        kw["key_len"] = np.array([exp["key_len"]])
    if "block_mask" in exp:
        kw["block_mask"] = np.array(exp["block_mask"], dtype=np.uint8)
        kw["block_size"] = exp["block_size"]
    O, LSE = oracle.forward(q, k, v, _val(inp["scale"]), **kw)
    np.testing.assert_allclose(O[0, 0], _arr(exp["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(LSE[0, 0], _arr(exp["lse"]), rtol=0, atol=1e-14)


# --------------------------------------------------------------------------- helpers

def _rand(rng, *shape):
    return rng.standard_normal(shape)


MASKS = [
    dict(),
    dict(causal=True),
    dict(key_len=np.array([5, 9])),
    dict(causal=True, key_len=np.array([7, 1])),
    dict(block_mask=np.array([[1, 0, 1], [0, 1, 0], [1, 1, 0]], dtype=np.uint8), block_size=4),
]


def _allowed_for(N, b, kw):
    L = None if kw.get("key_len") is None else int(kw["key_len"][b])
    return oracle.allowed_matrix(N, kw.get("causal", False), L, kw.get("block_mask"), kw.get("block_size"))


# --------------------------------------------------------------------------- P1 row sums

@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_row_sums_and_masked_zero(mi):
    kw = MASKS[mi]
    rng = np.random.default_rng(10 + mi)
    N, d = 12, 5
    for b in range(2):
        ok = _allowed_for(N, b, kw)
        _, p, lse = oracle.head_probabilities(_rand(rng, N, d), _rand(rng, N, d), 0.7, ok)
        has = ok.any(axis=1)
        np.testing.assert_allclose(p.sum(axis=1)[has], 1.0, rtol=0, atol=1e-12)
        assert np.all(p[~ok] == 0.0)
        assert np.all(p >= 0.0)
        assert np.all(np.isneginf(lse[~has]))
        assert np.all(np.isfinite(lse[has]))


# --------------------------------------------------------------------------- P4 closed forms

@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_scale_zero_is_mean_of_allowed_values(mi):
    kw = MASKS[mi]
    rng = np.random.default_rng(20 + mi)
    B, H, N, d = 2, 1, 12, 3
    q, k, v = (_rand(rng, B, H, N, d) for _ in range(3))
    O, LSE = oracle.forward(q, k, v, 0.0, **kw)
    for b in range(B):
        ok = _allowed_for(N, b, kw)
        for i in range(N):
            cnt = ok[i].sum()
            if cnt == 0:
                assert np.all(O[b, 0, i] == 0) and np.isneginf(LSE[b, 0, i])
                continue
            np.testing.assert_allclose(O[b, 0, i], v[b, 0][ok[i]].mean(axis=0), rtol=0, atol=1e-13)
            np.testing.assert_allclose(LSE[b, 0, i], math.log(cnt), rtol=0, atol=1e-13)


def test_single_key_and_causal_row0():
    rng = np.random.default_rng(3)
    q, k, v = (_rand(rng, 1, 1, 1, 4) for _ in range(3))
    O, LSE = oracle.forward(q, k, v, 0.37)
    np.testing.assert_allclose(O[0, 0, 0], v[0, 0, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(LSE[0, 0, 0], 0.37 * float(q[0, 0, 0] @ k[0, 0, 0]), rtol=0, atol=1e-14)
    q, k, v = (_rand(rng, 1, 2, 9, 4) for _ in range(3))
    O, LSE = oracle.forward(q, k, v, 0.5, causal=True)
    np.testing.assert_allclose(O[:, :, 0], v[:, :, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(LSE[:, :, 0], 0.5 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                               rtol=0, atol=1e-14)


def test_two_keys_is_logistic():
    """With two allowed keys, P_i1 = sigmoid(s_i1 - s_i0) (a textbook identity)."""
    rng = np.random.default_rng(4)
    q, k, v = (_rand(rng, 1, 1, 6, 3) for _ in range(3))
    O, _ = oracle.forward(q, k, v, 0.8, key_len=np.array([2]))
    s = 0.8 * q[0, 0] @ k[0, 0, :2].T
    w1 = 1.0 / (1.0 + np.exp(-(s[:, 1] - s[:, 0])))
    np.testing.assert_allclose(O[0, 0], (1 - w1)[:, None] * v[0, 0, 0] + w1[:, None] * v[0, 0, 1],
                               rtol=0, atol=1e-14)


# --------------------------------------------------------------------------- P5 reductions

def test_key_len_reduces_to_truncated_dense():
    rng = np.random.default_rng(5)
    N, d = 11, 4
    q, k, v, do = (_rand(rng, 1, 1, N, d) for _ in range(4))
    L = 6
    O, LSE = oracle.forward(q, k, v, 0.6, key_len=np.array([L]))
    # dense attention of every query against the first L keys only
    s = 0.6 * q[0, 0] @ k[0, 0, :L].T
    w = np.exp(s - s.max(axis=1, keepdims=True))
    ref = (w / w.sum(axis=1, keepdims=True)) @ v[0, 0, :L]
    np.testing.assert_allclose(O[0, 0], ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(LSE[0, 0], np.log(np.exp(s).sum(axis=1)), rtol=0, atol=1e-12)
    dQ, dK, dV = oracle.backward(q, k, v, do, 0.6, key_len=np.array([L]))
    assert np.all(dK[0, 0, L:] == 0) and np.all(dV[0, 0, L:] == 0)


def test_causal_row_equals_prefix_attention():
    rng = np.random.default_rng(6)
    N, d = 10, 3
    q, k, v = (_rand(rng, 1, 1, N, d) for _ in range(3))
    O, LSE = oracle.forward(q, k, v, 1.1, causal=True)
    for i in range(N):
        s = 1.1 * k[0, 0, :i + 1] @ q[0, 0, i]
        w = np.exp(s - s.max())
        np.testing.assert_allclose(O[0, 0, i], (w / w.sum()) @ v[0, 0, :i + 1], rtol=0, atol=1e-13)
        np.testing.assert_allclose(LSE[0, 0, i], np.log(np.exp(s).sum()), rtol=0, atol=1e-12)


def test_block_mask_all_ones_is_dense_and_diagonal_is_blockwise():
    rng = np.random.default_rng(7)
    N, d, bs = 12, 4, 4
    q, k, v, do = (_rand(rng, 1, 2, N, d) for _ in range(4))
    ones = np.ones((3, 3), dtype=np.uint8)
    Od, Ld = oracle.forward(q, k, v, 0.5)
    Ob, Lb = oracle.forward(q, k, v, 0.5, block_mask=ones, block_size=bs)
    np.testing.assert_array_equal(Od, Ob)
    np.testing.assert_array_equal(Ld, Lb)
    g_d = oracle.backward(q, k, v, do, 0.5)
    g_b = oracle.backward(q, k, v, do, 0.5, block_mask=ones, block_size=bs)
    for a, b in zip(g_d, g_b):
        np.testing.assert_array_equal(a, b)
    eye = np.eye(3, dtype=np.uint8)
    Oe, Le = oracle.forward(q, k, v, 0.5, block_mask=eye, block_size=bs)
    ge = oracle.backward(q, k, v, do, 0.5, block_mask=eye, block_size=bs)
    for blk in range(3):
        sl = slice(blk * bs, (blk + 1) * bs)
        Op, Lp = oracle.forward(q[:, :, sl], k[:, :, sl], v[:, :, sl], 0.5)
        np.testing.assert_allclose(Oe[:, :, sl], Op, rtol=0, atol=1e-14)
        np.testing.assert_allclose(Le[:, :, sl], Lp, rtol=0, atol=1e-14)
        gp = oracle.backward(q[:, :, sl], k[:, :, sl], v[:, :, sl], do[:, :, sl], 0.5)
        for a, b in zip(ge, gp):
            np.testing.assert_allclose(a[:, :, sl], b, rtol=0, atol=1e-13)


# --------------------------------------------------------------------------- P6 shift invariances

@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_shift_invariances(mi):
    kw = MASKS[mi]
    rng = np.random.default_rng(30 + mi)
    B, H, N, d = 2, 1, 12, 3
    q, k, v, do = (_rand(rng, B, H, N, d) for _ in range(4))
    c = rng.standard_normal(d)
    sc = 0.9
    O, LSE = oracle.forward(q, k, v, sc, **kw)
    g = oracle.backward(q, k, v, do, sc, **kw)
    Ok, LSEk = oracle.forward(q, k + c, v, sc, **kw)
    gk = oracle.backward(q, k + c, v, do, sc, **kw)
    Ov, _ = oracle.forward(q, k, v + c, sc, **kw)
    gv = oracle.backward(q, k, v + c, do, sc, **kw)
    has = np.isfinite(LSE)
    np.testing.assert_allclose(Ok, O, rtol=0, atol=1e-12)
    shift = sc * np.einsum("bhnd,d->bhn", q, c)
    np.testing.assert_allclose(LSEk[has], (LSE + shift)[has], rtol=0, atol=1e-12)
    np.testing.assert_allclose(Ov[has], (O + c)[has], rtol=0, atol=1e-12)
    for a, b in zip(gk, g):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)
    for a, b in zip(gv, g):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


# --------------------------------------------------------------------------- P7 finite differences

FD_MASKS = [dict(), dict(causal=True), dict(key_len=np.array([2])),
            dict(block_mask=np.array([[1, 0], [1, 1]], dtype=np.uint8), block_size=2)]


@pytest.mark.parametrize("N,d", [(2, 1), (3, 2), (4, 3), (5, 2)])
@pytest.mark.parametrize("mi", range(len(FD_MASKS)))
def test_finite_differences(N, d, mi):
    kw = dict(FD_MASKS[mi])
    if "block_mask" in kw and N % 2:
        pytest.skip("block size 2 needs even N")
    if "block_mask" in kw:
        kw["block_mask"] = np.ones((N // 2, N // 2), dtype=np.uint8)
        kw["block_mask"][0, -1] = 0 if N > 2 else 1
    rng = np.random.default_rng(100 * N + 10 * d + mi)
    q, k, v, do = (_rand(rng, 1, 1, N, d) for _ in range(4))
    sc = 0.7

    def loss(q_, k_, v_):
        O, _ = oracle.forward(q_, k_, v_, sc, **kw)
        return float(np.sum(do * O))

    grads = oracle.backward(q, k, v, do, sc, **kw)
    h = 1e-5
    for which, g in zip(range(3), grads):
        num = np.zeros_like(g)
        for idx in np.ndindex(*q.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.abs(num - g)
        assert np.all(err <= 1e-7 * np.abs(g) + 1e-9), (which, err.max())


# --------------------------------------------------------------------------- P8 gradient invariants

@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_gradient_invariants(mi):
    kw = MASKS[mi]
    rng = np.random.default_rng(40 + mi)
    B, H, N, d = 2, 2, 12, 5
    q, k, v, do = (_rand(rng, B, H, N, d) for _ in range(4))
    dQ, dK, dV = oracle.backward(q, k, v, do, 0.8, **kw)
    O, _ = oracle.forward(q, k, v, 0.8, **kw)
    for b in range(B):
        ok = _allowed_for(N, b, kw)
        has = ok.any(axis=1)
        seen = ok.any(axis=0)
        for h in range(H):
            # sum_j dS_ij = 0 for every row  =>  sum_j dK_j = 0
            np.testing.assert_allclose(dK[b, h].sum(axis=0), 0.0, rtol=0, atol=1e-12)
            # sum_j dV_j = sum_i (sum_j P_ij) dO_i = sum over rows with an allowed key of dO_i
            np.testing.assert_allclose(dV[b, h].sum(axis=0), do[b, h][has].sum(axis=0), rtol=0, atol=1e-12)
            assert np.all(dK[b, h][~seen] == 0) and np.all(dV[b, h][~seen] == 0)
            assert np.all(dQ[b, h][~has] == 0)
            _, _, _, dsum = oracle.head_backward(q[b, h], k[b, h], v[b, h], do[b, h], 0.8, ok)
            np.testing.assert_allclose(dsum, (do[b, h] * O[b, h]).sum(axis=1), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- P9 independent library

@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_matches_torch_sdpa_float64(mi):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    kw = MASKS[mi]
    rng = np.random.default_rng(50 + mi)
    B, H, N, d = 2, 3, 12, 8
    q, k, v, do = (_rand(rng, B, H, N, d) for _ in range(4))
    sc = 0.35
    O, LSE = oracle.forward(q, k, v, sc, **kw)
    dQ, dK, dV = oracle.backward(q, k, v, do, sc, **kw)
    mask = np.stack([_allowed_for(N, b, kw) for b in range(B)])[:, None]  # [B,1,N,N]
    has = mask.any(axis=-1)[..., None]  # rows with an allowed key
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(mask), scale=sc)
    to = torch.where(torch.tensor(has), to, torch.zeros_like(to))
    to.backward(torch.tensor(do))
    hb = np.broadcast_to(has, O.shape)
    np.testing.assert_allclose(O[hb], to.detach().numpy()[hb], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dQ, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dK, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dV, tv.grad.numpy(), rtol=0, atol=1e-11)
    s = sc * np.einsum("bhid,bhjd->bhij", q, k)
    s = np.where(mask, s, -np.inf)
    with np.errstate(divide="ignore"):
        ref_lse = np.log(np.exp(s).sum(axis=-1))
    np.testing.assert_allclose(LSE[hb[..., 0]], ref_lse[hb[..., 0]], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- sampled evaluation

SAMPLED_MASKS = MASKS + [dict(causal=True, key_len=np.array([40, 17]),
                              block_mask=(np.random.default_rng(7).random((12, 12)) < 0.4).astype(np.uint8),
                              block_size=5)]


@pytest.mark.parametrize("mi", range(len(SAMPLED_MASKS)))
def test_sampled_rows_and_keys_match_full_oracle(mi):
    """forward_rows / backward_rows / backward_keys (chunked, restricted to the keys each chunk
    may attend) reproduce forward() / backward() on every row and key, chunks smaller than N."""
    kw = SAMPLED_MASKS[mi]
    N = kw["block_mask"].shape[0] * kw["block_size"] if "block_mask" in kw else 12
    rng = np.random.default_rng(70 + mi)
    B, H, d = 2, 2, 8
    q, k, v, do = (_rand(rng, B, H, N, d) for _ in range(4))
    sc = 0.41
    O, LSE = oracle.forward(q, k, v, sc, **kw)
    dQ, dK, dV = oracle.backward(q, k, v, do, sc, **kw)
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            o, lse = oracle.forward_rows(q, k, v, sc, b, h, rows, **kw)
            np.testing.assert_allclose(o, O[b, h], rtol=0, atol=1e-12)
            np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(LSE[b, h]))
            fin = np.isfinite(lse)
            np.testing.assert_allclose(lse[fin], LSE[b, h][fin], rtol=0, atol=1e-12)
            dq = oracle.backward_rows(q, k, v, do, sc, b, h, rows, chunk=5, **kw)
            np.testing.assert_allclose(dq, dQ[b, h], rtol=0, atol=1e-12)
            keys = rng.permutation(N)[: N // 2]
            dk, dv = oracle.backward_keys(q, k, v, do, sc, b, h, keys, chunk=7, **kw)
            np.testing.assert_allclose(dk, dK[b, h][keys], rtol=0, atol=1e-12)
            np.testing.assert_allclose(dv, dV[b, h][keys], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- dropout

def test_philox_known_answers():
    """The generator behind the dropout bits reproduces the published known-answer vectors."""
    import json
    kat = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
    for vec in kat["vectors"]:
        ctr = np.array([int(x, 16) for x in vec["ctr"]], dtype=np.uint64)
        key = np.array([int(x, 16) for x in vec["key"]], dtype=np.uint64)
        out = [format(int(x), "08x") for x in oracle.philox4x32(ctr, key)]
        assert out == vec["out"]


# Pair (i, j) of the first known-answer block (counter (0, 0, 0, 0), key (0, 0)): byte j of word i
# of the published output 6627e8d5 e169c58d bc57ac4c 9b00dbd8, read off by hand (least significant
# byte first). A swap of rows and columns, of word and byte, or a wrong byte order fails here.
HAND_KEEP_BYTES = {(0, 0): 0xD5, (0, 1): 0xE8, (0, 2): 0x27, (0, 3): 0x66,
                   (1, 0): 0x8D, (1, 1): 0xC5, (1, 2): 0x69, (1, 3): 0xE1,
                   (2, 0): 0x4C, (2, 1): 0xAC, (2, 2): 0x57, (2, 3): 0xBC,
                   (3, 0): 0xD8, (3, 1): 0xDB, (3, 2): 0x00, (3, 3): 0x9B}


def _keep_byte(rows, cols, bh, seed, offset):
    """Recover the generator byte behind each pair from the keep decisions alone: the pair is kept
    at p8 = byte and dropped at p8 = byte + 1, so the byte is the number of p8 in 1..255 that keep it."""
    n = np.zeros((len(rows), len(cols)), dtype=np.int64)
    for p8 in range(1, 256):
        n += oracle.dropout_keep(rows, cols, bh, p8, seed, offset)
    return n


def test_dropout_keep_bytes_by_hand():
    """The (i, j) -> (counter, word, byte) map of the keep bits, pinned on the first published
    known-answer vector: seed 0, offset 0, instance 0 put every pair i, j < 4 at counter (0,0,0,0)."""
    got = _keep_byte(np.arange(4), np.arange(4), 0, 0, 0)
    for (i, j), byte in HAND_KEEP_BYTES.items():
        assert got[i, j] == byte, (i, j, got[i, j], byte)
    # pair (1, 2) takes byte 2 of e169c58d = 0x69 = 105: kept iff p8 <= 105
    assert oracle.dropout_keep([1], [2], 0, 105, 0, 0)[0, 0]
    assert not oracle.dropout_keep([1], [2], 0, 106, 0, 0)[0, 0]
    # and the rows 4.. / columns 4.. of the block belong to other counters (not the same bytes)
    other = _keep_byte(np.arange(4, 8), np.arange(4), 0, 0, 0)
    assert not np.array_equal(other, got)


@pytest.mark.parametrize("vi", [1, 2])
def test_dropout_keep_counter_and_key_words(vi):
    """The other published vectors fix which counter word holds i div 4, j div 4, the instance and
    the offset, and which key word holds which half of the seed: choosing rows, columns, instance,
    offset and seed so that the counter and key equal the vector's, the recovered bytes must be
    those of the published output words."""
    kat = _load("philox4x32_10_kat.json")["vectors"][vi]
    c = [int(x, 16) for x in kat["ctr"]]
    k = [int(x, 16) for x in kat["key"]]
    w = [int(x, 16) for x in kat["out"]]
    rows = 4 * c[0] + np.arange(4)
    cols = 4 * c[1] + np.arange(4)
    seed = k[0] | (k[1] << 32)
    got = _keep_byte(rows, cols, c[2], seed, c[3])
    want = np.array([[(w[i] >> (8 * j)) & 0xFF for j in range(4)] for i in range(4)])
    np.testing.assert_array_equal(got, want)


def test_hand_n2_inverted_dropout():
    """Inverted dropout in the forward (O = (P o Z) V / (1 - p), LSE of the softmax before dropout)
    and its backward, on the N = 2 hand case with keep bits read off the published vector."""
    g = _load("hand_n2_dropout.json")
    inp = g["inputs"]
    q, k, v, do = (_one_head(_arr(inp[n])) for n in ("q", "k", "v", "do"))
    drop = (inp["p8"], inp["seed"], inp["offset"])
    keep = oracle.dropout_keep(np.arange(2), np.arange(2), 0, *drop)
    np.testing.assert_array_equal(keep, np.array(g["keep"]))
    assert oracle.keep_scale(inp["p8"]) == 256.0 / 106.0
    O, LSE = oracle.forward(q, k, v, _val(inp["scale"]), dropout=drop)
    dQ, dK, dV = oracle.backward(q, k, v, do, _val(inp["scale"]), dropout=drop)
    np.testing.assert_allclose(O[0, 0], _arr(g["o"]), rtol=1e-15, atol=1e-14)
    np.testing.assert_allclose(LSE[0, 0], _arr(g["lse"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dV[0, 0], _arr(g["dv"]), rtol=1e-15, atol=1e-14)
    np.testing.assert_allclose(dQ[0, 0], _arr(g["dq"]), rtol=1e-15, atol=1e-14)
    np.testing.assert_allclose(dK[0, 0], _arr(g["dk"]), rtol=1e-15, atol=1e-14)
    ok = oracle.allowed_matrix(2)
    _, _, _, dsum = oracle.head_backward(q[0, 0], k[0, 0], v[0, 0], do[0, 0], _val(inp["scale"]), ok, keep,
                                         oracle.keep_scale(inp["p8"]))
    np.testing.assert_allclose(dsum, _arr(g["D"]), rtol=1e-15, atol=1e-14)


def test_dropout_keep_rate_and_indexing():
    N, p8 = 512, 26
    keep = oracle.dropout_keep(np.arange(N), np.arange(N), 3, p8, seed=0x1234_5678_9ABC, offset=7)
    rate = keep.mean()
    expect = (256 - p8) / 256
    assert abs(rate - expect) < 5 * np.sqrt(expect * (1 - expect) / keep.size)
    # any sub-block reads the same bits; other instances / offsets / seeds give other bits
    rows, cols = np.array([5, 77, 300]), np.array([0, 3, 4, 511])
    np.testing.assert_array_equal(oracle.dropout_keep(rows, cols, 3, p8, 0x1234_5678_9ABC, 7),
                                  keep[np.ix_(rows, cols)])
    for other in [dict(bh=4, seed=0x1234_5678_9ABC, offset=7), dict(bh=3, seed=0x1234_5678_9ABC, offset=8),
                  dict(bh=3, seed=0x1234_5678_9ABD, offset=7), dict(bh=3, seed=0x1235_5678_9ABC, offset=7)]:
        k2 = oracle.dropout_keep(np.arange(64), np.arange(64), other["bh"], p8, other["seed"], other["offset"])
        assert not np.array_equal(k2, keep[:64, :64])
    assert oracle.dropout_keep(np.arange(8), np.arange(8), 0, 0, 1, 2).all()  # p = 0 keeps everything


@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_dropout_zero_is_plain_attention_and_d_identity(mi):
    kw = MASKS[mi]
    rng = np.random.default_rng(90 + mi)
    B, H, N, d = 2, 2, 12, 8
    q, k, v, do = (_rand(rng, B, H, N, d) for _ in range(4))
    O, LSE = oracle.forward(q, k, v, 0.3, **kw)
    O0, LSE0 = oracle.forward(q, k, v, 0.3, dropout=(0, 5, 6), **kw)
    np.testing.assert_array_equal(O, O0)
    np.testing.assert_array_equal(LSE, LSE0)
    drop = (77, 123456789, 3)
    Od, LSEd = oracle.forward(q, k, v, 0.3, dropout=drop, **kw)
    np.testing.assert_array_equal(LSEd, LSE)  # LSE is the softmax's, before dropout
    for b in range(B):
        for h in range(H):
            ok = _allowed_for(N, b, kw)
            keep = oracle.dropout_keep(np.arange(N), np.arange(N), b * H + h, drop[0], drop[1], drop[2])
            _, _, _, dsum = oracle.head_backward(q[b, h], k[b, h], v[b, h], do[b, h], 0.3, ok, keep,
                                                 oracle.keep_scale(drop[0]))
            # D = rowsum(dO o O) holds with dropout too (the kernels' form of D)
            np.testing.assert_allclose(dsum, (do[b, h] * Od[b, h]).sum(axis=1), rtol=0, atol=1e-12)


@pytest.mark.parametrize("mi", range(len(FD_MASKS)))
def test_dropout_finite_differences(mi):
    """The dropout backward is the gradient of <dO, O> for fixed keep bits."""
    kw = dict(FD_MASKS[mi])
    N, d, drop = 4, 3, (90, 42, 1)
    if "block_mask" in kw:
        kw["block_mask"] = np.array([[1, 0], [1, 1]], dtype=np.uint8)
    rng = np.random.default_rng(95 + mi)
    q, k, v, do = (_rand(rng, 1, 1, N, d) for _ in range(4))
    sc = 0.7
    dQ, dK, dV = oracle.backward(q, k, v, do, sc, dropout=drop, **kw)
    keep = oracle.dropout_keep(np.arange(N), np.arange(N), 0, drop[0], drop[1], drop[2])
    assert not keep.all() and keep.any()  # the case does drop some entries

    def loss(q_, k_, v_):
        o, _ = oracle.forward(q_, k_, v_, sc, dropout=drop, **kw)
        return float((do * o).sum())

    h = 1e-5
    for X, G, which in ((q, dQ, 0), (k, dK, 1), (v, dV, 2)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            xp, xm = X.copy(), X.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(G, num, rtol=1e-7, atol=1e-9)


@pytest.mark.parametrize("mask", ["causal", "key_len", "block"])
def test_nan_key_poisons_exactly_the_rows_that_see_it(mask):
    """A NaN in key j reaches exactly the rows allowed to see key j: their scores for j are
    NaN, so their softmax (and O, LSE) is NaN; every other row masks j to -inf before the
    softmax and is identical to a run with a finite key j."""
    rng = np.random.default_rng(17)
    N, d, j = 8, 4, 5
    q, k, v = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    kw = {"causal": dict(causal=True), "key_len": dict(key_len=np.array([j], np.int32)),
          "block": dict(block_mask=np.array([[1, 0], [0, 1]], np.uint8), block_size=4)}[mask]
    sees = {"causal": np.arange(N) >= j, "key_len": np.zeros(N, bool), "block": np.arange(N) >= 4}[mask]
    k_nan = k.copy()
    k_nan[0, 0, j, 0] = np.nan
    o, lse = oracle.forward(q, k_nan, v, 0.5, **kw)
    o_ref, lse_ref = oracle.forward(q, k, v, 0.5, **kw)
    assert np.all(np.isnan(lse[0, 0, sees])) and np.all(np.isnan(o[0, 0, sees]))
    np.testing.assert_array_equal(o[0, 0, ~sees], o_ref[0, 0, ~sees])
    np.testing.assert_array_equal(lse[0, 0, ~sees], lse_ref[0, 0, ~sees])
