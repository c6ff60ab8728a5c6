"""Dropout on P: GPU parity with the oracle (same Philox keep bits on both sides)."""
import numpy as np
import pytest

import workloads
from helpers import compare, ensure_library, run_oracle, upload

pytestmark = pytest.mark.gpu

SEED = 0x0123_4567_89AB_CDEF
OFFSET = 11


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def _run(case, p, seed=SEED, offset=OFFSET):
    import torch
    import exact_attention_100_amd as fa
    t = upload(case)
    sc = float(case.scale)
    o, lse = fa.fwd(t["q"], t["k"], t["v"], scale=sc, causal=case.causal, key_len=t["key_len"],
                    dropout_p=p, seed=seed, offset=offset)
    dq, dk, dv = fa.bwd(t["q"], t["k"], t["v"], o, t["do"], lse, scale=sc, causal=case.causal,
                        key_len=t["key_len"], dropout_p=p, seed=seed, offset=offset)
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy().astype(np.float64) for k, v in
            dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv).items()}


@pytest.mark.parametrize("p", [0.1, 0.5])
@pytest.mark.parametrize("mask", ["none", "causal", "key_len", "causal+key_len"])
@pytest.mark.parametrize("d", [64, 128])
def test_dropout_matches_oracle(p, mask, d):
    case = workloads.make_case(2, 2, 300, d, mask=mask, seed=80 + d, key_len_range=(1, 300),
                               name=f"dropout-{mask}")
    print("[case]", case.name, "p", p, "d", d, flush=True)
    gpu = _run(case, p)
    p8 = int(round(p * 256))
    ref = run_oracle(case, dropout=(p8, SEED, OFFSET))
    print("[case] errors", compare(gpu, ref, case), flush=True)


def test_dropout_zero_equals_plain_and_seeds_matter():
    case = workloads.make_case(1, 2, 256, 128, mask="causal", seed=85, name="dropout-seeds")
    print("[case]", case.name, flush=True)
    plain = _run(case, 0.0)
    a = _run(case, 0.2)
    b = _run(case, 0.2)
    c = _run(case, 0.2, seed=SEED + 1)
    for k in plain:
        np.testing.assert_array_equal(a[k], b[k])  # deterministic for fixed (seed, offset)
    assert not np.array_equal(a["o"], c["o"])
    assert not np.array_equal(a["o"], plain["o"])
    np.testing.assert_array_equal(a["lse"], plain["lse"])  # LSE is the softmax's, before dropout


def _run_sparse(case, p, seed=SEED, offset=OFFSET):
    import torch
    import exact_attention_100_amd as fa
    t = upload(case)
    sc = float(case.scale)
    kw = dict(scale=sc, causal=case.causal, key_len=t["key_len"], dropout_p=p, seed=seed, offset=offset)
    o, lse = fa.blocksparse_fwd(t["q"], t["k"], t["v"], t["block_mask"], case.block_size, **kw)
    dq, dk, dv = fa.blocksparse_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, t["block_mask"], case.block_size, **kw)
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy().astype(np.float64) for k, v in
            dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv).items()}


@pytest.mark.parametrize("p", [0.1, 0.5])
@pytest.mark.parametrize("mask", ["block", "block+causal", "block+key_len", "block+causal+key_len"])
@pytest.mark.parametrize("d,bs", [(64, 128), (128, 128), (64, 256)])
def test_block_sparse_dropout_matches_oracle(p, mask, d, bs):
    """Dropout inside the block-sparse kernels: the keep bits of the pairs in kept blocks are those
    of the dense kernels (same counters), every other pair has probability 0 anyway."""
    N = 4 * bs
    case = workloads.make_case(2, 2, N, d, mask=mask, block_size=bs, block_p=0.5, seed=87 + d + bs,
                               key_len_range=(bs // 2, N - 1), name=f"sparse-dropout-{mask}")
    case.block_mask[2, 0] = 1  # at least one kept block below the diagonal
    print("[case]", case.name, "p", p, "d", d, "bs", bs, flush=True)
    gpu = _run_sparse(case, p)
    ref = run_oracle(case, dropout=(int(round(p * 256)), SEED, OFFSET))
    print("[case] errors", compare(gpu, ref, case), flush=True)


def test_block_sparse_dropout_all_ones_equals_dense_dropout():
    """With an all-ones block mask the block-sparse dropout kernels compute what the dense ones do."""
    import torch
    import exact_attention_100_amd as fa
    case = workloads.make_case(1, 2, 512, 128, mask="causal", seed=88, name="sparse-dropout-vs-dense")
    print("[case]", case.name, flush=True)
    t = upload(case)
    ones = torch.ones((4, 4), dtype=torch.uint8, device="cuda")
    kw = dict(causal=True, dropout_p=0.2, seed=SEED, offset=OFFSET)
    o1, l1 = fa.fwd(t["q"], t["k"], t["v"], **kw)
    o2, l2 = fa.blocksparse_fwd(t["q"], t["k"], t["v"], ones, 128, **kw)
    g1 = fa.bwd(t["q"], t["k"], t["v"], o1, t["do"], l1, **kw)
    g2 = fa.blocksparse_bwd(t["q"], t["k"], t["v"], o1, t["do"], l1, ones, 128, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)

