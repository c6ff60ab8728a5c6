"""Standard (exact) attention in float64 on the CPU: the oracle.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's
CPU-baseline leg may import or call this module; the HIP library never does,
and nothing here is shared with it.

What it computes, per (batch, head) instance with Q, K, V in R^{N x d}:
  S = scale * Q K^T, P = row-wise softmax(S), O = P V
  -- FlashAttention reading notes (hackmd), §Background › Standard Attention
  Implementation, the S / P / O equations. The pages write S = Q K^T; the
  caller's scale multiplies S (a reading: the workloads use 1/sqrt(d)).
Masking sets disallowed entries of S to -inf before the softmax (the notes'
description of the fused kernel lists masking next to dropout after the
softmax; it is read as mask-before-softmax so that masked keys get zero
probability):
  * causal: key j is allowed for query i iff j <= i;
  * key padding: keys j >= key_len[b] are masked for every query of batch b;
  * block-sparse: entry (i, j) is allowed iff block_mask[i // bs, j // bs] != 0
    (same notes, §Introduction › Block-sparse FlashAttention: zero blocks are
    skipped, i.e. they contribute nothing to the softmax).
A row with no allowed key has P = 0, O = 0 and LSE = -inf (a reading; the
pages never reach such a row).

The forward also returns LSE = m + ln(l) with m the row max and l the row sum
of exp(S - m): the pages' forward saves O, m and l (§Algorithm › Recomputation);
one log-sum-exp per row carries the same information.

The backward is the exact gradient of L = <dO, O> by the chain rule through the
three equations above (the pages defer it to the paper's appendix):
  dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
  dS = P o (dP - D 1^T),  dQ = scale * dS K,  dK = scale * dS^T Q.
It recomputes P from Q and K; it never uses any LSE produced elsewhere.

Dropout (the notes' list of fused steps puts dropout after the softmax): with keep
bits Z from dropout_keep (Philox4x32-10, oracle/philox.py) and drop probability p,
O = (P o Z) V / (1 - p) and LSE stays that of the softmax; the backward is the
chain rule through that product (head_backward).

forward_rows, backward_rows and backward_keys evaluate the same equations for
chosen query rows / key columns of one instance, a chunk of rows at a time and
only over the keys each chunk may attend, so that long sequences never need the
N x N matrices; they are pinned against forward() / backward().

Pins (tests/test_oracle.py): hand-solved N=2 and N=4 cases (tests/golden/),
row sums, closed forms (scale 0, N 1, causal row 0), reductions of every mask
to plain attention on a sub-range, shift invariances, central finite
differences of <dO, O>, gradient invariants and an independent library routine
(torch CPU float64 scaled_dot_product_attention with autograd).
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np

from .philox import philox4x32


def allowed_matrix(N: int, causal: bool = False, key_len: Optional[int] = None,
                   block_mask: Optional[np.ndarray] = None, block_size: Optional[int] = None,
                   rows: Optional[np.ndarray] = None, cols: Optional[np.ndarray] = None) -> np.ndarray:
    """Boolean [len(rows), len(cols)] (all rows / keys by default): entry (i, j) is True iff
    key cols[j] may be attended by query rows[i]."""
    r = np.arange(N) if rows is None else np.asarray(rows)
    j = np.arange(N) if cols is None else np.asarray(cols)
    ok = np.ones((r.size, j.size), dtype=bool)
    if causal:
        ok &= j[None, :] <= r[:, None]
    if key_len is not None:
        L = min(max(int(key_len), 0), N)
        ok &= j[None, :] < L
    if block_mask is not None:
        bs = int(block_size)
        ok &= np.asarray(block_mask)[r[:, None] // bs, j[None, :] // bs] != 0
    return ok


def head_probabilities(q: np.ndarray, k: np.ndarray, scale: float, allowed: np.ndarray):
    """S, P and LSE for one head (float64). q: [R, d] query rows, k: [N, d]."""
    s = float(scale) * (q @ k.T)
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1)                       # row max; -inf for a row with no allowed key
    empty = m == -np.inf                    # (a NaN score keeps its row non-empty: NaN propagates)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])         # exp(-inf) = 0 on masked entries
    l = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(empty[:, None], 0.0, e / np.where(empty, 1.0, l)[:, None])
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return s, p, lse


def dropout_keep(rows, cols, bh: int, p8: int, seed: int, offset: int) -> np.ndarray:
    """Dropout keep bits, Boolean [len(rows), len(cols)], of instance bh = b * H + h.

    The pair (i, j) takes byte (j mod 4) of word (i mod 4) of Philox4x32-10 at counter
    (i div 4, j div 4, bh, offset) with key (seed mod 2^32, seed div 2^32); it is kept iff
    that byte is >= p8 (the drop probability is p8 / 256)."""
    r = np.asarray(rows, dtype=np.int64)[:, None]
    c = np.asarray(cols, dtype=np.int64)[None, :]
    shape = np.broadcast_shapes(r.shape, c.shape)
    ctr = np.stack([np.broadcast_to(r >> 2, shape), np.broadcast_to(c >> 2, shape),
                    np.full(shape, bh, dtype=np.int64), np.full(shape, offset, dtype=np.int64)], axis=-1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    words = philox4x32(ctr.astype(np.uint64), key).astype(np.int64)
    w = np.take_along_axis(words, np.broadcast_to(r & 3, shape)[..., None], axis=-1)[..., 0]
    byte = (w >> (8 * np.broadcast_to(c & 3, shape))) & 0xFF
    return byte >= int(p8)


def keep_scale(p8: int) -> float:
    """1 / (1 - p) for the drop probability p = p8 / 256."""
    return 256.0 / (256.0 - int(p8))


def head_forward(q, k, v, scale, allowed, keep=None, kscale=1.0):
    """O and LSE for one head: O = P V, or with dropout O = (P o Z) V / (1 - p) (keep bits
    Z, kscale = 1 / (1 - p)); LSE is that of the softmax before dropout."""
    _, p, lse = head_probabilities(q, k, scale, allowed)
    if keep is not None:
        p = p * keep * kscale
    return p @ v, lse


def head_backward(q, k, v, do, scale, allowed, keep=None, kscale=1.0):
    """dQ, dK, dV for one head, the gradient of <dO, O>; also returns D = rowsum(P o dP).
    With dropout, O = Pd V with Pd = P o Z / (1 - p): dV = Pd^T dO and dP = (dO V^T) o Z / (1 - p),
    then the same softmax backward."""
    _, p, _ = head_probabilities(q, k, scale, allowed)
    pd = p if keep is None else p * keep * kscale
    dv = pd.T @ do
    dp = do @ v.T
    if keep is not None:
        dp = dp * keep * kscale
    dsum = (p * dp).sum(axis=1)
    ds = p * (dp - dsum[:, None])
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv, dsum


def _dropout_for(dropout, N, bh):
    """(keep bits, 1 / (1 - p)) of instance bh for dropout = (p8, seed, offset), or (None, 1)."""
    if dropout is None or int(dropout[0]) == 0:
        return None, 1.0
    p8, seed, offset = (int(x) for x in dropout)
    return dropout_keep(np.arange(N), np.arange(N), bh, p8, seed, offset), keep_scale(p8)


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _heads(B: int, H: int, heads: Optional[Iterable]) -> list:
    if heads is None:
        return [(b, h) for b in range(B) for h in range(H)]
    return [tuple(x) for x in heads]


def forward(Q, K, V, scale, causal=False, key_len=None, block_mask=None, block_size=None,
            heads=None, dropout=None):
    """Exact attention forward over [B, H, N, d] inputs.

    Returns O [B, H, N, d] and LSE [B, H, N] in float64. With `heads` (a list of
    (b, h)) only those instances are computed; the rest of the outputs are NaN.
    dropout = (p8, seed, offset) applies dropout_keep's bits to P (None: no dropout).
    """
    B, H, N, d = Q.shape
    O = np.full((B, H, N, d), np.nan)
    LSE = np.full((B, H, N), np.nan)
    for b, h in _heads(B, H, heads):
        L = None if key_len is None else int(key_len[b])
        ok = allowed_matrix(N, causal, L, block_mask, block_size)
        keep, ks = _dropout_for(dropout, N, b * H + h)
        O[b, h], LSE[b, h] = head_forward(_f64(Q[b, h]), _f64(K[b, h]), _f64(V[b, h]), scale, ok, keep, ks)
    return O, LSE


def forward_rows(Q, K, V, scale, b, h, rows, causal=False, key_len=None, block_mask=None,
                 block_size=None):
    """O and LSE of selected query rows of one instance (each row depends only on its own q)."""
    N = Q.shape[2]
    rows = np.asarray(rows)
    L = None if key_len is None else int(key_len[b])
    ok = allowed_matrix(N, causal, L, block_mask, block_size, rows=rows)
    return head_forward(_f64(Q[b, h][rows]), _f64(K[b, h]), _f64(V[b, h]), scale, ok)


# ----------------------------------------------------------------------------- sampled evaluation
#
# For long sequences the N x N matrices do not fit. The functions below evaluate
# the same equations for chosen query rows or key columns of one (b, h) instance,
# a chunk of query rows at a time. Each chunk only touches the union of the keys
# its rows may attend (masked keys contribute exp(-inf) = 0 to every sum), so a
# causal or block-sparse instance costs what its kept pairs cost. They are pinned
# against forward() / backward() on sizes where those fit (tests/test_oracle.py).


def _candidate_cols(N, rows, L, causal, block_mask, block_size):
    """A superset of the keys that query rows `rows` may attend: below the causal and key-length
    bounds, and inside the key blocks that the rows' query blocks keep."""
    hi = N
    if causal:
        hi = min(hi, int(np.max(rows)) + 1)
    if L is not None:
        hi = min(hi, max(int(L), 0))
    if block_mask is None:
        return np.arange(hi)
    bs = int(block_size)
    kept = np.nonzero(np.asarray(block_mask)[np.unique(np.asarray(rows) // bs)].any(axis=0))[0]
    c = (kept[:, None] * bs + np.arange(bs)[None, :]).ravel()
    return c[c < hi]


def _chunk_terms(Q, K, V, dO, scale, rows, L, causal, block_mask, block_size):
    """For query rows `rows` of one instance: the kept key columns `cols`, and on them
    P, dP (rows x cols), LSE and D = sum_j P_ij dP_ij per row (same equations as
    head_probabilities / head_backward)."""
    N = K.shape[0]
    cand = _candidate_cols(N, rows, L, causal, block_mask, block_size)
    ok = allowed_matrix(N, causal, L, block_mask, block_size, rows=rows, cols=cand)
    keep = ok.any(axis=0)
    cols, ok = cand[keep], ok[:, keep]
    if cols.size == 0:  # no row of the chunk has a key: P = 0, LSE = -inf
        z = np.zeros((len(rows), 0))
        return cols, z, z, np.full(len(rows), -np.inf), np.zeros(len(rows))
    q = _f64(Q[rows])
    _, p, lse = head_probabilities(q, _f64(K[cols]), scale, ok)
    dp = _f64(dO[rows]) @ _f64(V[cols]).T
    dsum = (p * dp).sum(axis=1)
    return cols, p, dp, lse, dsum


def backward_rows(Q, K, V, dO, scale, b, h, rows, causal=False, key_len=None, block_mask=None,
                  block_size=None, chunk=256):
    """dQ of the given query rows of instance (b, h): dQ_i = scale * sum_j dS_ij K_j with
    dS_ij = P_ij (dP_ij - D_i); each row depends only on its own P and dP."""
    rows = np.asarray(rows)
    L = None if key_len is None else int(key_len[b])
    q_, k_, v_, do_ = Q[b, h], K[b, h], V[b, h], dO[b, h]
    dq = np.zeros((rows.size, Q.shape[-1]))
    for c0 in range(0, rows.size, chunk):
        r = rows[c0:c0 + chunk]
        cols, p, dp, _, dsum = _chunk_terms(q_, k_, v_, do_, scale, r, L, causal, block_mask, block_size)
        ds = p * (dp - dsum[:, None])
        dq[c0:c0 + chunk] = float(scale) * (ds @ _f64(k_[cols]))
    return dq


def backward_keys(Q, K, V, dO, scale, b, h, keys, causal=False, key_len=None, block_mask=None,
                  block_size=None, chunk=256):
    """dK and dV of the given keys of instance (b, h): dV_j = sum_i P_ij dO_i and
    dK_j = scale * sum_i dS_ij Q_i over every query row i, whose LSE and D come from the
    same chunked evaluation (rows that attend none of the keys are skipped)."""
    keys = np.asarray(keys)
    N, d = Q.shape[2], Q.shape[3]
    L = None if key_len is None else int(key_len[b])
    q_, k_, v_, do_ = Q[b, h], K[b, h], V[b, h], dO[b, h]
    sees = allowed_matrix(N, causal, L, block_mask, block_size, cols=keys)  # [N, len(keys)]
    dk = np.zeros((keys.size, d))
    dv = np.zeros((keys.size, d))
    for r0 in range(0, N, chunk):
        r = np.arange(r0, min(r0 + chunk, N))
        ok_k = sees[r]
        if not ok_k.any():
            continue
        cols, p, dp, lse, dsum = _chunk_terms(q_, k_, v_, do_, scale, r, L, causal, block_mask, block_size)
        # the chosen keys' columns of P and dP (zero where a key is not kept for a row)
        s_k = float(scale) * (_f64(q_[r]) @ _f64(k_[keys]).T)
        with np.errstate(invalid="ignore"):
            p_k = np.where(ok_k, np.exp(np.where(ok_k, s_k, 0.0) - np.where(lse == -np.inf, 0.0, lse)[:, None]),
                           0.0)
        dp_k = _f64(do_[r]) @ _f64(v_[keys]).T
        ds_k = p_k * (dp_k - dsum[:, None])
        dv += p_k.T @ _f64(do_[r])
        dk += float(scale) * (ds_k.T @ _f64(q_[r]))
    return dk, dv


def backward(Q, K, V, dO, scale, causal=False, key_len=None, block_mask=None, block_size=None,
             heads=None, dropout=None):
    """Exact gradients dQ, dK, dV [B, H, N, d] (float64) of <dO, O>.

    With `heads` only those instances are computed; the rest are NaN. `dropout` as in forward().
    """
    B, H, N, d = Q.shape
    dQ = np.full((B, H, N, d), np.nan)
    dK = np.full((B, H, N, d), np.nan)
    dV = np.full((B, H, N, d), np.nan)
    for b, h in _heads(B, H, heads):
        L = None if key_len is None else int(key_len[b])
        ok = allowed_matrix(N, causal, L, block_mask, block_size)
        keep, ks = _dropout_for(dropout, N, b * H + h)
        dQ[b, h], dK[b, h], dV[b, h], _ = head_backward(
            _f64(Q[b, h]), _f64(K[b, h]), _f64(V[b, h]), _f64(dO[b, h]), scale, ok, keep, ks)
    return dQ, dK, dV
