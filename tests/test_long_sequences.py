"""Parity at N = 65536 (long sequences, O(N) memory): dense causal and block-sparse.

The oracle cannot form the N x N matrices here, so outputs are compared on sampled
query rows (O, LSE, dQ) and sampled keys (dK, dV) through the oracle's chunked
evaluation, which only visits the keys each chunk of rows may attend. Causal keys are
sampled near the end of the sequence (few rows attend them, so the oracle stays
cheap); block-sparse keys come from four key blocks anywhere in the sequence.
"""
import numpy as np
import pytest

import oracle
import workloads
from helpers import TOL_GRAD_FRO, TOL_LSE_BF16, TOL_O_BF16, ensure_library, rel_fro, run_gpu

pytestmark = pytest.mark.gpu

N_LONG = 65536


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


@pytest.mark.parametrize("kind", ["causal", "block"])
def test_64k_sampled_rows_and_keys(kind):
    d = 64
    if kind == "causal":
        case = workloads.make_case(1, 1, N_LONG, d, mask="causal", seed=60, name="long-causal")
    else:
        case = workloads.make_case(1, 1, N_LONG, d, mask="block", block_size=256, seed=61, name="long-block")
    print("[case]", case.name, "N", N_LONG, "d", d, flush=True)
    gpu = run_gpu(case)
    kw = dict(causal=case.causal, key_len=case.key_len, block_mask=case.block_mask,
              block_size=case.block_size)
    rng = np.random.default_rng(62)
    rows = np.unique(np.concatenate([[0, 1, 2, 255, 256, N_LONG - 2, N_LONG - 1],
                                     rng.choice(N_LONG, 25, replace=False)]))
    o, lse = oracle.forward_rows(case.q, case.k, case.v, float(case.scale), 0, 0, rows, **kw)
    assert np.max(np.abs(gpu["o"][0, 0, rows] - o)) <= TOL_O_BF16
    assert np.max(np.abs(gpu["lse"][0, 0, rows] - lse)) <= TOL_LSE_BF16
    dq = oracle.backward_rows(case.q, case.k, case.v, case.do, float(case.scale), 0, 0, rows, **kw)
    assert rel_fro(gpu["dq"][0, 0, rows], dq) <= TOL_GRAD_FRO
    if kind == "causal":
        keys = np.unique(np.concatenate([[N_LONG - 1, N_LONG - 1024],
                                         N_LONG - 1024 + rng.choice(1024, 14, replace=False)]))
    else:
        blocks = rng.choice(N_LONG // 256, 4, replace=False)
        keys = np.concatenate([b * 256 + rng.choice(256, 4, replace=False) for b in blocks])
    dk, dv = oracle.backward_keys(case.q, case.k, case.v, case.do, float(case.scale), 0, 0, keys, **kw)
    assert rel_fro(gpu["dk"][0, 0, keys], dk) <= TOL_GRAD_FRO
    assert rel_fro(gpu["dv"][0, 0, keys], dv) <= TOL_GRAD_FRO


@pytest.mark.parametrize("mask", ["block", "block+causal"])
def test_largest_block_mask_sampled_rows_and_keys(mask):
    """N = 131072 with 128-blocks: a 1024 x 1024 block mask, the most the library takes, so each
    workgroup's list of kept blocks is built from 16 ballot rounds over its mask row or column."""
    n, d, bs = 131072, 64, 128
    case = workloads.make_case(1, 1, n, d, mask=mask, block_size=bs, block_p=1.0 / 64, seed=63,
                               name="max-blocks")
    print("[case]", case.name, mask, "N", n, "d", d, "bs", bs, flush=True)
    gpu = run_gpu(case)
    kw = dict(causal=case.causal, key_len=case.key_len, block_mask=case.block_mask, block_size=bs)
    rng = np.random.default_rng(64)
    rows = np.unique(np.concatenate([[0, 127, 128, n - 129, n - 1], rng.choice(n, 20, replace=False)]))
    o, lse = oracle.forward_rows(case.q, case.k, case.v, float(case.scale), 0, 0, rows, **kw)
    assert np.max(np.abs(gpu["o"][0, 0, rows] - o)) <= TOL_O_BF16
    assert np.max(np.abs(gpu["lse"][0, 0, rows] - lse)) <= TOL_LSE_BF16
    dq = oracle.backward_rows(case.q, case.k, case.v, case.do, float(case.scale), 0, 0, rows, **kw)
    assert rel_fro(gpu["dq"][0, 0, rows], dq) <= TOL_GRAD_FRO
    blocks = np.concatenate([[0, n // bs - 1], rng.choice(n // bs, 3, replace=False)])
    keys = np.unique(np.concatenate([b * bs + rng.choice(bs, 4, replace=False) for b in blocks]))
    dk, dv = oracle.backward_keys(case.q, case.k, case.v, case.do, float(case.scale), 0, 0, keys, **kw)
    assert rel_fro(gpu["dk"][0, 0, keys], dk) <= TOL_GRAD_FRO
    assert rel_fro(gpu["dv"][0, 0, keys], dv) <= TOL_GRAD_FRO
