"""Parity at N = 65536 (long sequences, O(N) memory): dense causal and block-sparse.

The oracle cannot form the N x N matrices here, so outputs are compared on sampled
32-row slabs of queries (O, LSE, dQ) and 32-key slabs (dK, dV) through the oracle's
chunked evaluation, which only visits the keys each chunk of rows may attend. Causal
keys are sampled near the end of the sequence (few rows attend them, so the oracle
stays cheap); block-sparse keys come from slabs of four key blocks anywhere in the
sequence. Gradients are checked over all sampled slabs (relative Frobenius error) and
slab by slab (helpers.slab_errors).
"""
import numpy as np
import pytest

import oracle
import workloads
from helpers import (SLAB, TOL_GRAD_FRO, TOL_GRAD_SLAB, TOL_LSE_BF16, TOL_O_BF16, ensure_library, rel_fro,
                     run_gpu, slab_errors)

pytestmark = pytest.mark.gpu

N_LONG = 65536


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def _slabs(starts):
    """Rows of the 32-row slabs that start at `starts` (multiples of 32), in increasing order."""
    starts = np.unique(np.asarray(starts, dtype=np.int64))
    assert np.all(starts % SLAB == 0)
    return (starts[:, None] + np.arange(SLAB)[None, :]).ravel()


def _check_grads(gpu_rows, ref_rows):
    """Sampled slabs laid end to end: the whole-sample bound, then each slab."""
    assert rel_fro(gpu_rows, ref_rows) <= TOL_GRAD_FRO
    worst = slab_errors(gpu_rows[None], ref_rows[None]).max()
    assert worst <= TOL_GRAD_SLAB, worst
    return float(worst)


def _compare_sampled(case, gpu, rows, keys, kw):
    o, lse = oracle.forward_rows(case.q, case.k, case.v, float(case.scale), 0, 0, rows, **kw)
    assert np.max(np.abs(gpu["o"][0, 0, rows] - o)) <= TOL_O_BF16
    assert np.max(np.abs(gpu["lse"][0, 0, rows] - lse)) <= TOL_LSE_BF16
    dq = oracle.backward_rows(case.q, case.k, case.v, case.do, float(case.scale), 0, 0, rows, **kw)
    e_dq = _check_grads(gpu["dq"][0, 0, rows], dq)
    dk, dv = oracle.backward_keys(case.q, case.k, case.v, case.do, float(case.scale), 0, 0, keys, **kw)
    e_dk = _check_grads(gpu["dk"][0, 0, keys], dk)
    e_dv = _check_grads(gpu["dv"][0, 0, keys], dv)
    print("[case] worst slab errors dq, dk, dv", e_dq, e_dk, e_dv, flush=True)


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
    rows = _slabs(np.concatenate([[0, 256, N_LONG - SLAB], SLAB * rng.choice(N_LONG // SLAB, 3, replace=False)]))
    if kind == "causal":
        keys = _slabs([N_LONG - SLAB, N_LONG - 1024])
    else:
        blocks = rng.choice(N_LONG // 256, 4, replace=False)
        keys = _slabs(blocks * 256 + SLAB * rng.integers(0, 256 // SLAB, size=4))
    _compare_sampled(case, gpu, rows, keys, kw)


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
    rows = _slabs(np.concatenate([[0, 96, 128, n - 160, n - SLAB], SLAB * rng.choice(n // SLAB, 3, replace=False)]))
    blocks = np.concatenate([[0, n // bs - 1], rng.choice(n // bs, 3, replace=False)])
    keys = _slabs(blocks * bs + SLAB * rng.integers(0, bs // SLAB, size=blocks.size))
    _compare_sampled(case, gpu, rows, keys, kw)
