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
