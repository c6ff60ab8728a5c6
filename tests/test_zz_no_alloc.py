"""fa_bwd_noalloc (the backward whose workspace is the library's static per-device scratch)
against fa_bwd through the C ABI: bit-identical gradients, and the oracle's tolerances, on two
calls in a row where the second is smaller (the scratch keeps the first call's contents)."""
import numpy as np
import pytest

import workloads
from helpers import compare, ensure_library, run_oracle, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def _both(case):
    import torch
    import exact_attention_100_amd as fa
    t = upload(case)
    sc = float(case.scale)
    o, lse = fa.fwd(t["q"], t["k"], t["v"], scale=sc, causal=case.causal, key_len=t["key_len"])
    ref = fa.bwd(t["q"], t["k"], t["v"], o, t["do"], lse, scale=sc, causal=case.causal, key_len=t["key_len"])
    outs = tuple(torch.full_like(t["q"], float("nan")) for _ in range(3))
    got = fa.bwd_noalloc(t["q"], t["k"], t["v"], o, t["do"], lse, *outs, scale=sc, causal=case.causal,
                         key_len=t["key_len"])
    torch.cuda.synchronize()
    return o, lse, ref, got


def test_noalloc_backward_matches_fa_bwd_twice_second_smaller():
    first = workloads.make_case(2, 4, 1000, 128, mask="causal", seed=31, name="noalloc-1")
    second = workloads.make_case(1, 2, 300, 64, mask="key_len", seed=32, key_len_range=(1, 300),
                                 name="noalloc-2")
    for case in (first, second):
        print("[case]", case.name, "B,H,N,d", case.B, case.H, case.N, case.d, flush=True)
        o, lse, ref, got = _both(case)
        for a, b in zip(got, ref):
            assert bool((a == b).all()), "fa_bwd_noalloc differs from fa_bwd"
        gpu = {"o": o, "lse": lse, "dq": got[0], "dk": got[1], "dv": got[2]}
        gpu = {k: v.float().cpu().numpy().astype(np.float64) for k, v in gpu.items()}
        print("[case] errors", compare(gpu, run_oracle(case), case), flush=True)
