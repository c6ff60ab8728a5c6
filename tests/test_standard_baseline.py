"""The standard-attention baseline that the memory / runtime sweep measures this path against
(bench.standard_attention_step: separate torch ops that materialise S and P in HBM, the pages'
comparison point in Experiments > 4.4) computes attention and its gradients: checked against the
float64 oracle with the bf16 tolerances, with key padding and with dropout (keep bits from the
oracle's generator, so both sides drop the same pairs)."""
import numpy as np
import pytest

import oracle
import workloads
from bench import standard_attention_step
from helpers import compare, ensure_library, run_oracle, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


@pytest.mark.parametrize("mask", ["none", "causal", "key_len", "causal+key_len"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("p8", [0, 26])
def test_standard_attention_baseline_matches_oracle(mask, d, p8):
    import torch
    case = workloads.make_case(2, 2, 256, d, mask=mask, seed=140 + d, key_len_range=(1, 256),
                               name=f"standard-{mask}")
    print("[case]", case.name, "d", d, "p8", p8, flush=True)
    t = upload(case)
    keep = None
    drop = None
    if p8:
        drop = (p8, 99, 5)
        bits = np.stack([np.stack([oracle.dropout_keep(np.arange(case.N), np.arange(case.N), b * case.H + h, *drop)
                                   for h in range(case.H)]) for b in range(case.B)])
        keep = torch.from_numpy(bits).cuda()
    o, dq, dk, dv = standard_attention_step(t["q"], t["k"], t["v"], t["do"], float(case.scale), case.causal,
                                            key_len=t["key_len"], dropout_p=p8 / 256.0, keep=keep)
    torch.cuda.synchronize()
    ref = run_oracle(case, dropout=drop)
    gpu = {k: v.float().cpu().numpy().astype(np.float64) for k, v in dict(o=o, dq=dq, dk=dk, dv=dv).items()}
    gpu["lse"] = ref["lse"]  # (the baseline keeps no statistic)
    print("[case] errors", compare(gpu, ref, case), flush=True)
