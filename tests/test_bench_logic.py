"""Host-side logic of bench.py (no GPU): the kept-pair count that turns times into FLOP/s."""
import numpy as np
import pytest

import oracle
import workloads
from bench import kept_pairs


@pytest.mark.parametrize("mask,kl", [("none", None), ("causal", None), ("key_len", (1, 300)),
                                     ("causal+key_len", (0, 300)), ("block", None),
                                     ("block+causal", None), ("block+key_len", (50, 300)),
                                     ("block+causal+key_len", (0, 299))])
def test_kept_pairs_equals_brute_force(mask, kl):
    case = workloads.make_case(3, 2, 256, 16, mask=mask, block_size=64 if "block" in mask else None,
                               block_p=0.5, key_len_range=kl, seed=9)
    ref = 0
    for b in range(case.B):
        L = None if case.key_len is None else int(case.key_len[b])
        ref += int(oracle.allowed_matrix(case.N, case.causal, L, case.block_mask, case.block_size).sum())
    assert kept_pairs(case) == ref * case.H


def test_kept_pairs_of_the_named_causal_workloads():
    # N (N + 1) / 2 per instance for the causal configurations
    for name in ("C3", "C4a", "C4b"):
        c = workloads.CONFIGS[name]
        case = workloads.Case(name=name, B=c["B"], H=c["H"], N=c["N"], d=c["d"], dtype=c["dtype"], causal=True,
                              scale=np.float32(1), q=None, k=None, v=None, do=None)
        assert kept_pairs(case) == c["B"] * c["H"] * c["N"] * (c["N"] + 1) // 2


def test_run_parity_check_flags_a_wrong_slab():
    """The bench's parity of the benched run: exact outputs pass, a zeroed 32-row slab of dK fails."""
    from bench import _parity_of
    rng = np.random.default_rng(3)
    B, H, N, d = 1, 2, 96, 8
    ref = {n: rng.standard_normal((B, H, N, d)) for n in ("o", "dq", "dk", "dv")}
    ref["lse"] = rng.standard_normal((B, H, N))
    gpu = {n: ref[n][0, 1].copy() for n in ref}
    e = _parity_of(gpu, ref, (0, 1))
    assert e["within_tolerance"] and e["o_max_abs"] == 0.0 and e["dk_worst_slab"] == 0.0
    gpu["dk"][32:64] = 0.0
    e = _parity_of(gpu, ref, (0, 1))
    assert not e["within_tolerance"] and e["dk_worst_slab"] > 0.9 and e["dk_rel_fro"] < 0.7
