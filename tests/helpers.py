"""Shared helpers for the GPU tests: upload seeded cases, run the HIP path through
the C ABI binding, and compare with the float64 oracle."""
from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

# Tolerances: fp32 configs max |err| <= 1e-5 (O and LSE); bf16 configs max |err O| <= 2e-2 and
# relative Frobenius error of dQ, dK, dV <= 5e-2 over the compared tensor. Two internal checks on
# top of those bounds:
#  * bf16 LSE max |err| <= 1e-3: LSE is m + ln(l) with l the float32 row sum of the unrounded
#    exponentials, so only float32 and exp2 rounding remain;
#  * per 32-row slab of dQ, dK and dV (32 consecutive queries or keys of one instance; the last
#    slab of a ragged N is shorter), relative Frobenius error <= 5e-2 of max(|ref_slab|,
#    0.1 * RMS slab norm of the compared tensor). A missing or wrong slab scores about 1 and a
#    single zeroed row of typical size about 1/sqrt(32) = 0.18, so both fail even where the
#    whole-tensor norm would hide them. Slabs rather than single rows because D = rowsum(dO o O)
#    is formed from the stored bf16 O, whose rounding moves D by an amount that does not shrink
#    with the row's own gradient: rows whose exact gradient nearly cancels (causal row 0 of dQ
#    is exactly 0; a very peaked softmax) carry a relative error of 0.1-0.25 on their own, while
#    over a slab it averages against the neighbouring rows. The floor keeps slabs with a (near)
#    zero gradient (keys no query sees) from turning rounding into a large relative error.
TOL_F32 = 1e-5
TOL_O_BF16 = 2e-2
TOL_LSE_BF16 = 1e-3
TOL_GRAD_FRO = 5e-2
TOL_GRAD_SLAB = 5e-2
SLAB_FLOOR = 0.1
SLAB = 32


def ensure_library():
    from exact_attention_100_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from exact_attention_100_amd.build import build
        build()


def to_device(case: workloads.Case, name: str):
    import torch
    if case.dtype == workloads.BF16:
        bits = case.bits(name)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(getattr(case, name))).cuda()


def upload(case: workloads.Case):
    import torch
    t = {n: to_device(case, n) for n in ("q", "k", "v", "do")}
    t["key_len"] = None if case.key_len is None else torch.from_numpy(case.key_len).cuda()
    t["block_mask"] = None if case.block_mask is None else torch.from_numpy(case.block_mask).cuda()
    return t


def run_gpu(case: workloads.Case, backward: bool = True):
    """fwd (+ bwd) through the library; returns float64 numpy arrays."""
    import torch
    import exact_attention_100_amd as fa
    t = upload(case)
    sc = float(case.scale)
    if case.block_mask is not None:
        o, lse = fa.blocksparse_fwd(t["q"], t["k"], t["v"], t["block_mask"], case.block_size, scale=sc,
                                    causal=case.causal, key_len=t["key_len"])
    else:
        o, lse = fa.fwd(t["q"], t["k"], t["v"], scale=sc, causal=case.causal, key_len=t["key_len"])
    out = {"o": o, "lse": lse}
    if backward:
        if case.block_mask is not None:
            dq, dk, dv = fa.blocksparse_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, t["block_mask"],
                                            case.block_size, scale=sc, causal=case.causal,
                                            key_len=t["key_len"])
        else:
            dq, dk, dv = fa.bwd(t["q"], t["k"], t["v"], o, t["do"], lse, scale=sc, causal=case.causal,
                                key_len=t["key_len"])
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy().astype(np.float64) for k, v in out.items()}


def oracle_kwargs(case: workloads.Case):
    return dict(causal=case.causal, key_len=case.key_len, block_mask=case.block_mask,
                block_size=case.block_size)


def run_oracle(case: workloads.Case, backward: bool = True, heads=None, dropout=None):
    sc = float(case.scale)
    kw = oracle_kwargs(case)
    O, LSE = oracle.forward(case.q, case.k, case.v, sc, heads=heads, dropout=dropout, **kw)
    out = {"o": O, "lse": LSE}
    if backward:
        dQ, dK, dV = oracle.backward(case.q, case.k, case.v, case.do, sc, heads=heads, dropout=dropout, **kw)
        out.update(dq=dQ, dk=dK, dv=dV)
    return out


def rel_fro(a, ref):
    den = np.linalg.norm(ref)
    return np.linalg.norm(a - ref) / (den if den > 0 else 1.0)


def slab_errors(g, r, slab: int = SLAB):
    """Relative Frobenius error of each run of `slab` consecutive rows of a [..., N, d] gradient,
    per instance: |g_slab - r_slab| / max(|r_slab|, SLAB_FLOOR * RMS slab norm)."""
    N, d = g.shape[-2], g.shape[-1]
    g3 = g.reshape(-1, N, d)
    r3 = r.reshape(-1, N, d)
    err, ref = [], []
    for s0 in range(0, N, slab):
        err.append(np.linalg.norm((g3[:, s0:s0 + slab] - r3[:, s0:s0 + slab]).reshape(g3.shape[0], -1), axis=1))
        ref.append(np.linalg.norm(r3[:, s0:s0 + slab].reshape(r3.shape[0], -1), axis=1))
    err, ref = np.stack(err, axis=1), np.stack(ref, axis=1)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    den = np.maximum(ref, SLAB_FLOOR * rms)
    return np.where(den > 0, err / np.where(den > 0, den, 1.0), err)


def compare(gpu, ref, case: workloads.Case, heads=None, backward=True):
    """Assert the tolerances; returns a dict of the measured errors."""
    sel = (slice(None),) if heads is None else (tuple(h[0] for h in heads), tuple(h[1] for h in heads))
    errs = {}
    for name in ("o", "lse") + (("dq", "dk", "dv") if backward else ()):
        g, r = gpu[name][sel], ref[name][sel]
        assert np.all(np.isfinite(g) | (np.isneginf(g) & np.isneginf(r))), f"{name}: non-finite output"
    g_lse, r_lse = gpu["lse"][sel], ref["lse"][sel]
    assert np.array_equal(np.isneginf(g_lse), np.isneginf(r_lse)), "rows without keys differ"
    fin = np.isfinite(r_lse)
    errs["o"] = float(np.max(np.abs(gpu["o"][sel] - ref["o"][sel]))) if gpu["o"][sel].size else 0.0
    errs["lse"] = float(np.max(np.abs(g_lse[fin] - r_lse[fin]))) if fin.any() else 0.0
    if case.dtype == workloads.F32:
        assert errs["o"] <= TOL_F32, errs
        assert errs["lse"] <= TOL_F32, errs
    else:
        assert errs["o"] <= TOL_O_BF16, errs
        assert errs["lse"] <= TOL_LSE_BF16, errs
    if backward:
        for name in ("dq", "dk", "dv"):
            errs[name] = float(rel_fro(gpu[name][sel], ref[name][sel]))
            se = slab_errors(gpu[name][sel], ref[name][sel])
            errs[name + "_slab"] = float(se.max()) if se.size else 0.0
        for name in ("dq", "dk", "dv"):
            assert errs[name] <= TOL_GRAD_FRO, errs
            assert errs[name + "_slab"] <= TOL_GRAD_SLAB, errs
    return errs
