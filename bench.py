"""Benchmark: exact attention forward + backward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C4b]

One step = one fa_fwd + one fa_bwd (every kernel of the hot path) over one batch
of seeded synthetic bf16 inputs already resident in HBM. Prints one JSON line.

value    = whole-job algorithmic TFLOP/s = 14 d (kept query/key pairs) / step time
           (forward 4 d per pair: Q K^T and P V; backward 10 d: the Q K^T recompute,
           P^T dO, dO V^T, dS^T Q and dS K).
           Timed over K steps with no instrumentation between the kernels (warm: the
           inputs stay in L2 / MALL between steps). "cold" repeats the K steps, each
           after a 512 MiB write that evicts L2 and the 256 MiB MALL (median step).
roofline = the dominant kernel's algorithmic FLOP per launch / its mean launch time,
           against the bf16 MFMA peak. Launch times come from HIP events that the
           library records around each launch on the launch stream, over a second
           pass of K steps right after the first (events between kernels delay the
           next launch by a few microseconds each, so they stay out of the step time).
cpu_baseline = the float64 CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU
KERNEL_SOURCES = ["exact_attention_100_amd/csrc/fa_fwd.hip", "exact_attention_100_amd/csrc/fa_bwd.hip",
                  "exact_attention_100_amd/csrc/fa_common.hpp"]


def kept_pairs(case) -> int:
    """Number of (query, key) pairs the masks keep, summed over all instances."""
    import numpy as np
    B, H, N = case.B, case.H, case.N
    i = np.arange(N, dtype=np.int64)
    total = 0
    for b in range(B):
        L = N if case.key_len is None else int(min(max(case.key_len[b], 0), N))
        if case.block_mask is None:
            hi = np.full(N, L, dtype=np.int64)
            if case.causal:
                hi = np.minimum(hi, i + 1)  # row i keeps keys j < min(i + 1, L)
            total += int(hi.sum())
            continue
        bs = case.block_size
        for rb, cb in zip(*np.nonzero(case.block_mask)):
            rows = i[rb * bs:(rb + 1) * bs]
            hi = np.full(bs, min(cb * bs + bs, L), dtype=np.int64)
            if case.causal:
                hi = np.minimum(hi, rows + 1)
            total += int(np.maximum(hi - cb * bs, 0).sum())  # keys cb*bs <= j < hi of each row
    return total * H


def device_peak_bf16_tflops():
    """Dense bf16 MFMA peak implied by the device's own report: peak engine clock x CUs x 4096
    flop per clock per CU (None if the runtime does not report it)."""
    import ctypes
    import torch
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        khz = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, 0) != 0:  # hipDeviceAttributeClockRate (kHz)
            return None
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        return round(khz.value * 1e3 * cus * 4096 / 1e12, 1)
    except OSError:
        return None


def sources_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic_record(workload: str):
    """The committed rocprofv3 HBM-counter digest of a workload, if taken on the current sources."""
    path = os.path.join(ROOT, "profiles", f"attention_kernels_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        text = fh.read()
    rec = json.loads(text[text.index("{"):])  # the JSON follows a short header
    return rec if rec.get("sources_hash") == sources_hash() else None


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters, if taken on the current sources."""
    rec = _traffic_record(workload)
    k = None if rec is None else rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def _sq_record(workload: str):
    """The committed rocprofv3 SQ-counter digest of a workload, if taken on the current sources."""
    path = os.path.join(ROOT, "profiles", f"attention_kernels_{workload}_sq_counters.txt")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        text = fh.read()
    if "{" not in text:
        return None
    rec = json.loads(text[text.index("{"):])
    return rec if rec.get("sources_hash") == sources_hash() else None


def counter_source(kind: str, workload: str, rec) -> str:
    return (f"profiles/attention_kernels_{workload}_{kind}.txt: rocprofv3 counters from a separate run of the "
            f"same command on one MI355X (not this run's box), kernel sources_hash {rec['sources_hash']}")


# The two SQ counter sets (one rocprofv3 --pmc run each: at most 8 SQ and 2 GRBM counters per run).
SQ_SETS = (["SQ_WAVE_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
            "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_LDS_BANK_CONFLICT"],
           ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM", "SQ_ACTIVE_INST_VALU",
            "SQ_ACTIVE_INST_LDS", "GRBM_GUI_ACTIVE"])


def sq_digest(p1: str, p2: str, workload: str):
    """Per-kernel SQ counter summary from two rocprofv3 --pmc csv runs (SQ_SETS): the matrix cores'
    busy fraction, where the waves' time goes, and instructions per MFMA. Returns (record, text)."""
    import csv
    import glob
    import re
    vals, clocks = {}, {}
    for d in (p1, p2):
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for row in csv.DictReader(fh):
                    k = re.sub(r"^void fa::", "", row["Kernel_Name"])
                    k = k.replace("(fa::FwdKParams)", "").replace("(fa::BwdKParams)", "")
                    vals.setdefault(k, {}).setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
                    dur = int(row.get("End_Timestamp") or 0) - int(row.get("Start_Timestamp") or 0)
                    if row["Counter_Name"] == "GRBM_GUI_ACTIVE" and dur > 0:
                        # engine cycles per XCD over the dispatch's nanoseconds: the clock it ran at
                        clocks.setdefault(k, []).append(float(row["Counter_Value"]) / 8 / dur * 1e3)
    out = {"workload": workload, "sources_hash": sources_hash(), "kernels": {}}
    lines = []
    for k, cs in vals.items():
        name = next((v for frag, v in KERNEL_NAMES.items() if frag in k), None)
        if name is None:
            continue
        m = {c: sum(v) / len(v) for c, v in cs.items()}
        busy = (m["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024) / (m["GRBM_GUI_ACTIVE"] / 8)
        w, mf = m["SQ_WAVE_CYCLES"], m["SQ_INSTS_MFMA"]
        rec = {"symbol": k, "mfma_busy": round(busy, 3), "issuing": round(m["SQ_ACTIVE_INST_ANY"] / w, 3),
               "waiting": round(m["SQ_WAIT_ANY"] / w, 3), "issue_stalled": round(m["SQ_WAIT_INST_ANY"] / w, 3),
               "valu_per_mfma": round((m["SQ_INSTS_VALU"] - mf) / mf, 2), "lds_per_mfma": round(m["SQ_INSTS_LDS"] / mf, 2),
               "salu_per_mfma": round(m["SQ_INSTS_SALU"] / mf, 2), "lds_bank_conflicts": m["SQ_LDS_BANK_CONFLICT"]}
        if clocks.get(k):
            ck = sorted(clocks[k])
            rec["engine_clock_mhz"] = round(ck[len(ck) // 2])
        out["kernels"][name] = rec
        lines += [k, "  " + "  ".join(f"{c}={m[c]:.4g}" for c in sorted(m)),
                  f"  mfma_busy {busy:.3f}; wave time: issuing {rec['issuing']:.2f}, waiting {rec['waiting']:.2f}, "
                  f"issue-stalled {rec['issue_stalled']:.2f}; per MFMA: {rec['valu_per_mfma']:.2f} other VALU, "
                  f"{rec['lds_per_mfma']:.2f} LDS, {rec['salu_per_mfma']:.2f} SALU; LDS bank conflicts "
                  f"{m['SQ_LDS_BANK_CONFLICT']:.0f}"
                  + (f"; engine clock {rec['engine_clock_mhz']} MHz (median over dispatches of GRBM_GUI_ACTIVE / 8 "
                     f"over the dispatch's duration)" if "engine_clock_mhz" in rec else ""), ""]
    return out, "\n".join(lines)


# LDS counters (one rocprofv3 --pmc run): latency, bytes delivered, FIFO stalls, MFMA / VALU co-execution.
LDS_SET = ["LdsLatency", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_CMD_FIFO_FULL", "SQ_LDS_DATA_FIFO_FULL",
           "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_LDS_LOAD_BANDWIDTH", "GRBM_GUI_ACTIVE"]


def digest_lds(p: str, workload: str):
    """Per-kernel LDS summary of one rocprofv3 --pmc csv run over LDS_SET: the mean LDS latency, the LDS bytes
    loaded per compute-unit cycle (SQ_INSTS_LDS_LOAD_BANDWIDTH counts 64-byte units over the 256 CUs), the share
    of CU cycles with the LDS command FIFO full, the share of SIMD cycles in which a VALU instruction issued while
    the matrix core was busy, and the engine clock (GRBM_GUI_ACTIVE / 8 over the dispatch's duration)."""
    import csv
    import glob
    import re
    vals, durs = {}, {}
    for f in glob.glob(os.path.join(p, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                k = re.sub(r"^void fa::", "", row["Kernel_Name"]).split("(")[0]
                vals.setdefault(k, {}).setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
                if row["Counter_Name"] == "GRBM_GUI_ACTIVE":
                    durs.setdefault(k, []).append(int(row["End_Timestamp"]) - int(row["Start_Timestamp"]))
    print(f"workload {workload}, kernel sources_hash {sources_hash()}")
    for k, cs in vals.items():
        if not any(frag in k for frag in KERNEL_NAMES):
            continue
        m = {c: sum(v) / len(v) for c, v in cs.items()}
        cyc = m["GRBM_GUI_ACTIVE"] / 8  # engine cycles per XCD
        print(k, f"({len(durs.get(k, []))} dispatches)")
        print("  " + "  ".join(f"{c}={m[c]:.4g}" for c in sorted(m)))
        print(f"  LDS latency {m['LdsLatency']:.1f} cycles; LDS bytes loaded per CU-cycle "
              f"{m['SQ_INSTS_LDS_LOAD_BANDWIDTH'] * 64 / 256 / cyc:.1f}; LDS command FIFO full "
              f"{100 * m['SQ_LDS_CMD_FIFO_FULL'] / 256 / cyc:.2f}% of CU-cycles; VALU issued beside a busy matrix "
              f"core {100 * m['SQ_VALU_MFMA_COEXEC_CYCLES'] / 1024 / cyc:.1f}% of SIMD-cycles; engine clock "
              f"{cyc / (sum(durs[k]) / len(durs[k])) * 1e3:.0f} MHz", flush=True)


def digest_sq(p1: str, p2: str, workload: str):
    """Prints sq_digest's text and the JSON that bench.py reads from profiles/."""
    rec, text = sq_digest(p1, p2, workload)
    print(text, flush=True)
    print(json.dumps(rec, indent=1), flush=True)


def step_traffic_for(workload: str):
    """Measured HBM bytes of a whole step against the algorithmic bytes and the standard-attention
    byte model, from the same digest (None if absent or stale)."""
    rec = _traffic_record(workload)
    return None if rec is None else rec.get("step")


# Library timer names of the kernels, by a fragment of their symbol.
KERNEL_NAMES = {"fwd_bf16_kernel": "fa_fwd_bf16", "fwd_pp_kernel": "fa_fwd_bf16", "fwd_f32_kernel": "fa_fwd_f32",
                "bwd_dkdv_kernel": "fa_bwd_dkdv", "bwd_dkdv_pp_kernel": "fa_bwd_dkdv",
                "bwd_dq_kernel": "fa_bwd_dq", "bwd_dq_pp_kernel": "fa_bwd_dq"}


def calibrate_copy(nbytes: int = 1 << 30, launches: int = 3):
    """A plain device-to-device copy of known size, run under rocprofv3 --pmc to scale
    FETCH_SIZE / WRITE_SIZE into bytes."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(launches):
        torch.mul(src, 1.0, out=dst)  # one elementwise kernel: reads and writes nbytes
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": launches}), flush=True)


def _counter_means(d: str, counter: str):
    """Mean counter value per dispatch, by kernel symbol, from a rocprofv3 --output-format csv run."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] != counter:
                    continue
                vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def traffic_digest(fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str, workload: str):
    """Per-kernel HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (KiB) runs, each scaled by what the
    counter reads for the calibration copy of known size; the step's sum against the algorithmic bytes and
    the standard-attention byte model."""
    import workloads
    c = workloads.CONFIGS[workload]
    cf, cw = _counter_means(copy_fetch_dir, "FETCH_SIZE"), _counter_means(copy_write_dir, "WRITE_SIZE")
    # the calibration copy is the dispatch with the largest traffic in its run
    copy_bytes = 1 << 30
    kf = copy_bytes / (max(cf.values()) * 1024.0)
    kw = copy_bytes / (max(cw.values()) * 1024.0)
    fetch, write = _counter_means(fetch_dir, "FETCH_SIZE"), _counter_means(write_dir, "WRITE_SIZE")
    e = 2
    B, H, N, d = c["B"], c["H"], c["N"], c["d"]
    rows = B * H * N
    algo = {"fa_fwd_bf16": 4 * rows * d * e + 4 * rows, "fa_bwd_dkdv": 6 * rows * d * e + 8 * rows,
            "fa_bwd_dq": 6 * rows * d * e + 12 * rows}
    kernels = {}
    for sym, kib in fetch.items():
        name = next((v for k, v in KERNEL_NAMES.items() if k in sym), None)
        if name is None:
            continue
        wkib = next((w for s2, w in write.items() if s2 == sym), 0.0)
        rd, wr = kib * 1024.0 * kf, wkib * 1024.0 * kw
        kernels[name] = {"symbol": sym, "fetch_kib": round(kib, 1), "write_kib": round(wkib, 1),
                         "hbm_read_bytes": round(rd), "hbm_write_bytes": round(wr),
                         "hbm_bytes_per_launch": round(rd + wr), "algorithmic_bytes": algo.get(name),
                         "ratio_to_algorithmic": round((rd + wr) / algo[name], 3) if name in algo else None}
    # Standard attention's HBM bytes for the same step: the three-op implementation with S, P (and dP, dS)
    # written and read back at e bytes, fwd (4 N d + 4 N^2) e and bwd (8 N d + 7 N^2) e per head.
    standard = B * H * (12 * N * d + 11 * N * N) * e
    measured = sum(k["hbm_bytes_per_launch"] for k in kernels.values())
    algorithmic = sum(v for v in algo.values())
    out = {"workload": workload, "sources_hash": sources_hash(),
           "calibration": {"copy_bytes": copy_bytes, "fetch_scale": round(kf, 4), "write_scale": round(kw, 4)},
           "kernels": kernels,
           "step": {"hbm_bytes_measured": round(measured), "algorithmic_bytes": algorithmic,
                    "standard_attention_model_bytes": standard,
                    "standard_over_measured": round(standard / measured, 2)}}
    return out


def digest_counters(fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str, workload: str):
    """Prints traffic_digest's JSON (the form bench.py reads from profiles/)."""
    print(json.dumps(traffic_digest(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, workload), indent=1),
          flush=True)


def _rocprofv3():
    import shutil
    for cand in ("/opt/rocm/bin/rocprofv3", shutil.which("rocprofv3")):
        if cand and os.path.exists(cand):
            return cand
    return None


def _profile_child(prof: str, counters, out_dir: str, args, timeout_s: float) -> bool:
    """One rocprofv3 --pmc pass (its own child process, killed with its process group past
    timeout_s) over `python3 bench.py <args>`; True if it left a counter csv. rocprofv3 can end
    with a segmentation fault after the program has finished: the csv decides, not the status."""
    import glob
    import signal
    import subprocess
    cmd = [prof, "--pmc", *counters, "-d", out_dir, "-o", "p", "--output-format", "csv", "--",
           sys.executable, os.path.join(ROOT, "bench.py"), *args]
    env = dict(os.environ, TMPDIR=os.environ.get("TMPDIR", "/tmp"))
    p = subprocess.Popen(cmd, cwd=ROOT, env=env, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL,
                         start_new_session=True)
    try:
        p.wait(timeout=timeout_s)
    except subprocess.TimeoutExpired:
        os.killpg(p.pid, signal.SIGKILL)
        p.wait()
        return False
    return bool(glob.glob(os.path.join(out_dir, "**", "*counter_collection.csv"), recursive=True))


def measure_counters(workload: str, lib, timeout_s: float = 240.0):
    """HBM traffic and SQ counters of this workload measured now, on this machine: rocprofv3 --pmc passes
    (FETCH_SIZE, WRITE_SIZE, the two SQ sets, and FETCH_SIZE / WRITE_SIZE of the 1 GiB calibration copy),
    each over a 2-step run of this bench command in a child process. Returns (traffic, sq); either is
    None if its passes failed."""
    import tempfile
    prof = _rocprofv3()
    if prof is None:
        return None, None
    base = ["--workload", workload, "--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--counters", "off"]
    if lib:
        base += ["--lib", lib]
    tmp = tempfile.mkdtemp(prefix="fa_counters_")
    d = {k: os.path.join(tmp, k) for k in ("fetch", "write", "cfetch", "cwrite", "sq1", "sq2")}
    ok = {}
    for key, counters, args in (("fetch", ["FETCH_SIZE"], base), ("write", ["WRITE_SIZE"], base),
                                ("cfetch", ["FETCH_SIZE"], ["--calibrate-copy"]),
                                ("cwrite", ["WRITE_SIZE"], ["--calibrate-copy"]),
                                ("sq1", SQ_SETS[0], base), ("sq2", SQ_SETS[1], base)):
        print(f"bench.py: counter pass {key}", file=sys.stderr, flush=True)
        ok[key] = _profile_child(prof, counters, d[key], args, timeout_s)
    traffic = sq = None
    try:
        if all(ok[k] for k in ("fetch", "write", "cfetch", "cwrite")):
            traffic = traffic_digest(d["fetch"], d["write"], d["cfetch"], d["cwrite"], workload)
    except (KeyError, ValueError, ZeroDivisionError):
        traffic = None
    try:
        if ok["sq1"] and ok["sq2"]:
            sq = sq_digest(d["sq1"], d["sq2"], workload)[0]
    except (KeyError, ValueError, ZeroDivisionError):
        sq = None
    return traffic, sq


def _parity_of(gpu, ref, bh):
    """Errors of one instance's GPU outputs against the oracle's (host arithmetic only), with the bf16
    bounds: O max abs <= 2e-2, dQ / dK / dV relative Frobenius <= 5e-2 (also per 32-row slab of
    max(|slab|, 0.1 RMS slab norm)); LSE max abs <= 1e-3 as an internal check."""
    import numpy as np
    b, h = bh
    e = {}
    fin = np.isfinite(ref["lse"][b, h])
    e["o_max_abs"] = float(np.max(np.abs(gpu["o"] - ref["o"][b, h])))
    e["lse_max_abs"] = float(np.max(np.abs(gpu["lse"][fin] - ref["lse"][b, h][fin]))) if fin.any() else 0.0
    ok = e["o_max_abs"] <= 2e-2 and e["lse_max_abs"] <= 1e-3
    for n in ("dq", "dk", "dv"):
        g, r = gpu[n], ref[n][b, h]
        e[n + "_rel_fro"] = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
        nslab = (r.shape[0] + 31) // 32
        err = np.array([np.linalg.norm(g[32 * i:32 * i + 32] - r[32 * i:32 * i + 32]) for i in range(nslab)])
        ref_n = np.array([np.linalg.norm(r[32 * i:32 * i + 32]) for i in range(nslab)])
        den = np.maximum(ref_n, 0.1 * np.sqrt(np.mean(ref_n ** 2)))
        e[n + "_worst_slab"] = float(np.max(err / np.where(den > 0, den, 1.0)))
        ok = ok and e[n + "_rel_fro"] <= 5e-2 and e[n + "_worst_slab"] <= 5e-2
    e["within_tolerance"] = bool(ok and np.all(np.isfinite(gpu["o"])))
    return e


def cpu_baseline(case, budget_s: float, gpu_instance=None):
    """Time the float64 oracle (fwd + bwd) on whole heads of the workload until the budget is used.
    gpu_instance(b, h) -> the benched step's outputs of that instance (host arrays o, lse, dq, dk, dv):
    the oracle's outputs of the first timed instance are checked against them (parity of the run)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    # the first and the last instance of the launch first, then the rest in order
    n_inst = case.B * case.H
    order = [0, n_inst - 1] + list(range(1, n_inst - 1)) if n_inst > 1 else [0]
    heads = [(i // case.H, i % case.H) for i in order]
    done, parity = [], []
    t0 = time.perf_counter()
    for bh in heads:
        kw = dict(causal=case.causal, key_len=case.key_len, block_mask=case.block_mask, block_size=case.block_size,
                  heads=[bh])
        O, LSE = oracle.forward(case.q, case.k, case.v, float(case.scale), **kw)
        dQ, dK, dV = oracle.backward(case.q, case.k, case.v, case.do, float(case.scale), **kw)
        done.append(bh)
        if gpu_instance is not None and len(parity) < 2:
            el_ = time.perf_counter()
            ref = {"o": O, "lse": LSE, "dq": dQ, "dk": dK, "dv": dV}
            parity.append({"instance": list(bh), **_parity_of(gpu_instance(*bh), ref, bh)})
            t0 += time.perf_counter() - el_  # (the comparison is not oracle time)
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    flops = 14 * case.d * kept_pairs(case) * len(done) / (case.B * case.H)
    out = {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
           "sample": f"float64 fwd+bwd of {len(done)} of {case.B * case.H} (batch, head) instances "
                     f"at full N={case.N}, d={case.d}; {el:.1f} s wall"}
    return out, parity


def cpu_table(budget_s: float):
    """The float64 oracle per workload: forward and forward + backward wall time on whole heads (heads taken
    across batches first, until the budget is used), extrapolated to all heads by head count. One JSON line
    per workload."""
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    for name in ("C1", "C2", "C3", "C4a", "C4b", "C5"):
        case = workloads.make_config(name)
        heads = [(b, h) for h in range(case.H) for b in range(case.B)]
        kw = dict(causal=case.causal, key_len=case.key_len, block_mask=case.block_mask,
                  block_size=case.block_size)
        fwd_only = workloads.CONFIGS[name].get("fwd_only", False)
        timed = {}
        for leg in (("fwd",) if fwd_only else ("fwd", "fwd+bwd")):
            n, t0 = 0, time.perf_counter()
            for bh in heads:
                oracle.forward(case.q, case.k, case.v, float(case.scale), heads=[bh], **kw)
                if leg == "fwd+bwd":
                    oracle.backward(case.q, case.k, case.v, case.do, float(case.scale), heads=[bh], **kw)
                n += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
            timed[leg] = ((time.perf_counter() - t0) / n * len(heads), n)
        pairs = kept_pairs(case)
        row = {"workload": name, "heads": len(heads), "cores": int(threads),
               "fwd_s": round(timed["fwd"][0], 3), "fwd_heads_timed": timed["fwd"][1],
               "fwd_gflops": round(4 * case.d * pairs / timed["fwd"][0] / 1e9, 2)}
        if "fwd+bwd" in timed:
            row.update({"step_s": round(timed["fwd+bwd"][0], 3), "step_heads_timed": timed["fwd+bwd"][1],
                        "step_gflops": round(14 * case.d * pairs / timed["fwd+bwd"][0] / 1e9, 2)})
        print(json.dumps(row), flush=True)


def standard_attention_step(q, k, v, do, scale: float, causal: bool, key_len=None, dropout_p: float = 0.0,
                            keep=None):
    """The pages' baseline for the memory / runtime comparison, not part of the path:
    standard attention as separate framework ops that materialise S and P in HBM
    (FlashAttention reading notes, Background > Standard Attention Implementation),
    forward and the analytic backward, bf16 with float32 accumulation inside each
    product. Every transposed operand is made contiguous before its product.

    key_len (int32 [B] on the device): keys j >= key_len[b] are masked. Dropout on P
    (the notes' fused steps, Algorithm > Kernel Fusion) with drop probability dropout_p: the
    keep bits are `keep` (bool [B, H, N, N]) when given, else drawn by torch; survivors are
    scaled by 1 / (1 - dropout_p)."""
    import torch
    n = q.shape[-2]
    kt = k.transpose(-1, -2).contiguous()
    s = torch.matmul(q, kt).mul_(scale)
    if causal:
        s.masked_fill_(torch.ones(n, n, dtype=torch.bool, device=q.device).triu_(1), float("-inf"))
    if key_len is not None:
        cols = torch.arange(n, device=q.device)
        s.masked_fill_((cols[None, :] >= key_len[:, None].long())[:, None, None, :], float("-inf"))
    p = torch.softmax(s, dim=-1)
    del s
    if keep is None and dropout_p > 0.0:
        keep = torch.empty(p.shape, dtype=torch.bool, device=q.device).bernoulli_(1.0 - dropout_p)
    ks = 1.0 / (1.0 - dropout_p)
    pd = p if keep is None else p * keep * ks
    o = torch.matmul(pd, v)
    pt = pd.transpose(-1, -2).contiguous()
    dv = torch.matmul(pt, do)
    del pt, pd  # (pd may be p itself: only the name goes)
    vt = v.transpose(-1, -2).contiguous()
    ds = torch.matmul(do, vt)  # dP, turned into dS = P (dP - D) in place
    if keep is not None:
        ds.mul_(keep).mul_(ks)
    dd = (do.float() * o.float()).sum(-1, keepdim=True).to(q.dtype)
    ds.sub_(dd).mul_(p)
    del p
    dq = torch.matmul(ds, k).mul_(scale)
    dst = ds.transpose(-1, -2).contiguous()
    del ds
    dk = torch.matmul(dst, q).mul_(scale)
    return o, dq, dk, dv


SWEEP_SETTINGS = ("padding-dropout", "causal")


def memory_sweep(ns, setting: str = "padding-dropout", B: int = 1, H: int = 16, d: int = 64, reps: int = 3,
                 dropout_p: float = 0.1):
    """Peak device memory and time of one fwd + bwd step over N, for this path and for
    standard attention (the pages' memory-footprint and runtime benchmark, Experiments > 4.4;
    Theorem 1: extra memory O(N)). One JSON line per N; memory is the peak above the four
    resident inputs.

    setting "padding-dropout" (the pages' benchmark: dropout and a padding mask): key padding
    with a seeded key length uniform in [N/2, N], dropout p = 0.1; three lines: this path dense,
    this path block-sparse (128 x 128 blocks, diagonal + symmetric p = 1/8, combined with the
    padding), and standard attention. setting "causal": causal, no dropout; this path and
    standard attention."""
    import numpy as np
    import torch

    import exact_attention_100_amd as fa
    import workloads
    assert setting in SWEEP_SETTINGS, setting
    dev = torch.device("cuda:0")
    # One small call of each line first, so that one-time library set-up (the matrix library's
    # handles and workspace) is not charged to the first N.
    w = torch.zeros((1, 1, 128, d), dtype=torch.bfloat16, device=dev)
    standard_attention_step(w, w, w, w, 1.0, setting == "causal")
    o_w, l_w = fa.fwd(w, w, w)
    fa.bwd(w, w, w, o_w, w, l_w)
    torch.cuda.synchronize()
    del w, o_w, l_w
    for n in ns:
        mask = "key_len" if setting == "padding-dropout" else "causal"
        if setting == "padding-dropout" and n % 128 == 0:
            mask = "key_len+block"
        case = workloads.make_case(B, H, n, d, dtype=workloads.BF16, mask=mask, seed=100 + n.bit_length(),
                                   key_len_range=(max(n // 2, 1), n), block_size=128 if "block" in mask else None,
                                   block_p=0.125)
        t = {x: torch.from_numpy(case.bits(x).view(np.int16)).view(torch.bfloat16).to(dev)
             for x in ("q", "k", "v", "do")}
        kl = None if case.key_len is None else torch.from_numpy(case.key_len).to(dev)
        bm = None if case.block_mask is None else torch.from_numpy(case.block_mask).to(dev)
        sc = float(case.scale)
        causal = setting == "causal"
        p = dropout_p if setting == "padding-dropout" else 0.0
        row = {"N": n, "B": B, "H": H, "d": d, "setting": setting, "dropout_p": p,
               "key_len": None if kl is None else case.key_len.tolist()}
        lines = ["flash"] + (["flash_blocksparse"] if bm is not None else []) + ["standard"]
        for name in lines:
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            base = torch.cuda.memory_allocated(dev)
            torch.cuda.reset_peak_memory_stats(dev)
            try:
                def step():
                    if name == "flash":
                        o, lse = fa.fwd(t["q"], t["k"], t["v"], scale=sc, causal=causal, key_len=kl, dropout_p=p,
                                        seed=7)
                        return fa.bwd(t["q"], t["k"], t["v"], o, t["do"], lse, scale=sc, causal=causal,
                                      key_len=kl, dropout_p=p, seed=7)
                    if name == "flash_blocksparse":
                        o, lse = fa.blocksparse_fwd(t["q"], t["k"], t["v"], bm, 128, scale=sc, key_len=kl,
                                                    dropout_p=p, seed=7)
                        return fa.blocksparse_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, bm, 128, scale=sc,
                                                  key_len=kl, dropout_p=p, seed=7)
                    return standard_attention_step(t["q"], t["k"], t["v"], t["do"], sc, causal, key_len=kl,
                                                   dropout_p=p)
                step()
                torch.cuda.synchronize()
                peak = torch.cuda.max_memory_allocated(dev) - base
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    step()
                e1.record()
                torch.cuda.synchronize()
                row[name] = {"peak_extra_bytes": int(peak), "ms_per_step": round(e0.elapsed_time(e1) / reps, 4)}
            except torch.cuda.OutOfMemoryError:
                row[name] = "out of memory"
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        s_ = row["standard"]
        for name in lines[:-1]:
            f = row[name]
            if isinstance(f, dict) and isinstance(s_, dict):
                row["standard_over_" + name] = {"memory": round(s_["peak_extra_bytes"] / f["peak_extra_bytes"], 2),
                                                "time": round(s_["ms_per_step"] / f["ms_per_step"], 2)}
        print(json.dumps(row), flush=True)
        del t


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="C4b")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lib", default=None,
                    help="load this library file instead of the package's (tile-size variants)")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="dropout probability on P (dense workloads; 0: none, the headline step)")
    ap.add_argument("--calibrate-copy", action="store_true", help="only run a 1 GiB device copy (counter scale)")
    ap.add_argument("--cpu-table", action="store_true",
                    help="only time the float64 oracle (fwd, fwd + bwd) on every workload; --cpu-budget s per leg")
    ap.add_argument("--digest-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                           "COPY_WRITE_DIR"),
                    help="print per-kernel HBM traffic from rocprofv3 --pmc csv runs")
    ap.add_argument("--counters", default="auto", choices=("auto", "off"),
                    help="auto: measure HBM traffic and SQ counters of the benched workload in rocprofv3 child "
                         "runs on this box (falls back to the committed digests if that fails)")
    ap.add_argument("--digest-sq", nargs=2, metavar=("P1_DIR", "P2_DIR"),
                    help="print per-kernel SQ counter summaries from two rocprofv3 --pmc csv runs")
    ap.add_argument("--digest-lds", metavar="DIR",
                    help="print per-kernel LDS counter summaries from one rocprofv3 --pmc csv run over LDS_SET")
    ap.add_argument("--memory-sweep", nargs="*", type=int, metavar="N",
                    help="peak memory and time of this path and of standard attention over N "
                         "(B=1, H=16, d=64; default N = 128 .. 64K)")
    ap.add_argument("--sweep-setting", default="padding-dropout", choices=SWEEP_SETTINGS,
                    help="the memory sweep's masks: key padding + dropout 0.1 (with a block-sparse line), "
                         "or causal")
    args = ap.parse_args()
    if args.memory_sweep is not None:
        memory_sweep(args.memory_sweep or [1 << e for e in range(7, 17)], setting=args.sweep_setting)
        return
    if args.digest_counters:
        digest_counters(*args.digest_counters, workload=args.workload)
        return
    if args.digest_sq:
        digest_sq(*args.digest_sq, workload=args.workload)
        return
    if args.digest_lds:
        digest_lds(args.digest_lds, workload=args.workload)
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.cpu_table:
        cpu_table(args.cpu_budget)
        return
    if args.gpus != 1:
        print(f"bench.py: the library runs on exactly one GPU; --gpus {args.gpus} is not supported",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_attention_100_amd as fa
    import workloads
    from exact_attention_100_amd import _lib
    if args.lib:
        _lib.LIB_PATH = os.path.abspath(args.lib)
        if not os.path.exists(_lib.LIB_PATH):
            sys.exit(f"{args.lib} is not built (python -m exact_attention_100_amd.build --out {args.lib} -D ...)")
    elif not os.path.exists(_lib.LIB_PATH):
        from exact_attention_100_amd.build import build
        build()

    case = workloads.make_config(args.workload)
    assert case.dtype == workloads.BF16, "the bench measures bf16 workloads"
    assert args.dropout == 0.0 or case.block_mask is None, "dropout is for dense workloads"
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(case.bits(n).view(np.int16)).view(torch.bfloat16).to(dev)
         for n in ("q", "k", "v", "do")}
    key_len = None if case.key_len is None else torch.from_numpy(case.key_len).to(dev)
    bmask = None if case.block_mask is None else torch.from_numpy(case.block_mask).to(dev)
    sc = float(case.scale)
    o = torch.empty_like(t["q"])
    lse = torch.empty((case.B, case.H, case.N), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(t["q"]) for _ in range(3))
    if bmask is None:
        ws = torch.empty(fa.bwd_workspace_bytes(t["q"]), dtype=torch.uint8, device=dev)
    else:
        ws = torch.empty(fa.blocksparse_workspace_bytes(t["q"], case.block_size, True), dtype=torch.uint8,
                         device=dev)

    def step():
        if bmask is None:
            fa.fwd(t["q"], t["k"], t["v"], scale=sc, causal=case.causal, key_len=key_len, out=o, lse=lse,
                   dropout_p=args.dropout, seed=1234, offset=0)
            fa.bwd(t["q"], t["k"], t["v"], o, t["do"], lse, scale=sc, causal=case.causal, key_len=key_len,
                   dq=dq, dk=dk, dv=dv, workspace=ws, dropout_p=args.dropout, seed=1234, offset=0)
        else:
            fa.blocksparse_fwd(t["q"], t["k"], t["v"], bmask, case.block_size, scale=sc, causal=case.causal,
                               key_len=key_len, out=o, lse=lse, workspace=ws)
            fa.blocksparse_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, bmask, case.block_size, scale=sc,
                               causal=case.causal, key_len=key_len, dq=dq, dk=dk, dv=dv, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    pairs = kept_pairs(case)
    flops_step = 14 * case.d * pairs
    # MFMA work each kernel executes per launch (the dQ pass recomputes S and dP,
    # so the two backward kernels together execute 14 d per pair; the step metric
    # credits only the 10 d of a single-pass backward).
    kernel_flops = {"fa_fwd_bf16": 4 * case.d * pairs, "fa_bwd_dkdv": 8 * case.d * pairs,
                    "fa_bwd_dq": 6 * case.d * pairs}

    stream = torch.cuda.current_stream(dev)

    def timed_steps() -> float:
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(args.steps):
            step()
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop)

    total_ms = timed_steps()  # the step time: nothing recorded between the kernels
    with fa.KernelTimer() as timer:  # the same K steps again, each launch bracketed by events
        timed_ms = timed_steps()
        kt = {}
        for name in ("fa_fwd_bf16", "fa_bwd_dq", "fa_bwd_dkdv"):
            ms, n = timer.read(name)
            if n:
                kt[name] = {"mean_ms": ms / n, "launches": n, "share": ms / timed_ms}
    ms_step = total_ms / args.steps

    # Cold: before each of K steps a 512 MiB write evicts the inputs from L2 and the
    # 256 MiB MALL; each step is timed on its own (the write stays outside), median.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(args.steps):
        flush.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        cold.append((a, b))
    torch.cuda.synchronize()
    cold_ms = sorted(x.elapsed_time(y) for x, y in cold)[len(cold) // 2]
    del flush
    value = flops_step / (ms_step * 1e-3) / 1e12

    dom = max((k for k in kt if k in kernel_flops), key=lambda k: kt[k]["mean_ms"] * kt[k]["launches"])
    achieved = kernel_flops[dom] / (kt[dom]["mean_ms"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_for(dom, args.workload)}
    live_traffic = live_sq = None
    if args.counters == "auto" and args.dropout == 0.0:
        live_traffic, live_sq = measure_counters(args.workload, args.lib)
    here = ("this run: rocprofv3 --pmc passes over `bench.py --workload {w} --steps 2` started by this bench "
            "as child processes on this box ({what})")
    if live_traffic is not None and dom in live_traffic["kernels"]:
        roofline["traffic"] = live_traffic["kernels"][dom]["hbm_bytes_per_launch"]
        roofline["traffic_source"] = here.format(w=args.workload, what="FETCH_SIZE, WRITE_SIZE, each scaled by "
                                                 "the same counter on a 1 GiB copy")
        hbm_step = dict(live_traffic["step"], source=roofline["traffic_source"])
    else:
        trec = _traffic_record(args.workload)
        if roofline["traffic"] is not None:
            roofline["traffic_source"] = counter_source("hbm_traffic", args.workload, trec)
        hbm_step = step_traffic_for(args.workload)
        if hbm_step is not None:
            hbm_step = dict(hbm_step, source=counter_source("hbm_traffic", args.workload, trec))
    sq = live_sq if live_sq is not None else _sq_record(args.workload)
    mfma_busy = None
    if sq is not None:
        mfma_busy = {k: v["mfma_busy"] for k, v in sq["kernels"].items()}
        mfma_busy["source"] = (here.format(w=args.workload, what="SQ_VALU_MFMA_BUSY_CYCLES / 1024 over "
                                           "GRBM_GUI_ACTIVE / 8") if live_sq is not None
                               else counter_source("sq_counters", args.workload, sq))

    # The engine clock each kernel ran at (the published peak assumes 2.4 GHz; under this load the
    # chip runs slower), and the MFMA peak at that clock.
    engine_clock = None
    if sq is not None and any("engine_clock_mhz" in v for v in sq["kernels"].values()):
        engine_clock = {k: v["engine_clock_mhz"] for k, v in sq["kernels"].items() if "engine_clock_mhz" in v}
        rk = roofline.get("kernel")
        if rk in engine_clock:
            at_clock = PEAK_BF16_TFLOPS * engine_clock[rk] / 2400.0
            engine_clock["roofline_kernel_peak_at_clock"] = round(at_clock, 1)
            engine_clock["roofline_kernel_frac_at_clock"] = round(roofline["achieved"] / at_clock, 4)
        engine_clock["unit"] = "MHz"
        engine_clock["source"] = mfma_busy["source"].replace(
            "SQ_VALU_MFMA_BUSY_CYCLES / 1024 over GRBM_GUI_ACTIVE / 8", "GRBM_GUI_ACTIVE / 8 over each dispatch's duration")

    out = {
        "metric": "attention fwd+bwd TFLOP/s (bf16) and % of MI355X bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_instrumented": round(timed_ms / args.steps, 4),
        "cold": {"ms_per_step": round(cold_ms, 4), "value": round(flops_step / (cold_ms * 1e-3) / 1e12, 2),
                 "note": "median of K steps, each after a 512 MiB write that evicts L2 and MALL"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q, K, V, dO)",
        "config": {"workload": f"{args.workload}: {workloads.CONFIGS[args.workload]['desc']}", "B": case.B,
                   "H": case.H, "N": case.N, "d": case.d, "seed": case.seed,
                   "mask": "causal" if case.causal else ("block" if bmask is not None else
                                                         ("key_len" if key_len is not None else "none")),
                   "kept_pairs": pairs, "flop_per_step": flops_step, "dropout_p": args.dropout,
                   "library": os.path.relpath(_lib.LIB_PATH, ROOT)},
        "kernels": {k: {"mean_ms": round(v["mean_ms"], 4), "launches": v["launches"],
                        "share": round(v["share"], 4)} for k, v in kt.items()},
        "roofline": roofline,
        "mfma_busy": mfma_busy,
        "engine_clock": engine_clock,
        "hbm_step": hbm_step,
        "device_peak_bf16": {"value": device_peak_bf16_tflops(), "unit": "TFLOP/s",
                             "note": "reported peak engine clock x CUs x 4096 flop/clk/CU"},
    }
    if not args.no_cpu_baseline:
        def gpu_instance(b, h):
            # the outputs of the last timed step (every step writes the same values)
            return {n: x[b, h].float().cpu().numpy().astype(np.float64)
                    for n, x in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}
        torch.cuda.synchronize()
        out["cpu_baseline"], parity = cpu_baseline(case, args.cpu_budget, gpu_instance if args.dropout == 0.0 else None)
        if parity:
            out["parity"] = {"reference": "float64 CPU oracle, computed in the cpu_baseline leg on the same inputs",
                             "instances": parity,
                             "within_tolerance": all(x["within_tolerance"] for x in parity)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
