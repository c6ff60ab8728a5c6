"""Compile the HIP sources into exact_attention_100_amd/lib/libfa.so for gfx950.

Usage: python -m exact_attention_100_amd.build   (or call build()).
Tile-size variants for measurements (the kernels' -D knobs, e.g. FA_FWD_BC_D128=32):
       python -m exact_attention_100_amd.build --out exact_attention_100_amd/lib/variants/libfa_x.so -D NAME=VALUE ...
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libfa.so")
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_bwd.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed f32 VALU ops (v_pk_*_f32).
HIPCC_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I" + INCLUDE, "-I" + CSRC]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + out)


def build(verbose: bool = False, out: str | None = None, defines: tuple[str, ...] = ()) -> str:
    """Compile every HIP source and link libfa.so (or `out`, with extra -D `defines`); always
    rebuilds. Returns the library path."""
    hipcc = _hipcc()
    lib = LIB if out is None else os.path.abspath(out)
    objdir = OBJDIR if out is None else os.path.join(OBJDIR, os.path.splitext(os.path.basename(lib))[0])
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    dflags = ["-D" + d for d in defines]
    cmds = [[hipcc, *HIPCC_FLAGS, *dflags, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=min(len(cmds), 4)) as ex:
        for c, _ in zip(cmds, ex.map(_run, cmds)):
            if verbose:
                print(" ".join(c), flush=True)
    tmp = lib + ".tmp"
    _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, lib)
    if verbose:
        print("built", lib, flush=True)
    return lib


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("-q", action="store_true")
    ap.add_argument("--out", default=None, help="library path (default: the package's libfa.so)")
    ap.add_argument("-D", dest="defines", action="append", default=[], help="NAME=VALUE for every source")
    a = ap.parse_args()
    build(verbose=not a.q, out=a.out, defines=tuple(a.defines))
