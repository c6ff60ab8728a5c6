"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the library sources with the sanitizers on the host side only (device code is
built as usual and never runs) together with tests/abi_sanitize_main.cpp, which calls
every entry point with arguments its checks must reject: null and misaligned pointers,
empty, overflowing and unsupported shapes, strides no device can hold, bad scales,
dropout probabilities, block sizes and workspaces. The program exits 0 only if every
call returned the expected status without a sanitizer report.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_100_amd", "csrc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.timeout(600)
def test_abi_validation_under_sanitizers(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-w",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, *SAN]
    sources = [os.path.join(CSRC, f) for f in ("fa_api.hip", "fa_fwd.hip", "fa_bwd.hip")]
    sources.append(os.path.join(ROOT, "tests", "abi_sanitize_main.cpp"))
    objs = [str(tmp_path / (os.path.basename(s) + ".o")) for s in sources]

    def compile_one(so):
        src, obj = so
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        r = subprocess.run([hipcc, *flags, *lang, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr

    with ThreadPoolExecutor(max_workers=4) as ex:
        list(ex.map(compile_one, zip(sources, objs)))
    exe = str(tmp_path / "abi_sanitize")
    r = subprocess.run([hipcc, "--offload-arch=gfx950", *SAN, "-o", exe, *objs], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
