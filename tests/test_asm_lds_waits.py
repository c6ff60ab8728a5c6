"""The generated gfx950 code consumes no LDS read before its wait (see lds_waits.py).

Compiles the forward and backward sources to device assembly with the library's own
flags (hipcc cross-compiles without a GPU) and scans every kernel.
"""
import os
import subprocess
import tempfile

import pytest

from exact_attention_100_amd import build as B
from lds_waits import violations


def test_scanner_flags_a_consumer_above_its_wait():
    asm = "\n".join(["_Zk:", "  ds_read_b64_tr_b16 v[66:67], v1 offset:0", "  ds_read_b64_tr_b16 v[68:69], v2 offset:0",
                     "  v_mfma_f32_32x32x16_bf16 v[0:15], v[66:69], v[144:147], v[0:15]", "  s_waitcnt lgkmcnt(0)"])
    assert len(violations(asm)) == 1
    ok = asm.replace("  v_mfma", "  s_waitcnt lgkmcnt(0)\n  v_mfma")
    assert violations(ok) == []
    # a partial wait covers the older read only
    part = "\n".join(["_Zk:", "  ds_read_b128 v[0:3], v9", "  ds_read_b128 v[4:7], v9 offset:1024", "  s_waitcnt lgkmcnt(1)",
                      "  v_mov_b32 v20, v1", "  v_mov_b32 v21, v5"])
    assert [v.split(":")[0] for v in violations(part)] == ["line 6 in _Zk"]


@pytest.mark.parametrize("src", ["fa_fwd.hip", "fa_bwd.hip"])
def test_kernels_wait_for_their_lds_reads(src):
    try:
        hipcc = B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        flags = [f for f in B.HIPCC_FLAGS if f != "-fPIC"]
        r = subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out],
                           stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert r.returncode == 0, r.stdout[-2000:]
        found = violations(open(out).read())
    assert found == [], "\n".join(found[:20])
