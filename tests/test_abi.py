"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

from helpers import ROOT, ensure_library


@pytest.fixture(scope="module")
def lib():
    ensure_library()
    import exact_attention_100_amd as fa
    return fa.lib()


def _header_functions():
    with open(os.path.join(ROOT, "include", "fa.h")) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    names = _header_functions()
    for n in ("fa_fwd", "fa_bwd", "fa_fwd_dropout", "fa_bwd_dropout", "fa_blocksparse_fwd",
              "fa_blocksparse_bwd", "fa_blocksparse_fwd_dropout", "fa_blocksparse_bwd_dropout",
              "fa_bwd_workspace_bytes", "fa_blocksparse_workspace_bytes", "fa_bwd_noalloc",
              "fa_status_string", "fa_version"):
        assert n in names


def test_library_exports_every_header_symbol(lib):
    cdll = ctypes.CDLL(os.path.join(ROOT, "exact_attention_100_amd", "lib", "libfa.so"))
    for n in _header_functions():
        assert hasattr(cdll, n), n


def test_version_and_status_strings(lib):
    assert lib.fa_version() == 104
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.fa_status_string(code)
    assert b"unknown" in lib.fa_status_string(7)


def _desc(B=2, H=3, N=256, d=64, dtype=0):
    from exact_attention_100_amd import FaDesc
    return FaDesc(B, H, N, d, dtype, 0, H * N * d, N * d, d)


A = 4096  # a 16-byte aligned, never dereferenced address


def test_argument_errors_before_any_launch(lib):
    d = _desc()
    ref = ctypes.byref
    assert lib.fa_fwd(ref(d), None, A, A, 0.1, 0, None, A, A, None) == -1
    assert lib.fa_fwd(ref(d), A + 2, A, A, 0.1, 0, None, A, A, None) == -1  # misaligned
    assert lib.fa_fwd(ref(d), A, A, A, -0.5, 0, None, A, A, None) == -1
    assert lib.fa_fwd(ref(d), A, A, A, float("nan"), 0, None, A, A, None) == -1
    assert lib.fa_fwd(None, A, A, A, 0.1, 0, None, A, A, None) == -1
    for bad in (_desc(N=0), _desc(B=0), _desc(dtype=5)):
        assert lib.fa_fwd(ref(bad), A, A, A, 0.1, 0, None, A, A, None) == -1
    assert lib.fa_fwd(ref(_desc(d=96)), A, A, A, 0.1, 0, None, A, A, None) == -2
    odd = _desc()
    odd.stride_n = 65  # row stride not a multiple of 16 bytes
    assert lib.fa_fwd(ref(odd), A, A, A, 0.1, 0, None, A, A, None) == -1
    # row strides from 2^23 elements on are refused (32-bit lane offsets over 256-row tiles);
    # just below the limit the descriptor passes and the null output is what is refused
    wide = _desc(B=1, H=1)
    wide.stride_n = wide.stride_h = wide.stride_b = 1 << 23
    assert lib.fa_fwd(ref(wide), A, A, A, 0.1, 0, None, A, A, None) == -2
    assert lib.fa_bwd(ref(wide), A, A, A, A, A, A, 0.1, 0, None, A, A, A, A, 1 << 30, None) == -2
    wide.stride_n = (1 << 23) - 16
    assert lib.fa_fwd(ref(wide), A, A, A, 0.1, 0, None, None, A, None) == -1
    # backward: fp32 unsupported, workspace checks
    assert lib.fa_bwd(ref(_desc(dtype=1)), A, A, A, A, A, A, 0.1, 0, None, A, A, A, A, 1 << 30, None) == -2
    need = lib.fa_bwd_workspace_bytes(ref(d))
    assert lib.fa_bwd(ref(d), A, A, A, A, A, A, 0.1, 0, None, A, A, A, A, need - 1, None) == -3
    assert lib.fa_bwd(ref(d), A, A, A, A, A, A, 0.1, 0, None, A, A, A, None, need, None) == -3
    # dropout: p must lie in [0, 1); fp32 with dropout is unsupported; checked before any launch
    for p in (-0.1, 1.0, 1.5, float("nan"), 0.999):
        assert lib.fa_fwd_dropout(ref(d), A, A, A, 0.1, 0, None, p, 1, 0, A, A, None) == -1
        assert lib.fa_bwd_dropout(ref(d), A, A, A, A, A, A, 0.1, 0, None, p, 1, 0, A, A, A, A, 1 << 30,
                                  None) == -1
    assert lib.fa_fwd_dropout(ref(_desc(dtype=1)), A, A, A, 0.1, 0, None, 0.1, 1, 0, A, A, None) == -2
    assert lib.fa_bwd_dropout(ref(_desc(dtype=1)), A, A, A, A, A, A, 0.1, 0, None, 0.1, 1, 0, A, A, A, A,
                              1 << 30, None) == -2
    # block-sparse dropout: the block-size, mask, probability, dtype and workspace checks
    for p in (-0.1, 1.0, float("nan")):
        assert lib.fa_blocksparse_fwd_dropout(ref(d), A, A, A, 0.1, 0, None, A, 128, p, 1, 0, A, A, None) == -1
        assert lib.fa_blocksparse_bwd_dropout(ref(d), A, A, A, A, A, A, 0.1, 0, None, A, 128, p, 1, 0, A, A, A, A,
                                              1 << 30, None) == -1
    assert lib.fa_blocksparse_fwd_dropout(ref(d), A, A, A, 0.1, 0, None, None, 128, 0.1, 1, 0, A, A, None) == -1
    assert lib.fa_blocksparse_fwd_dropout(ref(d), A, A, A, 0.1, 0, None, A, 100, 0.1, 1, 0, A, A, None) == -1
    assert lib.fa_blocksparse_fwd_dropout(ref(_desc(dtype=1)), A, A, A, 0.1, 0, None, A, 128, 0.1, 1, 0, A, A,
                                          None) == -2
    need_bs = lib.fa_bwd_workspace_bytes(ref(d))
    assert lib.fa_blocksparse_bwd_dropout(ref(d), A, A, A, A, A, A, 0.1, 0, None, A, 128, 0.1, 1, 0, A, A, A, A,
                                          need_bs - 1, None) == -3
    # block-sparse: block size must be a multiple of 128 that divides N
    for bs in (64, 100, 192, 512):
        assert lib.fa_blocksparse_fwd(ref(d), A, A, A, 0.1, 0, None, A, bs, A, A, A, 1 << 30, None) == -1
    assert lib.fa_blocksparse_fwd(ref(d), A, A, A, 0.1, 0, None, None, 128, A, A, A, 1 << 30, None) == -1
    assert lib.fa_blocksparse_workspace_bytes(ref(d), 100, 0) == 0
    # more than 1024 blocks per side is unsupported
    big = _desc(B=1, H=1, N=128 * 1025)
    assert lib.fa_blocksparse_fwd(ref(big), A, A, A, 0.1, 0, None, A, 128, A, A, None, 0, None) == -2
    # the forward needs no workspace; the backward needs the fa_bwd one
    need = lib.fa_bwd_workspace_bytes(ref(d))
    assert lib.fa_blocksparse_workspace_bytes(ref(d), 128, 0) == 0
    assert lib.fa_blocksparse_workspace_bytes(ref(d), 128, 1) == need
    assert lib.fa_blocksparse_bwd(ref(d), A, A, A, A, A, A, 0.1, 1, None, A, 128, A, A, A, A, need - 1,
                                  None) == -3
    assert lib.fa_blocksparse_bwd(ref(d), A, A, A, A, A, A, 0.1, 1, None, A, 128, A, A, A, None, need,
                                  None) == -3


def test_noalloc_backward_checks_before_any_launch(lib):
    """fa_bwd_noalloc rejects what fa_bwd rejects, and problems beyond its static scratch (2^21 rows)
    with FA_ERR_SCRATCH, all before touching the GPU."""
    ref = ctypes.byref
    d = _desc()
    assert lib.fa_bwd_noalloc(ref(_desc(dtype=1)), A, A, A, A, A, A, 0.1, 0, None, A, A, A, None) == -2
    assert lib.fa_bwd_noalloc(ref(d), A, A, A, A, A, A, 0.1, 0, None, None, A, A, None) == -1
    assert lib.fa_bwd_noalloc(ref(d), A, A, A, A, A, A, -1.0, 0, None, A, A, A, None) == -1
    assert lib.fa_bwd_noalloc(ref(_desc(B=1, H=1, N=(1 << 21) + 1)), A, A, A, A, A, A, 0.1, 0, None, A, A, A,
                              None) == -5
    assert lib.fa_bwd_noalloc(ref(_desc(B=2, H=16, N=65537, d=128)), A, A, A, A, A, A, 0.1, 1, None, A, A, A,
                              None) == -5
    assert b"FA_ERR_SCRATCH" in lib.fa_status_string(-5)


def test_workspace_is_linear_in_sequence_length(lib):
    """Extra memory grows as O(N) (Theorem 1), never O(N^2)."""
    ws = [lib.fa_bwd_workspace_bytes(ctypes.byref(_desc(B=1, H=1, N=n, d=128))) for n in (4096, 8192, 16384)]
    per_row = [w / n for w, n in zip(ws, (4096, 8192, 16384))]
    assert max(per_row) - min(per_row) < 1.0
    assert per_row[0] <= (128 + 2) * 4 + 1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from exact_attention_100_amd import _lib
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_LIB", None)
    with pytest.raises(FileNotFoundError):
        _lib.lib()
