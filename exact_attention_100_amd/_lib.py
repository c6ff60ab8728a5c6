"""ctypes declarations of the C ABI in include/fa.h (libfa.so)."""
from __future__ import annotations

import ctypes
import os

# The in-tree build; EXACT_ATTENTION_LIB selects another build of the same sources (tile-size
# variants made by build.py --out, for measurements and their parity checks).
LIB_PATH = os.environ.get("EXACT_ATTENTION_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "lib", "libfa.so")

FA_OK = 0
FA_ERR_INVALID = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_WORKSPACE = -3
FA_ERR_HIP = -4
FA_ERR_SCRATCH = -5
FA_BF16 = 0
FA_F32 = 1

EXPORTS = ("fa_fwd", "fa_bwd_workspace_bytes", "fa_bwd", "fa_fwd_dropout", "fa_bwd_dropout",
           "fa_blocksparse_workspace_bytes", "fa_blocksparse_fwd", "fa_blocksparse_bwd", "fa_blocksparse_fwd_dropout",
           "fa_blocksparse_bwd_dropout", "fa_status_string",
           "fa_version", "fa_bwd_noalloc",
           "fa_timer_enable", "fa_timer_reset", "fa_timer_read")


class FaDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64)]


class FAError(RuntimeError):
    """A nonzero status from libfa, or the library itself missing."""

    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = f"{what}: " if what else ""
        try:
            msg += _load().fa_status_string(status).decode()
        except Exception:  # library missing
            msg += f"status {status}"
        super().__init__(msg)


_LIB = None

P = ctypes.c_void_p
I32 = ctypes.c_int32
F32 = ctypes.c_float
SZ = ctypes.c_size_t
DESC = ctypes.POINTER(FaDesc)


def _load():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(f"{LIB_PATH} is not built; run `python -m exact_attention_100_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "fa_fwd": (ctypes.c_int, [DESC, P, P, P, F32, ctypes.c_int, P, P, P, P]),
        "fa_bwd_workspace_bytes": (SZ, [DESC]),
        "fa_bwd": (ctypes.c_int, [DESC, P, P, P, P, P, P, F32, ctypes.c_int, P, P, P, P, P, SZ, P]),
        "fa_fwd_dropout": (ctypes.c_int, [DESC, P, P, P, F32, ctypes.c_int, P, F32, ctypes.c_uint64,
                                          ctypes.c_uint32, P, P, P]),
        "fa_bwd_dropout": (ctypes.c_int, [DESC, P, P, P, P, P, P, F32, ctypes.c_int, P, F32, ctypes.c_uint64,
                                          ctypes.c_uint32, P, P, P, P, SZ, P]),
        "fa_blocksparse_workspace_bytes": (SZ, [DESC, I32, ctypes.c_int]),
        "fa_blocksparse_fwd": (ctypes.c_int, [DESC, P, P, P, F32, ctypes.c_int, P, P, I32, P, P, P, SZ, P]),
        "fa_blocksparse_bwd": (ctypes.c_int, [DESC, P, P, P, P, P, P, F32, ctypes.c_int, P, P, I32, P, P, P,
                                              P, SZ, P]),
        "fa_bwd_noalloc": (ctypes.c_int, [DESC, P, P, P, P, P, P, F32, ctypes.c_int, P, P, P, P, P]),
        "fa_blocksparse_fwd_dropout": (ctypes.c_int, [DESC, P, P, P, F32, ctypes.c_int, P, P, I32, F32,
                                                      ctypes.c_uint64, ctypes.c_uint32, P, P, P]),
        "fa_blocksparse_bwd_dropout": (ctypes.c_int, [DESC, P, P, P, P, P, P, F32, ctypes.c_int, P, P, I32, F32,
                                                      ctypes.c_uint64, ctypes.c_uint32, P, P, P, P, SZ, P]),
        "fa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "fa_version": (ctypes.c_int, []),
        "fa_timer_enable": (ctypes.c_int, [ctypes.c_int]),
        "fa_timer_reset": (None, []),
        "fa_timer_read": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_int64)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def lib():
    """The loaded libfa.so (raises if it has not been built)."""
    return _load()
