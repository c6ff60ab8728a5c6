"""Exact attention for MI355X (gfx950): Python binding of libfa.so.

Argument marshalling only: torch tensors provide device memory and the current
HIP stream; every step of the computation runs in the library's HIP kernels.
There is no CPU or PyTorch fallback: if libfa.so is missing, every call raises.

    o, lse = fwd(q, k, v, causal=True)
    dq, dk, dv = bwd(q, k, v, o, do, lse, causal=True)
    o, lse = blocksparse_fwd(q, k, v, block_mask, 128)
    dq, dk, dv = blocksparse_bwd(q, k, v, o, do, lse, block_mask, 128)

q, k, v, o, do: [B, H, N, d] tensors on the GPU, bf16 (or fp32 for fwd), all
with the same strides and a contiguous last dimension; lse: float32 [B, H, N].
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

from ._lib import (FA_BF16, FA_F32, FA_OK, FAError, FaDesc, lib)  # noqa: F401

__all__ = ["fwd", "bwd", "bwd_noalloc", "blocksparse_fwd", "blocksparse_bwd", "bwd_workspace_bytes",
           "blocksparse_workspace_bytes", "FAError", "lib", "KernelTimer"]


def _torch():
    import torch
    return torch


def _desc(q) -> FaDesc:
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("expected a [B, H, N, d] tensor")
    if q.dtype == torch.bfloat16:
        dt = FA_BF16
    elif q.dtype == torch.float32:
        dt = FA_F32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if not q.is_cuda:
        raise ValueError("tensors must live on the GPU")
    B, H, N, d = q.shape
    sb, sh, sn, sd = q.stride()
    if sd != 1:
        raise ValueError("the last dimension must be contiguous")
    return FaDesc(B, H, N, d, dt, 0, sb, sh, sn)


def _same_layout(ref, *ts):
    for t in ts:
        if t.shape != ref.shape or t.stride() != ref.stride() or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("q, k, v, o, do and the gradients must share shape, strides, dtype and device")


def _empty_like(ref):
    torch = _torch()
    return torch.empty_strided(ref.shape, ref.stride(), dtype=ref.dtype, device=ref.device)


def _stream(ref) -> int:
    return _torch().cuda.current_stream(ref.device).cuda_stream


def _scale(scale, d) -> float:
    return float(1.0 / math.sqrt(d)) if scale is None else float(scale)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(status: int, what: str):
    if status != FA_OK:
        raise FAError(status, what)


def _key_len(key_len, q):
    torch = _torch()
    if key_len is None:
        return None
    if key_len.dtype != torch.int32 or key_len.device != q.device or key_len.numel() != q.shape[0]:
        raise ValueError("key_len must be an int32 [B] tensor on the same device")
    return key_len.contiguous()


def _lse_check(lse, q):
    torch = _torch()
    B, H, N, _ = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")


def bwd_workspace_bytes(q) -> int:
    d = _desc(q)
    return int(lib().fa_bwd_workspace_bytes(ctypes.byref(d)))


def blocksparse_workspace_bytes(q, block_size: int, backward: bool) -> int:
    d = _desc(q)
    return int(lib().fa_blocksparse_workspace_bytes(ctypes.byref(d), int(block_size), int(bool(backward))))


def _workspace(nbytes, ref, workspace):
    torch = _torch()
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=ref.device)


def fwd(q, k, v, scale=None, causal=False, key_len=None, out=None, lse=None, dropout_p=0.0, seed=0, offset=0):
    """Exact attention forward; returns (O, LSE). With dropout_p > 0, dropout on P with keep bits
    from (seed, offset) (fa_fwd_dropout); the backward must get the same three values."""
    torch = _torch()
    d = _desc(q)
    _same_layout(q, k, v)
    o = _empty_like(q) if out is None else out
    _same_layout(q, o)
    B, H, N, _ = q.shape
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _lse_check(lse, q)
    kl = _key_len(key_len, q)
    if dropout_p:
        st = lib().fa_fwd_dropout(ctypes.byref(d), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  _scale(scale, q.shape[-1]), int(bool(causal)), _ptr(kl), float(dropout_p),
                                  int(seed), int(offset), o.data_ptr(), lse.data_ptr(), _stream(q))
        _check(st, "fa_fwd_dropout")
        return o, lse
    st = lib().fa_fwd(ctypes.byref(d), q.data_ptr(), k.data_ptr(), v.data_ptr(), _scale(scale, q.shape[-1]),
                      int(bool(causal)), _ptr(kl), o.data_ptr(), lse.data_ptr(), _stream(q))
    _check(st, "fa_fwd")
    return o, lse


def bwd(q, k, v, o, do, lse, scale=None, causal=False, key_len=None, dq=None, dk=None, dv=None,
        workspace=None, dropout_p=0.0, seed=0, offset=0):
    """Exact attention backward; returns (dQ, dK, dV). Use the forward's scale, causal, key_len
    and dropout (dropout_p, seed, offset)."""
    d = _desc(q)
    _same_layout(q, k, v, o, do)
    _lse_check(lse, q)
    dq = _empty_like(q) if dq is None else dq
    dk = _empty_like(q) if dk is None else dk
    dv = _empty_like(q) if dv is None else dv
    _same_layout(q, dq, dk, dv)
    kl = _key_len(key_len, q)
    need = int(lib().fa_bwd_workspace_bytes(ctypes.byref(d)))
    ws = _workspace(need, q, workspace)
    if dropout_p:
        st = lib().fa_bwd_dropout(ctypes.byref(d), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  do.data_ptr(), lse.data_ptr(), _scale(scale, q.shape[-1]), int(bool(causal)),
                                  _ptr(kl), float(dropout_p), int(seed), int(offset), dq.data_ptr(),
                                  dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                                  _stream(q))
        _check(st, "fa_bwd_dropout")
        return dq, dk, dv
    st = lib().fa_bwd(ctypes.byref(d), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                      lse.data_ptr(), _scale(scale, q.shape[-1]), int(bool(causal)), _ptr(kl), dq.data_ptr(),
                      dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(), _stream(q))
    _check(st, "fa_bwd")
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, scale=None, causal=False, key_len=None):
    """fa_bwd_noalloc: the backward with its workspace in the library's static per-device scratch
    (no allocation anywhere; the caller passes the outputs dq, dk, dv). Calls that overlap on one
    GPU race on that scratch."""
    d = _desc(q)
    _same_layout(q, k, v, o, do)
    _same_layout(q, dq, dk, dv)
    _lse_check(lse, q)
    kl = _key_len(key_len, q)
    st = lib().fa_bwd_noalloc(ctypes.byref(d), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              do.data_ptr(), lse.data_ptr(), _scale(scale, q.shape[-1]), int(bool(causal)),
                              _ptr(kl), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _stream(q))
    _check(st, "fa_bwd_noalloc")
    return dq, dk, dv


def _mask_check(block_mask, q, block_size):
    torch = _torch()
    nb = q.shape[2] // int(block_size) if block_size else 0
    if (block_mask.dtype != torch.uint8 or block_mask.device != q.device or tuple(block_mask.shape) != (nb, nb)
            or not block_mask.is_contiguous()):
        raise ValueError("block_mask must be a contiguous uint8 [N/bs, N/bs] tensor on the same device")


def blocksparse_fwd(q, k, v, block_mask, block_size, scale=None, causal=False, key_len=None, out=None,
                    lse=None, workspace=None, dropout_p=0.0, seed=0, offset=0):
    """Block-sparse forward (zero blocks of block_mask skipped, combined by AND with the causal
    and key-length masks); returns (O, LSE). With dropout_p > 0, dropout on P as in fwd()
    (fa_blocksparse_fwd_dropout)."""
    torch = _torch()
    d = _desc(q)
    _same_layout(q, k, v)
    _mask_check(block_mask, q, block_size)
    kl = _key_len(key_len, q)
    o = _empty_like(q) if out is None else out
    B, H, N, _ = q.shape
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _lse_check(lse, q)
    if dropout_p:
        st = lib().fa_blocksparse_fwd_dropout(ctypes.byref(d), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                              _scale(scale, q.shape[-1]), int(bool(causal)), _ptr(kl),
                                              block_mask.data_ptr(), int(block_size), float(dropout_p), int(seed),
                                              int(offset), o.data_ptr(), lse.data_ptr(), _stream(q))
        _check(st, "fa_blocksparse_fwd_dropout")
        return o, lse
    need = int(lib().fa_blocksparse_workspace_bytes(ctypes.byref(d), int(block_size), 0))
    ws = None if (need == 0 and workspace is None) else _workspace(need, q, workspace)
    st = lib().fa_blocksparse_fwd(ctypes.byref(d), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  _scale(scale, q.shape[-1]), int(bool(causal)), _ptr(kl),
                                  block_mask.data_ptr(), int(block_size), o.data_ptr(), lse.data_ptr(),
                                  _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(q))
    _check(st, "fa_blocksparse_fwd")
    return o, lse


def blocksparse_bwd(q, k, v, o, do, lse, block_mask, block_size, scale=None, causal=False, key_len=None,
                    dq=None, dk=None, dv=None, workspace=None, dropout_p=0.0, seed=0, offset=0):
    """Block-sparse backward; returns (dQ, dK, dV). Use the forward's mask, scale, causal, key_len
    and dropout (dropout_p, seed, offset)."""
    d = _desc(q)
    _same_layout(q, k, v, o, do)
    _lse_check(lse, q)
    _mask_check(block_mask, q, block_size)
    kl = _key_len(key_len, q)
    dq = _empty_like(q) if dq is None else dq
    dk = _empty_like(q) if dk is None else dk
    dv = _empty_like(q) if dv is None else dv
    need = int(lib().fa_blocksparse_workspace_bytes(ctypes.byref(d), int(block_size), 1))
    ws = _workspace(need, q, workspace)
    if dropout_p:
        st = lib().fa_blocksparse_bwd_dropout(ctypes.byref(d), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                              o.data_ptr(), do.data_ptr(), lse.data_ptr(), _scale(scale, q.shape[-1]),
                                              int(bool(causal)), _ptr(kl), block_mask.data_ptr(), int(block_size),
                                              float(dropout_p), int(seed), int(offset), dq.data_ptr(),
                                              dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                                              ws.numel() * ws.element_size(), _stream(q))
        _check(st, "fa_blocksparse_bwd_dropout")
        return dq, dk, dv
    st = lib().fa_blocksparse_bwd(ctypes.byref(d), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  do.data_ptr(), lse.data_ptr(), _scale(scale, q.shape[-1]),
                                  int(bool(causal)), _ptr(kl), block_mask.data_ptr(), int(block_size),
                                  dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                                  ws.numel() * ws.element_size(), _stream(q))
    _check(st, "fa_blocksparse_bwd")
    return dq, dk, dv


class KernelTimer:
    """The library's kernel timer: HIP events around every launch while enabled."""

    def __enter__(self):
        _check(lib().fa_timer_enable(1), "fa_timer_enable")
        lib().fa_timer_reset()
        return self

    def __exit__(self, *exc):
        lib().fa_timer_enable(0)
        return False

    @staticmethod
    def read(kernel: str):
        """(total milliseconds, launch count) of `kernel` since the timer was entered."""
        ms = ctypes.c_double(0.0)
        n = ctypes.c_int64(0)
        _check(lib().fa_timer_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)), "fa_timer_read")
        return ms.value, n.value
