"""Deterministic attention backward for AMD Instinct MI355X (gfx950).

A thin PyTorch-facing binding over libattn_det.so. Every step of the
computation runs in the library's HIP kernels; this module only checks tensor
shapes/dtypes, allocates outputs and workspace with torch, and passes device
pointers and the current HIP stream through the C ABI (include/attn_det.h).

    o, lse = fwd(q, k, v, causal)
    dq, dk, dv = bwd(q, k, v, o, do, lse, causal, schedule="shift")
    dq, dk, dv = bwd_nondeterministic(q, k, v, o, do, lse, causal)

Tensors: q, k, v, o, do are bfloat16 CUDA (HIP) tensors [B, H, S, D],
contiguous; lse is float32 [B, H, S] (natural-log log-sum-exp of the scaled
scores, as fwd returns it).
"""

from __future__ import annotations

import ctypes
import math

from . import _lib
from ._lib import (AttnError, MASK_CAUSAL, MASK_FULL, SCHED_DESCENDING, SCHED_NAIVE,  # noqa: F401
                   SCHED_SHIFT, SCHED_SYMMETRIC_SHIFT)

SCHEDULES = {
    "naive": SCHED_NAIVE,
    "descending": SCHED_DESCENDING,
    "shift": SCHED_SHIFT,
    "symmetric_shift": SCHED_SYMMETRIC_SHIFT,
}


def _torch():
    import torch
    return torch


def _sched(schedule) -> int:
    if isinstance(schedule, str):
        if schedule not in SCHEDULES:
            raise ValueError(f"unknown schedule {schedule!r}; one of {sorted(SCHEDULES)}")
        return SCHEDULES[schedule]
    return int(schedule)


def _stream_ptr(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _check_qkv(*ts):
    torch = _torch()
    shape = ts[0].shape
    for t in ts:
        if t.dtype != torch.bfloat16:
            raise TypeError(f"expected bfloat16, got {t.dtype}")
        if t.device.type != "cuda":
            raise ValueError("tensors must live on the GPU")
        if t.dim() != 4 or t.shape != shape:
            raise ValueError(f"expected matching [B, H, S, D] tensors, got {tuple(t.shape)} vs {tuple(shape)}")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, S, D]")
    return shape


def _check_heads(q, k, v, *rest):
    """q (and rest) [B, H, S, D], k and v [B, Hkv, S, D] with H % Hkv == 0; returns (B, H, Hkv, S, D)."""
    B, H, S, D = _check_qkv(q, *rest)
    Bk, Hkv, Sk, Dk = _check_qkv(k, v)
    if (Bk, Sk, Dk) != (B, S, D) or Hkv <= 0 or H % Hkv:
        raise ValueError(f"k/v {tuple(k.shape)} do not match q {tuple(q.shape)} (need [B, Hkv, S, D], H % Hkv == 0)")
    return B, H, Hkv, S, D


def _check_lse(lse, shape):
    torch = _torch()
    if lse.dtype != torch.float32 or lse.shape != shape[:3] or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, S] tensor")


def tile(S: int, D: int, tile_request: int = 0) -> int:
    t = _lib.load().attn_bwd_tile(int(S), int(D), int(tile_request))
    _lib.check(t if t < 0 else 0, "attn_bwd_tile")
    return t


def workspace_size(B, H, S, D, causal, schedule="descending", tile_request=0, Hkv=None) -> int:
    """Workspace bytes; Hkv = number of K/V heads when query heads share them (default H)."""
    mask = MASK_CAUSAL if causal else MASK_FULL
    if Hkv is None or int(Hkv) == int(H):
        n = _lib.load().attn_bwd_workspace_size(int(B), int(H), int(S), int(D), mask, _sched(schedule),
                                               int(tile_request))
    else:
        n = _lib.load().attn_bwd_gqa_workspace_size(int(B), int(H), int(Hkv), int(S), int(D), mask,
                                                   _sched(schedule), int(tile_request))
    if n == 0:
        raise ValueError("invalid shape for the attention backward")
    return int(n)


def alloc_workspace(B, H, S, D, causal, schedule="descending", tile_request=0, device="cuda", Hkv=None):
    """Device workspace (uint8) for bwd/bwd_nondeterministic with these arguments."""
    torch = _torch()
    return torch.empty(workspace_size(B, H, S, D, causal, schedule, tile_request, Hkv), dtype=torch.uint8,
                       device=device)


def fwd(q, k, v, causal: bool, scale: float | None = None, out=None):
    """Attention forward producing (O bf16 [B,H,S,D], LSE fp32 [B,H,S]); k, v may have fewer heads (grouped)."""
    torch = _torch()
    B, H, Hkv, S, D = _check_heads(q, k, v)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
    mask = MASK_CAUSAL if causal else MASK_FULL
    if Hkv == H:
        st = _lib.load().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, S, D, scale, mask,
                                  _stream_ptr(q.device))
    else:
        st = _lib.load().attn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, S, D, scale, mask,
                                      _stream_ptr(q.device))
    _lib.check(st, "attn_fwd")
    return o, lse


def bwd(q, k, v, o, do, lse, causal: bool, schedule="descending", scale: float | None = None, tile_request: int = 0,
        workspace=None, out=None):
    """Deterministic attention backward; returns (dq, dk, dv) bf16 shaped like (q, k, v)."""
    return _bwd(q, k, v, o, do, lse, causal, _sched(schedule), scale, tile_request, workspace, out, True)


def bwd_nondeterministic(q, k, v, o, do, lse, causal: bool, scale: float | None = None, tile_request: int = 0,
                         workspace=None, out=None):
    """Atomic-dQ attention backward (run-to-run order not fixed); returns (dq, dk, dv)."""
    return _bwd(q, k, v, o, do, lse, causal, SCHED_NAIVE, scale, tile_request, workspace, out, False)


def _bwd(q, k, v, o, do, lse, causal, schedule, scale, tile_request, workspace, out, deterministic):
    torch = _torch()
    B, H, Hkv, S, D = _check_heads(q, k, v, o, do)
    _check_lse(lse, q.shape)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if workspace is None:
        workspace = alloc_workspace(B, H, S, D, causal, schedule, tile_request, q.device, Hkv)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
    lib = _lib.load()
    mask = MASK_CAUSAL if causal else MASK_FULL
    stream = _stream_ptr(q.device)
    if Hkv != H:
        if deterministic:
            st = lib.attn_bwd_deterministic_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), mask,
                                                schedule, _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv, S, D, scale,
                                                int(tile_request), _ptr(workspace), workspace.numel(), stream)
        else:
            st = lib.attn_bwd_nondeterministic_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), mask,
                                                   _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv, S, D, scale,
                                                   int(tile_request), _ptr(workspace), workspace.numel(), stream)
        _lib.check(st, "attn_bwd_gqa")
    elif deterministic:
        st = lib.attn_bwd_deterministic(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), mask, schedule,
                                        _ptr(dq), _ptr(dk), _ptr(dv), B, H, S, D, scale, int(tile_request),
                                        _ptr(workspace), workspace.numel(), stream)
        _lib.check(st, "attn_bwd_deterministic")
    else:
        st = lib.attn_bwd_nondeterministic(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), mask,
                                           _ptr(dq), _ptr(dk), _ptr(dv), B, H, S, D, scale, int(tile_request),
                                           _ptr(workspace), workspace.numel(), stream)
        _lib.check(st, "attn_bwd_nondeterministic")
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, do, lse, causal: bool, schedule="descending", scale: float | None = None,
                tile_request: int = 0, out=None):
    """attn_bwd_deterministic_noalloc: the deterministic backward with the library's static
    scratch as its workspace (no device allocation in the call when `out` is given); plain
    heads only. Calls that overlap in time on one device race (they share the scratch)."""
    torch = _torch()
    B, H, Hkv, S, D = _check_heads(q, k, v, o, do)
    if Hkv != H:
        raise ValueError("bwd_noalloc takes one K/V head per query head")
    _check_lse(lse, q.shape)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dq, dk, dv = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)) if out is None else out
    mask = MASK_CAUSAL if causal else MASK_FULL
    st = _lib.load().attn_bwd_deterministic_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), mask,
                                                    _sched(schedule), _ptr(dq), _ptr(dk), _ptr(dv), B, H, S, D,
                                                    scale, int(tile_request), _stream_ptr(q.device))
    _lib.check(st, "attn_bwd_deterministic_noalloc")
    return dq, dk, dv


def check_workspace(workspace) -> None:
    """Synchronise the current stream; raise AttnError if a dQ ordering wait timed out."""
    st = _lib.load().attn_bwd_check(_ptr(workspace), workspace.numel(), _stream_ptr(workspace.device))
    _lib.check(st, "attn_bwd_check")


def schedule_plan(n_tiles: int, causal: bool, schedule):
    """One head's plan as exported by the library: (n_workers, [(worker, step, q, kv, rank), ...])."""
    lib = _lib.load()
    mask = MASK_CAUSAL if causal else MASK_FULL
    need = ctypes.c_size_t(0)
    _lib.check(lib.attn_schedule_plan(int(n_tiles), mask, _sched(schedule), None, 0, ctypes.byref(need)),
               "attn_schedule_plan")
    buf = (ctypes.c_int32 * need.value)()
    _lib.check(lib.attn_schedule_plan(int(n_tiles), mask, _sched(schedule), buf, need.value, None),
               "attn_schedule_plan")
    vals = list(buf)
    n_workers, n_tasks = vals[0], vals[1]
    recs = [tuple(vals[2 + 5 * t: 7 + 5 * t]) for t in range(n_tasks)]
    return n_workers, recs


DQ_PROTOCOLS = {"auto": 0, "device": 1, "xcd_local": 2}


def set_dq_protocol(protocol="auto") -> None:
    """Debug: force the dQ hand-off protocol of deterministic calls ("auto", "device", "xcd_local")."""
    _lib.check(_lib.load().attn_debug_set_dq_protocol(DQ_PROTOCOLS[protocol]), "attn_debug_set_dq_protocol")


def set_wait_limit(iterations: int = 0, poison: bool = False) -> None:
    """Debug: bound on one dQ ordering wait (0 = default) and flag poisoning for the next calls."""
    _lib.load().attn_debug_set_wait_limit(int(iterations), 1 if poison else 0)


def wait_timeouts(reset: bool = True) -> int:
    """Synchronise the device; bounded waits that ran out since the last reset, in any call of this process."""
    n = _lib.load().attn_debug_wait_timeouts(1 if reset else 0)
    _lib.check(n if n < 0 else 0, "attn_debug_wait_timeouts")
    return n
