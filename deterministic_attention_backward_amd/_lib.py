"""ctypes loader for libattn_det.so (the C ABI declared in include/attn_det.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any operation.
"""

from __future__ import annotations

import ctypes
import os

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libattn_det.so")
PROFILE_LIB_PATH = os.path.join(_PKG_DIR, "libattn_det_profile.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_WORKSPACE = -3
ERR_ALIGNMENT = -4
ERR_HIP = -5
ERR_TIMEOUT = -6
ERR_SCRATCH_LIMIT = -7
NOALLOC_SCRATCH_BYTES = 128 << 20  # ATTN_NOALLOC_SCRATCH_MIB
WAIT_PROFILE_VALUES = 9  # uint64 values per workgroup from attn_debug_wait_profile

MASK_FULL, MASK_CAUSAL = 0, 1
SCHED_NAIVE, SCHED_DESCENDING, SCHED_SHIFT, SCHED_SYMMETRIC_SHIFT = 0, 1, 2, 3

EXPORTS = (
    "attn_status_string",
    "attn_fwd",
    "attn_bwd_tile",
    "attn_bwd_workspace_size",
    "attn_bwd_deterministic",
    "attn_bwd_nondeterministic",
    "attn_bwd_deterministic_noalloc",
    "attn_bwd_check",
    "attn_fwd_gqa",
    "attn_bwd_gqa_workspace_size",
    "attn_bwd_deterministic_gqa",
    "attn_bwd_nondeterministic_gqa",
    "attn_schedule_plan",
    "attn_debug_set_wait_limit",
    "attn_set_timing_events",
    "attn_debug_set_dq_protocol",
    "attn_probe_mfma",
    "attn_probe_atomic",
    "attn_debug_wait_profile",
    "attn_debug_wait_timeouts",
    "attn_debug_order_violations",
)

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


def load() -> ctypes.CDLL:
    """Load (once) and type the shared library; raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = _open(LIB_PATH)
    return _lib


_profile_lib = None


def load_profile() -> ctypes.CDLL:
    """The profiling build (dQ-turn and barrier wait cycles); raises if it is missing."""
    global _profile_lib
    if _profile_lib is None:
        _profile_lib = _open(PROFILE_LIB_PATH)
    return _profile_lib


def _open(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with "
            "`python -m deterministic_attention_backward_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_status_string.argtypes = [i]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.attn_fwd.restype = i
    lib.attn_bwd_tile.argtypes = [i, i, i]
    lib.attn_bwd_tile.restype = i
    lib.attn_bwd_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.attn_bwd_workspace_size.restype = sz
    lib.attn_bwd_deterministic.argtypes = [vp, vp, vp, vp, vp, vp, i, i, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp]
    lib.attn_bwd_deterministic.restype = i
    lib.attn_bwd_nondeterministic.argtypes = [vp, vp, vp, vp, vp, vp, i, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp]
    lib.attn_bwd_nondeterministic.restype = i
    lib.attn_bwd_deterministic_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.attn_bwd_deterministic_noalloc.restype = i
    lib.attn_bwd_check.argtypes = [vp, sz, vp]
    lib.attn_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.attn_fwd_gqa.restype = i
    lib.attn_bwd_gqa_workspace_size.argtypes = [i, i, i, i, i, i, i, i]
    lib.attn_bwd_gqa_workspace_size.restype = sz
    lib.attn_bwd_deterministic_gqa.argtypes = [vp, vp, vp, vp, vp, vp, i, i, vp, vp, vp, i, i, i, i, i, f, i, vp,
                                               sz, vp]
    lib.attn_bwd_deterministic_gqa.restype = i
    lib.attn_bwd_nondeterministic_gqa.argtypes = [vp, vp, vp, vp, vp, vp, i, vp, vp, vp, i, i, i, i, i, f, i, vp,
                                                  sz, vp]
    lib.attn_bwd_nondeterministic_gqa.restype = i
    lib.attn_bwd_check.restype = i
    lib.attn_schedule_plan.argtypes = [i, i, i, ctypes.POINTER(ctypes.c_int32), sz, ctypes.POINTER(sz)]
    lib.attn_schedule_plan.restype = i
    lib.attn_debug_set_wait_limit.argtypes = [ctypes.c_uint32, i]
    lib.attn_debug_set_wait_limit.restype = None
    lib.attn_set_timing_events.argtypes = [vp, vp]
    lib.attn_set_timing_events.restype = None
    lib.attn_debug_set_dq_protocol.argtypes = [i]
    lib.attn_debug_set_dq_protocol.restype = i
    lib.attn_probe_mfma.argtypes = [i, vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    lib.attn_probe_mfma.restype = i
    lib.attn_probe_atomic.argtypes = [vp, ctypes.c_size_t, i, vp, ctypes.POINTER(ctypes.c_double)]
    lib.attn_probe_atomic.restype = i
    lib.attn_debug_wait_profile.argtypes = [ctypes.POINTER(ctypes.c_uint64), i]
    lib.attn_debug_wait_profile.restype = i
    lib.attn_debug_wait_timeouts.argtypes = [i]
    lib.attn_debug_wait_timeouts.restype = i
    lib.attn_debug_order_violations.argtypes = [i]
    lib.attn_debug_order_violations.restype = i
    return lib


def status_string(status: int) -> str:
    return load().attn_status_string(int(status)).decode()


def check(status: int, what: str) -> None:
    if status != OK:
        raise AttnError(status, what)
