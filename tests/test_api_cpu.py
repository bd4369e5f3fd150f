"""Host-side checks of the C-ABI library: no GPU needed, no compute call made.

* the library loads and exports every function include/attn_det.h declares;
* argument validation returns the documented status before any HIP call;
* workspace sizing and tile choice;
* the schedule the library exports (the same formulas its kernels evaluate)
  equals the oracle's schedule, task for task and rank for rank.
"""

import ctypes
import os
import re

import pytest

import deterministic_attention_backward_amd as dab
from deterministic_attention_backward_amd import _lib
from oracle import schedule as Sch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_det.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|void|const char\*)\s+(attn_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(_lib.EXPORTS)


def test_header_constants_match_the_binding():
    text = open(HEADER).read()
    want = {"ATTN_WAIT_PROFILE_VALUES": _lib.WAIT_PROFILE_VALUES,
            "ATTN_NOALLOC_SCRATCH_MIB": _lib.NOALLOC_SCRATCH_BYTES >> 20}
    for name, value in want.items():
        m = re.search(rf"^#define\s+{name}\s+(\d+)", text, re.M)
        assert m and int(m.group(1)) == value, name


def test_atomic_probe_validates_before_any_hip_call():
    lib = _lib.load()
    g = ctypes.c_double()
    assert lib.attn_probe_atomic(None, 1 << 20, 10, None, ctypes.byref(g)) == _lib.ERR_INVALID_ARG
    assert lib.attn_probe_atomic(ctypes.c_void_p(4096), 100, 10, None, ctypes.byref(g)) == _lib.ERR_INVALID_ARG
    assert lib.attn_probe_atomic(ctypes.c_void_p(4096), 1 << 20, 0, None, ctypes.byref(g)) == _lib.ERR_INVALID_ARG
    assert lib.attn_probe_atomic(ctypes.c_void_p(4096 + 16), 1 << 20, 10, None, ctypes.byref(g)) == _lib.ERR_ALIGNMENT
    assert lib.attn_probe_atomic(ctypes.c_void_p(4096), 1 << 20, 10, None, None) == _lib.ERR_INVALID_ARG


def test_status_strings():
    for st in range(-7, 1):
        assert _lib.status_string(st) not in ("", "unknown status")
    assert _lib.status_string(-99) == "unknown status"


def test_tile_choice():
    lib = _lib.load()
    assert lib.attn_bwd_tile(256, 64, 0) == 64
    assert lib.attn_bwd_tile(257, 64, 0) == 128
    assert lib.attn_bwd_tile(4096, 128, 0) == 128
    assert lib.attn_bwd_tile(4096, 128, 64) == 64
    assert lib.attn_bwd_tile(100, 128, 128) == 128
    assert lib.attn_bwd_tile(100, 96, 0) == _lib.ERR_UNSUPPORTED
    assert lib.attn_bwd_tile(100, 64, 32) == _lib.ERR_INVALID_ARG
    assert lib.attn_bwd_tile(0, 64, 0) == _lib.ERR_INVALID_ARG


def test_order_checks_only_in_profiling_build():
    # the regular build carries no ordering checks and says so without touching a device
    assert _lib.load().attn_debug_order_violations(0) == _lib.ERR_UNSUPPORTED


def test_workspace_size():
    B, H, S, D = 4, 16, 2048, 128
    n = dab.workspace_size(B, H, S, D, False, "naive")
    # at least the fp32 dQ accumulator plus the two per-row fp32 vectors
    assert n >= B * H * S * D * 4 + 2 * B * H * S * 4
    assert n < B * H * S * D * 4 * 1.1
    # ragged S is padded to whole tiles
    assert dab.workspace_size(1, 1, 1000, 128, False) >= 1024 * 128 * 4
    # Symmetric Shift adds the parking area
    assert dab.workspace_size(4, 32, 4096, 128, True, "symmetric_shift") > dab.workspace_size(
        4, 32, 4096, 128, True, "descending")
    assert _lib.load().attn_bwd_workspace_size(1, 1, 128, 96, 0, 0, 0) == 0


class FakePtr:
    """16-byte aligned fake device addresses: validation must reject before dereferencing."""

    def __init__(self, base=1 << 20):
        self.base = base

    def __call__(self, k):
        return ctypes.c_void_p(self.base + 4096 * k)


def call_det(**over):
    lib = _lib.load()
    p = FakePtr()
    args = dict(q=p(1), k=p(2), v=p(3), o=p(4), dout=p(5), lse=p(6), mask=0, schedule=0, dq=p(7), dk=p(8),
                dv=p(9), B=1, H=2, S=256, D=64, scale=0.125, tile=0, ws=p(10), ws_bytes=1 << 30, stream=None)
    args.update(over)
    return lib.attn_bwd_deterministic(*args.values())


def test_validation_before_any_hip_call():
    # every case below must return its status without touching the (fake) pointers
    assert call_det(q=None) == _lib.ERR_INVALID_ARG
    assert call_det(dv=None) == _lib.ERR_INVALID_ARG
    assert call_det(B=0) == _lib.ERR_INVALID_ARG
    assert call_det(S=-3) == _lib.ERR_INVALID_ARG
    assert call_det(mask=2) == _lib.ERR_INVALID_ARG
    assert call_det(schedule=7) == _lib.ERR_INVALID_ARG
    assert call_det(tile=100) == _lib.ERR_INVALID_ARG
    assert call_det(scale=float("nan")) == _lib.ERR_INVALID_ARG
    assert call_det(D=96) == _lib.ERR_UNSUPPORTED
    assert call_det(schedule=_lib.SCHED_SYMMETRIC_SHIFT, mask=_lib.MASK_FULL) == _lib.ERR_UNSUPPORTED
    # odd tile count: S = 192 with T = 64 -> N = 3
    assert call_det(schedule=_lib.SCHED_SYMMETRIC_SHIFT, mask=_lib.MASK_CAUSAL, S=192) == _lib.ERR_UNSUPPORTED
    assert call_det(q=ctypes.c_void_p((1 << 20) + 8)) == _lib.ERR_ALIGNMENT
    assert call_det(ws=None) == _lib.ERR_WORKSPACE
    assert call_det(ws_bytes=1024) == _lib.ERR_WORKSPACE
    assert call_det(ws=ctypes.c_void_p((1 << 20) + 16)) == _lib.ERR_ALIGNMENT


def call_noalloc(**over):
    lib = _lib.load()
    p = FakePtr()
    args = dict(q=p(1), k=p(2), v=p(3), o=p(4), dout=p(5), lse=p(6), mask=0, schedule=0, dq=p(7), dk=p(8),
                dv=p(9), B=1, H=2, S=256, D=64, scale=0.125, tile=0, stream=None)
    args.update(over)
    return lib.attn_bwd_deterministic_noalloc(*args.values())


def test_noalloc_validation_before_any_hip_call():
    # the allocation-free entry point validates like the workspace one, then refuses
    # problems whose workspace exceeds its static scratch, all before any HIP call
    assert call_noalloc(q=None) == _lib.ERR_INVALID_ARG
    assert call_noalloc(B=0) == _lib.ERR_INVALID_ARG
    assert call_noalloc(D=96) == _lib.ERR_UNSUPPORTED
    assert call_noalloc(schedule=_lib.SCHED_SYMMETRIC_SHIFT, mask=_lib.MASK_FULL) == _lib.ERR_UNSUPPORTED
    assert call_noalloc(dk=ctypes.c_void_p((1 << 20) + 8)) == _lib.ERR_ALIGNMENT
    lib = _lib.load()
    # 4 x 32 x 4096 x 128: the fp32 dQ accumulator alone is 256 MiB
    assert lib.attn_bwd_workspace_size(4, 32, 4096, 128, 1, 2, 0) > _lib.NOALLOC_SCRATCH_BYTES
    assert call_noalloc(B=4, H=32, S=4096, D=128, mask=1, schedule=2) == _lib.ERR_SCRATCH_LIMIT
    # the largest sizes it takes are stated in the header: 4 x 16 x 2048 x 128 fits
    assert lib.attn_bwd_workspace_size(4, 16, 2048, 128, 0, 2, 0) <= _lib.NOALLOC_SCRATCH_BYTES
    assert "static scratch" in _lib.status_string(_lib.ERR_SCRATCH_LIMIT)


def test_fwd_validation():
    lib = _lib.load()
    p = FakePtr()
    assert lib.attn_fwd(None, p(1), p(2), p(3), p(4), 1, 1, 64, 64, 0.1, 0, None) == _lib.ERR_INVALID_ARG
    assert lib.attn_fwd(p(0), p(1), p(2), p(3), p(4), 1, 1, 64, 80, 0.1, 0, None) == _lib.ERR_UNSUPPORTED
    assert lib.attn_fwd(p(0), p(1), p(2), p(3), p(4), 1, 1, 64, 64, 0.1, 5, None) == _lib.ERR_INVALID_ARG
    assert lib.attn_fwd(p(0), p(1), ctypes.c_void_p((1 << 20) + 4), p(3), p(4), 1, 1, 64, 64, 0.1, 0,
                        None) == _lib.ERR_ALIGNMENT


def call_gqa(**over):
    lib = _lib.load()
    p = FakePtr()
    args = dict(q=p(1), k=p(2), v=p(3), o=p(4), dout=p(5), lse=p(6), mask=0, schedule=0, dq=p(7), dk=p(8),
                dv=p(9), B=1, H=4, Hkv=2, S=256, D=64, scale=0.125, tile=0, ws=p(10), ws_bytes=1 << 30, stream=None)
    args.update(over)
    return lib.attn_bwd_deterministic_gqa(*args.values())


def test_grouped_validation_and_workspace():
    lib = _lib.load()
    assert call_gqa(Hkv=3) == _lib.ERR_INVALID_ARG          # 4 query heads cannot share 3 K/V heads evenly
    assert call_gqa(Hkv=0) == _lib.ERR_INVALID_ARG
    assert call_gqa(dk=None) == _lib.ERR_INVALID_ARG
    assert call_gqa(D=96) == _lib.ERR_UNSUPPORTED
    assert call_gqa(ws_bytes=1024) == _lib.ERR_WORKSPACE
    p = FakePtr()
    assert lib.attn_fwd_gqa(p(0), p(1), p(2), p(3), p(4), 1, 4, 3, 64, 64, 0.1, 0, None) == _lib.ERR_INVALID_ARG
    assert lib.attn_bwd_gqa_workspace_size(1, 6, 4, 256, 64, 0, 0, 0) == 0
    # sharing K/V heads adds the per-query-head fp32 dK and dV (two [B, H, S_pad, D] tensors)
    B, H, S, D = 2, 8, 1000, 128
    plain = lib.attn_bwd_gqa_workspace_size(B, H, H, S, D, 1, 2, 0)
    assert plain == lib.attn_bwd_workspace_size(B, H, S, D, 1, 2, 0)
    assert lib.attn_bwd_gqa_workspace_size(B, H, 2, S, D, 1, 2, 0) >= plain + 2 * B * H * 1024 * D * 4


def plan_cases():
    for N in (1, 2, 3, 4, 5, 6, 8, 16, 31, 32, 64, 128):
        yield N, False, Sch.NAIVE
        yield N, False, Sch.DESCENDING
        yield N, False, Sch.SHIFT
        yield N, True, Sch.NAIVE
        yield N, True, Sch.DESCENDING
        yield N, True, Sch.SHIFT
        if N % 2 == 0:
            yield N, True, Sch.SYMMETRIC_SHIFT


@pytest.mark.parametrize("N,causal,sched", list(plan_cases()))
def test_plan_matches_oracle(N, causal, sched):
    n_workers, recs = dab.schedule_plan(N, causal, sched)
    ref = Sch.build(N, causal, sched)
    assert n_workers == len(ref.workers)
    assert sorted(recs) == ref.records()


def test_plan_rejections():
    lib = _lib.load()
    need = ctypes.c_size_t(0)
    assert lib.attn_schedule_plan(0, 0, 0, None, 0, ctypes.byref(need)) == _lib.ERR_INVALID_ARG
    assert lib.attn_schedule_plan(5, 1, _lib.SCHED_SYMMETRIC_SHIFT, None, 0, None) == _lib.ERR_UNSUPPORTED
    assert lib.attn_schedule_plan(4, 0, 0, None, 0, ctypes.byref(need)) == 0 and need.value == 2 + 5 * 16
    buf = (ctypes.c_int32 * 10)()
    assert lib.attn_schedule_plan(4, 0, 0, buf, 10, None) == _lib.ERR_INVALID_ARG


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.load()
