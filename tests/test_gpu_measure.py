"""GPU checks of the measurement helpers: the MFMA probe and the profiling build.

The profiling build (ATTN_PROFILE_WAIT=1) only adds clock reads around waits,
so its gradients must be bit-identical to the regular library's.
"""

import ctypes

import pytest
import torch

import attn_inputs
import deterministic_attention_backward_amd as dab
from deterministic_attention_backward_amd import _lib

pytestmark = pytest.mark.gpu

K = _lib.WAIT_PROFILE_VALUES


def test_mfma_probe_is_plausible():
    lib = _lib.load()
    tf, ghz = ctypes.c_double(), ctypes.c_double()
    st = lib.attn_probe_mfma(20000, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream),
                             ctypes.byref(tf), ctypes.byref(ghz))
    assert st == 0
    print(f"probe: {tf.value:.1f} TFLOP/s at {ghz.value:.3f} GHz", flush=True)
    # dense bf16 peak of the part is about 2.5 PFLOP/s at 2.4 GHz
    assert 100.0 < tf.value < 3000.0
    assert 0.3 < ghz.value < 3.5
    assert lib.attn_debug_wait_profile((ctypes.c_uint64 * _lib.WAIT_PROFILE_VALUES)(), 1) == _lib.ERR_UNSUPPORTED


def test_atomic_probe_is_plausible():
    lib = _lib.load()
    buf = torch.zeros(1 << 22, dtype=torch.float32, device="cuda")  # 16 MiB: 4096 blocks of 4 KB
    g = ctypes.c_double()
    st = torch.cuda.current_stream().cuda_stream
    assert lib.attn_probe_atomic(ctypes.c_void_p(buf.data_ptr()), buf.numel() * 4, 20, ctypes.c_void_p(st),
                                 ctypes.byref(g)) == 0
    assert 10.0 < g.value < 100000.0
    # two launches (warm-up and timed) of 8 workgroups x 4 waves per CU, 20 rounds of 16 adds of 1.0 per lane
    torch.cuda.synchronize()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert float(buf.sum()) == 2 * n_cu * 8 * 4 * 64 * 20 * 16


@pytest.mark.parametrize("causal,sched", [(False, "shift"), (True, "symmetric_shift"), (True, "naive")])
def test_profiling_build_is_bitwise_identical(causal, sched):
    B, H, S, D = 1, 4, 1024, 128
    x = attn_inputs.draw(B, H, S, D, 71)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = dab.fwd(q, k, v, causal)
    ref = dab.bwd(q, k, v, o, do, lse, causal, sched)
    torch.cuda.synchronize()
    prof = _lib.load_profile()
    saved = _lib._lib
    try:
        _lib._lib = prof
        got = dab.bwd(q, k, v, o, do, lse, causal, sched)
        torch.cuda.synchronize()
        buf = (ctypes.c_uint64 * (K * 1024))()
        n = prof.attn_debug_wait_profile(buf, 1024)
    finally:
        _lib._lib = saved
    for a, b in zip(ref, got):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert n > 0
    rows = [[buf[K * g + j] for j in range(K)] for g in range(n)]
    assert sum(r[5] for r in rows) > 0            # sub-tiles were counted
    assert sum(r[7] for r in rows) > 0            # and segments
    assert all(r[2] <= r[4] and r[0] <= r[1] for r in rows)  # waits are part of the total
    # barriers, KV-tile switches and unit claims are disjoint parts of the tile wave's time
    assert all(r[0] + r[6] + r[8] <= r[1] for r in rows)


@pytest.mark.parametrize("protocol", ["xcd_local", "device"])
def test_profiling_build_dq_order_checks_pass(protocol):
    """Every dQ hand-off of every schedule keeps the fixed order: the profiling
    build counts a contributor that finds its tile counter past its rank while
    waiting, or moved by someone else before it hands over."""
    prof = _lib.load_profile()
    assert _lib.load().attn_debug_order_violations(0) == _lib.ERR_UNSUPPORTED
    saved = _lib._lib
    try:
        _lib._lib = prof
        dab.set_dq_protocol(protocol)
        prof.attn_debug_order_violations(1)
        prof.attn_debug_wait_timeouts(1)
        cases = [(1, 4, 4, 1024, 128), (1, 4, 4, 1024, 64), (1, 8, 2, 1024, 128), (1, 16, 16, 4096, 128)]
        for B, H, Hkv, S, D in cases:
            for causal in (False, True):
                x = attn_inputs.draw_grouped(B, H, Hkv, S, D, 73) if Hkv != H else attn_inputs.draw(B, H, S, D, 73)
                q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
                o, lse = dab.fwd(q, k, v, causal)
                for sched in ("naive", "descending", "shift") + (("symmetric_shift",) if causal else ()):
                    print(f"order checks: {protocol} B={B} H={H} Hkv={Hkv} S={S} D={D} "
                          f"causal={causal} {sched}", flush=True)
                    dab.bwd(q, k, v, o, do, lse, causal, sched)
                    torch.cuda.synchronize()
                    assert prof.attn_debug_order_violations(1) == 0, (B, H, Hkv, S, D, causal, sched)
        assert prof.attn_debug_wait_timeouts(1) == 0
    finally:
        dab.set_dq_protocol("auto")
        _lib._lib = saved
