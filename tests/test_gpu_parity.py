"""GPU parity of the HIP path against the float64 oracle (MI355X only).

Small shapes (several tiles, ragged tails, both masks, both head sizes, both
tile edges) are compared element by element: every deterministic schedule and
the atomic variant must meet max|x - ref| <= 2e-2 and
||x - ref||_2 / ||ref||_2 <= 5e-3 for dQ, dK and dV. The oracle backward and
the HIP backward consume the same O and LSE (the HIP forward's), and the HIP
forward is checked against the oracle forward separately.
"""

import hashlib
import math
import sys

import numpy as np
import pytest
import torch

import attn_inputs
import deterministic_attention_backward_amd as dab
from oracle import attention as A

pytestmark = pytest.mark.gpu

TOL_ABS = 2e-2
TOL_REL = 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().float().cpu().double().numpy()


def assert_close(name, got, ref, tol_abs=TOL_ABS, tol_rel=TOL_REL):
    mx, rel = A.compare(got, ref)
    assert mx <= tol_abs and rel <= tol_rel, f"{name}: max_abs={mx:.3e} rel_l2={rel:.3e}"
    return mx, rel


class Case:
    """Inputs on the GPU, HIP forward outputs, and the oracle's gradients from them."""

    def __init__(self, B, H, S, D, causal, seed):
        torch.cuda.init()
        self.B, self.H, self.S, self.D, self.causal = B, H, S, D, causal
        self.scale = 1.0 / math.sqrt(D)
        x = attn_inputs.draw(B, H, S, D, seed)
        self.q, self.k, self.v, self.do = (x[n].cuda() for n in ("q", "k", "v", "do"))
        self.o, self.lse = dab.fwd(self.q, self.k, self.v, causal)
        torch.cuda.synchronize()
        self.nq, self.nk, self.nv, self.ndo = (f64(t) for t in (self.q, self.k, self.v, self.do))
        self.no, self.nlse = f64(self.o), f64(self.lse)
        self._ref = None

    def ref(self):
        if self._ref is None:
            self._ref = A.backward(self.nq, self.nk, self.nv, self.no, self.ndo, self.nlse, self.causal, self.scale)
        return self._ref

    def run(self, schedule=None, tile=0, out=None):
        if schedule is None:
            g = dab.bwd_nondeterministic(self.q, self.k, self.v, self.o, self.do, self.lse, self.causal,
                                         tile_request=tile, out=out)
        else:
            ws = dab.alloc_workspace(self.B, self.H, self.S, self.D, self.causal, schedule, tile)
            g = dab.bwd(self.q, self.k, self.v, self.o, self.do, self.lse, self.causal, schedule,
                        tile_request=tile, workspace=ws, out=out)
            dab.check_workspace(ws)
        torch.cuda.synchronize()
        return g


def schedules_for(S, D, causal, tile):
    T = dab.tile(S, D, tile)
    N = -(-S // T)
    out = ["naive", "descending", "shift"]
    if causal and N % 2 == 0:
        out.append("symmetric_shift")
    return out + [None]


# (B, H, S, D, causal, seed, tile)
SMALL = [
    (1, 2, 256, 64, False, 1, 64),     # the small full-mask workload, 64x64 tiles (N = 4)
    (1, 2, 256, 64, True, 1, 64),
    (2, 2, 1000, 128, False, 11, 0),   # ragged: N = 8 at T = 128
    (1, 3, 1000, 128, True, 12, 0),
    (1, 2, 700, 64, True, 13, 0),      # N = 6, ragged, D = 64 with 128-row sub-tiles
    (1, 2, 333, 64, False, 14, 0),     # N = 3 (odd)
    (2, 1, 512, 128, True, 15, 64),    # T = 64 with D = 128, N = 8
    (1, 2, 640, 64, False, 16, 128),
    (1, 1, 1, 64, False, 17, 0),       # a single position
    (1, 1, 1, 128, True, 18, 0),
    (1, 2, 17, 128, True, 19, 0),      # shorter than one tile
    (1, 1, 130, 64, True, 20, 128),    # N = 2, one full tile and a 2-row tail
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%dH%dS%dD%d%s_t%d" % (c[0], c[1], c[2], c[3],
                                                                              "c" if c[4] else "f", c[6]))
def test_forward_parity(case):
    B, H, S, D, causal, seed, tile = case
    say(f"forward parity {case}")
    c = Case(B, H, S, D, causal, seed)
    o_ref, lse_ref = A.forward(c.nq, c.nk, c.nv, causal, c.scale)
    assert_close("O", c.no, o_ref)
    assert np.abs(c.nlse - lse_ref).max() <= 1e-3


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%dH%dS%dD%d%s_t%d" % (c[0], c[1], c[2], c[3],
                                                                              "c" if c[4] else "f", c[6]))
@pytest.mark.parametrize("protocol", ["auto", "device"])
def test_backward_parity(case, protocol):
    B, H, S, D, causal, seed, tile = case
    c = Case(B, H, S, D, causal, seed)
    dq_r, dk_r, dv_r = c.ref()
    try:
        dab.set_dq_protocol(protocol)
        for sched in schedules_for(S, D, causal, tile):
            say(f"backward parity {case} schedule={sched or 'atomic'} dq protocol={protocol}")
            dq, dk, dv = c.run(sched, tile)
            for name, g, r in (("dQ", dq, dq_r), ("dK", dk, dk_r), ("dV", dv, dv_r)):
                assert_close(f"{sched or 'atomic'} {name}", f64(g), r)
    finally:
        dab.set_dq_protocol("auto")


# Grids smaller than 8 x the workers of a head, so that some XCD queues have a
# single workgroup, and head counts that leave the last run of interleaved
# heads (naive, Descending) partial: every unit must still run exactly once,
# whichever queue claims which heads first.
SMALL_GRID = [
    (1, 5, 300, 64, False, 41),   # 3 workers per head, 15 units: runs of 4 heads, the last one partial
    (1, 5, 300, 64, True, 42),
    (1, 7, 200, 128, True, 43),   # 2 workers per head, 14 units
    (2, 3, 130, 128, False, 44),  # 2 workers per head, 12 units
]


@pytest.mark.parametrize("case", SMALL_GRID, ids=lambda c: "B%dH%dS%dD%d%s" % (c[0], c[1], c[2], c[3],
                                                                                "c" if c[4] else "f"))
def test_small_grids_run_every_unit(case):
    B, H, S, D, causal, seed = case
    c = Case(B, H, S, D, causal, seed)
    dq_r, dk_r, dv_r = c.ref()
    for sched in ("naive", "descending"):
        say(f"small grid {case} schedule={sched}")
        first = c.run(sched)
        for name, g, r in (("dQ", first[0], dq_r), ("dK", first[1], dk_r), ("dV", first[2], dv_r)):
            assert_close(f"{sched} {name}", f64(g), r)
        for _ in range(5):  # (which queue claims which heads differs from call to call)
            again = c.run(sched)
            assert all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(first, again))


DET_CASES = [
    (2, 4, 1024, 128, False, 31),
    (2, 4, 1024, 128, True, 32),
    (1, 4, 2048, 64, True, 33),
]


@pytest.mark.parametrize("case", DET_CASES, ids=lambda c: "B%dH%dS%dD%d%s" % (c[0], c[1], c[2], c[3],
                                                                              "c" if c[4] else "f"))
@pytest.mark.parametrize("protocol", ["auto", "device"])
def test_bitwise_reproducible_20_runs(case, protocol):
    B, H, S, D, causal, seed = case
    c = Case(B, H, S, D, causal, seed)
    try:
        dab.set_dq_protocol(protocol)
        for sched in schedules_for(S, D, causal, 0)[:-1]:
            say(f"determinism {case} schedule={sched} dq protocol={protocol}")
            digests = set()
            for _ in range(20):
                out = tuple(torch.full_like(c.q, float("nan")) for _ in range(3))
                dq, dk, dv = c.run(sched, 0, out=out)
                h = hashlib.sha256()
                for t in (dq, dk, dv):
                    h.update(t.view(torch.int16).cpu().numpy().tobytes())
                digests.add(h.hexdigest())
            assert len(digests) == 1, f"{sched}: {len(digests)} distinct results in 20 runs"
    finally:
        dab.set_dq_protocol("auto")


def test_forward_bitwise_reproducible():
    c = Case(1, 4, 1500, 128, True, 41)
    ref = (c.o.clone(), c.lse.clone())
    for _ in range(5):
        o, lse = dab.fwd(c.q, c.k, c.v, True)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref[0].view(torch.int16))
        assert torch.equal(lse.view(torch.int32), ref[1].view(torch.int32))


@pytest.mark.expects_timeout
def test_wait_bound_reports_timeout():
    # a poisoned counter can never reach its turn; the bounded wait must give up,
    # record the timeout and let every workgroup finish normally
    c = Case(1, 2, 512, 64, False, 51)
    ws = dab.alloc_workspace(1, 2, 512, 64, False, "naive", 0)
    say("timeout path: poisoned counter, wait bound 2000 iterations")
    dab.wait_timeouts(reset=True)
    try:
        dab.set_wait_limit(2000, poison=True)
        dq, dk, dv = dab.bwd(c.q, c.k, c.v, c.o, c.do, c.lse, False, "naive", workspace=ws)
        # the failure shows in the gradients themselves, with no host check
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            assert bool(torch.isnan(t.float()).all()), f"{name} of a call whose wait ran out is not all NaN"
        with pytest.raises(dab.AttnError) as err:
            dab.check_workspace(ws)
        assert err.value.status == -6
    finally:
        dab.set_wait_limit(0, poison=False)
    # the process-wide count saw it too (one dQ wave per expired wait and workgroup)
    assert dab.wait_timeouts(reset=True) >= 1
    # the next call is clean again
    dq, dk, dv = c.run("naive")
    assert dab.wait_timeouts(reset=False) == 0
    dq_r, dk_r, dv_r = c.ref()
    assert_close("dQ after timeout", f64(dq), dq_r)


def test_rejects_unsupported_on_device():
    c = Case(1, 1, 384, 64, True, 61)  # N = 3: Symmetric Shift needs an even tile count
    with pytest.raises(dab.AttnError):
        dab.bwd(c.q, c.k, c.v, c.o, c.do, c.lse, True, "symmetric_shift")


@pytest.mark.parametrize("sched", ["naive", "shift"])
def test_workspace_reuse_sees_fresh_accumulators(sched):
    # One workspace, many calls with different inputs: every call's dQ must match
    # the atomic variant's on the same inputs (a running sum left in a cache by an
    # earlier call, or by an earlier contributor, would show up as a large error).
    B, H, S, D = 2, 8, 2048, 128
    ws = dab.alloc_workspace(B, H, S, D, False, sched)
    for seed in range(80, 86):
        x = attn_inputs.draw(B, H, S, D, seed)
        q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
        o, lse = dab.fwd(q, k, v, False)
        say(f"workspace reuse: schedule={sched} seed={seed}")
        dq, dk, dv = dab.bwd(q, k, v, o, do, lse, False, sched, workspace=ws)
        dab.check_workspace(ws)
        rq, rk, rv = dab.bwd_nondeterministic(q, k, v, o, do, lse, False)
        torch.cuda.synchronize()
        for name, a, b in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
            err = (a.float() - b.float()).abs().max().item()
            assert err <= 2e-2, f"{sched} seed {seed} {name}: {err:.3e}"


@pytest.mark.parametrize("scale", [0.0, -0.7], ids=["zero", "negative"])
@pytest.mark.parametrize("case", [(1, 2, 300, 128, True, 83), (1, 2, 200, 64, False, 84)],
                         ids=lambda c: "B%dH%dS%dD%d%s" % (c[0], c[1], c[2], c[3], "c" if c[4] else "f"))
def test_forward_with_a_zero_or_negative_scale(case, scale):
    """The forward tracks the row maximum of the scaled scores: with a negative
    scale that is the smallest raw score, and with a zero scale every visible
    key gets the same weight while masked keys (the diagonal tiles and the
    ragged tail) must still get none."""
    B, H, S, D, causal, seed = case
    scale = scale / math.sqrt(D)
    say(f"forward with scale {scale:.4f}: B={B} H={H} S={S} D={D} causal={causal}")
    x = attn_inputs.draw(B, H, S, D, seed)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o, lse = dab.fwd(q, k, v, causal, scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = A.forward(f64(q), f64(k), f64(v), causal, scale)
    assert_close("O", f64(o), o_ref)
    assert np.abs(f64(lse) - lse_ref).max() <= 1e-3


@pytest.mark.parametrize("case", [(1, 3, 300, 128, True, 81), (2, 2, 256, 64, False, 82)],
                         ids=lambda c: "B%dH%dS%dD%d%s" % (c[0], c[1], c[2], c[3], "c" if c[4] else "f"))
def test_parity_with_a_caller_softmax_scale(case):
    """A softmax scale other than 1/sqrt(D) reaches every step: the forward's
    scores and LSE, the backward's P (through scale log2 e) and dK's factor.
    The scale is 0.6 / sqrt(D), below the default, so the gradients are no
    larger than at the default scale and the target's tolerance applies as
    it stands (a kernel that used the default scale instead would miss by
    far more)."""
    B, H, S, D, causal, seed = case
    scale = 0.6 / math.sqrt(D)
    say(f"caller scale {scale:.4f}: B={B} H={H} S={S} D={D} causal={causal}")
    x = attn_inputs.draw(B, H, S, D, seed)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = dab.fwd(q, k, v, causal, scale)
    torch.cuda.synchronize()
    nq, nk, nv, ndo, no, nlse = (f64(t) for t in (q, k, v, do, o, lse))
    o_ref, lse_ref = A.forward(nq, nk, nv, causal, scale)
    assert_close("O", no, o_ref)
    assert np.abs(nlse - lse_ref).max() <= 1e-3
    dq_r, dk_r, dv_r = A.backward(nq, nk, nv, no, ndo, nlse, causal, scale)
    N = -(-S // dab.tile(S, D))
    scheds = ["naive", "descending", "shift"] + (["symmetric_shift"] if causal and N % 2 == 0 else [])
    for sched in scheds + [None]:
        say(f"caller scale {scale:.4f}: schedule={sched or 'atomic'}")
        if sched is None:
            dq, dk, dv = dab.bwd_nondeterministic(q, k, v, o, do, lse, causal, scale)
        else:
            dq, dk, dv = dab.bwd(q, k, v, o, do, lse, causal, sched, scale)
        torch.cuda.synchronize()
        for name, g, r in (("dQ", dq, dq_r), ("dK", dk, dk_r), ("dV", dv, dv_r)):
            assert_close(f"{sched or 'atomic'} {name}", f64(g), r)


def test_calls_run_on_the_callers_stream():
    """Forward and backward issued under a side stream (default priority)
    give the default stream's bits: every launch and the workspace set-up go
    to the caller's stream, in order."""
    B, H, S, D = 2, 4, 640, 128
    say(f"side stream: B={B} H={H} S={S} D={D}")
    x = attn_inputs.draw(B, H, S, D, 91)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = dab.fwd(q, k, v, True)
    ref = dab.bwd(q, k, v, o, do, lse, True, "shift")
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o2, lse2 = dab.fwd(q, k, v, True)
        got = dab.bwd(q, k, v, o2, do, lse2, True, "shift")
        nondet = dab.bwd_nondeterministic(q, k, v, o2, do, lse2, True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)
    for a, b in zip(ref, got):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for a, b in zip(ref, nondet):
        assert (a.float() - b.float()).abs().max().item() <= 2e-2


def test_c1_with_oracle_forward_and_fp32_study():
    """The small full-mask workload exactly as configured: B=1, H=2, S=256,
    D=64, 64x64 tiles (N = 4), seed 1, O and LSE from the oracle's float64
    forward (O rounded to bf16, LSE to fp32), both schedules the
    configuration names (naive and Shift) plus the others and the atomic
    variant, against the float64 oracle backward fed the same O and LSE.

    The configuration draws float32 Q/K/V/dO; the kernel takes bf16, so both
    sides consume the bf16 roundings. The float64 oracle run on the unrounded
    float32 draws (its own forward and backward) is reported beside it: the
    gap between that and the HIP gradients is what rounding the inputs to
    bf16 costs, not a kernel error, and is only bounded loosely here."""
    w = attn_inputs.WORKLOADS["C1"]
    x = attn_inputs.draw_workload(w)
    to64 = attn_inputs.to_f64
    nq, nk, nv, ndo = (to64(x[n]) for n in ("q", "k", "v", "do"))
    o64, lse64 = A.forward(nq, nk, nv, w.causal, w.scale)
    o_bf = torch.from_numpy(o64).to(torch.bfloat16)
    lse_f = torch.from_numpy(lse64).to(torch.float32)
    ref = A.backward(nq, nk, nv, to64(o_bf), ndo, to64(lse_f), w.causal, w.scale)
    # the unrounded study: float32 draws, the oracle's own forward and backward
    q32, k32, v32, do32 = (to64(x[n + "32"]) for n in ("q", "k", "v", "do"))
    o32, lse32 = A.forward(q32, k32, v32, w.causal, w.scale)
    ref32 = A.backward(q32, k32, v32, o32, do32, lse32, w.causal, w.scale)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = o_bf.cuda(), lse_f.cuda()
    assert dab.tile(w.S, w.D, w.tile) == 64
    for sched in ["naive", "shift", "descending", None]:
        ws = dab.alloc_workspace(w.B, w.H, w.S, w.D, w.causal, sched or "naive", w.tile)
        say(f"C1 with the oracle forward's O/LSE: schedule={sched or 'atomic'}")
        if sched is None:
            g = dab.bwd_nondeterministic(q, k, v, o, do, lse, w.causal, w.scale, w.tile, ws)
        else:
            g = dab.bwd(q, k, v, o, do, lse, w.causal, sched, w.scale, w.tile, ws)
            dab.check_workspace(ws)
        torch.cuda.synchronize()
        for name, got, r, r32 in zip(("dQ", "dK", "dV"), g, ref, ref32):
            mx, rel = assert_close(f"C1 {sched or 'atomic'} {name}", f64(got), r)
            mx32, rel32 = A.compare(f64(got), r32)
            say(f"  {name}: vs bf16-input oracle max_abs={mx:.3e} rel_l2={rel:.3e}; "
                f"vs unrounded fp32-input oracle max_abs={mx32:.3e} rel_l2={rel32:.3e}")
            assert rel32 <= 5e-2, f"C1 {name}: the bf16 rounding of the inputs moved the result by {rel32:.3e}"
