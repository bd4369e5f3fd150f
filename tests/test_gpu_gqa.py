"""GPU parity of grouped-query attention (query heads sharing K/V heads).

The HIP forward and backward with Hkv < H are compared with the float64
oracle's grouped functions (oracle.attention.forward_grouped /
backward_grouped) element by element for every schedule and the atomic
variant; the group sum of dK/dV is bitwise reproducible over 20 runs; and a
grouped call with Hkv == H gives the plain call's bits.

Tolerance: relative L2 <= 5e-3 per tensor as for the plain path, and per
element |x - ref| <= 2e-2 + 2^-8 |ref|. The second term is the rounding of a
bf16 output (8 significant bits) of the element's own size: a K/V head's dK
and dV sum G query heads' contributions, so they grow up to G times larger
than in the plain case, where the fixed 2e-2 covers the rounding of elements
below about 4 in magnitude.
"""

import ctypes
import hashlib
import math
import sys

import numpy as np
import pytest
import torch

import attn_inputs
import deterministic_attention_backward_amd as dab
from deterministic_attention_backward_amd import _lib
from oracle import attention as A

pytestmark = pytest.mark.gpu

TOL_ABS = 2e-2
TOL_REL = 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().float().cpu().double().numpy()


def assert_close(name, got, ref):
    mx, rel = A.compare(got, ref)
    excess = float(np.max(np.abs(got - ref) - 2.0 ** -8 * np.abs(ref)))
    assert excess <= TOL_ABS and rel <= TOL_REL, f"{name}: max_abs={mx:.3e} beyond rounding={excess:.3e} rel_l2={rel:.3e}"


class GCase:
    def __init__(self, B, H, Hkv, S, D, causal, seed):
        torch.cuda.init()
        self.B, self.H, self.Hkv, self.S, self.D, self.causal = B, H, Hkv, S, D, causal
        self.scale = 1.0 / math.sqrt(D)
        x = attn_inputs.draw_grouped(B, H, Hkv, S, D, seed)
        self.q, self.k, self.v, self.do = (x[n].cuda() for n in ("q", "k", "v", "do"))
        self.o, self.lse = dab.fwd(self.q, self.k, self.v, causal)
        torch.cuda.synchronize()
        self.nq, self.nk, self.nv, self.ndo = (f64(t) for t in (self.q, self.k, self.v, self.do))
        self.no, self.nlse = f64(self.o), f64(self.lse)

    def ref(self):
        return A.backward_grouped(self.nq, self.nk, self.nv, self.no, self.ndo, self.nlse, self.causal, self.scale)

    def run(self, schedule, out=None):
        if schedule is None:
            g = dab.bwd_nondeterministic(self.q, self.k, self.v, self.o, self.do, self.lse, self.causal, out=out)
        else:
            ws = dab.alloc_workspace(self.B, self.H, self.S, self.D, self.causal, schedule, 0, Hkv=self.Hkv)
            g = dab.bwd(self.q, self.k, self.v, self.o, self.do, self.lse, self.causal, schedule, workspace=ws,
                        out=out)
            dab.check_workspace(ws)
        torch.cuda.synchronize()
        return g


# (B, H, Hkv, S, D, causal, seed)
CASES = [
    (1, 4, 2, 333, 128, False, 51),   # ragged, N = 3
    (2, 4, 1, 512, 128, True, 52),    # one K/V head for four query heads, N = 4
    (1, 6, 2, 700, 64, True, 53),     # D = 64, 128-row sub-tiles, N = 6
    (1, 8, 2, 256, 64, False, 54),    # 64x64 tiles (N = 4)
]


def schedules(S, D, causal):
    N = -(-S // dab.tile(S, D))
    out = ["naive", "descending", "shift"]
    if causal and N % 2 == 0:
        out.append("symmetric_shift")
    return out + [None]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dKV%dS%dD%d%s" % (c[0], c[1], c[2], c[3], c[4],
                                                                              "c" if c[5] else "f"))
@pytest.mark.parametrize("protocol", ["auto", "device"])
def test_grouped_forward_and_backward_parity(case, protocol):
    B, H, Hkv, S, D, causal, seed = case
    say(f"grouped parity {case} dq protocol={protocol}")
    c = GCase(B, H, Hkv, S, D, causal, seed)
    o_ref, lse_ref = A.forward_grouped(c.nq, c.nk, c.nv, causal, c.scale)
    assert_close("O", c.no, o_ref)
    assert np.abs(c.nlse - lse_ref).max() <= 1e-3
    dq_r, dk_r, dv_r = c.ref()
    try:
        dab.set_dq_protocol(protocol)
        for sched in schedules(S, D, causal):
            say(f"grouped parity {case} schedule={sched or 'atomic'} dq protocol={protocol}")
            dq, dk, dv = c.run(sched)
            assert tuple(dk.shape) == (B, Hkv, S, D) and tuple(dv.shape) == (B, Hkv, S, D)
            for name, g, r in (("dQ", dq, dq_r), ("dK", dk, dk_r), ("dV", dv, dv_r)):
                assert_close(f"{sched or 'atomic'} {name}", f64(g), r)
    finally:
        dab.set_dq_protocol("auto")


def test_grouped_bitwise_reproducible_20_runs():
    c = GCase(2, 8, 2, 1024, 128, True, 61)
    for sched in ("shift", "symmetric_shift"):
        say(f"grouped determinism schedule={sched}")
        digests = set()
        for _ in range(20):
            out = (torch.full_like(c.q, float("nan")), torch.full_like(c.k, float("nan")),
                   torch.full_like(c.v, float("nan")))
            dq, dk, dv = c.run(sched, out=out)
            h = hashlib.sha256()
            for t in (dq, dk, dv):
                h.update(t.view(torch.int16).cpu().numpy().tobytes())
            digests.add(h.hexdigest())
        assert len(digests) == 1, f"{sched}: {len(digests)} distinct results in 20 runs"


def test_grouped_entry_with_own_kv_heads_matches_plain_call():
    B, H, S, D = 1, 3, 400, 128
    x = attn_inputs.draw(B, H, S, D, 71)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = dab.fwd(q, k, v, True)
    plain = dab.bwd(q, k, v, o, do, lse, True, "shift")
    lib = _lib.load()
    ws = torch.empty(lib.attn_bwd_gqa_workspace_size(B, H, H, S, D, 1, 2, 0), dtype=torch.uint8, device="cuda")
    got = tuple(torch.empty_like(t) for t in (q, k, v))
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.attn_bwd_deterministic_gqa(p(q), p(k), p(v), p(o), p(do), p(lse), 1, 2, p(got[0]), p(got[1]), p(got[2]),
                                        B, H, H, S, D, 1.0 / math.sqrt(D), 0, p(ws), ws.numel(), stream)
    assert st == 0
    o2 = torch.empty_like(o)
    lse2 = torch.empty_like(lse)
    st = lib.attn_fwd_gqa(p(q), p(k), p(v), p(o2), p(lse2), B, H, H, S, D, 1.0 / math.sqrt(D), 1, stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16)) and torch.equal(lse2, lse)
    for a, b in zip(got, plain):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.expects_timeout
def test_grouped_timeout_writes_nan():
    """A grouped call whose dQ wait runs out writes NaN into dq and into the
    group-summed dk and dv (the group sum reads the call's failure flag)."""
    c = GCase(1, 4, 2, 512, 64, False, 57)
    ws = dab.alloc_workspace(c.B, c.H, c.S, c.D, False, "naive", 0, Hkv=c.Hkv)
    say("grouped timeout path: poisoned counter, wait bound 2000 iterations")
    try:
        dab.set_wait_limit(2000, poison=True)
        dq, dk, dv = dab.bwd(c.q, c.k, c.v, c.o, c.do, c.lse, False, "naive", workspace=ws)
        torch.cuda.synchronize()
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            assert bool(torch.isnan(t.float()).all()), f"{name} of a call whose wait ran out is not all NaN"
        with pytest.raises(dab.AttnError):
            dab.check_workspace(ws)
    finally:
        dab.set_wait_limit(0, poison=False)
    assert dab.wait_timeouts(reset=True) >= 1
    dq, dk, dv = c.run("naive")
    assert not bool(torch.isnan(dk.float()).any())
