"""The allocation-free backward entry point against the workspace one (MI355X only).

attn_bwd_deterministic_noalloc runs the same kernels as attn_bwd_deterministic
with the library's static device scratch as its workspace. Two calls in a
row, the second on a smaller problem (so it runs on whatever the first left
in the scratch), must each give the workspace entry point's bits and meet the
float64 oracle within max-abs 2e-2 and relative L2 5e-3.
"""

import math
import sys

import pytest
import torch

import attn_inputs
import deterministic_attention_backward_amd as dab
from deterministic_attention_backward_amd import _lib
from oracle import attention as A

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().float().cpu().double().numpy()


# (B, H, S, D, causal, schedule, seed): the second is smaller than the first
CALLS = [(2, 4, 1024, 128, True, "shift", 91), (1, 2, 384, 64, False, "naive", 92)]


def test_noalloc_matches_workspace_entry_point_twice():
    torch.cuda.init()
    for B, H, S, D, causal, sched, seed in CALLS:
        say(f"noalloc call: B={B} H={H} S={S} D={D} causal={causal} schedule={sched}")
        x = attn_inputs.draw(B, H, S, D, seed)
        q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
        o, lse = dab.fwd(q, k, v, causal)
        out = tuple(torch.full_like(q, float("nan")) for _ in range(3))
        torch.cuda.synchronize()
        got = dab.bwd_noalloc(q, k, v, o, do, lse, causal, sched, out=out)
        ref = dab.bwd(q, k, v, o, do, lse, causal, sched)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name}: not the workspace call's bits"
        oracle = A.backward(f64(q), f64(k), f64(v), f64(o), f64(do), f64(lse), causal, 1.0 / math.sqrt(D))
        for name, a, r in zip(("dq", "dk", "dv"), got, oracle):
            mx, rel = A.compare(f64(a), r)
            assert mx <= 2e-2 and rel <= 5e-3, f"{name}: max_abs={mx:.3e} rel_l2={rel:.3e}"


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    x = torch.empty(8, dtype=torch.bfloat16, device="cuda")  # never dereferenced: refused on the host
    lib = _lib.load()
    p = x.data_ptr()
    st = lib.attn_bwd_deterministic_noalloc(p, p, p, p, p, p, 1, 2, p, p, p, 4, 32, 4096, 128, 0.0884, 0, None)
    assert st == _lib.ERR_SCRATCH_LIMIT
