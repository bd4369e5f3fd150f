"""GPU parity on a seeded sweep of small random shapes (MI355X only).

Beyond the hand-picked shapes of test_gpu_parity.py: lengths drawn anywhere
in [1, 700] (so tile counts odd and even, ragged tails of every size), one
to four heads, one or two batches, both head sizes, both masks, every tile
request, and grouped K/V heads. Each backward of every deterministic
schedule and of the atomic variant is compared element by element with the
float64 oracle on the HIP forward's O and LSE (which are checked against
the oracle forward first), to the same bar as
test_gpu_parity.py (grouped dK/dV: the widened per-element bound of
test_gpu_gqa.py). The shapes come from a fixed seed, so a failure names a
shape that reproduces.
"""

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


def _shapes():
    rng = np.random.default_rng(20261202)
    plain, grouped = [], []
    for i in range(16):
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 5))
        S = int(rng.integers(1, 701))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        tile = int(rng.choice([0, 64, 128]))
        plain.append((B, H, S, D, causal, tile, 500 + i))
    for i in range(6):
        Hkv = int(rng.integers(1, 3))
        G = int(rng.choice([2, 4]))
        S = int(rng.integers(1, 513))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        grouped.append((1, Hkv * G, Hkv, S, D, causal, 600 + i))
    return plain, grouped


PLAIN, GROUPED = _shapes()


def _schedules(S, D, causal, tile):
    T = dab.tile(S, D, tile)
    N = -(-S // T)
    out = ["naive", "descending", "shift"]
    if causal and N % 2 == 0:
        out.append("symmetric_shift")
    return out + [None]


@pytest.mark.parametrize("case", PLAIN, ids=lambda c: "B%dH%dS%dD%d%s_t%d" % (c[0], c[1], c[2], c[3],
                                                                              "c" if c[4] else "f", c[5]))
def test_random_shape_parity(case):
    B, H, S, D, causal, tile, seed = case
    say(f"random shape {case}")
    x = attn_inputs.draw(B, H, S, D, seed)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = dab.fwd(q, k, v, causal)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(D)
    o_ref, lse_ref = A.forward(f64(q), f64(k), f64(v), causal, scale)
    mx, rel = A.compare(f64(o), o_ref)
    assert mx <= TOL_ABS and rel <= TOL_REL, f"{case} forward O: max_abs={mx:.3e} rel_l2={rel:.3e}"
    assert np.abs(f64(lse) - lse_ref).max() <= 1e-3, f"{case} forward LSE"
    ref = A.backward(f64(q), f64(k), f64(v), f64(o), f64(do), f64(lse), causal, scale)
    for sched in _schedules(S, D, causal, tile):
        say(f"  schedule={sched or 'atomic'}")
        if sched is None:
            got = dab.bwd_nondeterministic(q, k, v, o, do, lse, causal, tile_request=tile)
        else:
            got = dab.bwd(q, k, v, o, do, lse, causal, sched, tile_request=tile)
        torch.cuda.synchronize()
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            mx, rel = A.compare(f64(g), r)
            assert mx <= TOL_ABS and rel <= TOL_REL, f"{case} {sched or 'atomic'} {name}: max_abs={mx:.3e} rel_l2={rel:.3e}"


@pytest.mark.parametrize("case", GROUPED, ids=lambda c: "B%dH%dKV%dS%dD%d%s" % (c[0], c[1], c[2], c[3], c[4],
                                                                                "c" if c[5] else "f"))
def test_random_grouped_shape_parity(case):
    B, H, Hkv, S, D, causal, seed = case
    say(f"random grouped shape {case}")
    x = attn_inputs.draw_grouped(B, H, Hkv, S, D, seed)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = dab.fwd(q, k, v, causal)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(D)
    ref = A.backward_grouped(f64(q), f64(k), f64(v), f64(o), f64(do), f64(lse), causal, scale)
    for sched in _schedules(S, D, causal, 0):
        say(f"  schedule={sched or 'atomic'}")
        if sched is None:
            got = dab.bwd_nondeterministic(q, k, v, o, do, lse, causal)
        else:
            got = dab.bwd(q, k, v, o, do, lse, causal, sched)
        torch.cuda.synchronize()
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            gg = f64(g)
            mx, rel = A.compare(gg, r)
            widen = 0.0 if name == "dQ" else 2.0 ** -8  # dK/dV sum the group's shares before rounding to bf16
            excess = float(np.max(np.abs(gg - r) - widen * np.abs(r))) if r.size else 0.0
            assert excess <= TOL_ABS and rel <= TOL_REL, f"{case} {sched or 'atomic'} {name}: max_abs={mx:.3e} rel_l2={rel:.3e}"
