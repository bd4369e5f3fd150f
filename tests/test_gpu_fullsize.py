"""Full-size parity on the benchmark workloads (MI355X only).

At the full shapes the oracle cannot compute whole tensors in seconds, so
each case checks (1) sampled rows of dQ, dK and dV against the oracle's
row-restricted backward (the same formulas, O(S*D) per row) and (2) two
column-sum identities that hold at any size: sum_j dK_j = 0 and
sum_j dV_j = sum_i dO_i per head. The calls are the ones bench.py times
(same shapes, tiles, schedules and workspace sizing).
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def schedules(w, N):
    out = ["naive", "descending"]
    out += ["shift"] + (["symmetric_shift"] if (w.causal and N % 2 == 0) else [])
    return out + [None]


def sample_rows(S, T):
    rows = {0, 1, T - 1, T, S // 2 - 1, S // 2, S - T, S - 2, S - 1, 3 * S // 4 + 5}
    return sorted(r for r in rows if 0 <= r < S)


@pytest.mark.parametrize("name", ["C2", "C3", "C3F", "C4", "C5"])
def test_fullsize_sampled_parity(name):
    w = attn_inputs.WORKLOADS[name]
    T = dab.tile(w.S, w.D, w.tile)
    N = -(-w.S // T)
    x = attn_inputs.draw_workload(w)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = dab.fwd(q, k, v, w.causal, w.scale)
    torch.cuda.synchronize()
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    rows = sample_rows(w.S, T)
    f64 = lambda t: t.float().cpu().double().numpy()
    refs = {}
    for b, h in heads:
        args = [f64(t[b, h]) for t in (q, k, v, o, do)]
        refs[(b, h)] = A.backward_rows_head(*args[:4], args[4], f64(lse[b, h]), w.causal, w.scale, rows, rows)
    out = tuple(torch.empty_like(q) for _ in range(3))
    for sched in schedules(w, N):
        say(f"full-size {name} {w.describe()} T={T} schedule={sched or 'atomic'}")
        ws = dab.alloc_workspace(w.B, w.H, w.S, w.D, w.causal, sched or "naive", w.tile)
        if sched is None:
            dq, dk, dv = dab.bwd_nondeterministic(q, k, v, o, do, lse, w.causal, w.scale, w.tile, ws, out)
        else:
            dq, dk, dv = dab.bwd(q, k, v, o, do, lse, w.causal, sched, w.scale, w.tile, ws, out)
            dab.check_workspace(ws)
        torch.cuda.synchronize()
        for (b, h), (rq, rk, rv) in refs.items():
            for label, got, ref in (("dQ", dq[b, h, rows], rq), ("dK", dk[b, h, rows], rk), ("dV", dv[b, h, rows], rv)):
                mx, rel = A.compare(f64(got), ref)
                assert mx <= 2e-2 and rel <= 5e-3, f"{name} {sched} head {(b, h)} {label}: {mx:.3e} {rel:.3e}"
        # column sums per head: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i
        dk_sum = dk.float().sum(dim=2)
        dv_sum = dv.float().sum(dim=2)
        do_sum = do.float().sum(dim=2)
        dk_scale = dk.float().abs().sum(dim=2)
        assert torch.all(dk_sum.abs() <= 1e-2 * dk_scale + 1e-3), f"{name} {sched}: sum dK"
        assert torch.all((dv_sum - do_sum).abs() <= 1e-2 * do.float().abs().sum(dim=2) + 1e-3), f"{name} {sched}: sum dV"
        del ws
