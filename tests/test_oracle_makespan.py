"""Pins for the multi-head makespan model (CPU only).

The model is pinned by: its one-head case, which must be the pages' DAG and
so reproduce the hand-derived critical-path closed forms; a hand-worked
two-head golden (tests/golden/makespan_two_heads.json) that includes the gap
§2.2 A of the Dutch and Japanese technical summaries speaks of; bounds any
list schedule obeys (total work over P, the longest chain, one processor
running everything in sequence); and deadlock cases worked out by hand.
"""

import json
import os

import pytest

from oracle import makespan as M
from oracle import schedule as Sch
from test_oracle_schedule import NS, WEIGHTS, cases, closed_form

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BY_NAME = {v: k for k, v in Sch.NAMES.items()}


@pytest.mark.parametrize("N,causal,sched", list(cases()))
@pytest.mark.parametrize("c,r", WEIGHTS)
def test_one_head_is_the_dag(N, causal, sched, c, r):
    plan = Sch.build(N, causal, sched)
    for P in (len(plan.workers), len(plan.workers) + 3):
        got = M.makespan(plan, 1, P, c, r)
        assert got == pytest.approx(closed_form(N, causal, sched, c, r))
        assert got == pytest.approx(Sch.critical_path(plan, c, r))


def test_golden_two_heads():
    g = json.load(open(os.path.join(GOLDEN, "makespan_two_heads.json")))
    for case in g["cases"]:
        plan = Sch.build(case["N"], case["causal"], BY_NAME[case["schedule"]])
        res = M.simulate(plan, case["heads"], case["processors"], case["c"], case["r"])
        assert res is not None, case["name"]
        assert res["makespan"] == case["makespan"], case["name"]
        want = {(h, w): (p, s, e) for h, w, p, s, e in case["spans"]}
        assert res["spans"] == want, case["name"]


def test_descending_closes_the_gap_between_heads():
    # the pages' §2.2 A claim, on the smallest case (hand-worked in the golden) and at larger sizes:
    # with several heads in flight, Descending never loses to naive on a causal mask
    for N in (2, 4, 8, 16):
        for heads in (2, 3, 5):
            for P in (N, N + N // 2, 2 * N):
                for c, r in ((1.0, 0.0), (1.0, 0.25), (1.0, 1.0)):
                    nv = M.makespan(Sch.build(N, True, Sch.NAIVE), heads, P, c, r)
                    ds = M.makespan(Sch.build(N, True, Sch.DESCENDING), heads, P, c, r)
                    assert ds <= nv + 1e-9, (N, heads, P, c, r)
    assert M.makespan(Sch.build(2, True, Sch.DESCENDING), 2, 2, 1.0, 0.0) < \
        M.makespan(Sch.build(2, True, Sch.NAIVE), 2, 2, 1.0, 0.0)


@pytest.mark.parametrize("N,causal,sched", [x for x in cases() if x[0] in (2, 3, 4, 8)])
def test_list_schedule_bounds(N, causal, sched):
    plan = Sch.build(N, causal, sched)
    tasks = sum(len(t) for t in plan.workers)
    longest = max(len(t) for t in plan.workers)
    for heads in (1, 2, 5):
        for P in (len(plan.workers), 2 * len(plan.workers) + 1):
            for c, r in WEIGHTS:
                res = M.simulate(plan, heads, P, c, r)
                assert res is not None
                ms = res["makespan"]
                assert ms >= heads * tasks * (c + r) / P - 1e-9
                assert ms >= longest * (c + r) - 1e-9
                # every unit's span is its work plus the waits charged to its processor
                assert sum(res["busy"]) == pytest.approx(heads * tasks * (c + r) + sum(res["wait"]))
                assert all(e <= ms for _, _, e in res["spans"].values())


@pytest.mark.parametrize("sched", [Sch.NAIVE, Sch.DESCENDING])
@pytest.mark.parametrize("causal", [False, True])
def test_one_processor_runs_everything_in_sequence(sched, causal):
    # naive and Descending order each dQ tile by ascending KV tile = ascending worker, so a
    # lone processor never waits: the makespan is the total work
    for N in (1, 3, 6):
        plan = Sch.build(N, causal, sched)
        tasks = sum(len(t) for t in plan.workers)
        for c, r in WEIGHTS:
            res = M.simulate(plan, 3, 1, c, r)
            assert res["makespan"] == pytest.approx(3 * tasks * (c + r))
            assert res["wait"] == [0.0]


def test_deadlock_when_a_head_does_not_fit():
    # full-mask Shift: the second contribution to dQ tile i comes from worker i-1 at step 1,
    # which waits for worker i at step 0; with P < N the last running worker waits for a
    # worker no processor will take
    for N in (2, 3, 4, 8):
        plan = Sch.build(N, False, Sch.SHIFT)
        assert M.makespan(plan, 1, N - 1, 1.0, 1.0) is None
        assert M.makespan(plan, 3, N, 1.0, 1.0) == pytest.approx(3 * N * 2.0)
    # causal Shift: worker j waits for worker j+1 (a later ticket), same failure
    assert M.makespan(Sch.build(4, True, Sch.SHIFT), 1, 3, 1.0, 0.0) is None
    # naive waits only for earlier tickets: any processor count finishes
    for N in NS[:6]:
        for P in range(1, N + 1):
            assert M.makespan(Sch.build(N, False, Sch.NAIVE), 2, P, 1.0, 1.0) is not None


def test_ticket_order_validation():
    plan = Sch.build(3, False, Sch.SHIFT)
    assert M.ticket_order(plan, 2, [2, 0, 1]) == [(0, 2), (0, 0), (0, 1), (1, 2), (1, 0), (1, 1)]
    with pytest.raises(ValueError):
        M.ticket_order(plan, 1, [0, 0, 1])
    with pytest.raises(ValueError):
        M.simulate(plan, 1, 0)


# Per-XCD shapes of the benchmark workloads: one XCD's queue holds B*H/8 heads and its
# 32 workgroups are the processors (one resident workgroup per CU at D = 128). The kernel
# deals a head's workers in ascending KV-tile order; the model finds no better order among
# the two natural ones for any schedule at these shapes.
XCD_SHAPES = [  # (N, causal, heads per XCD)
    (16, False, 8),    # B=4, H=16, S=2048 full
    (32, True, 16),    # B=4, H=32, S=4096 causal
    (32, False, 16),   # B=4, H=32, S=4096 full
]


@pytest.mark.parametrize("N,causal,heads", XCD_SHAPES)
def test_ascending_worker_order_is_never_worse(N, causal, heads):
    for sched in (Sch.NAIVE, Sch.DESCENDING, Sch.SHIFT, Sch.SYMMETRIC_SHIFT):
        if sched == Sch.SYMMETRIC_SHIFT and not causal:
            continue
        plan = Sch.build(N, causal, sched)
        n = len(plan.workers)
        for r in (0.0, 0.25, 0.75):
            best, res = M.best_worker_order(plan, heads, 32, {"ascending": range(n), "descending": range(n)[::-1]},
                                            1.0, r)
            assert best == "ascending", (Sch.NAMES[sched], r, res)
