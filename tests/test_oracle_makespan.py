"""Pins for the multi-head makespan model (CPU only).

The model is pinned by: its one-head case, which must be the pages' DAG and
so reproduce the hand-derived critical-path closed forms; a hand-worked
two-head golden (tests/golden/makespan_two_heads.json) that includes the gap
§2.2 A of the Dutch and Japanese technical summaries speaks of; bounds any
list schedule obeys (total work over P, the longest chain, one processor
running everything in sequence); and deadlock cases worked out by hand. The
pipelined reading (hand-off off the processor) is pinned by reducing to the
DAG model at its defaults, by a closed form for full-mask Shift, by a
hand-worked golden (tests/golden/makespan_pipelined.json), and by the proof
sketched at test_causal_shift_last_tile_first_never_waits.
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
# deals a head's workers in ascending KV-tile order except for causal Shift; for the other
# schedules the model finds no better order among the two natural ones at these shapes.
XCD_SHAPES = [  # (N, causal, heads per XCD)
    (16, False, 8),    # B=4, H=16, S=2048 full
    (32, True, 16),    # B=4, H=32, S=4096 causal
    (32, False, 16),   # B=4, H=32, S=4096 full
]


@pytest.mark.parametrize("N,causal,heads", XCD_SHAPES)
def test_ascending_worker_order_is_never_worse(N, causal, heads):
    # causal Shift is the exception, covered below: its dQ chains run from the
    # last KV tile down, and the kernel deals its workers in that order
    for sched in (Sch.NAIVE, Sch.DESCENDING, Sch.SHIFT, Sch.SYMMETRIC_SHIFT):
        if (sched == Sch.SYMMETRIC_SHIFT and not causal) or (sched == Sch.SHIFT and causal):
            continue
        plan = Sch.build(N, causal, sched)
        n = len(plan.workers)
        for r in (0.0, 0.25, 0.75):
            best, res = M.best_worker_order(plan, heads, 32, {"ascending": range(n), "descending": range(n)[::-1]},
                                            1.0, r)
            assert best == "ascending", (Sch.NAMES[sched], r, res)


# ---- the pipelined reading (the hand-off runs off the processor)

@pytest.mark.parametrize("N,causal,sched", [x for x in cases() if x[0] in (1, 2, 3, 4, 6)])
def test_pipelined_defaults_are_the_dag_model(N, causal, sched):
    plan = Sch.build(N, causal, sched)
    n = len(plan.workers)
    for heads, P in ((1, n), (2, n), (3, n + 1), (2, max(1, n - 1))):
        for c, r in WEIGHTS:
            a = M.simulate(plan, heads, P, c, r)
            b = M.simulate_pipelined(plan, heads, P, c, r)
            assert (a is None) == (b is None)
            if a is not None:
                assert a["spans"] == b["spans"] and a["wait"] == b["wait"]


def test_pipelined_full_shift_closed_form():
    # conflict-free steps and a hand-off no longer than a compute: every hand-off
    # overlaps the next compute, so one head takes its N nsub computes plus the
    # last hand-off
    for N in (2, 4, 8):
        plan = Sch.build(N, False, Sch.SHIFT)
        for nsub in (1, 2):
            for r in (0.0, 0.5, 1.0):
                for gate in ("done", "start"):
                    res = M.simulate_pipelined(plan, 1, N, 1.0, r, nsub=nsub, lag=1, gate=gate)
                    assert res["makespan"] == pytest.approx(N * nsub + r)
                    assert sum(res["wait"]) == 0.0
                # a set-up before the first compute and a delay before each hand-off
                # (no longer than a compute) add once; every unit spans the whole run
                for setup, delay in ((2.0, 0.0), (0.0, 0.5), (3.0, 1.0)):
                    res = M.simulate_pipelined(plan, 1, N, 1.0, r, nsub=nsub, lag=1, setup=setup, delay=delay,
                                               gate="start")
                    want = setup + N * nsub + delay + r
                    assert res["makespan"] == pytest.approx(want)
                    assert all(sp == (w, 0.0, pytest.approx(want)) for w, (sp) in
                               zip(range(N), [res["spans"][(0, w)] for w in range(N)]))


def test_golden_pipelined():
    g = json.load(open(os.path.join(GOLDEN, "makespan_pipelined.json")))
    plan = Sch.build(2, True, Sch.SHIFT)
    for case in g["cases"]:
        res = M.simulate_pipelined(plan, 2, 2, 1.0, 1.0, M.ticket_order(plan, 2, case["worker_order"]), nsub=1,
                                   lag=1, gate="start")
        assert res["makespan"] == case["makespan"], case["name"]
        assert sum(res["wait"]) == case["wait"], case["name"]
        assert res["spans"] == {(h, w): (p, s, e) for h, w, p, s, e in case["spans"]}, case["name"]


PIPE_PARAMS = [  # (c, r, delay, lag, setup, nsub, gate)
    (1.0, 0.0, 0.0, 0, 0.0, 1, "done"), (1.0, 1.0, 0.0, 0, 0.0, 1, "done"), (1.0, 0.25, 0.0, 0, 0.0, 1, "done"),
    (1.0, 0.5, 1.0, 1, 3.0, 2, "start"), (1.0, 1.0, 1.0, 1, 3.0, 2, "start"), (2.0, 1.0, 1.0, 1, 0.0, 2, "done"),
    (1.0, 1.0, 0.5, 1, 0.0, 1, "start"), (1.0, 1.0, 1.0, 2, 1.0, 2, "start"),
]


@pytest.mark.parametrize("N", [2, 3, 4, 5, 8, 12])
def test_causal_shift_last_tile_first_never_waits(N):
    # causal Shift's dQ tile i takes KV tiles i, i-1, ..., 0, so worker j waits on
    # worker j+1. Dealt last KV tile first, worker j+1 starts no later than worker j
    # and is one task ahead on every dQ tile they share, so (by induction from the
    # last worker, which is always first on its tiles) no hand-off ever waits
    plan = Sch.build(N, True, Sch.SHIFT)
    order = list(range(N))[::-1]
    for P in (N, N + 1, N + N // 2, 2 * N):
        for heads in (1, 2, 3, 5):
            res = M.simulate(plan, heads, P, 1.0, 1.0, M.ticket_order(plan, heads, order))
            assert sum(res["wait"]) == 0.0
            for c, r, delay, lag, setup, nsub, gate in PIPE_PARAMS:
                res = M.simulate_pipelined(plan, heads, P, c, r, M.ticket_order(plan, heads, order), nsub=nsub,
                                           lag=lag, setup=setup, delay=delay, gate=gate)
                assert sum(res["wait"]) == 0.0, (P, heads, c, r, delay, lag, setup, nsub, gate)


def test_causal_shift_first_tile_first_waits_at_the_kernel_shape():
    # ascending tickets: the next head's workers start one after another as the
    # previous head's shortest units drain, each after its own predecessor in the
    # dQ chain, so hand-offs wait (the kernel measures these waits as a large loss)
    plan = Sch.build(32, True, Sch.SHIFT)
    for c, r, delay, lag, setup, nsub, gate in PIPE_PARAMS[3:5]:
        res = M.simulate_pipelined(plan, 16, 32, c, r, None, nsub=nsub, lag=lag, setup=setup, delay=delay,
                                   gate=gate)
        assert sum(res["wait"]) > 0.0


# Interleaved heads: the kernel deals naive and Descending units in runs of
# up to four heads, worker by worker. The model is what chose that.

def test_interleaved_ticket_order_is_a_permutation_in_worker_order():
    plan = Sch.build(5, True, BY_NAME["descending"])
    for heads in (1, 3, 7, 8):
        for ilv in (1, 2, 4):
            tk = M.interleaved_ticket_order(plan, heads, ilv)
            assert sorted(tk) == sorted(M.ticket_order(plan, heads))
            for h in range(heads):  # each head's workers in ascending order
                assert [w for hh, w in tk if hh == h] == list(range(len(plan.workers)))
    assert M.interleaved_ticket_order(plan, 7, 1) == M.ticket_order(plan, 7)
    # hand-worked: two heads of two workers, then one left over
    small = Sch.build(2, False, BY_NAME["naive"])
    assert M.interleaved_ticket_order(small, 3, 2) == [(0, 0), (1, 0), (0, 1), (1, 1), (2, 0), (2, 1)]
    with pytest.raises(ValueError):
        M.interleaved_ticket_order(small, 3, 0)


@pytest.mark.parametrize("sched", ["naive", "descending"])
@pytest.mark.parametrize("causal", [False, True])
def test_interleaved_naive_and_descending_never_deadlock(sched, causal):
    # their workers wait only on lower workers of the same head, so any
    # number of processors drains the queue, also fewer than a head's workers
    plan = Sch.build(6, causal, BY_NAME[sched])
    for P in (1, 2, 5, 7):
        for ilv in (2, 4):
            tk = M.interleaved_ticket_order(plan, 5, ilv)
            assert M.makespan(plan, 5, P, 1.0, 0.5, tk) is not None
            assert M.simulate_pipelined(plan, 5, P, 1.0, 0.5, tk, nsub=2, lag=1, gate="start", setup=3.0,
                                        delay=1.0) is not None


def test_interleaving_shortens_the_causal_4k_queue():
    # One XCD queue of the causal 4k workload: 16 heads of 32 KV tiles on 32
    # workgroups, the pipelined reading with the kernel's shape (two sub-tiles
    # per task, lag 1, gate "start", set-up 3 intervals, hand-off one interval
    # after its sub-tile, r = 0.5). Four heads at a time shorten naive by
    # about a third (its serial chains leave gaps the other heads fill) and
    # Descending by about 2%, the measured direction (+43% and +2-3%).
    kw = dict(nsub=2, lag=1, gate="start", setup=3.0, delay=1.0)
    res = {}
    for name in ("naive", "descending"):
        plan = Sch.build(32, True, BY_NAME[name])
        for ilv in (1, 4):
            r = M.simulate_pipelined(plan, 16, 32, 1.0, 0.5, M.interleaved_ticket_order(plan, 16, ilv), **kw)
            res[(name, ilv)] = r["makespan"]
    assert res[("naive", 4)] < 0.7 * res[("naive", 1)]
    assert res[("descending", 4)] < res[("descending", 1)]
    assert res[("descending", 4)] > 0.95 * res[("descending", 1)]
