"""Pins for the schedule oracle (CPU only).

The schedules are checked against hand-worked tables (tests/golden), against
properties the DASH pages claim (coverage, one KV tile per worker, conflict
freedom of Shift and Symmetric Shift, Lemma 1's depth condition, balance of
Symmetric Shift), and against critical-path closed forms derived by hand for
the weighted DAG (compute weight c, reduction weight r):

    full mask   naive, descending : N(c+r) + (N-1) r
                shift             : N(c+r)            (= the longest worker chain)
    causal      naive             : N(c+r) + (N-1) r
                descending        : N(c+r)
                shift             : N(c+r)
                symmetric shift   : (N+1)(c+r) with N/2 workers of N+1 tasks each

Derivation (naive, full): the reduction of task (q tile i, KV tile j) ends at
E(i,j) = max(E(i-1,j) + c, E(i,j-1)) + r, whose solution is
(i+1)(c+r) + j r. Descending, causal: E(i,j) = max(E(i+1,j) + c, E(i,j-1)) + r
solves to (N-i)(c+r) + j r, largest at i = j = 0. Shift, causal: the
predecessor of (i, j) is (i, j+1), so E(i,j) = max(E(i-1,j) + c, E(i,j+1)) + r
solves to (i-j+1)(c+r), largest at i = N-1, j = 0. Shift and Symmetric Shift
never wait: each dQ tile's previous contribution finishes one step earlier.
"""

import itertools
import json
import os

import pytest

from oracle import schedule as Sch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NS = [1, 2, 3, 4, 5, 6, 8, 12, 16, 32]
WEIGHTS = [(1.0, 0.0), (1.0, 1.0), (3.0, 1.0), (1.0, 0.25), (0.0, 1.0)]


def cases():
    for N in NS:
        yield N, False, Sch.NAIVE
        yield N, False, Sch.DESCENDING
        yield N, False, Sch.SHIFT
        yield N, True, Sch.NAIVE
        yield N, True, Sch.DESCENDING
        yield N, True, Sch.SHIFT
        if N % 2 == 0:
            yield N, True, Sch.SYMMETRIC_SHIFT


@pytest.mark.parametrize("N,causal,sched", list(cases()))
def test_structure(N, causal, sched):
    plan = Sch.build(N, causal, sched)
    assert Sch.coverage_ok(plan)
    assert Sch.chains_ok(plan)
    assert Sch.deadlock_free(plan)
    # every accumulation order is a permutation of the tile's contributors
    for i, order in enumerate(plan.orders):
        want = sorted(j for j in range(N) if Sch.active(i, j, causal))
        assert sorted(order) == want
    if sched in (Sch.SHIFT, Sch.SYMMETRIC_SHIFT):
        assert Sch.conflict_free(plan)
        for c, r in WEIGHTS:
            assert Sch.lemma1_edges(plan, c, r) == []


def closed_form(N, causal, sched, c, r):
    if sched == Sch.SHIFT:
        return N * (c + r)
    if sched == Sch.SYMMETRIC_SHIFT:
        return (N + 1) * (c + r)
    if causal and sched == Sch.DESCENDING:
        return N * (c + r)
    return N * (c + r) + (N - 1) * r


@pytest.mark.parametrize("N,causal,sched", list(cases()))
@pytest.mark.parametrize("c,r", WEIGHTS)
def test_critical_path_closed_forms(N, causal, sched, c, r):
    plan = Sch.build(N, causal, sched)
    assert Sch.critical_path(plan, c, r) == pytest.approx(closed_form(N, causal, sched, c, r))


def test_naive_violates_lemma1_when_reductions_cost():
    # ascending order makes each worker wait for its left neighbour's reduction
    plan = Sch.build(8, False, Sch.NAIVE)
    assert Sch.lemma1_edges(plan, 1.0, 1.0) != []
    assert Sch.lemma1_edges(plan, 1.0, 0.0) == []


def test_shift_is_optimal_among_all_orders_small():
    # brute force over every set of accumulation orders for the Shift traversal (N = 3):
    # none beats the pages' order, which reaches the lower bound N(c+r)
    N, c, r = 3, 1.0, 1.0
    plan = Sch.build(N, False, Sch.SHIFT)
    best = None
    for perms in itertools.product(*[list(itertools.permutations(range(N)))] * N):
        trial = Sch.Plan(N, False, Sch.SHIFT, plan.workers, [list(p) for p in perms])
        cp = Sch.critical_path(trial, c, r)
        if cp is not None:
            best = cp if best is None else min(best, cp)
    assert best == pytest.approx(N * (c + r)) == pytest.approx(Sch.critical_path(plan, c, r))


def test_golden_shift():
    g = json.load(open(os.path.join(GOLDEN, "shift_n5.json")))
    plan = Sch.build(g["N"], False, Sch.SHIFT)
    assert [[i for _, i, _ in tasks] for tasks in plan.workers] == g["traversal"]
    assert plan.orders == g["orders"]


def test_golden_shift_causal():
    g = json.load(open(os.path.join(GOLDEN, "shift_causal_n4.json")))
    plan = Sch.build(g["N"], True, Sch.SHIFT)
    assert [[i for _, i, _ in tasks] for tasks in plan.workers] == g["traversal"]
    assert plan.orders == g["orders"]


def test_golden_symmetric_shift():
    g = json.load(open(os.path.join(GOLDEN, "symmetric_shift_n4.json")))
    plan = Sch.build(g["N"], True, Sch.SYMMETRIC_SHIFT)
    assert [[list(t) for t in tasks] for tasks in plan.workers] == g["workers"]
    assert plan.orders == g["orders"]


@pytest.mark.parametrize("N", [2, 4, 6, 8, 16, 32, 64])
def test_symmetric_shift_geometry(N):
    plan = Sch.build(N, True, Sch.SYMMETRIC_SHIFT)
    h = N // 2
    assert len(plan.workers) == h
    for p, tasks in enumerate(plan.workers):
        assert len(tasks) == N + 1                         # balanced: folded into a square
        assert {j for _, _, j in tasks} == {p, N - 1 - p}  # symmetric pair of KV tiles
        phase1 = tasks[:h]
        assert all(i >= h and j == p for _, i, j in phase1)  # dense lower-left rectangle
        assert sorted(i for _, i, _ in phase1) == list(range(h, N))


def test_descending_reverses_traversal():
    for causal in (False, True):
        a = Sch.build(7, causal, Sch.NAIVE)
        d = Sch.build(7, causal, Sch.DESCENDING)
        for ta, td in zip(a.workers, d.workers):
            assert [i for _, i, _ in td] == [i for _, i, _ in ta][::-1]
        assert a.orders == d.orders


def test_cycle_is_detected():
    # planted mistake: Shift traversal with each dQ tile's order reversed closes a cycle
    # (worker 0 would wait at step 0 for worker 1's step N-1, and vice versa)
    plan = Sch.build(4, False, Sch.SHIFT)
    bad = Sch.Plan(4, False, Sch.SHIFT, plan.workers, [o[::-1] for o in plan.orders])
    assert not Sch.deadlock_free(bad)
    assert Sch.critical_path(bad) is None
    # ascending accumulation on the same traversal is acyclic but slower than the step order
    slow = Sch.Plan(4, False, Sch.SHIFT, plan.workers, [list(range(4)) for _ in range(4)])
    assert Sch.critical_path(slow, 1.0, 1.0) > Sch.critical_path(plan, 1.0, 1.0)


def test_invalid_requests():
    with pytest.raises(ValueError):
        Sch.build(5, True, Sch.SYMMETRIC_SHIFT)
    with pytest.raises(ValueError):
        Sch.build(4, False, Sch.SYMMETRIC_SHIFT)
