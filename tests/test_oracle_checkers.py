"""Pins for the oracle's checkers (CPU only).

Every GPU parity assertion goes through ``oracle.attention.compare``, and the
schedule tests lean on ``coverage_ok``, ``chains_ok`` and ``conflict_free``.
A checker that is only ever asserted true proves nothing: replaced by a
constant it would still pass. These tests feed each checker inputs whose
answer is worked out by hand here, including inputs that must be rejected.

compare(x, y) returns (max |x - y|, ||x - y||_2 / ||y||_2), and ||x - y||_2
itself when ||y||_2 = 0. The schedule predicates state the properties the
DASH technical summaries (Dutch and Japanese, §2.1 and §2.2 B) ask of a plan:
every unmasked task done exactly once, a KV tile's tasks on one processor in
consecutive steps, and no two processors on one dQ tile in the same step.
"""

import copy
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import schedule as Sch


# --------------------------------------------------------------------------- compare


def test_compare_hand_worked_pair():
    # d = x - y = (0, 0, -2): max |d| = 2, ||d|| = 2, ||y|| = sqrt(1 + 4 + 25)
    mx, rel = A.compare([1.0, 2.0, 3.0], [1.0, 2.0, 5.0])
    assert mx == 2.0
    assert rel == pytest.approx(2.0 / math.sqrt(30.0), rel=1e-15)


def test_compare_two_dimensional_pair():
    x = np.array([[0.5, -1.0], [2.0, 4.0]])
    y = np.array([[0.0, -1.0], [2.5, 3.0]])
    # d = (0.5, 0, -0.5, 1): max 1, ||d||^2 = 0.25 + 0.25 + 1 = 1.5, ||y||^2 = 1 + 6.25 + 9 = 16.25
    mx, rel = A.compare(x, y)
    assert mx == 1.0
    assert rel == pytest.approx(math.sqrt(1.5 / 16.25), rel=1e-15)


def test_compare_zero_reference_gives_absolute_norm():
    # ||y|| = 0: the relative figure falls back to ||x - y|| = ||(3, 4)|| = 5
    mx, rel = A.compare([3.0, 4.0], [0.0, 0.0])
    assert (mx, rel) == (4.0, 5.0)


def test_compare_sign_flip():
    # x = -y: d = -2y, so max |d| = 2 max |y| and the relative error is exactly 2
    y = np.array([0.25, -1.5, 3.0, -0.125])
    mx, rel = A.compare(-y, y)
    assert mx == 6.0
    assert rel == pytest.approx(2.0, rel=1e-15)


def test_compare_identical_and_empty():
    y = np.linspace(-3, 3, 11)
    assert A.compare(y, y) == (0.0, 0.0)
    assert A.compare(np.zeros(0), np.zeros(0)) == (0.0, 0.0)


@pytest.mark.parametrize("pos", [0, 7, 63])
def test_compare_sees_one_wrong_element_anywhere(pos):
    y = np.ones(64)
    x = y.copy()
    x[pos] += 0.75
    mx, rel = A.compare(x, y)
    assert mx == 0.75
    assert rel == pytest.approx(0.75 / 8.0, rel=1e-15)  # ||y|| = sqrt(64)


def test_compare_is_not_symmetric():
    # the reference is the second argument: ||x - y|| / ||y||
    _, r1 = A.compare([2.0], [1.0])
    _, r2 = A.compare([1.0], [2.0])
    assert (r1, r2) == (1.0, 0.5)


def test_compare_lifts_to_float64():
    # float32 inputs are compared in float64: 1 + 2^-30 is not lost
    x = np.array([1.0 + 2.0 ** -30])
    y = np.array([1.0], dtype=np.float32)
    mx, _ = A.compare(x, y)
    assert mx == 2.0 ** -30


# --------------------------------------------------------------------------- schedule predicates


def _valid(N=4, causal=False, sched=Sch.SHIFT):
    plan = Sch.build(N, causal, sched)
    assert Sch.coverage_ok(plan) and Sch.chains_ok(plan) and Sch.conflict_free(plan)
    return copy.deepcopy(plan)


def test_coverage_rejects_a_dropped_task():
    plan = _valid()
    plan.workers[2].pop()  # worker 2 never does its last task
    assert not Sch.coverage_ok(plan)


def test_coverage_rejects_a_duplicated_task():
    plan = _valid()
    step, i, j = plan.workers[1][0]
    plan.workers[1].append((len(plan.workers[1]), i, j))  # the same (query, KV) tile pair twice
    assert not Sch.coverage_ok(plan)


def test_coverage_rejects_a_masked_task():
    # causal: task (query 0, KV 3) lies above the diagonal and has no unmasked work
    plan = _valid(4, True, Sch.SHIFT)
    plan.workers[3].append((len(plan.workers[3]), 0, 3))
    assert not Sch.coverage_ok(plan)


def test_coverage_rejects_a_task_moved_to_a_masked_cell():
    plan = _valid(4, True, Sch.NAIVE)
    s, i, j = plan.workers[2][0]          # (2, 2)
    plan.workers[2][0] = (s, 1, j)        # (1, 2) is masked and (2, 2) is now missing
    assert not Sch.coverage_ok(plan)


def test_chains_reject_a_kv_tile_split_across_workers():
    plan = _valid()
    # worker 0 hands one of its tasks (KV tile 0) to worker 1, which owns KV tile 1
    s, i, j = plan.workers[0].pop()
    plan.workers[1].append((len(plan.workers[1]), i, j))
    assert Sch.coverage_ok(plan)          # still every task once ...
    assert not Sch.chains_ok(plan)        # ... but KV tile 0 now lives on two workers


def test_chains_reject_a_step_gap():
    plan = _valid()
    s, i, j = plan.workers[3][-1]
    plan.workers[3][-1] = (s + 1, i, j)   # steps 0, 1, 2, 4
    assert Sch.coverage_ok(plan)
    assert not Sch.chains_ok(plan)


def test_chains_reject_steps_out_of_order():
    plan = _valid()
    w = plan.workers[1]
    (s0, i0, j0), (s1, i1, j1) = w[0], w[1]
    w[0], w[1] = (s1, i0, j0), (s0, i1, j1)  # steps 1, 0, 2, 3
    assert not Sch.chains_ok(plan)


def test_conflict_free_rejects_two_workers_on_one_dq_tile():
    plan = _valid()
    # at step 0 worker j is on query tile j; move worker 1's step-0 task onto query tile 0
    s, i, j = plan.workers[1][0]
    plan.workers[1][0] = (s, 0, j)
    assert not Sch.conflict_free(plan)


def test_conflict_free_rejects_the_naive_traversal():
    # naive: every worker starts on query tile 0, the conflict the pages' Shift removes
    assert not Sch.conflict_free(Sch.build(4, False, Sch.NAIVE))
    assert not Sch.conflict_free(Sch.build(4, False, Sch.DESCENDING))


def test_conflict_free_accepts_distinct_tiles_at_equal_steps():
    plan = Sch.Plan(2, False, Sch.SHIFT, [[(0, 0, 0), (1, 1, 0)], [(0, 1, 1), (1, 0, 1)]], [[0, 1], [1, 0]])
    assert Sch.conflict_free(plan) and Sch.coverage_ok(plan) and Sch.chains_ok(plan)
