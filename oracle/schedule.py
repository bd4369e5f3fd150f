"""dQ scheduling strategies and the DAG model of the DASH pages (test infrastructure).

Only tests use this module. It restates, for one attention head split into N
query tiles and N key/value (KV) tiles (indices 0..N-1), the strategies that
the DASH pages describe, and the DAG they reason with:

* Baseline ("naive"): the worker that owns KV tile j walks the query tiles in
  ascending order; dQ tile i is accumulated in ascending KV order. (Dutch and
  Japanese technical summaries, §1: a fixed accumulation order, serialised by
  barriers.)
* Descending Q-Tile Iteration: the same workers walk the query tiles from the
  last one down to the first; the accumulation order is unchanged. (§2.2 A of
  both technical summaries; "from N to 0" is read as N-1 down to 0, the
  0-based tiles that §2.2 B uses.)
* Shift Scheduling (full mask): the worker that owns KV tile j starts on query
  tile j and continues cyclically j+1, ..., N-1, 0, ..., j-1, so at every step
  the workers touch distinct dQ tiles and each dQ tile receives its
  contributions one step after another. (§2.2 B, "Full Masks".) The pages'
  sequence i, i+1, ..., i-1 is read as the traversal of the other tile
  dimension by the worker owning a fixed KV tile, because §2.1 keeps all work
  of one KV tile on one processor. On a causal mask (the English abstract of
  the shd-paper.top digest credits Shift Scheduling for both masks) the same
  cyclic walk leaves out the fully masked query tiles 0..j-1: worker j walks
  j, ..., N-1, and dQ tile i receives KV tiles i, i-1, ..., 0 in step order.
* Symmetric Shift (causal mask, N even): worker p owns KV tiles p and N-1-p.
  Phase 1 covers the dense lower-left rectangle (query tiles N/2..N-1 against
  KV tiles 0..N/2-1) with a cyclic shift; phase 2 covers the two remaining
  triangles, the lower-right one folded onto the upper-left one so that they
  fill an N/2 x N/2 square, again with a cyclic shift; the diagonal of that
  square holds two tasks and takes two steps. (§2.2 B, "Causal Masks".)

For Shift and Symmetric Shift the accumulation order of each dQ tile is the
order of the steps at which its contributions are made (the pages: the
reductions come out ordered without conflict).

The DAG (§2.1 of both technical summaries): each task (i, j) is a compute node
C(i,j) followed by a reduction node R(i,j). Edges: a worker's nodes form one
unbroken chain (the KV tile stays on one processor); the accumulation order of
dQ tile i adds edges R(i, previous contributor) -> R(i, j). The objective is
the critical-path length. Lemma 1 (§2.2 B): an added zero-weight edge u -> v
leaves the critical path unchanged when u is finished no later than v could
start; checked here as finish(u) <= start(v) in the chain-only DAG.
"""

from __future__ import annotations

from dataclasses import dataclass, field

NAIVE, DESCENDING, SHIFT, SYMMETRIC_SHIFT = 0, 1, 2, 3
NAMES = {NAIVE: "naive", DESCENDING: "descending", SHIFT: "shift", SYMMETRIC_SHIFT: "symmetric_shift"}
FULL, CAUSAL = 0, 1


def active(i: int, j: int, causal: bool) -> bool:
    """Task (query tile i, KV tile j) has unmasked work (equal tile edges)."""
    return (not causal) or i >= j


@dataclass
class Plan:
    """One head's schedule: per-worker task lists and per-dQ-tile orders."""

    N: int
    causal: bool
    schedule: int
    workers: list = field(default_factory=list)   # workers[w] = [(step, q_tile, kv_tile), ...]
    orders: list = field(default_factory=list)    # orders[i] = [kv tiles in accumulation order]

    def rank(self, i: int, j: int) -> int:
        return self.orders[i].index(j)

    def records(self):
        """Sorted (worker, step, q_tile, kv_tile, rank) tuples of every task."""
        out = []
        for w, tasks in enumerate(self.workers):
            for step, i, j in tasks:
                out.append((w, step, i, j, self.rank(i, j)))
        return sorted(out)


def _kv_ascending_orders(N: int, causal: bool):
    return [[j for j in range(N) if active(i, j, causal)] for i in range(N)]


def _orders_by_step(N: int, workers):
    """Accumulation order of each dQ tile = order of the steps of its contributions."""
    contrib = [[] for _ in range(N)]
    for tasks in workers:
        for step, i, j in tasks:
            contrib[i].append((step, j))
    orders = []
    for i in range(N):
        steps = [s for s, _ in contrib[i]]
        if len(set(steps)) != len(steps):
            raise ValueError(f"dQ tile {i} receives two contributions in one step")
        orders.append([j for _, j in sorted(contrib[i])])
    return orders


def build(N: int, causal: bool, schedule: int) -> Plan:
    """The schedule of one head with N query tiles and N KV tiles."""
    if N < 1:
        raise ValueError("N must be positive")
    plan = Plan(N, causal, schedule)
    if schedule in (NAIVE, DESCENDING):
        for j in range(N):
            q_tiles = [i for i in range(N) if active(i, j, causal)]
            if schedule == DESCENDING:
                q_tiles = q_tiles[::-1]
            plan.workers.append([(s, i, j) for s, i in enumerate(q_tiles)])
        plan.orders = _kv_ascending_orders(N, causal)
    elif schedule == SHIFT:
        for j in range(N):
            seq = [i for i in list(range(j, N)) + list(range(0, j)) if active(i, j, causal)]
            plan.workers.append([(s, i, j) for s, i in enumerate(seq)])
        plan.orders = _orders_by_step(N, plan.workers)
    elif schedule == SYMMETRIC_SHIFT:
        if not causal or N % 2:
            raise ValueError("Symmetric Shift needs a causal mask and an even tile count")
        h = N // 2
        for p in range(h):
            tasks = []
            # phase 1: dense rectangle, query tiles h..N-1 against KV tile p, shifted
            for s in range(h):
                tasks.append((s, h + (p + s) % h, p))
            # phase 2: folded square; column p holds upper-left entries (a, p), a >= p,
            # and the lower-right triangle's entries mapped (i, j) -> (N-1-i, N-1-j)
            step = h
            for u in range(h):
                a = (p + u) % h
                if a == p:                     # diagonal: both tasks, two steps
                    tasks.append((step, p, p))
                    tasks.append((step + 1, N - 1 - p, N - 1 - p))
                    step += 2
                elif a > p:
                    tasks.append((step, a, p))
                    step += 1
                else:
                    tasks.append((step, N - 1 - a, N - 1 - p))
                    step += 1
            plan.workers.append(tasks)
        plan.orders = _orders_by_step(N, plan.workers)
    else:
        raise ValueError(f"unknown schedule {schedule}")
    return plan


# --------------------------------------------------------------------------- checks

def coverage_ok(plan: Plan) -> bool:
    """Every active task appears exactly once, and no masked task appears."""
    seen = {}
    for tasks in plan.workers:
        for _, i, j in tasks:
            seen[(i, j)] = seen.get((i, j), 0) + 1
    want = {(i, j) for i in range(plan.N) for j in range(plan.N) if active(i, j, plan.causal)}
    return set(seen) == want and all(c == 1 for c in seen.values())


def chains_ok(plan: Plan) -> bool:
    """Each worker's steps are 0, 1, 2, ... and each KV tile stays on one worker."""
    owner = {}
    for w, tasks in enumerate(plan.workers):
        if [s for s, _, _ in tasks] != list(range(len(tasks))):
            return False
        for _, _, j in tasks:
            if owner.setdefault(j, w) != w:
                return False
    return True


def conflict_free(plan: Plan) -> bool:
    """At every step, no two workers touch the same dQ tile."""
    by_step = {}
    for tasks in plan.workers:
        for s, i, _ in tasks:
            by_step.setdefault(s, []).append(i)
    return all(len(v) == len(set(v)) for v in by_step.values())


def _graph(plan: Plan, with_order: bool):
    """Node list, weights key and predecessor lists of the DAG."""
    preds = {}
    for tasks in plan.workers:
        prev = None
        for _, i, j in tasks:
            preds.setdefault(("C", i, j), [])
            preds.setdefault(("R", i, j), [])
            preds[("R", i, j)].append(("C", i, j))
            if prev is not None:
                preds[("C", i, j)].append(("R",) + prev)
            prev = (i, j)
    if with_order:
        for i, order in enumerate(plan.orders):
            for a, b in zip(order, order[1:]):
                preds[("R", i, b)].append(("R", i, a))
    return preds


def _longest(preds, c: float, r: float):
    """(start, finish) times of every node by longest path; None if a cycle exists."""
    indeg = {n: len(p) for n, p in preds.items()}
    succ = {n: [] for n in preds}
    for n, ps in preds.items():
        for p in ps:
            succ[p].append(n)
    ready = [n for n, d in indeg.items() if d == 0]
    start, finish = {}, {}
    done = 0
    while ready:
        n = ready.pop()
        start[n] = max((finish[p] for p in preds[n]), default=0.0)
        finish[n] = start[n] + (c if n[0] == "C" else r)
        done += 1
        for s in succ[n]:
            indeg[s] -= 1
            if indeg[s] == 0:
                ready.append(s)
    if done != len(preds):
        return None
    return start, finish


def critical_path(plan: Plan, c: float = 1.0, r: float = 0.0):
    """Critical-path length with compute weight c and reduction weight r.

    Returns None when the order edges close a cycle (the schedule deadlocks).
    """
    res = _longest(_graph(plan, True), c, r)
    if res is None:
        return None
    return max(res[1].values(), default=0.0)


def deadlock_free(plan: Plan) -> bool:
    return _longest(_graph(plan, True), 1.0, 1.0) is not None


def lemma1_edges(plan: Plan, c: float = 1.0, r: float = 1.0):
    """Order edges u -> v with finish(u) > start(v) in the chain-only DAG.

    An empty list means every added accumulation-order edge satisfies Lemma 1's
    depth condition, so the critical path equals the longest worker chain.
    """
    start, finish = _longest(_graph(plan, False), c, r)
    bad = []
    for i, order in enumerate(plan.orders):
        for a, b in zip(order, order[1:]):
            if finish[("R", i, a)] > start[("R", i, b)]:
                bad.append((i, a, b))
    return bad
