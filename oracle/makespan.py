"""Makespan of a dQ schedule over several heads on a fixed number of processors (test infrastructure).

Only tests use this module. It extends the one-head DAG of the DASH pages
(Dutch and Japanese technical summaries, §2.1: a compute node C(i,j) and a
reduction node R(i,j) per task, each worker one unbroken chain, the dQ
accumulation order adding R -> R edges) to a persistent grid that runs many
heads: P identical processors take "units" (one worker of one head) from a
single ticket queue, in ticket order, each as soon as it is free, and run a
unit's chain to its end before taking the next ticket. A reduction that
reaches its turn early holds its processor until the previous contribution
to the same dQ tile has finished. §2.2 A of both summaries is about exactly
this setting: with several heads in flight, the idle time a head's short
workers leave behind (its "gaps") is taken by the next head's units.

Readings (the pages do not spell the multi-head setting out):
* processors free at the same instant take tickets in processor order;
* a processor is held while its unit waits for a dQ turn (a workgroup of the
  persistent kernel spins; it does not switch units);
* the heads are independent: no edge joins two heads.

With at least as many processors as units every unit starts at time 0 and
the model is the pages' one-head DAG, so its makespan is that DAG's critical
path. With fewer processors, a unit can wait for a unit holding a later
ticket that no processor will ever take (every processor held by a waiting
unit): the model reports that deadlock as None.

simulate_pipelined() is a second reading, closer to a kernel that overlaps
the dQ hand-off with the next sub-tile's compute: the reduction runs off the
processor, tasks may be cut into sub-tiles, a unit pays a set-up cost, and
the processor may run a bounded number of sub-tiles ahead of its hand-offs.
At its defaults it is simulate() exactly.
"""

from __future__ import annotations

import heapq

from . import schedule as Sch


def ticket_order(plan: Sch.Plan, heads: int, worker_order=None):
    """Head-major ticket list [(head, worker)]: all workers of head 0 in
    worker_order (default ascending), then head 1, and so on."""
    order = list(range(len(plan.workers))) if worker_order is None else list(worker_order)
    if sorted(order) != list(range(len(plan.workers))):
        raise ValueError("worker_order must be a permutation of the plan's workers")
    return [(h, w) for h in range(heads) for w in order]


def interleaved_ticket_order(plan: Sch.Plan, heads: int, ilv: int):
    """Tickets [(head, worker)] dealt in runs of `ilv` heads, worker by
    worker: worker 0 of each head of the run, then worker 1 of each, and so
    on; a last run may hold fewer heads. ilv = 1 is ticket_order(plan, heads)."""
    if ilv < 1:
        raise ValueError("ilv must be at least 1")
    n = len(plan.workers)
    out = []
    for first in range(0, heads, ilv):
        run = range(first, min(heads, first + ilv))
        out += [(h, w) for w in range(n) for h in run]
    return out


def simulate(plan: Sch.Plan, heads: int, processors: int, c: float = 1.0, r: float = 0.0,
             tickets=None):
    """Run every unit of `heads` copies of `plan` on `processors` processors.

    tickets: the queue as a list of (head, worker), default ticket_order(plan, heads).
    Returns a dict with the makespan, each unit's (processor, start, end), and
    each processor's busy and waiting time, or None if the run deadlocks.
    """
    if processors < 1:
        raise ValueError("need at least one processor")
    tickets = ticket_order(plan, heads) if tickets is None else list(tickets)
    # predecessor of task (i, j) in dQ tile i's accumulation order (None for the first)
    pred = {}
    for i, order in enumerate(plan.orders):
        for k, j in enumerate(order):
            pred[(i, j)] = order[k - 1] if k else None
    chains = [[(i, j) for _, i, j in sorted(tasks)] for tasks in plan.workers]

    done = {}             # (head, i, j) -> finish time of R(i, j)
    waiting = {}          # (head, i, j) -> the unit waiting for that reduction (its one successor)
    units = []            # per started unit: [head, worker, processor, task index, start, ready time]
    spans = {}
    wait_time = [0.0] * processors
    next_ticket = 0
    events = []           # (time, kind, tie, seq, payload); kind 0 = R done, 1 = C done, 2 = processor free
    seq = 0

    def push(t, kind, tie, payload):
        nonlocal seq
        heapq.heappush(events, (t, kind, tie, seq, payload))
        seq += 1

    for p in range(processors):
        push(0.0, 2, p, p)

    while events:
        t, kind, _, _, x = heapq.heappop(events)
        if kind == 2:                         # processor x takes the next ticket
            if next_ticket >= len(tickets):
                continue
            h, w = tickets[next_ticket]
            next_ticket += 1
            if not chains[w]:
                spans[(h, w)] = (x, t, t)
                push(t, 2, x, x)
                continue
            units.append([h, w, x, 0, t, None])
            push(t + c, 1, x, len(units) - 1)
        elif kind == 1:                       # unit x finished C of its current task
            h, w, p, k, _, _ = units[x]
            i, j = chains[w][k]
            units[x][5] = t
            before = pred[(i, j)]
            if before is None or (h, i, before) in done:
                # events run in time order: a finished predecessor finished by now
                push(t + r, 0, p, x)
            else:
                waiting[(h, i, before)] = x
        else:                                 # unit x finished R of its current task
            h, w, p, k, start, _ = units[x]
            i, j = chains[w][k]
            done[(h, i, j)] = t
            y = waiting.pop((h, i, j), None)
            if y is not None:
                wait_time[units[y][2]] += t - units[y][5]
                push(t + r, 0, units[y][2], y)
            if k + 1 < len(chains[w]):
                units[x][3] = k + 1
                push(t + c, 1, p, x)
            else:
                spans[(h, w)] = (p, start, t)
                push(t, 2, p, p)

    if waiting or next_ticket < len(tickets) or len(spans) != len(tickets):
        return None
    busy = [0.0] * processors
    for (h, w), (p, s, e) in spans.items():
        busy[p] += e - s
    return {
        "makespan": max((e for _, _, e in spans.values()), default=0.0),
        "spans": spans,
        "busy": busy,
        "wait": wait_time,
    }


def makespan(plan: Sch.Plan, heads: int, processors: int, c: float = 1.0, r: float = 0.0, tickets=None):
    """The makespan alone (None on deadlock)."""
    res = simulate(plan, heads, processors, c, r, tickets)
    return None if res is None else res["makespan"]


def best_worker_order(plan: Sch.Plan, heads: int, processors: int, candidates: dict, c: float = 1.0,
                      r: float = 0.0):
    """Among named worker orders {name: order}, the one with the smallest
    makespan (ties: first in the dict), and every candidate's makespan."""
    results = {}
    for name, order in candidates.items():
        results[name] = makespan(plan, heads, processors, c, r, ticket_order(plan, heads, order))
    finite = {k: v for k, v in results.items() if v is not None}
    best = min(finite, key=lambda k: (finite[k], list(candidates).index(k))) if finite else None
    return best, results


def simulate_pipelined(plan: Sch.Plan, heads: int, processors: int, c: float = 1.0, r: float = 0.0,
                       tickets=None, nsub: int = 1, lag: int = 0, setup: float = 0.0, delay: float = 0.0,
                       gate: str = "done"):
    """The same queue and processors, with the reduction taken off the processor.

    A reading of how a persistent kernel overlaps the dQ hand-off with compute
    (the pages' DAG charges the reduction to the worker's chain): each task is
    cut into `nsub` sub-tiles of compute time c each; sub-tile h of task (i, j)
    contributes to dQ sub-tile (i, h), in the same KV order as the task. A
    sub-tile's hand-off starts (takes its turn) no earlier than `delay` after
    its compute has finished, once the unit's previous hand-off is done (a unit
    hands over in order) and the previous contributor to the same dQ sub-tile
    has finished its hand-off; it lasts r. The processor runs at most `lag`
    sub-tiles ahead of its hand-offs: compute of sub-tile x waits until
    hand-off x - 1 - lag has finished (gate "done") or started (gate "start":
    the processor waits for the turn to be taken, not for the add). A unit
    first spends `setup` on its own (loading its KV tile) and holds its
    processor until its last hand-off is done.

    With the defaults (nsub = 1, lag = 0, setup = 0, delay = 0, gate "done")
    this is simulate(): the next task's compute waits for the previous
    reduction, which then occupies the chain exactly as in the DAG. Returns the
    same dict (or None on deadlock).
    """
    if processors < 1 or nsub < 1 or lag < 0 or gate not in ("done", "start"):
        raise ValueError("need processors >= 1, nsub >= 1, lag >= 0, gate 'done' or 'start'")
    tickets = ticket_order(plan, heads) if tickets is None else list(tickets)
    pred = {}
    for i, order in enumerate(plan.orders):
        for k, j in enumerate(order):
            pred[(i, j)] = order[k - 1] if k else None
    chains = [[(i, j, hf) for _, i, j in sorted(tasks) for hf in range(nsub)] for tasks in plan.workers]

    done = {}       # (head, i, half, j) -> hand-off finish time
    waiting = {}    # (head, i, half, j) -> unit whose next hand-off follows that one
    units = []      # dicts per started unit
    spans = {}
    wait_time = [0.0] * processors
    next_ticket = 0
    events = []     # (time, kind, tie, seq, payload)
    seq = 0
    # kinds: 0 hand-off done, 1 compute done, 2 processor free, 3 set-up done, 4 hand-off may start

    def push(t, kind, tie, payload):
        nonlocal seq
        heapq.heappush(events, (t, kind, tie, seq, payload))
        seq += 1

    def try_compute(u, t):
        """Start unit u's next compute at time t if the lag allows it."""
        st = units[u]
        x = st["nc"]
        if st["busy_c"] or not st["ready"] or x >= len(st["chain"]):
            return
        need = x - 1 - lag           # the hand-off the processor may not run ahead of
        passed = st["nh"] + (1 if (gate == "start" and st["busy_h"]) else 0)
        if need >= 0 and passed <= need:
            return
        st["busy_c"] = True
        push(t + c, 1, st["p"], u)

    def try_handoff(u, t):
        """Start unit u's next hand-off at time t if its conditions hold."""
        st = units[u]
        x = st["nh"]
        if st["busy_h"] or x >= len(st["chain"]) or x not in st["may"]:
            return
        i, j, hf = st["chain"][x]
        before = pred[(i, j)]
        key = (st["h"], i, hf, before)
        if before is not None and key not in done:
            waiting[key] = u
            st["wait_from"] = t
            return
        st["busy_h"] = True
        push(t + r, 0, st["p"], u)
        try_compute(u, t)

    for p in range(processors):
        push(0.0, 2, p, p)

    while events:
        t, kind, _, _, x = heapq.heappop(events)
        if kind == 2:                                   # processor x takes the next ticket
            if next_ticket >= len(tickets):
                continue
            h, w = tickets[next_ticket]
            next_ticket += 1
            if not chains[w]:
                spans[(h, w)] = (x, t, t)
                push(t, 2, x, x)
                continue
            units.append({"h": h, "w": w, "p": x, "start": t, "chain": chains[w], "nc": 0, "nh": 0,
                          "may": set(), "busy_c": False, "busy_h": False, "ready": setup <= 0,
                          "wait_from": None})
            u = len(units) - 1
            if setup > 0:
                push(t + setup, 3, x, u)
            else:
                try_compute(u, t)
        elif kind == 3:                                 # unit x finished its set-up
            units[x]["ready"] = True
            try_compute(x, t)
        elif kind == 1:                                 # unit x finished computing sub-tile nc
            st = units[x]
            st["nc"] += 1
            st["busy_c"] = False
            if delay > 0:
                push(t + delay, 4, st["p"], (x, st["nc"] - 1))
            else:
                st["may"].add(st["nc"] - 1)
                try_handoff(x, t)
            try_compute(x, t)
        elif kind == 4:                                 # a finished sub-tile's hand-off may start
            u, y = x
            units[u]["may"].add(y)
            try_handoff(u, t)
        else:                                           # unit x finished hand-off nh
            st = units[x]
            i, j, hf = st["chain"][st["nh"]]
            key = (st["h"], i, hf, j)
            done[key] = t
            st["nh"] += 1
            st["busy_h"] = False
            y = waiting.pop(key, None)
            if y is not None:
                wait_time[units[y]["p"]] += t - units[y]["wait_from"]
                units[y]["wait_from"] = None
                try_handoff(y, t)
            if st["nh"] == len(st["chain"]):
                spans[(st["h"], st["w"])] = (st["p"], st["start"], t)
                push(t, 2, st["p"], st["p"])
            else:
                try_handoff(x, t)
                try_compute(x, t)

    if waiting or next_ticket < len(tickets) or len(spans) != len(tickets):
        return None
    busy = [0.0] * processors
    for (h, w), (p, s, e) in spans.items():
        busy[p] += e - s
    return {"makespan": max((e for _, _, e in spans.values()), default=0.0), "spans": spans, "busy": busy,
            "wait": wait_time}
