"""Model of the main kernel's XCD-queue unit claims (host logic, CPU only).

The persistent backward kernel hands out units (one worker of one head) from
one ticket queue per XCD. With interleaving (naive and Descending), runs of
`ilv` heads share a run of ilv x workers tickets, worker by worker; the first
ticket of a run claims the run's heads from a counter shared by all XCDs,
after the queue's previous run has claimed; a ticket whose slot lies past the
last head takes another ticket, and a run that starts past it ends the queue.
This model plays that protocol out under random interleavings of the
workgroups (a worker completes only once the worker before it in its head has
started, as the dQ order of these schedules requires) and checks that every
unit runs exactly once and that no wait is left hanging, for grids where some
XCD queues hold a single workgroup. It also shows why the simpler rule (a
workgroup leaves as soon as one of its tickets lies past the last head) is
wrong once heads are interleaved: units of a claimed head are left over.
"""

import itertools
import random

import pytest


def play(grid, BH, n_workers, ilv, seed, leave_on_any_past_end=False, n_xcd=8):
    rng = random.Random(seed)
    counter = 0
    ticket = [0] * n_xcd
    slots = {}
    started, done = set(), set()
    wgs = [{"x": g % n_xcd, "st": "claim"} for g in range(grid)]
    while True:
        live = [w for w in wgs if w["st"] != "gone"]
        if not live:
            break
        rng.shuffle(live)
        for w in live:
            if w["st"] == "claim":
                k = ticket[w["x"]]
                ticket[w["x"]] += 1
                span = ilv * n_workers
                w.update(st="slot", grp=k // span, rem=k % span)
                break
            if w["st"] == "slot":
                x, grp, rem = w["x"], w["grp"], w["rem"]
                if leave_on_any_past_end:
                    # one slot per head: the first ticket of each head claims it
                    key, first_ticket = (x, grp * ilv + rem % ilv), rem < ilv
                else:
                    key, first_ticket = (x, grp), rem == 0
                first = BH
                if key[1] < BH:
                    if first_ticket:
                        if not leave_on_any_past_end and grp > 0:
                            if (x, grp - 1) not in slots:
                                continue  # the queue's previous run has not claimed yet
                            if slots[(x, grp - 1)] >= BH:
                                slots[key] = BH
                                w["st"] = "gone"
                                break
                        step = 1 if leave_on_any_past_end else ilv
                        first = min(counter, BH)
                        counter += step
                        slots[key] = first
                    else:
                        if key not in slots:
                            continue
                        first = slots[key]
                head = first if leave_on_any_past_end else first + rem % ilv
                if first >= BH:
                    w["st"] = "gone"
                elif head >= BH:
                    w["st"] = "claim"
                else:
                    unit = (head, rem // ilv)
                    assert unit not in started, f"unit {unit} claimed twice"
                    started.add(unit)
                    w.update(st="run", unit=unit, left=rng.randint(1, 4))
                break
            if w["st"] == "run":
                h, wk = w["unit"]
                if wk > 0 and (h, wk - 1) not in started:
                    continue
                w["left"] -= 1
                if w["left"] == 0:
                    done.add(w["unit"])
                    w["st"] = "claim"
                break
        else:
            return None  # every live workgroup waits: a hang
    return done


@pytest.mark.parametrize("ilv", [1, 2, 4])
def test_every_unit_runs_once(ilv):
    for grid, BH, nw in itertools.product([1, 3, 8, 12, 17, 32], [1, 2, 3, 4, 5, 9], [1, 2, 3, 5, 16]):
        for seed in range(3):
            done = play(grid, BH, nw, ilv, seed)
            assert done is not None, (grid, BH, nw, ilv, seed)
            assert done == {(h, w) for h in range(BH) for w in range(nw)}, (grid, BH, nw, ilv, seed)


def test_leaving_on_any_past_end_ticket_loses_units():
    # 12 workgroups (XCDs 4..7 hold one each), 4 heads of 3 workers, 4 heads per run
    lost = [play(12, 4, 3, 4, seed, leave_on_any_past_end=True) for seed in range(5)]
    assert any(d is not None and len(d) < 12 for d in lost)
    # one head at a time it was right
    assert play(12, 4, 3, 1, 0, leave_on_any_past_end=True) == {(h, w) for h in range(4) for w in range(3)}
