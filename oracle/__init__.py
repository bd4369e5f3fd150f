"""CPU oracle for the deterministic attention backward (test infrastructure).

This package is test infrastructure. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. The product path
(the HIP library and its Python binding) never calls it and shares no code
with it.

Contents:
  * ``attention`` - plain float64 attention forward and backward (the
    definition written out), plus an unfused brute-force backward that forms
    each row's softmax Jacobian explicitly.
  * ``schedule`` - the four dQ scheduling strategies of the DASH pages
    (ascending, Descending Q-Tile, Shift, Symmetric Shift) as task lists and
    accumulation orders, plus the DAG model: critical path, conflict freedom,
    Lemma 1 depth monotonicity and deadlock freedom.
  * ``makespan`` - that DAG run for many heads on a fixed number of
    processors fed from one ticket queue (the persistent grid's setting):
    makespan, per-unit spans, busy and waiting time, deadlock detection;
    ticket orders one head after another or in interleaved runs of heads.

Every function is pinned by ``tests/test_oracle_*.py`` against things the
oracle does not compute itself: finite differences, closed forms, invariants,
torch's float64 autograd and ``scaled_dot_product_attention``, brute force
over tiny cases, list-scheduling bounds, a hand-worked two-head makespan
golden, and hand-worked inputs (including ones that must be rejected) for
the checkers ``attention.compare``, ``schedule.coverage_ok``,
``schedule.chains_ok`` and ``schedule.conflict_free``.
"""

from . import attention, makespan, schedule  # noqa: F401
