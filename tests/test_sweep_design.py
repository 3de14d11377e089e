"""Host-only checks of the small-shape GPU sweep's design (tests/
test_gpu_sweep.py): every pair of drawn factor values, and every factor value
with every element type, occurs in some case; the cases reach every kind of
step (drifting, compacting, overlapping in-place move, staged, longer than
the cache) for every element type, by the oracle's plan."""
from __future__ import annotations

import itertools

import numpy as np

import oracle
from tests.test_gpu_sweep import DTYPES, FACTORS, _kind, all_cases, draw_factors


def test_case_count():
    # sum over C of C * (2C + 1) shapes, times three element types
    assert len(all_cases()) == 3 * sum(C * (2 * C + 1) for C in range(1, 13))


def test_factor_pairs_all_occur():
    seen = set()
    for i, (C, W, S, dt) in enumerate(all_cases()):
        f, _ = draw_factors(i)
        items = [("dtype", dt)] + sorted(f.items())
        for a, b in itertools.combinations(items, 2):
            seen.add((a, b))
    names = ["dtype"] + sorted(FACTORS)
    values = {"dtype": DTYPES, **FACTORS}
    for x, y in itertools.combinations(names, 2):
        for vx in values[x]:
            for vy in values[y]:
                assert ((x, vx), (y, vy)) in seen, (x, vx, y, vy)


def test_every_step_kind_occurs_per_element_type_and_part():
    kinds = {}
    for i, (C, W, S, dt) in enumerate(all_cases()):
        f, rng = draw_factors(i)
        P = rng.integers(0, 3 * C + 3, size=f["B"])
        p = oracle.make_params(f["B"], S, f["Hkv"] * f["group"], f["Hkv"], f["D"], C, W,
                               int((P + S).max()))
        st, plan = oracle.plan(p, (P + S - 1).astype(np.int32))
        assert st == 0
        for b in range(f["B"]):
            key = (dt, C <= 9, _kind(plan[b], S, C))
            kinds[key] = kinds.get(key, 0) + 1
    for dt in DTYPES:
        for part in (True, False):
            for k in ("drifting", "compacting", "overlapping move", "staged",
                      "longer than the cache"):
                assert kinds.get((dt, part, k), 0) > 0, (dt, part, k)
