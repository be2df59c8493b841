"""Pins for the routing oracle (oracle/route.py)."""
import json
import math
import os

import numpy as np
import pytest

from oracle.route import route, route_row

GOLD = os.path.join(os.path.dirname(__file__), "golden", "route_cases.json")


def test_golden_cases():
    for c in json.load(open(GOLD))["cases"]:
        ids, w = route_row(c["logits"], c["k"])
        assert ids == c["ids"], c
        if c["w"] is not None:
            np.testing.assert_allclose(w, c["w"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("E,k,seed", [(16, 2, 0), (256, 8, 1), (256, 6, 2), (7, 7, 3)])
def test_against_lexsort_and_softmax_properties(E, k, seed):
    rng = np.random.default_rng(seed)
    # coarse values so that ties are frequent
    logits = rng.integers(-4, 5, size=(64, E)).astype(np.float32) * np.float32(0.5)
    ids, ws = route(logits, k)
    for t in range(64):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))[:k]
        assert list(order) == ids[t]
        w = np.array(ws[t])
        assert abs(w.sum() - 1.0) < 1e-15
        assert np.all(np.diff(w) <= 0)
        for j in range(k):
            assert math.isclose(w[j] / w[0], math.exp(float(logits[t, ids[t][j]]) - float(logits[t, ids[t][0]])),
                                rel_tol=1e-14)


def test_full_sort_brute_force():
    rng = np.random.default_rng(5)
    for _ in range(50):
        E = int(rng.integers(1, 40))
        k = int(rng.integers(1, E + 1))
        row = rng.normal(size=E).astype(np.float32)
        row[rng.integers(0, E, size=3)] = row[0]
        ids, _ = route_row(row, k)
        # brute force: an id is selected iff fewer than k ids beat it
        beats = lambda a, b: (row[a] > row[b]) or (row[a] == row[b] and a < b)
        sel = [i for i in range(E) if sum(beats(j, i) for j in range(E)) < k]
        assert sorted(sel) == sorted(ids)
