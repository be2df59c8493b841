"""Pins for the LRU simulator (oracle/lru_sim.py)."""
import json
import os

import numpy as np
import pytest

from oracle.brute_lru import BruteLRU
from oracle.lru_sim import FILL, HIT, HOST, LRUSim, fill_count

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _key(k):
    return None if k is None else tuple(k)


def test_hand_traced_steps():
    g = json.load(open(os.path.join(GOLD, "lru_trace_tiny.json")))
    sim = LRUSim(g["L"], g["E"], g["C"], g["K"], 1000, 1000)
    for s in g["steps"]:
        sim.set_bandwidth(s["bp"], s["bh"])
        r = sim.step(s["layer"], s["ids"])
        for f in ("uniq", "h", "m", "q", "fills", "victims", "host_list", "rewritten", "cls"):
            assert r[f] == s[f], (f, r[f], s[f])
        assert r["evicted"] == [_key(e) for e in s["evicted"]]


def test_qstar_table():
    for r in json.load(open(os.path.join(GOLD, "qstar_table.json")))["rows"]:
        assert fill_count(r["m"], r["bp"], r["bh"], r["K"], r["n_avail"]) == r["q"], r


def test_qstar_degenerate_and_errors():
    # BP >= BH -> every miss is filled (up to the caps); BP = 0 -> none are
    for m in range(0, 97):
        for bp, bh in [(1000, 1000), (2000, 1000), (1001, 1000), (5, 1)]:
            assert fill_count(m, bp, bh, 1000, 1000) == m
        assert fill_count(m, 0, 1000, 1000, 1000) == 0
        assert fill_count(m, 999, 1000, 1000, 1000) <= m
    with pytest.raises(ValueError):
        fill_count(3, 1, 0, 8, 8)


def _random_trace(rng, L, E, T, k, n):
    out = []
    for _ in range(n):
        l = int(rng.integers(0, L))
        ids = [list(rng.choice(E, size=k, replace=False)) for _ in range(T)]
        out.append((l, [[int(e) for e in row] for row in ids]))
    return out


@pytest.mark.parametrize("seed", range(12))
def test_against_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    L, E = 2, 8
    C = int(rng.integers(0, 7))
    K = int(rng.integers(1, 5))
    T = int(rng.integers(1, 3))
    k = int(rng.integers(1, 4))
    bp, bh = [(1000, 1000), (500, 1000), (300, 1000), (2000, 1000)][seed % 4]
    sim, ref = LRUSim(L, E, C, K, bp, bh), BruteLRU(C, K, bp, bh)
    for n, (l, ids) in enumerate(_random_trace(rng, L, E, T, k, 60)):
        if n == 30:
            newC = int(rng.integers(0, 7))
            sim.rebuild(newC)
            ref.rebuild(newC)
        a, b = sim.step(l, ids), ref.step(l, ids)
        for f in ("h", "m", "q", "victims", "evicted"):
            assert a[f] == b[f], (n, f, a[f], b[f])
        assert set(sim.resid.items()) == set(ref.where.items())


@pytest.mark.parametrize("seed", range(6))
def test_textbook_lru_set(seed):
    """q = m and enough candidates: residents are the C most recent distinct keys."""
    rng = np.random.default_rng(200 + seed)
    L, E, T, k = 3, 10, 2, 3
    C = int(rng.integers(T * k, 12))
    sim, ref = LRUSim(L, E, C, T * k, 1000, 1000), BruteLRU(C, T * k, 1000, 1000)
    for l, ids in _random_trace(rng, L, E, T, k, 80):
        r = sim.step(l, ids)
        ref.step(l, ids)
        assert r["q"] == r["m"] and r["host_list"] == []
        assert sim.resident_keys() == ref.most_recent_distinct(C)


@pytest.mark.parametrize("seed", range(4))
def test_mattson_inclusion(seed):
    """With every miss filled, the resident set of C slots is inside that of C+1."""
    rng = np.random.default_rng(300 + seed)
    L, E, T, k = 2, 12, 1, 3
    trace = _random_trace(rng, L, E, T, k, 120)
    sims = [LRUSim(L, E, C, k, 1000, 1000) for C in range(k, 16)]
    hits = [0] * len(sims)
    for l, ids in trace:
        for i, s in enumerate(sims):
            hits[i] += s.step(l, ids)["h"]
        for a, b in zip(sims, sims[1:]):
            assert a.resident_keys() <= b.resident_keys()
    assert hits == sorted(hits)


@pytest.mark.parametrize("seed", range(6))
def test_step_invariants(seed):
    rng = np.random.default_rng(400 + seed)
    L, E, T, k = 3, 16, 3, 4
    C, K = 7, 3
    bp, bh = [(300, 1000), (1000, 1000), (700, 1000)][seed % 3]
    sim = LRUSim(L, E, C, K, bp, bh)
    for l, ids in _random_trace(rng, L, E, T, k, 80):
        r = sim.step(l, ids)
        flat = sorted(set(e for row in ids for e in row))
        assert r["uniq"] == flat
        assert r["h"] + r["m"] == len(flat)
        assert r["q"] <= min(r["m"], K, C - r["h"])
        assert len(r["host_list"]) == r["m"] - r["q"]
        assert len(set(r["victims"])) == len(r["victims"]) == r["q"]
        for t, row in enumerate(ids):
            for j, e in enumerate(row):
                s = r["rewritten"][t][j]
                c = r["cls"][r["pos"][t][j]]
                if s >= 0:
                    assert c in (HIT, FILL) and sim.slot_key[s] == (l, e)
                else:
                    assert c == HOST and r["host_list"][-s - 1] == e and (l, e) not in sim.resid


def test_budget_zero_is_all_host():
    sim = LRUSim(2, 8, 0, 4, 1000, 1000)
    r = sim.step(0, [[1, 2, 3]])
    assert (r["h"], r["m"], r["q"], r["host_list"]) == (0, 3, 0, [1, 2, 3])
    assert r["rewritten"] == [[-1, -2, -3]]
