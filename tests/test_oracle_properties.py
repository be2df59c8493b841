"""Property tests (hypothesis) for the oracle's routing and shared-LRU simulator.

Generated traces and logits, checked against independent models and against the facts the
FreeToken write-up states:
- the cache step ("Implementation notes", "1. Bandwidth-adaptive execution") equals the
  brute-force LRU over the whole access history on every step, across rebuilds and changes of
  BP:BH;
- q = m whenever BP >= BH (within the caps K and C - h); q <= m always; filled experts become
  resident, host-side experts leave residency unchanged;
- with every miss filled, the residents are the C most recently used distinct keys;
- routing: the k largest logits with ties to the lower id (a brute force over all k-subsets on
  small E), weights summing to 1 with ratios exp(l_i - l_j).
"""
import itertools
import math

from hypothesis import given, settings, strategies as st

from oracle.brute_lru import BruteLRU
from oracle.lru_sim import LRUSim, fill_count
from oracle.route import route_row

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True)


@st.composite
def traces(draw):
    L = draw(st.integers(1, 3))
    E = draw(st.integers(2, 9))
    k = draw(st.integers(1, min(3, E)))
    T = draw(st.integers(1, 3))
    C = draw(st.integers(0, 8))
    K = draw(st.integers(1, 6))
    n = draw(st.integers(1, 40))
    ratios = st.sampled_from([(0, 1000), (300, 1000), (500, 1000), (999, 1000), (1000, 1000), (2000, 1000)])
    steps = []
    for _ in range(n):
        layer = draw(st.integers(0, L - 1))
        ids = [draw(st.lists(st.integers(0, E - 1), min_size=k, max_size=k, unique=True)) for _ in range(T)]
        event = draw(st.sampled_from(["step"] * 8 + ["rebuild", "bandwidth"]))
        arg = draw(st.integers(0, 8)) if event == "rebuild" else draw(ratios) if event == "bandwidth" else None
        steps.append((layer, ids, event, arg))
    return L, E, C, K, draw(ratios), steps


@SETTINGS
@given(traces())
def test_lru_sim_equals_brute_force(tr):
    L, E, C, K, (bp, bh), steps = tr
    sim, ref = LRUSim(L, E, C, K, bp, bh), BruteLRU(C, K, bp, bh)
    for layer, ids, event, arg in steps:
        if event == "rebuild":
            sim.rebuild(arg)
            ref.rebuild(arg)
        elif event == "bandwidth":
            sim.set_bandwidth(*arg)
            ref.bp, ref.bh = arg
        before = dict(sim.resid)
        a, b = sim.step(layer, ids), ref.step(layer, ids)
        for f in ("h", "m", "q", "victims", "evicted"):
            assert a[f] == b[f], (f, a[f], b[f])
        assert set(sim.resid.items()) == set(ref.where.items())
        # the split: q <= m, all misses filled when BP >= BH (within the caps)
        assert a["q"] <= a["m"]
        if sim.bp >= sim.bh:
            assert a["q"] == min(a["m"], sim.K, sim.C - a["h"])
        # filled experts are resident afterwards; host-side experts are not, and never were
        for u in a["fills"]:
            assert (layer, u) in sim.resid
        for u in a["host_list"]:
            assert (layer, u) not in sim.resid and (layer, u) not in before


@SETTINGS
@given(st.integers(1, 3), st.integers(4, 12), st.integers(1, 2), st.integers(1, 3), st.integers(0, 10 ** 6))
def test_every_miss_filled_keeps_the_most_recent(L, E, T, k, seed):
    import random
    rng = random.Random(seed)
    k = min(k, E)
    C = rng.randint(T * k, 12)
    sim, ref = LRUSim(L, E, C, T * k, 1000, 1000), BruteLRU(C, T * k, 1000, 1000)
    for _ in range(40):
        layer = rng.randrange(L)
        ids = [rng.sample(range(E), k) for _ in range(T)]
        r = sim.step(layer, ids)
        ref.step(layer, ids)
        assert r["q"] == r["m"] and r["host_list"] == []
        assert sim.resident_keys() == ref.most_recent_distinct(C)


@SETTINGS
@given(st.integers(0, 200), st.integers(0, 5000), st.integers(1, 5000), st.integers(0, 80), st.integers(0, 80))
def test_fill_count_closed_form(m, bp, bh, K, avail):
    q = fill_count(m, bp, bh, K, avail)
    assert 0 <= q <= m and q <= K and q <= max(avail, 0)
    # the largest q with q * BH <= m * BP, within the caps
    assert q == max(0, min([m, K, avail] + [max(i for i in range(m + 1) if i * bh <= m * bp)]))


@SETTINGS
@given(st.integers(1, 7), st.data())
def test_route_row_is_the_top_k_with_ties_to_lower_ids(E, data):
    k = data.draw(st.integers(1, E))
    logits = data.draw(st.lists(st.integers(-3, 3), min_size=E, max_size=E))  # many ties
    ids, w = route_row(logits, k)
    # brute force: among all k-subsets, the one with the largest logit multiset, then smallest ids
    best = min(itertools.combinations(range(E), k),
               key=lambda s: (sorted((-logits[i] for i in s)), sorted(s)))
    assert sorted(ids) == sorted(best)
    assert ids == sorted(ids, key=lambda i: (-logits[i], i))
    assert abs(sum(w) - 1.0) < 1e-12
    for a in range(k):
        for b in range(k):
            assert abs(w[a] / w[b] - math.exp(logits[ids[a]] - logits[ids[b]])) < 1e-9
