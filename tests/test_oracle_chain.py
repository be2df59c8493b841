"""Pins for the chained-block oracle (oracle/chain.py): router logits, bf16 rounding, residual."""
import os

import numpy as np

from oracle import chain, moe

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden_bf16():
    rows = []
    for line in open(os.path.join(GOLD, "bf16_rne.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        v, b = line.split()
        val = float.fromhex(v) if "0x" in v and "p" in v else float(v)
        rows.append((val, int(b, 16)))
    return rows


def test_bf16_rounding_matches_hand_derived_values():
    rows = _golden_bf16()
    got = chain.round_bf16(np.array([v for v, _ in rows]))
    assert [int(g) for g in got] == [b for _, b in rows]


def test_bf16_round_trip_of_representable_values():
    rng = np.random.default_rng(3)
    bits = rng.integers(0x0080, 0x7F00, size=2000).astype(np.uint16)  # positive normals
    bits = np.concatenate([bits, bits | np.uint16(0x8000)])
    assert np.array_equal(chain.round_bf16(chain.widen_bf16(bits)), bits)


def test_rounding_is_to_the_nearest_bf16():
    # brute force: the chosen bf16 is no farther than either neighbour
    rng = np.random.default_rng(4)
    v = rng.normal(0, 3, 3000)
    b = chain.round_bf16(v).astype(np.int64)
    mid = chain.widen_bf16(b.astype(np.uint16))
    for d in (-1, 1):
        nb = chain.widen_bf16((b + d).astype(np.uint16))
        assert np.all(np.abs(v - mid) <= np.abs(v - nb))


def test_gate_logits_exact_on_integers_and_brute_force_dot():
    rng = np.random.default_rng(5)
    W = rng.integers(-8, 9, size=(7, 12)).astype(np.float64)
    x = rng.integers(-5, 6, size=(3, 12)).astype(np.float64)
    got = chain.gate_logits(W, x)
    for t in range(3):
        for e in range(7):
            assert got[t, e] == sum(int(W[e, h]) * int(x[t, h]) for h in range(12))


def test_gate_logits_linear_in_x():
    rng = np.random.default_rng(6)
    W, x = rng.normal(size=(16, 64)), rng.normal(size=(2, 64))
    assert np.array_equal(chain.gate_logits(W, 2.0 * x), 2.0 * chain.gate_logits(W, x))


def _tiny_experts(H, I, E, zero_down, rng):
    mats = {}
    for e in range(E):
        m = {"gate": rng.normal(0, 0.1, (I, H)).astype(np.float32),
             "up": rng.normal(0, 0.1, (I, H)).astype(np.float32),
             "down": np.zeros((H, I), np.float32) if zero_down else rng.normal(0, 0.1, (H, I)).astype(np.float32)}
        mats[e] = m
    return lambda e: mats[e]


def test_block_with_zero_down_weights_returns_its_input():
    rng = np.random.default_rng(7)
    H, I, E, k = 64, 32, 8, 2
    get = _tiny_experts(H, I, E, True, rng)
    x = rng.normal(size=(3, H)).astype(np.float32)
    W = rng.normal(0, 0.2, (E, H)).astype(np.float32)
    nxt, ids, ws, margin = chain.block(moe.F32, x, W, k, get)
    assert np.array_equal(nxt, x)
    xb = chain.round_bf16(x.astype(np.float64))
    Wb = chain.round_bf16(W.astype(np.float64))
    nxt_b, _, _, _ = chain.block(moe.BF16, xb, Wb, k, lambda e: {kk: chain.round_bf16(v.astype(np.float64))
                                                                 for kk, v in get(e).items()})
    assert np.array_equal(nxt_b, xb)


def test_block_routes_on_the_data_and_adds_the_residual():
    rng = np.random.default_rng(8)
    H, I, E, k = 64, 32, 8, 2
    get = _tiny_experts(H, I, E, False, rng)
    x = rng.normal(size=(2, H)).astype(np.float32)
    W = rng.normal(0, 0.2, (E, H)).astype(np.float32)
    nxt, ids, ws, margin = chain.block(moe.F32, x, W, k, get)
    for t in range(2):
        lg = [sum(float(W[e, h]) * float(x[t, h]) for h in range(H)) for e in range(E)]
        order = sorted(range(E), key=lambda e: (-np.float32(lg[e]), e))
        assert list(ids[t]) == order[:k]
        srt = sorted((np.float32(v) for v in lg), reverse=True)
        assert abs(margin[t] - (float(srt[k - 1]) - float(srt[k]))) == 0.0
        ref = x[t].astype(np.float64)
        for e, w in zip(ids[t], ws[t]):
            m = get(e)
            g, u = m["gate"].astype(np.float64) @ x[t], m["up"].astype(np.float64) @ x[t]
            ref = ref + w * (m["down"].astype(np.float64) @ (g / (1 + np.exp(-g)) * u))
        assert np.allclose(nxt[t], ref.astype(np.float32), rtol=1e-6, atol=1e-7)
