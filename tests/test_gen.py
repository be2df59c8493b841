"""The seeded input generator (gen/): decode routing logits with step-to-step overlap.

The k experts a token routes to at step s keep each of step s-1's experts with probability p and
draw the rest from the E - k experts outside that set; where fewer remain than are needed (2k > E),
the shortfall is kept from the previous set. Checked on the CPU: every row has k distinct top
logits, every step terminates, consecutive sets share at least max(0, 2k - E) experts, and the
measured overlap follows p where the experts outside suffice.
"""
import numpy as np
import pytest

import gen
from gen.configs import TINY


def top_sets(lg, k):
    # the k largest logits of each row (the generator's logits are distinct)
    return np.argsort(-lg, axis=-1, kind="stable")[..., :k]


@pytest.mark.parametrize("E,k,p", [(16, 15, 0.9), (16, 15, 0.0), (3, 2, 0.0), (8, 8, 0.5), (5, 3, 0.3)])
def test_overlap_when_few_experts_remain(E, k, p):
    cfg = TINY.with_(L=2, E=E, k=k, p=p)
    lg = gen.decode_logits(cfg, steps=32, T=5)
    assert lg.shape == (32, 2, 5, E)
    sets = top_sets(lg, k)
    for s in range(1, 32):
        for l in range(2):
            for t in range(5):
                a, b = set(sets[s - 1, l, t]), set(sets[s, l, t])
                assert len(b) == k
                assert len(a & b) >= max(0, 2 * k - E)


def test_overlap_follows_p():
    cfg = TINY.with_(L=1, E=256, k=8, p=0.6)
    sets = top_sets(gen.decode_logits(cfg, steps=400, T=4), 8)
    ov = np.mean([len(set(sets[s, 0, t]) & set(sets[s - 1, 0, t])) / 8 for s in range(1, 400) for t in range(4)])
    assert abs(ov - 0.6) < 0.03, ov
