"""Routing oracle: top-k experts by logit and their combine weights.

Follows the FreeToken write-up ("Why personal MoE is hard": each token is
routed to k of E experts per layer, e.g. 6 of 256). The write-up names top-k
routing only; the reading used here is: the k largest logits, ties to the
lower expert id, ordered by (logit descending, id ascending); combine weights
are the softmax over the k selected logits, computed in fp64.

Pins (tests/test_oracle_route.py): hand-worked cases with ties under
tests/golden/, numpy.lexsort as a library special case, sum of weights = 1,
weight ratios equal exp of logit differences.
"""
import math


def route_row(logits_row, k):
    """One token: (ids[k], w[k]) with ids ordered by (logit desc, id asc)."""
    vals = [float(v) for v in logits_row]
    order = sorted(range(len(vals)), key=lambda i: (-vals[i], i))[:k]
    top = vals[order[0]]
    ex = [math.exp(vals[i] - top) for i in order]
    s = 0.0
    for e in ex:
        s += e
    return order, [e / s for e in ex]


def route(logits, k):
    """logits [T][E] (any nested sequence / 2-D array) -> (ids [T][k], w [T][k])."""
    ids, ws = [], []
    for row in logits:
        i, w = route_row(row, k)
        ids.append(i)
        ws.append(w)
    return ids, ws
