"""Brute-force LRU over the full access history (tiny inputs only).

An independent model of the shared LRU expert cache (FreeToken write-up,
"Semantic-aware caching" and "Implementation notes"): it stores nothing but
the list of cache-side accesses (clock, rank, key) and, at every step,
re-derives each resident key's last access by scanning that whole list.

Victims for the q fills are the empty slots first (ascending slot index), then
resident keys in increasing order of last access, skipping those hit in the
current step. With every miss filled and enough candidates (q = m, K >= U,
C >= U), the resident set must be exactly the C most recently used distinct
keys of the history: the textbook LRU property.
"""


class BruteLRU:
    def __init__(self, C, K, bp, bh):
        self.C, self.K, self.bp, self.bh = C, K, bp, bh
        self.history = []  # (clock, rank, key) of every cache-side access
        self.where = {}    # key -> slot for resident keys
        self.clock = 0

    def rebuild(self, C):
        self.C = C
        self.where = {}

    def last_access(self, key):
        best = None
        for (c, r, k) in self.history:
            if k == key and (best is None or (c, r) > best):
                best = (c, r)
        return best

    def step(self, layer, ids):
        U = sorted(set(int(e) for row in ids for e in row))
        hits = [u for u in U if (layer, u) in self.where]
        misses = [u for u in U if (layer, u) not in self.where]
        m, h = len(misses), len(hits)
        q = max(0, min(m, (m * self.bp) // self.bh, self.K, self.C - h))
        used = set(self.where.values())
        empty = [s for s in range(self.C) if s not in used]
        hit_keys = set((layer, u) for u in hits)
        residents = [k for k in self.where if k not in hit_keys]
        residents.sort(key=lambda k: self.last_access(k))
        order = [(s, None) for s in empty] + [(self.where[k], k) for k in residents]
        chosen = order[:q]
        for (s, k), f in zip(chosen, misses[:q]):
            if k is not None:
                del self.where[k]
            self.where[(layer, f)] = s
        side = set(hits) | set(misses[:q])
        for rank, u in enumerate(U):
            if u in side:
                self.history.append((self.clock, rank, (layer, u)))
        self.clock += 1
        return dict(h=h, m=m, q=q, victims=[s for s, _ in chosen], evicted=[k for _, k in chosen])

    def most_recent_distinct(self, n):
        """The n most recently accessed distinct keys of the history."""
        seen, out = set(), []
        for (c, r, k) in sorted(self.history, reverse=True):
            if k not in seen:
                seen.add(k)
                out.append(k)
            if len(out) == n:
                break
        return set(out)
