"""Literal shared-LRU expert-cache simulator with the q* miss split.

Follows the FreeToken write-up:
  * "Design": the host pool is the source of truth; leftover GPU memory is one
    elastic expert cache shared by all MoE layers.
  * "Bandwidth-adaptive execution", decode: misses are split between GPU
    cache fills and host-side compute, q* ~ m * BP / BH; filled experts become
    resident, host-computed ones leave residency unchanged; BH -> BP gives
    q* -> m, pure on-demand fill.
  * "Semantic-aware caching": a shared LRU expert cache across tokens.
  * "Implementation notes": one device pass dedups the routed experts,
    classifies them against the residency table, derives the fill count,
    picks the K least-recently-used victim slots in one scan and rewrites
    logical routing ids to cache slots.
  * "Elastic edge resource management": the cache is rebuilt at safe points
    for a new memory budget, without reloading the host pool.

Readings where the write-up is silent (each also listed in the design notes):
  q* = min(m, floor(m*BP/BH), K, C - h) in integers; the first q misses in
  ascending expert id are filled; the i-th oldest victim takes the i-th fill;
  the LRU clock advances once per call; inside a call recency follows
  ascending expert id; empty slots are oldest, in ascending slot order; slots
  hit in the call are never victims; rewritten ids are the slot (cache side)
  or -(1 + index in the host list); a rebuild leaves the cache cold.

Data structures are deliberately plain: a dict for residency, a list of slot
keys, an OrderedDict for recency and a sorted list of free slots.

Pins (tests/test_oracle_lru.py): brute-force LRU from the full history
(brute_lru.py), the textbook "C most recent distinct keys" property when every
miss is filled, Mattson inclusion across cache sizes, hand-worked q* tables and
hand-traced step fixtures under tests/golden/.
"""
from collections import OrderedDict

HIT, FILL, HOST = 0, 1, 2


def fill_count(m, bp, bh, K, n_avail):
    """q = min(m, floor(m*BP/BH), K, n_avail), integers; BH >= 1, BP >= 0."""
    if bh < 1 or bp < 0:
        raise ValueError("BH must be >= 1 and BP >= 0")
    return max(0, min(m, (m * bp) // bh, K, n_avail))


class LRUSim:
    def __init__(self, L, E, C, K, bp, bh):
        self.L, self.E, self.K = L, E, K
        self.bp, self.bh = bp, bh
        self.clock = 0
        self._reset(C)
        self.stats = [dict(hits=0, misses=0, fills=0, host=0, evictions=0) for _ in range(L)]

    def _reset(self, C):
        self.C = C
        self.resid = {}
        self.slot_key = [None] * C
        self.recency = OrderedDict()
        self.free = list(range(C))  # kept sorted

    def set_bandwidth(self, bp, bh):
        if bh < 1 or bp < 0:
            raise ValueError("BH must be >= 1 and BP >= 0")
        self.bp, self.bh = bp, bh

    def rebuild(self, C):
        """Cold cache of C slots; the clock continues."""
        self._reset(C)

    def step(self, layer, ids):
        """One expert_cache_step for `layer` with routed ids [T][k]; returns a dict."""
        l = layer
        flat = [int(e) for row in ids for e in row]
        U = sorted(set(flat))
        is_hit = [(l, u) in self.resid for u in U]
        M = [u for u, hit in zip(U, is_hit) if not hit]
        m = len(M)
        h = len(U) - m
        q = fill_count(m, self.bp, self.bh, self.K, self.C - h)
        F = M[:q]
        Hs = M[q:]
        hit_slots = set(self.resid[(l, u)] for u, hit in zip(U, is_hit) if hit)

        victims, evicted = [], []
        walk = iter(list(self.recency.keys()))  # LRU end first
        for _ in range(q):
            if self.free:
                v = self.free.pop(0)
            else:
                v = next(s for s in walk if s not in hit_slots and s not in victims)
            victims.append(v)
            evicted.append(self.slot_key[v])

        for v, f in zip(victims, F):
            old = self.slot_key[v]
            if old is not None:
                del self.resid[old]
            self.slot_key[v] = (l, f)
            self.resid[(l, f)] = v

        fills = set(F)
        cls, slot = [], []
        for u, hit in zip(U, is_hit):
            if hit or u in fills:
                s = self.resid[(l, u)]
                if s in self.recency:
                    self.recency.move_to_end(s)
                else:
                    self.recency[s] = None
                cls.append(HIT if hit else FILL)
                slot.append(s)
            else:
                cls.append(HOST)
                slot.append(-(1 + Hs.index(u)))

        rewritten = [[slot[U.index(int(e))] for e in row] for row in ids]
        pos = [[U.index(int(e)) for e in row] for row in ids]
        st = self.stats[l]
        st["hits"] += h
        st["misses"] += m
        st["fills"] += q
        st["host"] += m - q
        st["evictions"] += sum(1 for ev in evicted if ev is not None)
        self.clock += 1
        return dict(uniq=U, pos=pos, cls=cls, slot=slot, h=h, m=m, q=q, nhost=m - q, fills=F,
                    victims=victims, evicted=evicted, host_list=Hs, rewritten=rewritten)

    def resident_keys(self):
        return set(self.resid.keys())

    def state_arrays(self):
        """(resid [L*E] slot or -1, slot_key [C] l*E+e or -1) for comparison with device state."""
        resid = [-1] * (self.L * self.E)
        for (l, e), s in self.resid.items():
            resid[l * self.E + e] = s
        sk = [-1 if k is None else k[0] * self.E + k[1] for k in self.slot_key]
        return resid, sk
