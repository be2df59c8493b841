"""CPU oracle for the MoE layer step with a GPU expert cache.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import, call, link or execute anything in this package.
The product path (expert_cached_decode_amd) never does, and shares no code with
it: the two take the same seeded inputs from gen/ and nothing else.

Parts (FreeToken edge-MoE write-up, "Design: three mechanisms" and
"Implementation notes"):
  route.py      routing: top-k by logit, softmax over the selected k
  lru_sim.py    literal shared-LRU cache simulator with the q* miss split
  brute_lru.py  brute-force LRU from the full access history (tiny inputs)
  moe_ref.c     plain-loop fp64 MoE layer (the definition, no cache at all)
  moe.py        ctypes wrapper around moe_ref.c plus per-token drivers

Every function here is pinned by tests that do not re-type its formula
(brute force, closed forms, library special cases, invariants); see each
module's header for its pins.
"""
