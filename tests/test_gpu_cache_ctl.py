"""expert_cache_step on the GPU vs the literal LRU simulator (oracle/lru_sim.py),
and the same decisions taken inside moe_decode_layer with fused routing (read
back through ec_last_step).

Every step of every trace is compared bit-exactly: unique experts, counts
(h, m, q, host), classes, slots, fills, victims, evicted keys, host list and
rewritten ids; the residency table and slot keys are compared at the end, and
the device LRU keys must order the occupied slots exactly as the simulator's
recency list. Cache control reads no expert bytes, so these traces use the
workloads' L, E, k, C, K, T and BP:BH with small H = I = 64 experts (the
decisions do not depend on H, I or the weight dtype).
"""
import numpy as np
import pytest

import gen
from gen.configs import BF16, DSV4_DECODE, QWEN_DECODE, STRESS, TINY, budget_slots
from oracle.lru_sim import LRUSim
from tests.harness import make_ctx, make_pool, route_ids

pytestmark = pytest.mark.gpu


def _small(cfg):
    return cfg.with_(H=64, I=64, wdtype=BF16)


def run_trace(cfg, steps, p=None, T=None, C=None, K=None, bp=None, bh=None, rebuild=None, ids_override=None,
              check_every=1, fused=False):
    """fused: each step is moe_decode_layer on the step's logits (routing inside the control
    kernel, then fill and GEMVs on zero inputs) and its decisions are read with ec_last_step;
    otherwise expert_cache_step on the oracle-routed ids."""
    import torch
    import expert_cached_decode_amd as EC
    from expert_cached_decode_amd.binding import memcpy_async
    T = cfg.T if T is None else T
    C = cfg.slots if C is None else C
    K = cfg.K if K is None else K
    bp = cfg.bp if bp is None else bp
    bh = cfg.bh if bh is None else bh
    rebuild = rebuild or {}
    sc = _small(cfg)
    pool = make_pool(sc, layer_period=1)
    ctx = make_ctx(sc, pool, C=C, K=K, bp=bp, bh=bh, T=T)
    sim = LRUSim(cfg.L, cfg.E, C, ctx.cfg.victim_k or min(64, min(cfg.E, T * cfg.k)), bp, bh)
    Kc = ctx.cfg.victim_k or min(64, min(cfg.E, T * cfg.k))
    if ids_override is None:
        logits = gen.decode_logits(cfg, steps=steps, p=cfg.p if p is None else p, T=T)
    n = T * cfg.k
    Umax = min(cfg.E, n)
    rec = 8 + 5 * Umax + 3 * Kc + n  # ints logged per step
    log = torch.empty((steps * cfg.L, rec), dtype=torch.int32, device="cuda")
    ids_dev = torch.empty((steps * cfg.L, T, cfg.k), dtype=torch.int32, device="cuda")
    all_ids = []
    for s in range(steps):
        for l in range(cfg.L):
            ids = ids_override(s, l) if ids_override else route_ids(logits[s, l], cfg.k)
            all_ids.append(ids)
    ids_dev.copy_(torch.from_numpy(np.stack(all_ids)))
    if fused:
        assert ids_override is None
        lg_dev = torch.from_numpy(np.ascontiguousarray(logits.reshape(steps * cfg.L, T, cfg.E), np.float32)).cuda()
        xz = torch.zeros((T, sc.H), dtype=torch.int16, device="cuda")
        yo = torch.empty((T, sc.H), dtype=torch.int16, device="cuda")
        views = EC.last_step(ctx)
    results = []
    i = 0
    for s in range(steps):
        if s in rebuild:
            torch.cuda.synchronize()
            newC = ctx.rebuild(rebuild[s])
            assert newC == budget_slots(cfg.L, cfg.E, rebuild[s])  # the library's C, the reading's formula
            sim.rebuild(newC)
        for l in range(cfg.L):
            if fused:
                EC.moe_decode_layer(ctx, l, xz, lg_dev[i], T, yo)
                v = views
            else:
                v = EC.expert_cache_step(ctx, l, ids_dev[i], T)
            row = log[i]
            o = 0
            for ptr, cnt in ((v.counts, 8), (v.uniq, Umax), (v.cls, Umax), (v.slot, Umax), (v.fills, Kc),
                             (v.victims, Kc), (v.evicted, Kc), (v.host_list, Umax), (v.rewritten, n)):
                memcpy_async(row.data_ptr() + 4 * o, ptr, 4 * cnt)
                o += cnt
            results.append(sim.step(l, all_ids[i].tolist()))
            i += 1
    torch.cuda.synchronize()
    got = log.cpu().numpy()
    for i, r in enumerate(results):
        g = got[i]
        U = len(r["uniq"])
        o = 8
        cnt = list(g[:6])
        assert cnt == [U, r["h"], r["m"], r["q"], r["nhost"], r["h"] + r["q"]], (i, cnt, r)
        uniq = list(g[o:o + U]); o += Umax
        cls = list(g[o:o + U]); o += Umax
        slot = list(g[o:o + U]); o += Umax
        fills = list(g[o:o + r["q"]]); o += Kc
        victims = list(g[o:o + r["q"]]); o += Kc
        evicted = list(g[o:o + r["q"]]); o += Kc
        host = list(g[o:o + r["nhost"]]); o += Umax
        rew = list(g[o:o + n])
        assert uniq == r["uniq"], i
        assert cls == r["cls"], i
        assert slot == r["slot"], i
        assert fills == r["fills"], i
        assert victims == r["victims"], (i, victims, r["victims"])
        assert evicted == [-1 if e is None else e[0] * cfg.E + e[1] for e in r["evicted"]], i
        assert host == r["host_list"], i
        assert rew == [x for row in r["rewritten"] for x in row], i
    resid, sk, lru, clk = ctx.debug_state()
    sresid, ssk = sim.state_arrays()
    assert list(resid) == sresid and list(sk) == ssk
    assert clk == steps * cfg.L
    occupied = [s for s in range(len(sk)) if sk[s] >= 0]
    assert [s for s in sorted(occupied, key=lambda s: int(lru[s]))] == list(sim.recency.keys())
    assert all(int(lru[s]) == s for s in range(len(sk)) if sk[s] < 0)
    st = ctx.stats()
    assert st["device_error"] == 0
    assert st["hits"] == sum(r["h"] for r in results) and st["fills"] == sum(r["q"] for r in results)
    ctx.close()
    return results


def test_tiny_trace():
    res = run_trace(TINY, TINY.steps)
    assert sum(r["nhost"] for r in res) > 0 and sum(r["q"] for r in res) > 0


def test_qwen_decode_full_trace():
    res = run_trace(QWEN_DECODE, QWEN_DECODE.steps)
    assert all(r["nhost"] == 0 for r in res)  # BP = BH: every miss is filled


@pytest.mark.parametrize("bp,steps", [(300, 1024), (1000, 256), (2000, 256)])
def test_dsv4_decode_ratios(bp, steps):
    res = run_trace(DSV4_DECODE, steps, bp=bp, bh=1000)
    if bp >= 1000:
        assert all(r["q"] == r["m"] for r in res)


@pytest.mark.parametrize("p", [0.0, 0.9])
def test_stress_batch16_k64(p):
    run_trace(STRESS, 48, p=p, T=16)


def test_stress_rebuild_40_15_40():
    c5 = STRESS.with_(T=1, slots=budget_slots(43, 256, 4000))
    run_trace(c5, 96, T=1, rebuild={32: 1500, 64: 4000})


def test_budget_zero_and_tiny_caches():
    run_trace(TINY.with_(L=2), 40, C=0)
    run_trace(TINY.with_(L=2), 40, C=1, K=2, bp=1000, bh=1000)
    run_trace(TINY.with_(L=3, k=4), 40, T=3, C=5, K=64, bp=700, bh=1000)


def test_slot_table_beyond_registers():
    """C > 5120: the control kernel holds 5120 slot entries in registers and reads the rest of the
    table from memory in the victim scan (also after a rebuild that grows the cache past it)."""
    c = STRESS.with_(T=1, slots=6000)
    run_trace(c, 40, T=1, K=64, bp=700, bh=1000)
    run_trace(c, 40, T=1, K=64, bp=1000, bh=1000, fused=True, rebuild={8: 10000})
    run_trace(STRESS, 8, T=16, C=8000, p=0.3)


def test_max_pairs_and_wide_expert_table():
    cfg = TINY.with_(L=2, E=4096, k=16, slots=300, K=64, T=64, p=0.3)
    run_trace(cfg, 6)


def test_duplicate_ids_in_a_step():
    cfg = TINY.with_(L=2, E=16, k=3, slots=4, K=3, T=4)
    rng = np.random.default_rng(9)
    run_trace(cfg, 30, ids_override=lambda s, l: rng.integers(0, 5, size=(4, 3)).astype(np.int32))


def test_fused_routing_one_token_traces():
    # batch-1 steps with routing fused into the control kernel: every decision bit-exact
    res = run_trace(TINY, TINY.steps, fused=True)  # BP:BH 500:1000: host list in use
    assert sum(r["nhost"] for r in res) > 0 and sum(r["q"] for r in res) > 0
    run_trace(QWEN_DECODE, 64, fused=True)
    res = run_trace(DSV4_DECODE, 128, bp=300, bh=1000, fused=True)
    assert sum(r["nhost"] for r in res) > 0
    run_trace(TINY.with_(L=2), 40, C=0, fused=True)
    run_trace(TINY.with_(L=2), 40, C=1, K=2, bp=1000, bh=1000, fused=True)
    c5 = STRESS.with_(T=1, slots=budget_slots(43, 256, 4000))
    run_trace(c5, 48, T=1, rebuild={16: 1500, 32: 4000}, fused=True)
    # the form's limits: k = 16 (64 candidates in the second routing stage), k = 1 with a ragged
    # E = 200 (the last wavefront holds 8 logits), C just above one register row per thread
    run_trace(TINY.with_(L=3, E=256, k=16, slots=300, K=16, p=0.4), 24, fused=True)
    run_trace(TINY.with_(L=3, E=200, k=1, slots=257, K=1, p=0.3), 40, fused=True)


def test_fused_routing_general_forms():
    # fused routing outside the one-token form: E > 256, k > 16, T > 1
    run_trace(TINY.with_(L=2, E=512, k=4, slots=64, K=4), 20, fused=True)
    run_trace(TINY.with_(L=2, E=64, k=20, slots=64, K=20), 20, fused=True)
    run_trace(STRESS, 12, T=16, p=0.5, fused=True)
    # several tokens per wavefront (four per pass, one per DPP row): ragged T over three passes,
    # k = 16 with E not a multiple of 16, and 1024 threads with T > 32 (no token masks)
    run_trace(TINY.with_(L=2, E=256, k=4, slots=64, K=8, p=0.4), 12, T=37, fused=True)
    run_trace(TINY.with_(L=2, E=200, k=16, slots=64, K=16, p=0.4), 12, T=5, fused=True)
    run_trace(TINY.with_(L=2, E=256, k=8, slots=128, K=32, p=0.4), 8, T=40, fused=True)


def test_invalid_id_sets_device_error():
    import torch
    import expert_cached_decode_amd as EC
    sc = _small(TINY)
    pool = make_pool(sc)
    ctx = make_ctx(sc, pool)
    bad = torch.tensor([[3, 99]], dtype=torch.int32, device="cuda")
    EC.expert_cache_step(ctx, 0, bad, 1)
    with pytest.raises(EC.ECError):
        ctx.stats()
    st = ctx.stats(allow_bad_ids=True)
    assert st["device_error"] == 1 and st["steps"] == 0
    with pytest.raises(EC.ECError):
        EC.binding.check(EC.lib().ec_get_stats(ctx.handle, EC.binding.ctypes.byref(EC.binding.ec_stats()), 0),
                         ctx.handle)
    ctx.close()


def random_traces(n=10, seed=20261204):
    """Seeded draws over the control step's accepted ranges: 1..6 layers, 2..4096 experts (log-
    uniform), top-1..32, 1..64 tokens with T k <= 1024, 0..min(L E, 12000) slots (past the 5120 held
    in registers sometimes), K 0..64, BP:BH on both sides of 1, routing overlap 0..0.9, routing
    separate or fused into the control kernel, and a rebuild at step 12 in a third of the traces."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        L = int(rng.integers(1, 7))
        E = int(round(2 ** rng.uniform(1, 12)))
        k = int(rng.integers(1, min(32, E) + 1))
        T = int(rng.integers(1, 65))
        if T * k > 1024:
            continue
        C = int(rng.integers(0, min(L * E, 12000) + 1))
        K = int(rng.integers(0, 65))
        bp, bh = [(300, 1000), (1000, 1000), (2000, 1000), (700, 300)][int(rng.integers(0, 4))]
        p = float(rng.choice([0.0, 0.3, 0.6, 0.9]))
        fused = bool(rng.integers(0, 2))
        rebuild = {12: int(rng.integers(0, 10001))} if rng.random() < 1 / 3 else None
        out.append((L, E, k, T, C, K, bp, bh, p, fused, rebuild))
    return out


@pytest.mark.parametrize("i,trace", list(enumerate(random_traces())))
def test_random_traces(i, trace):
    """24-step traces at seeded random shapes: every decision of every step bit-exact against the
    simulator, and the final residency, slot keys and LRU order."""
    L, E, k, T, C, K, bp, bh, p, fused, rebuild = trace
    print("trace", i, dict(L=L, E=E, k=k, T=T, C=C, K=K, bp=bp, bh=bh, p=p, fused=fused, rebuild=rebuild),
          flush=True)
    cfg = TINY.with_(L=L, E=E, k=k, T=T, slots=C, K=K, bp=bp, bh=bh, p=p, seed=TINY.seed + 3000 + i)
    run_trace(cfg, 24, T=T, rebuild=rebuild, fused=fused)
