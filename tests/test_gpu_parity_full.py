"""Layer outputs against the fp64 oracle at the workloads' full sizes, through the C ABI.

- Qwen3.6-35B-A3B-shaped decode (40 layers, 64.4 GB pinned bank, 3072 slots, batch 1): every
  layer of every step of a multi-step run.
- Prefill on those shapes: one full 40-layer chunk of 8192 tokens, 256 seeded rows per layer
  (rows are independent, so a row sample checks the chunk at full fidelity).
- DeepSeek-V4-Flash-shaped MXFP4 decode (43 layers, 2752 slots) at BP:BH 300, 1000 and
  2000 : 1000. The outputs do not depend on the split, so each layer step is checked once,
  at one of the three ratios. At 1000 and 2000 the steps run without the host branch.
- The stress shapes: batch 1 across cache_rebuild 40% -> 15% -> 40% (without the host
  branch), and batch 16 with K = 64 (misses beyond K go to the host branch); every 16th
  layer step.

Outputs pass at per-row relative error <= 1e-2 (max |g - o| / max |o| over the row), and every
cache decision total equals the literal LRU simulator's. The MXFP4 workloads hold 16 distinct
pool layers drawn as layer 0 (layer l reads pool layer l mod 16); the oracle is told the same.
"""
import numpy as np
import pytest

import gen
from gen.configs import DSV4_DECODE, QWEN_DECODE, QWEN_PREFILL, STRESS, budget_slots
from oracle.lru_sim import LRUSim
from tests.harness import (make_ctx, make_pool, oracle_layer, out_to_host, prefetch_experts, route_ids,
                           row_rel_err, x_to_device)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

TOL = 1e-2


@pytest.fixture(scope="module")
def qwen_pool():
    pool = make_pool(QWEN_DECODE)
    yield pool
    pool.close()


@pytest.fixture(scope="module")
def dsv4_pool():
    pool = make_pool(DSV4_DECODE, L=16, layer_period=1)
    yield pool
    pool.close()


def decode_run(cfg, ctx, steps, T=1, rebuild=None, sim=None):
    """All layers of `steps` decode steps through moe_decode_layer (eager); returns the outputs
    [steps, L, T, H] (host, widened), the inputs and the logits. With `sim`, the simulator takes
    the same steps (and rebuilds) and the decision totals are compared."""
    import torch
    import expert_cached_decode_amd as EC
    L = cfg.L
    logits = gen.decode_logits(cfg, steps=steps, T=T)
    lg_dev = torch.from_numpy(logits).cuda()
    xs = np.stack([np.stack([gen.decode_x(cfg, s, l, T) for l in range(L)]) for s in range(steps)])
    xs_dev = x_to_device(cfg, xs.reshape(steps * L * T, cfg.H)).reshape(steps, L, T, cfg.H)
    outs = torch.empty_like(xs_dev)
    tot = dict(hits=0, misses=0, fills=0, host=0)
    for s in range(steps):
        if rebuild and s in rebuild:
            torch.cuda.synchronize()
            C = ctx.rebuild(rebuild[s])
            assert C == budget_slots(L, cfg.E, rebuild[s])
            if sim is not None:
                sim.rebuild(C)
        for l in range(L):
            EC.moe_decode_layer(ctx, l, xs_dev[s, l], lg_dev[s, l], T, outs[s, l])
            if sim is not None:
                r = sim.step(l, route_ids(logits[s, l], cfg.k).tolist())
                tot["hits"] += r["h"]; tot["misses"] += r["m"]; tot["fills"] += r["q"]; tot["host"] += r["nhost"]
    torch.cuda.synchronize()
    st = ctx.stats()
    assert st["device_error"] == 0
    if sim is not None:
        assert {k: st[k] for k in tot} == tot
    got = out_to_host(cfg, outs.reshape(steps * L * T, cfg.H)).reshape(steps, L, T, cfg.H)
    return got, xs, logits, st


def check_layer_steps(cfg, keys, got, xs, logits, layer_period=0, tokens=None):
    """Oracle rows for each (step, layer) in keys, grouped by layer so each layer's experts are
    drawn once; returns the worst row error."""
    worst = 0.0
    for l in sorted({l for _, l in keys}):
        src = l % layer_period if layer_period else l
        sl = [s for s, l2 in keys if l2 == l]
        need = set()
        for s in sl:
            rows = range(logits.shape[2]) if tokens is None else tokens
            need.update(route_ids(logits[s, l][list(rows)], cfg.k).ravel().tolist())
        prefetch_experts(cfg, src, sorted(need))
        for s in sl:
            ref, _, _ = oracle_layer(cfg, l, xs[s, l], logits[s, l], layer_period=layer_period, tokens=tokens)
            g = got[s, l] if tokens is None else got[s, l][tokens]
            e = row_rel_err(g, ref)
            assert e <= TOL, ((s, l), e)
            worst = max(worst, e)
    return worst


def test_qwen_decode_every_layer_of_every_step(qwen_pool):
    cfg = QWEN_DECODE
    steps = 12
    ctx = make_ctx(cfg, qwen_pool)
    sim = LRUSim(cfg.L, cfg.E, cfg.slots, cfg.K, cfg.bp, cfg.bh)
    got, xs, logits, st = decode_run(cfg, ctx, steps, sim=sim)
    ctx.close()
    assert st["host_branch"] == 0 and st["fills"] > 0 and st["hits"] > 0
    keys = [(s, l) for s in range(steps) for l in range(cfg.L)]
    worst = check_layer_steps(cfg, keys, got, xs, logits)
    print("qwen decode: %d layer steps, worst row error %.3g" % (len(keys), worst))


def test_prefill_full_chunk_256_rows_every_layer(qwen_pool):
    """One 8192-token chunk through all 40 layers (full-layer double buffering on), 256 seeded rows
    of every layer against the oracle; the expert weights are the decode bank's."""
    import torch
    import expert_cached_decode_amd as EC
    cfg, pcfg = QWEN_DECODE, QWEN_PREFILL
    T = pcfg.T
    ctx = make_ctx(cfg, qwen_pool, C=0, T=1, prefill=T)
    rng = np.random.default_rng(pcfg.seed)
    compute = torch.cuda.current_stream()
    out = torch.empty((T, cfg.H), dtype=torch.int16, device="cuda")
    worst = 0.0
    for l in range(cfg.L):
        x = gen.prefill_x(pcfg, l)
        lg = gen.prefill_logits(pcfg, l)
        EC.moe_prefill_layer(ctx, l, torch.from_numpy(x.view(np.int16)).cuda(), torch.from_numpy(lg).cuda(), T,
                             out, compute, ctx.copy_stream)
        rows = sorted(set([0, T - 1]) | set(rng.choice(np.arange(1, T - 1), 254, replace=False).tolist()))
        got = gen.bf16_to_f32(out[torch.tensor(rows, device="cuda")].cpu().numpy().view(np.uint16))
        prefetch_experts(cfg, l, route_ids(lg[rows], cfg.k).ravel())
        ref, _, _ = oracle_layer(cfg, l, x, lg, tokens=rows)
        e = row_rel_err(got.astype(np.float64), ref)
        assert e <= TOL, (l, e)
        worst = max(worst, e)
    ctx.close()
    print("prefill: 40 layers x 256 rows, worst row error %.3g" % worst)


def test_dsv4_full_size_each_layer_step_once(dsv4_pool):
    cfg = DSV4_DECODE
    steps = 6
    got_all, keys_all = {}, {}
    for idx, bp in enumerate((300, 1000, 2000)):
        c = cfg.with_(bp=bp, bh=1000)
        ctx = make_ctx(c, dsv4_pool, pool_layers=16)
        sim = LRUSim(c.L, c.E, c.slots, c.K, bp, 1000)
        got, xs, logits, st = decode_run(c, ctx, steps, sim=sim)
        ctx.close()
        # BP >= BH with K and C >= U_max: every miss is filled and the steps run without the
        # host branch (the down GEMV form with the host-side merge compiled out)
        assert st["host_branch"] == (1 if bp < 1000 else 0), (bp, st)
        assert (st["host"] > 0) == (bp < 1000)
        got_all[bp] = got
        keys_all[bp] = [(s, l) for s in range(steps) for l in range(c.L) if (s * c.L + l) % 3 == idx]
    for bp in (300, 1000, 2000):
        worst = check_layer_steps(cfg, keys_all[bp], got_all[bp], xs, logits, layer_period=1)
        print("dsv4 BP:BH %d:1000: %d layer steps, worst row error %.3g" % (bp, len(keys_all[bp]), worst))


def test_stress_batch1_rebuild_40_15_40(dsv4_pool):
    """Batch 1 on the stress shapes (4096-slot class cache, K = 64, BP = BH) across safe-point
    rebuilds 40% -> 15% -> 40%: decisions against the simulator rebuilt at the same steps, every
    16th layer step against the oracle; the steps run without the host branch."""
    c = STRESS.with_(T=1, seed=DSV4_DECODE.seed, slots=budget_slots(43, 256, 4000), bp=1000, bh=1000)
    steps = 48
    ctx = make_ctx(c, dsv4_pool, pool_layers=16)
    sim = LRUSim(c.L, c.E, c.slots, c.K, c.bp, c.bh)
    got, xs, logits, st = decode_run(c, ctx, steps, rebuild={16: 1500, 32: 4000}, sim=sim)
    ctx.close()
    assert st["host_branch"] == 0
    keys = [(s, l) for s in range(steps) for l in range(c.L) if (s * c.L + l) % 16 == 0]
    worst = check_layer_steps(c, keys, got, xs, logits, layer_period=1)
    print("stress batch 1 across rebuilds: %d layer steps, worst row error %.3g" % (len(keys), worst))


def test_stress_batch16_every_16th_layer_step(dsv4_pool):
    """Batch 16, K = 64, 4096 slots: up to 96 unique experts per layer step, so misses beyond K
    are computed by the host branch; all 16 token rows of every 16th layer step."""
    c = STRESS.with_(seed=DSV4_DECODE.seed)
    steps = 4
    ctx = make_ctx(c, dsv4_pool, pool_layers=16)
    sim = LRUSim(c.L, c.E, c.slots, c.K, c.bp, c.bh)
    got, xs, logits, st = decode_run(c, ctx, steps, T=c.T, sim=sim)
    ctx.close()
    assert st["host_branch"] == 1 and st["host"] > 0
    keys = [(s, l) for s in range(steps) for l in range(c.L) if (s * c.L + l) % 16 == 0]
    worst = check_layer_steps(c, keys, got, xs, logits, layer_period=1)
    print("stress batch 16: %d layer steps x 16 tokens, worst row error %.3g" % (len(keys), worst))
