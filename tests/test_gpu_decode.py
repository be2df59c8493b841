"""moe_decode_layer on the GPU vs the fp64 oracle MoE layer.

Outputs must be within 1e-2 per-row relative error of the oracle (bf16 and
MXFP4 weights, fp32 accumulation, bf16 output); fp32 workloads are checked
to 1e-5. Cache counters must equal the literal LRU simulator's. The layer
output must not depend on the cache size or on the BP:BH split.
"""
import numpy as np
import pytest

import gen
from gen.configs import BF16, DSV4_DECODE, F32, MXFP4, QWEN_DECODE, STRESS, TINY
from oracle.lru_sim import LRUSim
from tests.harness import (empty_out, make_ctx, make_pool, oracle_layer, out_to_host, route_ids, row_rel_err,
                           x_to_device)

pytestmark = pytest.mark.gpu


def run_decode(cfg, ctx, steps, L, T, keep):
    """Run steps x layers through moe_decode_layer; return {(s, l): out} for keep(s, l)."""
    import torch
    import expert_cached_decode_amd as EC
    logits = gen.decode_logits(cfg, steps=steps, T=T, L=L)
    lg_dev = torch.from_numpy(logits).cuda()
    outs = {}
    out = empty_out(cfg, T)
    for s in range(steps):
        for l in range(L):
            x = gen.decode_x(cfg, s, l, T)
            xd = x_to_device(cfg, x)
            EC.moe_decode_layer(ctx, l, xd, lg_dev[s, l], T, out)
            if keep(s, l):
                torch.cuda.synchronize()
                outs[(s, l)] = (out_to_host(cfg, out), x, logits[s, l])
    torch.cuda.synchronize()
    return outs, logits


def check_against_oracle(cfg, outs, tol, layer_period=0, max_checks=None):
    worst = 0.0
    items = sorted(outs.items())
    if max_checks:
        items = items[:max_checks]
    for (s, l), (got, x, lg) in items:
        ref, _, _ = oracle_layer(cfg, l, x, lg, layer_period=layer_period)
        e = row_rel_err(got, ref)
        worst = max(worst, e)
        assert e <= tol, ((s, l), e)
    return worst


def sim_counts(cfg, logits, L, T, C, K, bp, bh):
    sim = LRUSim(L, cfg.E, C, K, bp, bh)
    tot = dict(hits=0, misses=0, fills=0, host=0)
    for s in range(logits.shape[0]):
        for l in range(L):
            r = sim.step(l, route_ids(logits[s, l], cfg.k).tolist())
            tot["hits"] += r["h"]; tot["misses"] += r["m"]; tot["fills"] += r["q"]; tot["host"] += r["nhost"]
    return tot


def test_tiny_all_steps():
    pool = make_pool(TINY)
    ctx = make_ctx(TINY, pool)
    outs, logits = run_decode(TINY, ctx, TINY.steps, TINY.L, 1, lambda s, l: True)
    worst = check_against_oracle(TINY, outs, 1e-5)
    st = ctx.stats()
    ref = sim_counts(TINY, logits, TINY.L, 1, TINY.slots, TINY.K, TINY.bp, TINY.bh)
    assert {k: st[k] for k in ref} == ref
    assert ref["host"] > 0 and ref["fills"] > 0  # both sides of the split were exercised
    print("tiny worst row error", worst)
    ctx.close()


def test_qwen_shapes_two_layers():
    cfg = QWEN_DECODE.with_(L=2, slots=64)
    pool = make_pool(cfg)
    ctx = make_ctx(cfg, pool)
    outs, logits = run_decode(cfg, ctx, 24, 2, 1, lambda s, l: s % 3 == 0)
    check_against_oracle(cfg, outs, 1e-2)
    st = ctx.stats()
    ref = sim_counts(cfg, logits, 2, 1, 64, cfg.K, cfg.bp, cfg.bh)
    assert {k: st[k] for k in ref} == ref
    ctx.close()


@pytest.mark.parametrize("wd,k,T,H,I", [
    (BF16, 1, 1, 512, 256), (BF16, 3, 1, 512, 256), (BF16, 5, 2, 512, 256), (BF16, 6, 1, 512, 256),
    (BF16, 7, 3, 512, 256), (MXFP4, 3, 1, 512, 256), (MXFP4, 6, 4, 512, 256), (MXFP4, 7, 2, 512, 256),
    (MXFP4, 5, 2, 1024, 2048), (F32, 6, 2, 256, 128)])
def test_down_group_sizes(wd, k, T, H, I):
    """The down GEMV's pair groups (2, 4, 6, 8) with full and partial last groups, one and several
    tokens, guarded and full MXFP4 rows, with a host split: outputs against the oracle."""
    cfg = TINY.with_(L=2, E=32, k=k, H=H, I=I, wdtype=wd, slots=24, K=4, T=T, bp=500, bh=1000, p=0.5)
    pool = make_pool(cfg)
    ctx = make_ctx(cfg, pool)
    outs, logits = run_decode(cfg, ctx, 10, 2, T, lambda s, l: s % 3 == 1)
    check_against_oracle(cfg, outs, 1e-5 if wd == F32 else 1e-2)
    st = ctx.stats()
    ref = sim_counts(cfg, logits, 2, T, 24, 4, 500, 1000)
    assert {k_: st[k_] for k_ in ref} == ref
    assert st["host"] > 0 and (st["fills"] > 0 or k * T < 2)  # one pair per step: floor(m / 2) = 0
    ctx.close()


@pytest.mark.parametrize("wd,H,I,T", [(BF16, 1024, 256, 1), (BF16, 2048, 128, 1), (BF16, 4096, 256, 1),
                                       (MXFP4, 2048, 256, 1), (MXFP4, 4096, 128, 1), (MXFP4, 8192, 256, 1),
                                       (BF16, 2048, 128, 3), (BF16, 4096, 256, 2), (MXFP4, 2048, 256, 2),
                                       (MXFP4, 4096, 128, 3)])
def test_gate_up_forms(wd, H, I, T):
    """The gate/up GEMV's forms: x staged in LDS (bf16 rows of 4 and 8 chunks per lane, MXFP4 rows
    of 1, 2 and 4; with several tokens, each pair's token in turn behind a block barrier), MXFP4 block
    scales as byte loads (1 chunk) or as words handed out by ds_bpermute (2 and 4 chunks: one and two
    words per lane), and the register form (bf16, 2 chunks); with a host split. Outputs against the
    oracle, counters against the LRU simulator."""
    cfg = TINY.with_(L=2, E=32, k=4, H=H, I=I, wdtype=wd, slots=24, K=4, T=T, bp=500, bh=1000, p=0.5)
    pool = make_pool(cfg)
    ctx = make_ctx(cfg, pool)
    outs, logits = run_decode(cfg, ctx, 10, 2, T, lambda s, l: s % 3 == 1)
    check_against_oracle(cfg, outs, 1e-2)
    st = ctx.stats()
    ref = sim_counts(cfg, logits, 2, T, 24, 4, 500, 1000)
    assert {k_: st[k_] for k_ in ref} == ref
    assert st["host"] > 0 and st["fills"] > 0
    ctx.close()


def random_shapes(n=12, seed=20261202):
    """Seeded draws over the shapes the library accepts: any dtype; H and I multiples of 64 (up to
    512 for f32, 1024 for bf16, 2048 for MXFP4, so that whole and guarded rows of every width
    occur); 2..320 experts; top-k up to 32 (a quarter of the draws) or 8; 1..8 tokens; cache slots
    0..2E over two layers; K 0..64 (0: the library's default, min(64, U_max)); BP:BH on both sides
    of 1. Pools above 384 MB are redrawn."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        wd = int(rng.choice([F32, BF16, MXFP4, BF16, MXFP4]))
        maxd = {F32: 512, BF16: 1024, MXFP4: 2048}[wd]
        H = 64 * int(rng.integers(1, maxd // 64 + 1))
        I = 64 * int(rng.integers(1, maxd // 64 + 1))
        E = int(rng.integers(2, 321))
        k = int(rng.integers(1, min(32, E) + 1)) if rng.random() < 0.25 else int(rng.integers(1, min(8, E) + 1))
        T = int(rng.integers(1, 9))
        if T * k > 1024:
            continue
        es = {F32: 12 * H * I, BF16: 6 * H * I, MXFP4: 3 * H * I // 2 + 3 * H * I // 32}[wd]
        if 2 * E * es > (384 << 20):
            continue
        C = int(rng.integers(0, 2 * E + 1))
        K = int(rng.integers(0, 65))
        bp, bh = [(300, 1000), (1000, 1000), (2000, 1000), (500, 1000), (700, 300)][int(rng.integers(0, 5))]
        out.append((wd, H, I, E, k, T, C, K, bp, bh))
    return out


@pytest.mark.parametrize("i,shape", list(enumerate(random_shapes())))
def test_random_shapes(i, shape):
    """Decode at seeded random shapes within the accepted ranges: outputs of every second step of both
    layers against the oracle, cache counters of all steps against the literal LRU simulator."""
    wd, H, I, E, k, T, C, K, bp, bh = shape
    print("shape", i, dict(wd=wd, H=H, I=I, E=E, k=k, T=T, C=C, K=K, bp=bp, bh=bh), flush=True)
    cfg = TINY.with_(L=2, E=E, k=k, H=H, I=I, wdtype=wd, slots=C, K=K, T=T, bp=bp, bh=bh, p=0.5,
                     seed=TINY.seed + 1000 + i)
    pool = make_pool(cfg)
    ctx = make_ctx(cfg, pool)
    outs, logits = run_decode(cfg, ctx, 6, 2, T, lambda s, l: s % 2 == 1)
    check_against_oracle(cfg, outs, 1e-5 if wd == F32 else 1e-2)
    st = ctx.stats()
    K_eff = K if K else min(64, min(E, T * k))  # victim_k 0 selects min(64, U_max)
    ref = sim_counts(cfg, logits, 2, T, C, K_eff, bp, bh)
    assert {k_: st[k_] for k_ in ref} == ref
    ctx.close()


@pytest.mark.parametrize("wd,split", [(BF16, (300, 1000, 40)), (BF16, (1000, 1000, 40)), (BF16, (2000, 1000, 40)),
                                      (BF16, (300, 1000, 0)), (BF16, (1000, 1000, 1024)),
                                      (MXFP4, (1000, 1000, 24)), (MXFP4, (2000, 1000, 64)),
                                      (MXFP4, (300, 1000, 24))])
def test_output_independent_of_split_and_capacity(wd, split):
    """Same inputs, different BP:BH and cache sizes: outputs agree with the oracle (and so with each
    other). MXFP4 at BP >= BH runs without the host branch (its down GEMV form merges no host terms)."""
    bp, bh, C = split
    base = QWEN_DECODE if wd == BF16 else DSV4_DECODE.with_(H=1024, I=1024)
    cfg = base.with_(L=4, slots=C, bp=bp, bh=bh, K=base.k)
    pool = make_pool(cfg)
    ctx = make_ctx(cfg, pool)
    outs, logits = run_decode(cfg, ctx, 12, 4, 1, lambda s, l: s in (0, 5, 11) and l in (0, 3))
    check_against_oracle(cfg, outs, 1e-2)
    st = ctx.stats()
    assert st["host_branch"] == (0 if (bp >= bh and C >= cfg.k) else 1)
    ref = sim_counts(cfg, logits, 4, 1, C, cfg.K, bp, bh)
    assert {k: st[k] for k in ref} == ref
    ctx.close()


def test_mxfp4_host_split_ratios():
    """Full DeepSeek-V4-Flash expert shapes (H 4096, I 2048, MXFP4) on three layers at BP:BH 300, 1000
    and 2000 : 1000; the last two run without the host branch. Every kept output against the oracle."""
    cfg = DSV4_DECODE.with_(L=3, slots=192)
    pool = make_pool(cfg)
    for bp in (300, 1000, 2000):
        ctx = make_ctx(cfg, pool, bp=bp, bh=1000)
        outs, logits = run_decode(cfg, ctx, 6, 3, 1, lambda s, l: s in (1, 5))
        st = ctx.stats()
        assert st["host_branch"] == (1 if bp < 1000 else 0)
        ref = sim_counts(cfg, logits, 3, 1, 192, cfg.K, bp, 1000)
        assert {k: st[k] for k in ref} == ref
        if bp == 300:
            assert ref["host"] > 0
        ctx.close()
        check_against_oracle(cfg, outs, 1e-2)


def test_batch16_mxfp4():
    cfg = STRESS.with_(L=2, slots=256, K=64, T=16)
    pool = make_pool(cfg)
    ctx = make_ctx(cfg, pool, bp=500, bh=1000)
    outs, logits = run_decode(cfg, ctx, 3, 2, 16, lambda s, l: s == 2)
    for (s, l), (got, x, lg) in outs.items():
        toks = [0, 7, 15]
        ref, _, _ = oracle_layer(cfg, l, x, lg, tokens=toks)
        assert row_rel_err(got[toks], ref) <= 1e-2
    ctx.close()


def test_host_pool_layer_aliasing():
    """pool_layers = 2 for 4 layers: layer l reads pool layer l % 2 (fills and host branch)."""
    cfg = QWEN_DECODE.with_(L=4, slots=24, bp=500, bh=1000)
    pool = make_pool(cfg, L=2)
    ctx = make_ctx(cfg, pool, pool_layers=2)
    outs, logits = run_decode(cfg, ctx, 6, 4, 1, lambda s, l: s in (2, 5))
    for (s, l), (got, x, lg) in sorted(outs.items()):
        ref, _, _ = oracle_layer(cfg, l % 2, x, lg)
        assert row_rel_err(got, ref) <= 1e-2, (s, l)
    assert ctx.stats()["host"] > 0
    ctx.close()


def test_budget_zero_runs_every_expert_on_the_host():
    """C = 0: q = 0 at every step, every routed expert is computed by the host branch."""
    cfg = QWEN_DECODE.with_(L=3, slots=0, bp=1000, bh=1000)
    pool = make_pool(cfg)
    ctx = make_ctx(cfg, pool)
    outs, logits = run_decode(cfg, ctx, 5, 3, 1, lambda s, l: True)
    check_against_oracle(cfg, outs, 1e-2)
    st = ctx.stats()
    ref = sim_counts(cfg, logits, 3, 1, 0, cfg.K, 1000, 1000)
    assert {k: st[k] for k in ref} == ref
    assert st["fills"] == 0 and st["hits"] == 0 and st["host"] == st["misses"] == 5 * 3 * cfg.k
    assert st["host_only"] == 0
    ctx.close()


def test_pageable_pool_selects_host_only_mode():
    """A host pool in ordinary pageable memory (pinning failed): BP is 0 on the device,
    nothing is filled, every expert runs on the host, outputs still match the oracle."""
    import expert_cached_decode_amd as EC
    cfg = QWEN_DECODE.with_(L=2, slots=32, bp=2000, bh=1000)
    pinned = make_pool(cfg)
    pageable = np.array(pinned.numpy(), copy=True)  # same bytes, ordinary memory
    pinned.close()
    ctx = EC.Context(cfg.L, cfg.E, cfg.k, cfg.H, cfg.I, cfg.wdtype, max_tokens=1, cache_slots=cfg.slots,
                     victim_k=cfg.K, bp=cfg.bp, bh=cfg.bh, host_pool=pageable.ctypes.data,
                     host_pool_bytes=pageable.nbytes, host_threads=8)
    outs, logits = run_decode(cfg, ctx, 4, 2, 1, lambda s, l: True)
    check_against_oracle(cfg, outs, 1e-2)
    st = ctx.stats()
    assert st["host_only"] == 1
    assert st["fills"] == 0 and st["hits"] == 0 and st["host"] == st["misses"] == 4 * 2 * cfg.k
    ctx.set_bandwidth(5000, 1000)  # still no fills: the device keeps BP = 0
    run_decode(cfg, ctx, 2, 2, 1, lambda s, l: False)
    assert ctx.stats()["fills"] == 0
    ctx.close()
    del pageable


def test_bandwidth_calibration_drives_the_split():
    """Measured BP and BH (MB/s) are applied on the device; the step decisions then follow
    the oracle simulator run with the same integers."""
    cfg = QWEN_DECODE.with_(L=2, slots=24)
    pool = make_pool(cfg)
    ctx = make_ctx(cfg, pool, bp=1000, bh=1000)
    bp, bh = ctx.calibrate_bandwidth(probe_experts=4, apply=True)
    print("calibrated BP %d MB/s, BH %d MB/s" % (bp, bh))
    assert bp > 1000 and bh >= 1
    outs, logits = run_decode(cfg, ctx, 4, 2, 1, lambda s, l: s == 3)
    check_against_oracle(cfg, outs, 1e-2)
    st = ctx.stats()
    ref = sim_counts(cfg, logits, 2, 1, cfg.slots, cfg.K, bp, bh)
    assert {k: st[k] for k in ref} == ref
    bp2, bh2 = ctx.calibrate_bandwidth(probe_experts=2, apply=False)  # a later safe point
    assert bp2 > 0 and bh2 >= 1
    ctx.close()


def test_calibration_in_host_only_mode_reports_no_link():
    import expert_cached_decode_amd as EC
    cfg = TINY.with_(L=1)
    pinned = make_pool(cfg)
    pageable = np.array(pinned.numpy(), copy=True)
    pinned.close()
    ctx = EC.Context(cfg.L, cfg.E, cfg.k, cfg.H, cfg.I, cfg.wdtype, max_tokens=1, cache_slots=cfg.slots,
                     victim_k=cfg.K, bp=cfg.bp, bh=cfg.bh, host_pool=pageable.ctypes.data,
                     host_pool_bytes=pageable.nbytes)
    bp, bh = ctx.calibrate_bandwidth(probe_experts=2, apply=True)
    assert bp == 0 and bh >= 1
    ctx.close()
    del pageable


def test_decode_outputs_across_rebuilds():
    """cache_rebuild at safe points (40% -> 15% -> 40% of the experts, cold each time, clock going
    on): outputs keep matching the oracle and decisions the simulator rebuilt at the same steps."""
    import torch
    import expert_cached_decode_amd as EC
    from gen.configs import budget_slots
    cfg = QWEN_DECODE.with_(L=3, slots=budget_slots(3, 256, 4000), bp=700, bh=1000)
    pool = make_pool(cfg)
    ctx = make_ctx(cfg, pool)
    steps, L = 12, 3
    logits = gen.decode_logits(cfg, steps=steps, T=1, L=L)
    lg_dev = torch.from_numpy(logits).cuda()
    out = empty_out(cfg, 1)
    sim = LRUSim(L, cfg.E, cfg.slots, cfg.K, cfg.bp, cfg.bh)
    plan = {4: 1500, 8: 4000}
    for s in range(steps):
        if s in plan:
            C = ctx.rebuild(plan[s])
            assert C == budget_slots(L, cfg.E, plan[s])
            sim.rebuild(C)
        for l in range(L):
            x = gen.decode_x(cfg, s, l, 1)
            EC.moe_decode_layer(ctx, l, x_to_device(cfg, x), lg_dev[s, l], 1, out)
            r = sim.step(l, route_ids(logits[s, l], cfg.k).tolist())
            if (s + l) % 3 == 0:
                torch.cuda.synchronize()
                ref, _, _ = oracle_layer(cfg, l, x, logits[s, l])
                assert row_rel_err(out_to_host(cfg, out), ref) <= 1e-2, (s, l)
    resid, sk, lru, clk = ctx.debug_state()
    assert clk == steps * L
    occ = sorted((int(k) for k in sk if k >= 0))
    assert occ == sorted(l * cfg.E + e for (l, e) in sim.resid.keys())
    ctx.close()


def test_decode_from_a_bank_file(tmp_path):
    """Fast start ("Elastic edge resource management", "Implementation notes"): the expert bank is
    written as a bank file in its final layout, read back with parallel direct I/O into pinned
    memory, and that memory serves as the host pool of a decode with fills and the host branch.
    Outputs against the oracle (whose weights come from gen/, not from the file)."""
    import expert_cached_decode_amd as EC
    cfg = QWEN_DECODE.with_(L=3, E=64, slots=40, bp=500, bh=1000)
    src = gen.pool_array(cfg)
    shape = EC.make_shape(cfg.L, cfg.E, cfg.k, cfg.H, cfg.I, cfg.wdtype)
    path = str(tmp_path / "bank.ecb")
    EC.bank_write(path, shape, cfg.L, src.ctypes.data, src.nbytes)
    pinned = EC.PinnedBuffer(src.nbytes)
    sec, mode = EC.bank_read(path, shape, cfg.L, pinned.ptr, pinned.nbytes, threads=8)
    print("bank file of %.2f GB read in %.3f s (mode %d)" % (src.nbytes / 1e9, sec, mode))
    del src
    ctx = make_ctx(cfg, pinned)
    outs, logits = run_decode(cfg, ctx, 8, cfg.L, 1, lambda s, l: True)
    check_against_oracle(cfg, outs, 1e-2)
    st = ctx.stats()
    ref = sim_counts(cfg, logits, cfg.L, 1, cfg.slots, cfg.K, cfg.bp, cfg.bh)
    assert {k: st[k] for k in ref} == ref
    assert st["fills"] > 0 and st["host"] > 0
    ctx.close()
    pinned.close()


def test_host_wait_bound_flags_missing_partials():
    """The host branch's failure path, forced from the host: with the host paused and the down
    GEMV's wait for the host's partial sums bounded to 64 polls, a step with a host-side expert
    ends without them, every workgroup finishes, and ec_get_stats reports device error bit 2."""
    import torch
    import expert_cached_decode_amd as EC
    cfg = TINY  # BP:BH 500:1000: a cold step's two misses are one fill and one host-side expert
    pool = make_pool(cfg)
    ctx = make_ctx(cfg, pool)
    assert ctx.stats()["host_branch"] == 1
    logits = torch.from_numpy(gen.decode_logits(cfg, steps=2)).cuda()
    out = empty_out(cfg, 1)
    ctx.host_branch_test_hooks(True, 64)
    EC.moe_decode_layer(ctx, 0, x_to_device(cfg, gen.decode_x(cfg, 0, 0)), logits[0, 0], 1, out)
    torch.cuda.synchronize()
    with pytest.raises(EC.ECError, match="did not deliver"):
        ctx.stats()
    s = EC.binding.ec_stats()
    assert EC.lib().ec_get_stats(ctx.handle, EC.binding.ctypes.byref(s), 1) == -7
    assert s.device_error & 2 and s.host == 1
    ctx.host_branch_test_hooks(False, 0)
    ctx.close()
