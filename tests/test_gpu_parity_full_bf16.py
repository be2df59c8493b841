"""Layer outputs against the fp64 oracle at the bf16 workload's full size, through the C ABI.

- Qwen3.6-35B-A3B-shaped decode (40 layers, 64.4 GB pinned bank, 3072 slots, batch 1): every
  layer of every step of a multi-step run.
- Prefill on those shapes: one full 40-layer chunk of 8192 tokens, 256 seeded rows per layer
  (rows are independent, so a row sample checks the chunk at full fidelity).

Outputs pass at per-row relative error <= 1e-2 (max |g - o| / max |o| over the row), and every
cache decision total equals the literal LRU simulator's. The 64.4 GB bank is pinned once for the
module (the host can pin one full-size bank at a time).
"""
import numpy as np
import pytest

import gen
from gen.configs import QWEN_DECODE, QWEN_PREFILL
from oracle.lru_sim import LRUSim
from tests.harness import make_ctx, make_pool, oracle_layer, prefetch_experts, route_ids, row_rel_err
from tests.parity_full import TOL, check_layer_steps, decode_run

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def qwen_pool():
    pool = make_pool(QWEN_DECODE)
    yield pool
    pool.close()


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
