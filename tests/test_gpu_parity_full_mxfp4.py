"""Layer outputs against the fp64 oracle at the MXFP4 workloads' full sizes, through the C ABI.

- DeepSeek-V4-Flash-shaped MXFP4 decode (43 layers, 2752 slots) at BP:BH 300, 1000 and
  2000 : 1000. The outputs do not depend on the split, so each layer step is checked once,
  at one of the three ratios. At 1000 and 2000 the steps run without the host branch.
- The stress shapes: batch 1 across cache_rebuild 40% -> 15% -> 40% (without the host
  branch), and batch 16 with K = 64 (misses beyond K go to the host branch); every 16th
  layer step.

Outputs pass at per-row relative error <= 1e-2, and every cache decision total equals the literal
LRU simulator's. The workloads hold 16 distinct pool layers drawn as layer 0 (layer l reads pool
layer l mod 16; the oracle is told the same), pinned once for the module.
"""
import pytest

from gen.configs import DSV4_DECODE, STRESS, budget_slots
from oracle.lru_sim import LRUSim
from tests.harness import make_ctx, make_pool
from tests.parity_full import check_layer_steps, decode_run

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def dsv4_pool():
    pool = make_pool(DSV4_DECODE, L=16, layer_period=1)
    yield pool
    pool.close()


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
