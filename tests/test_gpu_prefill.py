"""moe_prefill_layer on the GPU vs the fp64 oracle on sampled rows, plus the
double-buffer invariants: overlap on and off give bit-identical outputs, and
repeated chunks (wrap-around prefetch) reproduce the same outputs."""
import numpy as np
import pytest

import gen
from gen.configs import DSV4_DECODE, QWEN_PREFILL
from tests.harness import make_ctx, make_pool, oracle_layer, row_rel_err

pytestmark = pytest.mark.gpu


def run_prefill(cfg, ctx, layers, T, overlap=True):
    import torch
    import expert_cached_decode_amd as EC
    ctx.set_prefill_overlap(overlap)
    outs = []
    compute = torch.cuda.current_stream()
    for l in layers:
        x = gen.prefill_x(cfg, l % cfg.L, T)
        lg = gen.prefill_logits(cfg, l % cfg.L, T)
        xd = torch.from_numpy(x.view(np.int16)).cuda()
        ld = torch.from_numpy(lg).cuda()
        out = torch.empty((T, cfg.H), dtype=torch.int16, device="cuda")
        EC.moe_prefill_layer(ctx, l % cfg.L, xd, ld, T, out, compute, ctx.copy_stream)
        outs.append((out, x, lg))
    torch.cuda.synchronize()
    return [(o.cpu().numpy().view(np.uint16), x, lg) for o, x, lg in outs]


def check_rows(cfg, layer, got_bits, x, lg, rows):
    ref, _, _ = oracle_layer(cfg, layer, x, lg, tokens=rows)
    got = gen.bf16_to_f32(got_bits[rows]).astype(np.float64)
    e = row_rel_err(got, ref)
    assert e <= 1e-2, (layer, e)
    return e


@pytest.mark.parametrize("T", [512, 333, 1])
def test_prefill_bf16_parity(T):
    cfg = QWEN_PREFILL.with_(L=2)
    pool = make_pool(cfg)
    ctx = make_ctx(cfg, pool, C=0, T=1, prefill=T)
    res = run_prefill(cfg, ctx, [0, 1], T)
    rng = np.random.default_rng(T)
    for l, (o, x, lg) in enumerate(res):
        rows = sorted(set([0, T - 1] + list(rng.choice(T, min(T, 10), replace=False))))
        check_rows(cfg, l, o, x, lg, rows)
    ctx.close()


def test_prefill_overlap_on_off_identical_and_repeatable():
    cfg = QWEN_PREFILL.with_(L=3)
    pool = make_pool(cfg)
    ctx = make_ctx(cfg, pool, C=0, T=1, prefill=256)
    a = run_prefill(cfg, ctx, [0, 1, 2, 0, 1, 2], 256, overlap=True)
    b = run_prefill(cfg, ctx, [0, 1, 2], 256, overlap=False)
    for i in range(3):
        assert np.array_equal(a[i][0], b[i][0])
        assert np.array_equal(a[i][0], a[i + 3][0])
    ctx.close()


def test_prefill_full_chunk_two_layers():
    cfg = QWEN_PREFILL.with_(L=2)
    pool = make_pool(cfg)
    ctx = make_ctx(cfg, pool, C=0, T=1, prefill=8192)
    res = run_prefill(cfg, ctx, [0, 1], 8192)
    rng = np.random.default_rng(7)
    for l, (o, x, lg) in enumerate(res):
        ids = np.argsort(-lg, axis=1)[:, :8]
        assert len(np.unique(ids)) == cfg.E  # the routing union covers every expert
        check_rows(cfg, l, o, x, lg, sorted(rng.choice(8192, 16, replace=False)))
    ctx.close()


def test_prefill_mxfp4_one_layer():
    cfg = DSV4_DECODE.with_(L=1, slots=0, T=512)
    pool = make_pool(cfg)
    ctx = make_ctx(cfg, pool, C=0, T=1, prefill=512)
    res = run_prefill(cfg, ctx, [0], 512)
    o, x, lg = res[0]
    check_rows(cfg, 0, o, x, lg, [0, 5, 100, 511])
    ctx.close()


@pytest.mark.parametrize("E,k,T,H", [(300, 5, 777, 256), (37, 3, 171, 320), (1024, 8, 64, 256)])
def test_prefill_grouping_odd_shapes(E, k, T, H):
    """Expert counts that are not powers of two (the placement ranks lanes by one ballot per bit of
    the expert id) and pair counts T k that are not multiples of the 512-pair segments or of a
    wavefront: every checked row must still meet the oracle, which it cannot if a pair is placed
    under the wrong expert or twice. H = 320 takes the down GEMM's 64-wide N tiles (H is not a
    multiple of 128)."""
    cfg = QWEN_PREFILL.with_(L=1, E=E, k=k, K=k, H=H, I=128)
    pool = make_pool(cfg)
    ctx = make_ctx(cfg, pool, C=0, T=1, prefill=T)
    (o, x, lg), = run_prefill(cfg, ctx, [0], T)
    rng = np.random.default_rng(E + T)
    check_rows(cfg, 0, o, x, lg, sorted(set([0, T - 1] + list(rng.choice(T, min(T, 24), replace=False)))))
    ctx.close()


def test_prefill_mxfp4_odd_shapes():
    """MXFP4 weights (decoded to bf16 in the tile loads) through the same grouping and GEMMs at odd
    shapes: 40 experts, top-3, 300 tokens, H = 320 (the down GEMM's 64-wide tiles), I = 256."""
    cfg = DSV4_DECODE.with_(L=1, E=40, k=3, K=3, H=320, I=256, slots=0, T=300)
    pool = make_pool(cfg)
    ctx = make_ctx(cfg, pool, C=0, T=1, prefill=300)
    (o, x, lg), = run_prefill(cfg, ctx, [0], 300)
    check_rows(cfg, 0, o, x, lg, [0, 1, 77, 150, 298, 299])
    ctx.close()


def random_prefill_shapes(n=8, seed=20261203):
    """Seeded draws over prefill shapes: bf16 or MXFP4 weights; 2..600 experts; top-1..12; 1..2500
    tokens; H a multiple of 64 up to 2048 (64- and 128-wide down tiles both occur) and I a multiple
    of 64 up to 1024. Pools above 384 MB are redrawn."""
    from gen.configs import BF16, MXFP4
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        wd = int(rng.choice([BF16, MXFP4]))
        H = 64 * int(rng.integers(1, 33))
        I = 64 * int(rng.integers(1, 17))
        E = int(rng.integers(2, 601))
        k = int(rng.integers(1, min(12, E) + 1))
        T = int(rng.integers(1, 2501))
        es = 6 * H * I if wd == BF16 else 3 * H * I // 2 + 3 * H * I // 32
        if E * es > (384 << 20):
            continue
        out.append((wd, H, I, E, k, T))
    return out


@pytest.mark.parametrize("i,shape", list(enumerate(random_prefill_shapes())))
def test_prefill_random_shapes(i, shape):
    """Prefill at seeded random shapes: the first and last rows and 14 sampled ones against the
    oracle."""
    wd, H, I, E, k, T = shape
    print("shape", i, dict(wd=wd, H=H, I=I, E=E, k=k, T=T), flush=True)
    base = QWEN_PREFILL if wd == QWEN_PREFILL.wdtype else DSV4_DECODE
    cfg = base.with_(L=1, E=E, k=k, K=k, H=H, I=I, slots=0, T=T, seed=base.seed + 2000 + i)
    pool = make_pool(cfg)
    ctx = make_ctx(cfg, pool, C=0, T=1, prefill=T)
    (o, x, lg), = run_prefill(cfg, ctx, [0], T)
    rng = np.random.default_rng(1000 + i)
    check_rows(cfg, 0, o, x, lg, sorted(set([0, T - 1] + list(rng.choice(T, min(T, 14), replace=False)))))
    ctx.close()
