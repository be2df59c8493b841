"""A decode step captured as one graph (all layers, fixed shapes, device-resident
counts; the host branch answers a mailbox the kernels write, so the graph holds
kernels only) replays bit-identically to the eager calls:
every replay's outputs and the final cache state (residency, slot keys, LRU keys,
clock) match an eager run on an identical context. Replays alternate with eager
work and synchronisations on the same process."""
import numpy as np
import pytest

import gen
from gen.configs import DSV4_DECODE, QWEN_DECODE
from tests.harness import make_ctx, make_pool

pytestmark = pytest.mark.gpu


def inputs(cfg, steps, L):
    import torch
    logits = torch.from_numpy(gen.decode_logits(cfg, steps=steps, L=L)).cuda()        # [S, L, 1, E]
    xs = np.stack([np.stack([gen.decode_x(cfg, s, l) for l in range(L)]) for s in range(steps)])
    x = torch.from_numpy(xs.view(np.int16)).cuda()                                    # [S, L, 1, H]
    return logits, x


def eager_run(cfg, pool, L, steps, logits, x, **kw):
    import torch
    import expert_cached_decode_amd as EC
    ctx = make_ctx(cfg, pool, L=L, **kw)
    outs = torch.empty((L, 1, cfg.H), dtype=torch.int16, device="cuda")
    res = []
    for s in range(steps):
        for l in range(L):
            EC.moe_decode_layer(ctx, l, x[s, l], logits[s, l], 1, outs[l])
        torch.cuda.synchronize()
        res.append(outs.clone())
    state = ctx.debug_state()
    ctx.close()
    return res, state


def graph_run(cfg, pool, L, steps, logits, x, **kw):
    import torch
    import expert_cached_decode_amd as EC
    ctx = make_ctx(cfg, pool, L=L, **kw)
    xs = torch.empty((L, 1, cfg.H), dtype=torch.int16, device="cuda")
    ls = torch.empty((L, 1, cfg.E), dtype=torch.float32, device="cuda")
    outs = torch.empty((L, 1, cfg.H), dtype=torch.int16, device="cuda")
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        for l in range(L):
            EC.moe_decode_layer(ctx, l, xs[l], ls[l], 1, outs[l], cap)
    torch.cuda.synchronize()
    res = []
    scratch = torch.zeros(1 << 20, device="cuda")
    for s in range(steps):
        xs.copy_(x[s]); ls.copy_(logits[s])
        g.replay()
        torch.cuda.synchronize()
        res.append(outs.clone())
        scratch.add_(1.0)  # unrelated eager work between replays
        torch.cuda.synchronize()
    state = ctx.debug_state()
    ctx.close()
    return res, state


@pytest.mark.parametrize("cfg,kw", [
    (QWEN_DECODE.with_(L=4, slots=48), dict(C=48)),
    (DSV4_DECODE.with_(L=2, slots=24, H=1024, I=512), dict(C=24, bp=300, bh=1000)),
], ids=["bf16-no-host-branch", "mxfp4-host-branch"])
def test_graph_replay_matches_eager(cfg, kw):
    L, steps = cfg.L, 12
    pool = make_pool(cfg)
    logits, x = inputs(cfg, steps, L)
    a, sa = eager_run(cfg, pool, L, steps, logits, x, **kw)
    b, sb = graph_run(cfg, pool, L, steps, logits, x, **kw)
    for s in range(steps):
        assert np.array_equal(a[s].cpu().numpy(), b[s].cpu().numpy()), s
    for u, v in zip(sa[:3], sb[:3]):
        assert np.array_equal(u, v)
    assert sa[3] == sb[3] == steps * L


def test_chained_block_graph_matches_eager():
    """moe_decode_block (router GEMV, decode layer, residual) chained over the layers of a token
    and captured as one graph: every replay equals the eager chain, with the host branch on."""
    import torch
    import expert_cached_decode_amd as EC
    cfg = QWEN_DECODE.with_(L=3, slots=20, bp=500, bh=1000)
    L, steps = cfg.L, 8
    pool = make_pool(cfg)
    W = [torch.from_numpy(gen.router_weights(cfg, l).view(np.int16)).cuda() for l in range(L)]
    x0 = torch.from_numpy(np.stack([gen.decode_x(cfg, s, 0) for s in range(steps)]).view(np.int16)).cuda()

    def chain(ctx, src, bufs, stream=None):
        cur = src
        for l in range(L):
            EC.moe_decode_block(ctx, l, cur, W[l], 1, bufs[l], stream)
            cur = bufs[l]

    ctx = make_ctx(cfg, pool)
    bufs = [torch.empty((1, cfg.H), dtype=torch.int16, device="cuda") for _ in range(L)]
    eager = []
    for s in range(steps):
        chain(ctx, x0[s], bufs)
        torch.cuda.synchronize()
        eager.append(bufs[-1].clone())
    st_e = ctx.debug_state()
    ctx.close()

    ctx = make_ctx(cfg, pool)
    src = torch.empty((1, cfg.H), dtype=torch.int16, device="cuda")
    bufs = [torch.empty((1, cfg.H), dtype=torch.int16, device="cuda") for _ in range(L)]
    g, cap = torch.cuda.CUDAGraph(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        chain(ctx, src, bufs, cap)
    torch.cuda.synchronize()
    for s in range(steps):
        src.copy_(x0[s])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs[-1], eager[s]), s
    st_g = ctx.debug_state()
    ctx.close()
    for u, v in zip(st_e[:3], st_g[:3]):
        assert np.array_equal(u, v)
    assert st_e[3] == st_g[3]


def test_stale_graph_after_epoch_change_is_flagged_not_addressed():
    """A graph captured while the host branch was compiled out (BP >= BH and the cache holds a whole
    step), replayed after ec_set_bandwidth switched the branch on: the control step now sends misses
    to the host, and the captured down GEMV, which has no host branch, must skip those pairs (never
    address a slot from a negative id) and raise the device error that names the epoch change."""
    import torch
    import expert_cached_decode_amd as EC
    cfg = QWEN_DECODE.with_(L=2, slots=48)
    L = cfg.L
    pool = make_pool(cfg)
    logits, x = inputs(cfg, 1, L)
    ctx = make_ctx(cfg, pool, C=48, bp=1000, bh=1000)
    assert ctx.stats()["host_branch"] == 0
    e0 = ctx.epoch()
    outs = torch.empty((L, 1, cfg.H), dtype=torch.int16, device="cuda")
    g, cap = torch.cuda.CUDAGraph(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        for l in range(L):
            EC.moe_decode_layer(ctx, l, x[0, l], logits[0, l], 1, outs[l], cap)
    torch.cuda.synchronize()
    ctx.set_bandwidth(0, 1000)  # no fills: every miss of the cold cache is a host-side pair
    assert ctx.epoch() != e0 and ctx.stats()["host_branch"] == 1
    g.replay()
    torch.cuda.synchronize()
    with pytest.raises(EC.ECError, match="epoch"):
        ctx.stats()
    s = EC.binding.ec_stats()
    assert EC.lib().ec_get_stats(ctx.handle, EC.binding.ctypes.byref(s), 0) == -7
    assert s.device_error & 4
    ctx.close()
