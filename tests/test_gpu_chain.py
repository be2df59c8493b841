"""Router GEMV and chained decode blocks on the GPU against the oracle (oracle/chain.py).

The chains run free on both sides: each layer's output is the next layer's input,
and routing comes from the data. Where the oracle's top-k set is within a small
margin of a tie, the two chains may legitimately route differently from then on;
the comparison of that token stream stops there (the margin is reported)."""
import numpy as np
import pytest

import gen
from gen.configs import BF16, F32, QWEN_DECODE, TINY
from oracle import chain
from tests.harness import make_ctx, make_pool, row_rel_err

pytestmark = pytest.mark.gpu


def _dev(a):
    import torch
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def _host(t, f32):
    a = t.cpu().numpy()
    return a.astype(np.float32) if f32 else a.view(np.uint16)


@pytest.mark.parametrize("shape", [(QWEN_DECODE, 4), (TINY, 3), (QWEN_DECODE.with_(E=37, H=192), 2),
                                   (QWEN_DECODE.with_(H=4096), 1)],
                         ids=["qwen-bf16", "tiny-f32", "ragged-bf16", "wide-bf16"])
def test_gate_logits_parity(shape):
    import torch
    import expert_cached_decode_amd as EC
    cfg, T = shape
    f32 = cfg.wdtype == F32
    W = gen.router_weights(cfg, 3)
    x = gen.decode_x(cfg, 5, 3, T)
    lg = torch.empty((T, cfg.E), dtype=torch.float32, device="cuda")
    EC.moe_gate_logits(_dev(W), _dev(x), F32 if f32 else BF16, T, cfg.E, cfg.H, lg)
    torch.cuda.synchronize()
    got = lg.cpu().numpy().astype(np.float64)
    wv = W.astype(np.float64) if f32 else chain.widen_bf16(W)
    xv = x.astype(np.float64) if f32 else chain.widen_bf16(x)
    ref = chain.gate_logits(wv, xv)
    scale = np.abs(xv) @ np.abs(wv).T  # sum of |terms|: the fp32 accumulation error scales with it
    assert np.all(np.abs(got - ref) <= 1e-5 * scale + 1e-30)


def _run_chain(cfg, L, T, steps, margin_min, tol, margin_first=1e-4):
    import torch
    import expert_cached_decode_amd as EC
    f32 = cfg.wdtype == F32
    pool = make_pool(cfg, L=L)
    ctx = make_ctx(cfg.with_(L=L), pool, T=T)
    Ws = [gen.router_weights(cfg, l) for l in range(L)]
    Wd = [_dev(w) for w in Ws]
    a = torch.empty((T, cfg.H), dtype=torch.float32 if f32 else torch.int16, device="cuda")
    b = torch.empty_like(a)
    compared, stopped, worst = 0, 0, 0.0
    for s in range(steps):
        x_ref = gen.decode_x(cfg, s, 0, T)
        a.copy_(_dev(x_ref))
        cur, nxt = a, b
        live = True
        for l in range(L):
            EC.moe_decode_block(ctx, l, cur, Wd[l], T, nxt)
            x_ref, ids, ws, margin = chain.block(cfg.wdtype, x_ref, Ws[l], cfg.k,
                                                 lambda e, l=l: gen.expert_logical(cfg, l, e))
            if live:
                # layer 0 sees identical inputs on both sides; later layers inputs that differ by rounding
                if float(np.min(margin)) < (margin_first if l == 0 else margin_min):
                    live, stopped = False, stopped + 1
                else:
                    torch.cuda.synchronize()
                    got = _host(nxt, f32)
                    gv = got.astype(np.float64) if f32 else chain.widen_bf16(got)
                    rv = x_ref.astype(np.float64) if f32 else chain.widen_bf16(x_ref)
                    e = row_rel_err(gv, rv)
                    worst = max(worst, e)
                    assert e <= tol, (s, l, e)
                    compared += 1
            cur, nxt = nxt, cur
    st = ctx.stats()
    ctx.close()
    return compared, stopped, worst, st


def test_chained_blocks_f32_with_host_split():
    cfg = TINY.with_(L=6, E=64, k=4, H=512, I=256, slots=40, K=4, bp=700, bh=1000)
    compared, stopped, worst, st = _run_chain(cfg, 6, 2, 5, 1e-4, 1e-4)
    print("f32 chain: %d layer outputs compared, %d streams stopped at near-ties, worst %.2e" % (compared, stopped, worst))
    assert compared >= 24 and st["host"] > 0 and st["fills"] > 0


def test_chained_blocks_bf16_qwen_shapes():
    cfg = QWEN_DECODE.with_(slots=48)
    compared, stopped, worst, st = _run_chain(cfg, 3, 1, 4, 0.02, 1e-2)
    print("bf16 chain: %d layer outputs compared, %d streams stopped at near-ties, worst %.2e" % (compared, stopped, worst))
    assert compared >= 4


def test_decode_block_rejects_aliasing():
    import torch
    import expert_cached_decode_amd as EC
    cfg = TINY
    pool = make_pool(cfg)
    ctx = make_ctx(cfg, pool)
    x = torch.zeros((1, cfg.H), dtype=torch.float32, device="cuda")
    W = _dev(gen.router_weights(cfg, 0))
    with pytest.raises(EC.ECError):
        EC.moe_decode_block(ctx, 0, x, W, 1, x)
    ctx.close()
