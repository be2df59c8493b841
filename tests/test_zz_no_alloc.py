"""moe_decode_layer_static (the variant for callers that cannot allocate: its step buffers live in the
library's static device scratch) against moe_decode_layer, through the C ABI.

Two contexts with the same configuration and bank take the same calls: one through each entry
point. Calls come in pairs, the second with fewer tokens than the first. Outputs must be
bit-identical (the kernels are the same), and so must every decision read with ec_last_step,
the counters and the final cache state; the outputs also match the fp64 oracle to the 1e-2 bar.
"""
import numpy as np
import pytest

import gen
from gen.configs import DSV4_DECODE, QWEN_DECODE
from tests.harness import make_ctx, make_pool, oracle_layer, row_rel_err, x_to_device

pytestmark = pytest.mark.gpu


def _run(cfg, pool, plan, static):
    import torch
    import expert_cached_decode_amd as EC
    from expert_cached_decode_amd.binding import memcpy_async
    ctx = make_ctx(cfg, pool)
    fn = EC.moe_decode_layer_static if static else EC.moe_decode_layer
    n = cfg.T * cfg.k
    outs, decisions = [], []
    for s, l, T in plan:
        logits = torch.from_numpy(gen.decode_logits(cfg, steps=s + 1, T=T, L=cfg.L)[s, l]).cuda()
        x = x_to_device(cfg, gen.decode_x(cfg, s, l, T))
        out = torch.empty((T, cfg.H), dtype=torch.int16, device="cuda")
        fn(ctx, l, x, logits, T, out)
        v = EC.last_step(ctx)
        rec = torch.empty(8 + 3 * n, dtype=torch.int32, device="cuda")
        memcpy_async(rec.data_ptr(), v.counts, 4 * 8)
        memcpy_async(rec.data_ptr() + 4 * 8, v.rewritten, 4 * T * cfg.k)
        memcpy_async(rec.data_ptr() + 4 * (8 + n), v.victims, 4 * cfg.K)
        memcpy_async(rec.data_ptr() + 4 * (8 + 2 * n), v.host_list, 4 * min(n, cfg.E))
        torch.cuda.synchronize()
        r = rec.cpu().numpy()
        q, nhost = int(r[3]), int(r[4])
        decisions.append((r[:6].tolist(), r[8:8 + T * cfg.k].tolist(), r[8 + n:8 + n + q].tolist(),
                          r[8 + 2 * n:8 + 2 * n + nhost].tolist()))
        outs.append(out.cpu().numpy().copy())
    st = ctx.stats()
    state = ctx.debug_state()
    ctx.close()
    return outs, decisions, st, state


@pytest.mark.parametrize("name,cfg", [
    ("bf16_host_branch", QWEN_DECODE.with_(L=2, slots=40, bp=500, bh=1000, T=4, K=8)),
    ("mxfp4_no_host_branch", DSV4_DECODE.with_(L=2, H=2048, I=1024, slots=48, bp=1000, bh=1000, T=4, K=24)),
])
def test_static_scratch_matches_workspace_entry_point(name, cfg):
    pool = make_pool(cfg)
    # calls in pairs, the second with fewer tokens; both layers; the cache fills and evicts
    plan = [(s, l, T) for s in range(6) for l in range(cfg.L) for T in (4, 2)]
    a = _run(cfg, pool, plan, static=False)
    b = _run(cfg, pool, plan, static=True)
    for i, (oa, ob) in enumerate(zip(a[0], b[0])):
        assert np.array_equal(oa, ob), (name, i, plan[i])
    assert a[1] == b[1], name
    for k in ("hits", "misses", "fills", "host", "evictions", "steps", "clock"):
        assert a[2][k] == b[2][k], (name, k)
    for x, y in zip(a[3][:3], b[3][:3]):
        assert np.array_equal(x, y), name
    assert a[2]["fills"] > 0 and (a[2]["host"] > 0) == (cfg.bp < cfg.bh)
    # and against the oracle, on every call of the first two steps
    import torch  # noqa: F401
    worst = 0.0
    for i, (s, l, T) in enumerate(plan[:4 * cfg.L]):
        lg = gen.decode_logits(cfg, steps=s + 1, T=T, L=cfg.L)[s, l]
        x = gen.decode_x(cfg, s, l, T)
        ref, _, _ = oracle_layer(cfg, l, x, lg)
        got = gen.bf16_to_f32(b[0][i].view(np.uint16)).astype(np.float64)
        worst = max(worst, row_rel_err(got, ref))
    assert worst <= 1e-2, (name, worst)
    print("%s: %d calls bit-identical to moe_decode_layer; worst row error against the oracle %.3g"
          % (name, len(plan), worst))
