"""Helpers of the full-size parity tests (test_gpu_parity_full_*.py): decode runs through the C ABI
with decision totals against the literal LRU simulator, and oracle checks grouped by layer."""
import numpy as np

import gen
from gen.configs import budget_slots
from tests.harness import oracle_layer, out_to_host, prefetch_experts, route_ids, row_rel_err, x_to_device

TOL = 1e-2


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
