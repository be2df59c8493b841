"""Test-side plumbing: build contexts over seeded expert banks, run the HIP path,
run the oracle on the same inputs, compare. Inputs come from gen/ only."""
from collections import OrderedDict
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import gen
from gen.configs import F32


def row_rel_err(got, ref):
    """max over rows t of max_h |g - o| / max_h |o| (rows of all zeros compare absolutely)."""
    got = np.asarray(got, np.float64).reshape(ref.shape)
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1), num)))


def widen_x(cfg, x):
    return (x.astype(np.float64) if cfg.wdtype == F32 else gen.bf16_to_f32(x).astype(np.float64))


def x_to_device(cfg, x):
    import torch
    if cfg.wdtype == F32:
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()


def out_to_host(cfg, t):
    a = t.cpu().numpy()
    if cfg.wdtype == F32:
        return a.astype(np.float64)
    return gen.bf16_to_f32(a.view(np.uint16)).astype(np.float64)


def empty_out(cfg, T):
    import torch
    return torch.empty((T, cfg.H), dtype=torch.float32 if cfg.wdtype == F32 else torch.int16, device="cuda")


def make_pool(cfg, L=None, layer_period=0):
    import expert_cached_decode_amd as EC
    L = cfg.L if L is None else L
    pb = EC.PinnedBuffer(L * cfg.E * cfg.expert_bytes)
    gen.fill_pool_ptr(cfg, pb.ptr, 0, L, layer_period)
    return pb


def make_ctx(cfg, pool, L=None, C=None, K=None, bp=None, bh=None, T=None, prefill=0, threads=8, pool_layers=0):
    import expert_cached_decode_amd as EC
    L = cfg.L if L is None else L
    return EC.Context(L, cfg.E, cfg.k, cfg.H, cfg.I, cfg.wdtype, max_tokens=cfg.T if T is None else T,
                      cache_slots=cfg.slots if C is None else C, victim_k=cfg.K if K is None else K,
                      bp=cfg.bp if bp is None else bp, bh=cfg.bh if bh is None else bh, host_pool=pool,
                      host_threads=threads, prefill_max_tokens=prefill, pool_layers=pool_layers)


_EXPERTS = OrderedDict()  # (seed, dtype, H, I, sigma, layer, expert) -> logical matrices, LRU
_EXPERT_CACHE_BYTES = 8 << 30


def _nbytes(m):
    return sum(sum(a.nbytes for a in v) if isinstance(v, tuple) else v.nbytes for v in m.values())


def expert_mats(cfg, layer, e):
    """Logical matrices of one expert from gen/, cached (the draws are pure functions of the key)."""
    key = (cfg.seed, cfg.wdtype, cfg.H, cfg.I, cfg.sigma, layer, e)
    m = _EXPERTS.get(key)
    if m is None:
        m = gen.expert_logical(cfg, layer, e)
        _EXPERTS[key] = m
        total = sum(_nbytes(v) for v in _EXPERTS.values())
        while total > _EXPERT_CACHE_BYTES and len(_EXPERTS) > 1:
            total -= _nbytes(_EXPERTS.popitem(last=False)[1])
    else:
        _EXPERTS.move_to_end(key)
    return m


def prefetch_experts(cfg, layer, experts, threads=8):
    """Draw the given experts of a layer on host threads (gen's C calls release the GIL)."""
    todo = [e for e in dict.fromkeys(int(e) for e in experts)
            if (cfg.seed, cfg.wdtype, cfg.H, cfg.I, cfg.sigma, layer, e) not in _EXPERTS]
    with ThreadPoolExecutor(threads) as ex:
        mats = list(ex.map(lambda e: gen.expert_logical(cfg, layer, e), todo))
    for e, m in zip(todo, mats):
        _EXPERTS[(cfg.seed, cfg.wdtype, cfg.H, cfg.I, cfg.sigma, layer, e)] = m
    total = sum(_nbytes(v) for v in _EXPERTS.values())
    while total > _EXPERT_CACHE_BYTES and len(_EXPERTS) > 1:
        total -= _nbytes(_EXPERTS.popitem(last=False)[1])


def oracle_layer(cfg, layer, x, logits, layer_period=0, tokens=None):
    """fp64 oracle output rows for one layer: x [T,H] (bf16 bits or f32), logits [T,E]."""
    from oracle import moe
    src_layer = layer % layer_period if layer_period else layer
    get = lambda e: expert_mats(cfg, src_layer, e)
    out, ids, w = moe.moe_tokens(cfg.wdtype, widen_x(cfg, x), logits, cfg.k, get, tokens=tokens)
    return out, ids, w


def route_ids(logits, k):
    """Routed ids by (logit desc, id asc) via numpy lexsort (input preparation)."""
    T, E = logits.shape
    out = np.empty((T, k), np.int32)
    for t in range(T):
        out[t] = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))[:k]
    return out
