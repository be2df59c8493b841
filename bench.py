"""Benchmark: one MoE layer step with a GPU expert cache on one MI355X.

Default (the headline): a step is one batch-1 decode token through all 40 MoE
layers of the Qwen3.6-35B-A3B-shaped workload (E = 256, top-8, H = 2048,
I = 512, bf16 experts, 64.4 GB pinned expert bank, 3072-slot shared LRU cache,
routing with 60% step-to-step overlap, BP:BH = 1000:1000): route -> cache
control -> fill -> gate/up GEMV -> down GEMV + exact merge, per layer, captured
in one hipGraph per token. Inputs (router logits and layer inputs of every
step) are resident in HBM before the timed region. `value` is tok/s of steady
decode: the --steps timed steps follow the generation's first 64 tokens (the
cache's fill transient from empty, timed on its own as `cache_fill_transient`)
and then --warmup steps; `steady_state` times further steps after them.

Also measured in the same run:
- `roofline`: D9 expert streaming (gate/up + down GEMV per layer step) on the
  all-hit leg (a warm cache, no fills in the timed steps); the same figure on
  the workload's own steps is `roofline_workload`. Kernel durations come from
  HIP event pairs each launch stamps from its own dispatch, in eager passes.
- the measured BP:BH split, measured peaks, prefill seconds per 8192-token
  chunk with full-layer double buffering against the sustained host-link
  bound, the CPU oracle on a bounded sample (cpu_baseline);
- the DeepSeek-V4-Flash-shaped MXFP4 decode at BP:BH 300:1000 and 1000:1000,
  the cache-control step alone on the stress shapes (batch 16, 4096 slots,
  K = 64), and a cold start from a bank file.
Prints one JSON line. Other workloads (`--workload dsv4 | stress`) measure the
MXFP4 decode and the batch-16 / K = 64 stress case as the headline instead.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_gemv_qwen35b.json")


def measured_traffic(kernel_prefixes):
    """HBM bytes per layer step of the given kernels (FETCH_SIZE + WRITE_SIZE per launch, scaled by
    the copy calibration, summed) from the committed counter runs, or None when the kernels' source
    has changed since they were taken or a kernel is missing."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    src = open(os.path.join(ROOT, "expert_cached_decode_amd", "csrc", "decode.hip"), "rb").read()
    if hashlib.sha256(src).hexdigest() != rec.get("decode_hip_sha256"):
        return None
    total = 0
    for prefix in kernel_prefixes:
        hits = [k for name, k in rec["kernels"].items() if prefix in name]
        if not hits:
            return None
        total += int(hits[0]["fetch_bytes"] + hits[0]["write_bytes"])
    return total


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def workload(args):
    from gen.configs import DSV4_DECODE, QWEN_DECODE, STRESS, budget_slots
    if args.workload == "qwen":
        cfg = QWEN_DECODE
        text = ("Qwen3.6-35B-A3B-shaped MoE decode: 40 layers, 256 experts, top-8, hidden 2048, expert "
                "intermediate 512, bf16 experts (64.4 GB pinned bank), shared LRU cache of 3072 slots (30%)")
    elif args.workload == "dsv4":
        cfg = DSV4_DECODE.with_(bp=1000, bh=1000)
        text = ("DeepSeek-V4-Flash-shaped MoE decode: 43 layers, 256 experts, top-6, hidden 4096, expert "
                "intermediate 2048, MXFP4 experts (147.2 GB bank, held as 16 distinct pinned layers of 3.42 GB), "
                "shared LRU cache of 2752 slots (25%)")
    else:
        cfg = STRESS.with_(T=args.tokens or 16)
        text = ("stress: DeepSeek-V4-Flash shapes (MXFP4), 4096-slot cache, K = 64")
    if args.bpbh and args.bpbh != "calibrate":
        bp, bh = (int(v) for v in args.bpbh.split(":"))
        cfg = cfg.with_(bp=bp, bh=bh)
    if args.p is not None:
        cfg = cfg.with_(p=args.p)
    if args.tokens and args.workload != "stress":
        cfg = cfg.with_(T=args.tokens)
    text += ", batch %d, %d%% step-to-step routing overlap" % (cfg.T, round(100 * cfg.p))
    return cfg, text


def gemv_bytes(cfg):
    """Algorithmic bytes per cache-side expert: (gate + up) and down, codes plus MXFP4 scales."""
    n = cfg.H * cfg.I
    if cfg.wdtype == 2:
        return 2 * (n // 2 + n // 32), n // 2 + n // 32
    es = 4 if cfg.wdtype == 0 else 2
    return 2 * n * es, n * es


class DecodeWorkload:
    """One decode workload on one context: the pinned expert bank, seeded inputs resident in HBM,
    one hipGraph per token (all layers) over fixed staging buffers, and the eager kernel-timing
    pass. Steps index the generated inputs modulo their count."""

    def __init__(self, cfg, P, period, n_inputs, prefill_T=0, host_threads=0):
        import torch
        import gen
        import expert_cached_decode_amd as EC
        self.cfg, self.P, self.period = cfg, P, period
        L, T = cfg.L, cfg.T
        t0 = time.time()
        self.pool = EC.PinnedBuffer(P * cfg.E * cfg.expert_bytes)
        gen.fill_pool_ptr(cfg, self.pool.ptr, 0, P, layer_period=period)
        log("%s: expert bank %.1f GB pinned (%d pool layers) and drawn in %.1f s"
            % (cfg.name, self.pool.nbytes / 1e9, P, time.time() - t0))
        self.ctx = EC.Context(L, cfg.E, cfg.k, cfg.H, cfg.I, cfg.wdtype, max_tokens=T, cache_slots=cfg.slots,
                              victim_k=cfg.K, bp=cfg.bp, bh=cfg.bh, host_pool=self.pool,
                              prefill_max_tokens=prefill_T, host_threads=host_threads, pool_layers=P)
        self.budget_bp = -(-cfg.slots * 10000 // (L * cfg.E))  # the budget giving exactly cfg.slots
        while self.ctx.rebuild_slots(self.budget_bp)[0] > cfg.slots:
            self.budget_bp -= 1
        assert self.ctx.rebuild_slots(self.budget_bp)[0] == cfg.slots
        t0 = time.time()
        self.n_inputs = n_inputs
        self.logits_host = gen.decode_logits(cfg, steps=n_inputs)
        self.logits = torch.from_numpy(self.logits_host).cuda()  # [S, L, T, E]
        self.xs = torch.empty((n_inputs, L, T, cfg.H), dtype=torch.int16, device="cuda")
        for s in range(n_inputs):
            self.xs[s].copy_(torch.from_numpy(np.stack([gen.decode_x(cfg, s, l) for l in range(L)]).view(np.int16)))
        log("%s: decode inputs for %d steps generated in %.1f s" % (cfg.name, n_inputs, time.time() - t0))
        self.x_stage = torch.empty((L, T, cfg.H), dtype=torch.int16, device="cuda")
        self.lg_stage = torch.empty((L, T, cfg.E), dtype=torch.float32, device="cuda")
        self.outs = torch.empty((L, T, cfg.H), dtype=torch.int16, device="cuda")
        self.graph = None
        self.prime_us = 0  # queue primer ahead of each step of a kernel pass (0: none)
        self.enqueue_us = 0.0

    def token_layers(self, xsrc, lsrc, strm):
        import expert_cached_decode_amd as EC
        for l in range(self.cfg.L):
            EC.moe_decode_layer(self.ctx, l, xsrc[l], lsrc[l], self.cfg.T, self.outs[l], strm)

    def capture(self):
        """(Re-)capture the token graph (after a rebuild or a change of the host branch)."""
        import torch
        self.graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.graph(self.graph, stream=side):
            self.token_layers(self.x_stage, self.lg_stage, side)
        torch.cuda.synchronize()
        self.epoch = self.ctx.epoch()

    def step(self, s):
        i = s % self.n_inputs
        self.x_stage.copy_(self.xs[i])
        self.lg_stage.copy_(self.logits[i])
        self.graph.replay()

    def timed(self, s0, n):
        """Graph replays of steps s0 .. s0+n-1 between events on the current stream: (ms per step,
        stats of those steps). Raises if the context reports a device error."""
        import torch
        assert self.ctx.epoch() == self.epoch, "graph is stale"
        torch.cuda.synchronize()
        self.ctx.stats(reset=True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in range(s0, s0 + n):
            self.step(s)
        e1.record()
        torch.cuda.synchronize()
        st = self.ctx.stats(reset=True)
        assert st["device_error"] == 0
        return e0.elapsed_time(e1) / n, st

    def kernel_pass(self, steps):
        """Eager pass over the given steps with each decode kernel stamping a HIP event pair from its
        own dispatch on the launch stream; per-kind (us per launch, launches) and the pass's stats.
        With prime_us set, each step's launches are queued behind a primer of that many us, so its
        kernels run back to back as in a graph replay (the host's launch cost per kernel exceeds the
        short kernels' durations: unprimed, each would start on an idle queue)."""
        import torch
        import expert_cached_decode_amd as EC
        stream = torch.cuda.current_stream()
        torch.cuda.synchronize()
        self.ctx.stats(reset=True)
        self.ctx.kernel_timing(True)
        self.enqueue_us = 0.0
        pending = 0
        for n_step, s in enumerate(steps):
            i = s % self.n_inputs
            if pending + self.cfg.L > 1024:
                # the library holds 1024 event pairs per kernel kind and drains them (synchronising)
                # when they run out: drain here, between steps, rather than inside a primed step
                for k in ("ctl", "fill", "gate_up", "down"):
                    self.ctx.kernel_time(k)
                pending = 0
            pending += self.cfg.L
            if self.prime_us:
                EC.binding.queue_delay(self.prime_us, stream)
            t0 = time.perf_counter()
            self.token_layers(self.xs[i], self.logits[i], stream)
            if n_step > 0:  # the first step of a pass also pays Python's own warm-up
                self.enqueue_us = max(self.enqueue_us, 1e6 * (time.perf_counter() - t0))
        torch.cuda.synchronize()
        st = self.ctx.stats(reset=True)
        assert st["device_error"] == 0
        kt = {k: self.ctx.kernel_time(k) for k in ("ctl", "fill", "gate_up", "down")}
        self.ctx.kernel_timing(False)
        return {k: (v[0] * 1e3 / max(v[1], 1), v[1]) for k, v in kt.items()}, st

    def d9(self, kt, st, leg):
        """D9 expert streaming of a kernel pass: algorithmic cache-side expert bytes per layer step
        (gate/up: 2 I H weights, down: H I weights, with MXFP4 scales) over the average durations of
        the gate/up and down kernels."""
        cfg = self.cfg
        n = max(kt["gate_up"][1], 1)
        side = st["hits"] + st["fills"]  # cache-side experts over the pass
        gub, dnb = gemv_bytes(cfg)
        gu_b, dn_b = side * gub / n, side * dnb / n
        gu_us, dn_us = kt["gate_up"][0], kt["down"][0]
        gbs = (gu_b + dn_b) / ((gu_us + dn_us) * 1e-6) / 1e9
        out = {"bound": "hbm",
               "kernel": "D9 expert streaming: gate/up SwiGLU GEMV (gu_kernel) + down GEMV with exact merge "
                         "(down_kernel), per layer step",
               "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
               "traffic": None, "bytes_per_launch": int(gu_b + dn_b), "us_per_launch": round(gu_us + dn_us, 3),
               "launches": int(n), "leg": leg,
               "gate_up": {"bytes_per_launch": int(gu_b), "us_per_launch": round(gu_us, 3),
                           "achieved": round(gu_b / (gu_us * 1e-6) / 1e9, 1),
                           "frac": round(gu_b / (gu_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
               "down": {"bytes_per_launch": int(dn_b), "us_per_launch": round(dn_us, 3),
                        "achieved": round(dn_b / (dn_us * 1e-6) / 1e9, 1),
                        "frac": round(dn_b / (dn_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
               "ctl_us_per_launch": round(kt["ctl"][0], 3),
               "timing": "HIP event pair stamped by each launch's own dispatch on its stream "
                         "(hipExtLaunchKernelGGL), eager pass" + (
                             ", each step queued behind a %d us primer (ec_queue_delay; host enqueue %.0f us "
                             "per step at most)" % (self.prime_us, self.enqueue_us) if self.prime_us
                             else ", unprimed (kernels may start on an idle queue)")}
        if self.prime_us and self.enqueue_us > self.prime_us:
            log("warning: a step took %.0f us to enqueue, longer than the %d us primer" % (self.enqueue_us, self.prime_us))
        log("%s D9 (%s): gate/up %.2f + down %.2f us = %.2f us for %.1f MB -> %.0f GB/s, %.1f%% of 8 TB/s; ctl %.2f us"
            % (cfg.name, leg, gu_us, dn_us, gu_us + dn_us, (gu_b + dn_b) / 1e6, gbs, 100 * gbs / HBM_PEAK_GBS,
               kt["ctl"][0]))
        return out

    def all_hit(self, s0, window=8, reps=4, eager_only=False):
        """All-hit leg: a cold rebuild to the configured budget, one warm pass over `window` steps
        (they touch at most window * L * k <= C distinct experts, so nothing is evicted), then the
        same steps again: every routed expert is a hit, nothing is filled, so no expert byte read in
        the timed steps was written moments before (each pass streams window * L * k experts, far more
        than the 256 MB last-level cache holds). Returns the D9 roofline of an eager kernel pass and
        the tok/s of graph replays of the same warm steps (eager_only: the kernel pass alone, with an
        eager warm pass, so that no graph is launched)."""
        cfg = self.cfg
        window = min(window, cfg.slots // (cfg.L * cfg.k * cfg.T))
        if window < 1:
            return None
        self.ctx.rebuild(self.budget_bp)
        if eager_only:
            self.kernel_pass(range(s0, s0 + window))
        else:
            self.capture()
            for s in range(s0, s0 + window):
                self.step(s)
        kt, st = self.kernel_pass([s0 + (i % window) for i in range(window * reps)])
        assert st["misses"] == 0 and st["fills"] == 0 and st["host"] == 0, st
        out = self.d9(kt, st, "all-hit: warm cache, every routed expert a hit, no fills")
        if eager_only:
            return out
        ms = []
        for r in range(reps):
            m, st2 = self.timed(s0, window)
            assert st2["misses"] == 0
            ms.append(m)
        out["tok_s_all_hit"] = round(1e3 * cfg.T / float(np.median(ms)), 2)
        out["ms_per_step_all_hit"] = round(float(np.median(ms)), 4)
        log("%s all-hit decode: %.2f tok/s (graph replays of %d warm steps)" % (cfg.name, out["tok_s_all_hit"], window))
        return out

    def close(self):
        self.ctx.close()
        self.graph = None
        self.pool.close()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", choices=["qwen", "dsv4", "stress"], default="qwen")
    ap.add_argument("--bpbh", default=None,
                    help="BP:BH integers, e.g. 300:1000, or 'calibrate' (measured on this machine and applied)")
    ap.add_argument("--p", type=float, default=None, help="step-to-step routing overlap")
    ap.add_argument("--tokens", type=int, default=0, help="decode batch T")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the legs beyond the headline workload (DSV4 legs, control step, cold start)")
    ap.add_argument("--timing-steps", type=int, default=64)
    ap.add_argument("--steady-steps", type=int, default=128,
                    help="steps timed after the headline steps for the steady-state figure")
    ap.add_argument("--host-threads", type=int, default=0, help="host-branch worker threads (0 = library default)")
    ap.add_argument("--sweep-locality", action="store_true",
                    help="stress workload: tok/s and miss rate against routing overlap at batch 1 and 16")
    ap.add_argument("--no-peaks", action="store_true", help="skip the HBM copy and bf16 GEMM peak measurements")
    ap.add_argument("--sweep-ps", default="0,0.3,0.6,0.9", help="locality sweep: overlaps p (comma list)")
    ap.add_argument("--sweep-T", default="1,16", help="locality sweep: tokens per step (comma list)")
    ap.add_argument("--sweep-steps", type=int, default=48, help="locality sweep: timed steps per point")
    ap.add_argument("--sweep-warm", type=int, default=16, help="locality sweep: warm-up steps per point")
    ap.add_argument("--rebuild-recovery", action="store_true",
                    help="stress workload: batch-1 miss rate by window across cache_rebuild 40%% -> 15%% -> 40%%")
    ap.add_argument("--cold-start-gb", type=float, default=3.3,
                    help="time a cold start: write about this many GB of the bank as a bank file and read it "
                         "back into pinned memory with parallel direct I/O (0 = skip)")
    ap.add_argument("--measured-split-steps", type=int, default=128,
                    help="extra decode run with the measured BP:BH applied (0 = skip)")
    ap.add_argument("--prefill-chunks", type=int, default=4)
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration for rocprofv3 --pmc runs)")
    ap.add_argument("--prime-us", type=int, default=8000,
                    help="kernel passes: queue each step's launches behind a primer of this many us (0: off)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="for profiler runs: the prefill leg alone (no calibration and no decode leg); "
                         "prints its JSON")
    ap.add_argument("--counters-only", action="store_true",
                    help="for rocprofv3 --pmc runs: eager decode steps only (W warm-up, then --timing-steps "
                         "timed, then the all-hit window), no graph replays and no other leg; prints the D9 lines")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.steady_steps < 1 or args.timing_steps < 1:
        print("bench.py: need --steps, --steady-steps and --timing-steps >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    import torch
    from gen.configs import MXFP4, QWEN_PREFILL

    cfg, text = workload(args)
    torch.cuda.set_device(0)
    if args.calib_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    K, W, T, L = args.steps, args.warmup, cfg.T, cfg.L
    SS, TS = args.steady_steps, args.timing_steps
    # The cache starts empty. Its first FILL_TOKENS tokens are the fill transient (every routed
    # expert a miss at first); decode throughput is taken after them, as in a long generation.
    FILL_TOKENS = 64
    ss0 = FILL_TOKENS + W + K
    n_inputs = ss0 + SS + TS
    # The MXFP4 bank (147 GB) exceeds what the host can pin (about 64 GiB): the host pool then
    # holds P = 16 layers and layer l reads pool layer l mod 16 (bytes per fill unchanged). Its
    # layers are drawn once (period 1) and copied; every byte is still distinct memory.
    P = 16 if cfg.wdtype == MXFP4 else L
    period = 1 if cfg.wdtype == MXFP4 else 0
    prefill_T = QWEN_PREFILL.T if (args.workload == "qwen" and not args.no_prefill) else 0
    wl = DecodeWorkload(cfg, P, period, n_inputs, prefill_T=prefill_T, host_threads=args.host_threads)
    wl.prime_us = args.prime_us
    ctx = wl.ctx
    if args.prefill_only:
        if not prefill_T:
            sys.exit("--prefill-only needs the qwen workload with prefill on")
        print(json.dumps({"prefill": bench_prefill(wl, QWEN_PREFILL, args.prefill_chunks)}), flush=True)
        wl.close()
        return
    # measured BP and BH (MB/s): applied with --bpbh calibrate, else reported only
    bp_meas, bh_meas = ctx.calibrate_bandwidth(min(32, cfg.E // 4), apply=(args.bpbh == "calibrate"))
    log("calibration: BP %d MB/s over the link, BH %d MB/s on the host branch%s"
        % (bp_meas, bh_meas, " (applied)" if args.bpbh == "calibrate" else ""))
    bp_used, bh_used = (bp_meas, bh_meas) if args.bpbh == "calibrate" else (cfg.bp, cfg.bh)
    if args.counters_only:
        wl.kernel_pass(range(W))
        log("counters: %d eager warm-up steps done" % W)
        wl.d9(*wl.kernel_pass(range(W, W + TS)), "workload: eager steps continuing the warm-up")
        wl.all_hit(W + TS, eager_only=True)
        wl.close()
        return
    text += ", BP:BH %d:%d%s" % (bp_used, bh_used, " (measured)" if args.bpbh == "calibrate" else "")
    text += "; timed after the cache's first %d tokens (its fill from empty) and the warm-up steps" % FILL_TOKENS

    # the fill transient (graph replays of the first FILL_TOKENS steps from an empty cache), then the
    # headline: W warm-up steps, then exactly K timed steps (graph replays)
    wl.capture()
    ms_fill, st_fill = wl.timed(0, FILL_TOKENS)
    fill_transient = {"steps": FILL_TOKENS, "tok_s": round(1e3 * T / ms_fill, 3), "ms_per_step": round(ms_fill, 4),
                      "miss_rate": round(st_fill["misses"] / max(st_fill["hits"] + st_fill["misses"], 1), 4),
                      "fills_per_step": round(st_fill["fills"] / FILL_TOKENS, 3)}
    log("cache fill transient (steps 0..%d from an empty cache): %.2f tok/s, miss rate %.3f"
        % (FILL_TOKENS, fill_transient["tok_s"], fill_transient["miss_rate"]))
    for s in range(FILL_TOKENS, FILL_TOKENS + W):
        wl.step(s)
    t_wall = time.time()
    ms_per_step, st = wl.timed(FILL_TOKENS + W, K)
    t_wall = time.time() - t_wall
    tok_s = 1000.0 * T / ms_per_step
    lookups = st["hits"] + st["misses"]
    log("decode: %d steps at %.3f ms (wall %.3f s): %.2f tok/s; miss rate %.3f, fills/step %.2f, host/step %.2f"
        % (K, ms_per_step, t_wall, tok_s, st["misses"] / max(lookups, 1), st["fills"] / K, st["host"] / K))
    # steady state: SS more steps continuing the headline ones
    ms_ss, st_ss = wl.timed(ss0, SS)
    steady = {"tok_s": round(1e3 * T / ms_ss, 3), "ms_per_step": round(ms_ss, 4), "from_step": ss0, "steps": SS,
              "miss_rate": round(st_ss["misses"] / max(st_ss["hits"] + st_ss["misses"], 1), 4),
              "fills_per_step": round(st_ss["fills"] / SS, 3), "host_per_step": round(st_ss["host"] / SS, 3)}
    log("steady state (steps %d..%d): %.2f tok/s, miss rate %.3f" % (ss0, ss0 + SS, steady["tok_s"], steady["miss_rate"]))
    # kernel timing on the workload itself (eager, continuing the same steps)
    kt, st2 = wl.kernel_pass(range(ss0 + SS, ss0 + SS + TS))
    d9_workload = wl.d9(kt, st2, "workload: steps continuing the timed run (fills and hits)")
    fill_ms = kt["fill"][0] * kt["fill"][1] / 1e3
    fill_gbs = st2["fills"] * cfg.expert_bytes / max(fill_ms * 1e-3, 1e-9) / 1e9

    result = {
        "metric": "MoE decode tok/s (batch 1) + % HBM roofline; prefill s per 8192-token chunk",
        "value": round(tok_s, 3), "unit": "tok/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp4" if cfg.wdtype == MXFP4 else "bf16", "data": "synthetic",
        "config": {"workload": text, "global_batch": T, "layers": L, "cache_slots": cfg.slots,
                   "host_pool_layers": P, "graph": True, "tokens_before_warmup": FILL_TOKENS},
        "cache_fill_transient": fill_transient,
        "steady_state": steady,
        "roofline_workload": d9_workload,
        "other_kernels_us": {"ctl": round(kt["ctl"][0], 3),
                             "fill_per_expert": round(fill_ms * 1e3 / max(st2["fills"], 1), 2)},
        "bandwidth_mbps": {"bp_measured": bp_meas, "bh_measured": bh_meas, "bp_used": bp_used, "bh_used": bh_used},
        "cache": {"miss_rate": round(st["misses"] / max(lookups, 1), 4), "fills_per_step": round(st["fills"] / K, 3),
                  "host_per_step": round(st["host"] / K, 3), "fill_link_GBs": round(fill_gbs, 2)},
        "token_bound": token_bound(cfg, st_ss, SS, bp_meas, bh_meas, steady["tok_s"]),
    }
    log("per-token bound at steady state (HBM at 8 TB/s + larger of link at the measured BP and host at the "
        "measured BH): %.3f ms per step, %.2f tok/s; achieved %.1f%%" % (
            result["token_bound"]["ms_per_step"], result["token_bound"]["tok_s"], 100 * result["token_bound"]["frac"]))
    if args.bpbh != "calibrate" and args.measured_split_steps > 0:
        result["measured_split"] = bench_measured_split(wl, args.measured_split_steps)
        wl.ctx.set_bandwidth(cfg.bp, cfg.bh)
        torch.cuda.synchronize()
    # all-hit leg (the D9 roofline without fills before the reads): the headline roofline
    hit = wl.all_hit(ss0)  # None when one step's experts exceed the cache (batch 16 on the stress shapes)
    result["roofline"] = dict(hit if hit is not None else d9_workload,
                              traffic=measured_traffic(("gu_kernel", "down_kernel")) if args.workload == "qwen" else None)
    result["roofline"]["workload_frac"] = d9_workload["frac"]
    if args.workload == "stress":
        wl.ctx.rebuild(wl.budget_bp)
        result["cache_ctl"] = bench_cache_ctl(wl.ctx, cfg)
        result["rebuild"] = bench_rebuild(wl.ctx, cfg)
        if args.sweep_locality:
            result["locality_sweep"] = bench_locality_sweep(
                wl.ctx, cfg, ps=tuple(float(v) for v in args.sweep_ps.split(",")),
                Ts=tuple(int(v) for v in args.sweep_T.split(",")), warm=args.sweep_warm, steps=args.sweep_steps)
        if args.rebuild_recovery:
            result["rebuild_recovery"] = bench_rebuild_recovery(wl.ctx, cfg)
    if not args.no_peaks:
        result["peaks"] = bench_peaks()
        gub, dnb = gemv_bytes(cfg)
        side = cfg.k * cfg.T  # cache-side experts of an all-hit batch-1 layer step
        sizes = {"d9_layer_step": side * (gub + dnb), "gate_up": side * gub, "down": side * dnb}
        if args.workload == "qwen":
            from gen.configs import DSV4_DECODE
            g4, d4 = gemv_bytes(DSV4_DECODE)
            sizes["d9_layer_step_mxfp4_dsv4"] = DSV4_DECODE.k * (g4 + d4)
            sizes["gate_up_mxfp4_dsv4"] = DSV4_DECODE.k * g4
            sizes["down_mxfp4_dsv4"] = DSV4_DECODE.k * d4
        ceil = bench_burst_ceilings(sizes)
        result["peaks"]["hbm_burst"] = ceil
        # D9 is two dependent streams (down reads what gate/up writes): its ceiling is a gate/up-sized
        # burst followed by a down-sized one; one burst of all the bytes is the bound of a fused form
        two = ceil["gate_up"]["us_median"] + ceil["down"]["us_median"]
        two_frac = sizes["d9_layer_step"] / (two * 1e-6) / 1e9 / HBM_PEAK_GBS
        result["roofline"]["burst_ceiling"] = {
            "two_dependent_bursts": {"us": round(two, 3), "frac": round(two_frac, 4)},
            "one_burst": ceil["d9_layer_step"]}
        result["roofline"]["frac_of_burst_ceiling"] = round(result["roofline"]["frac"] / two_frac, 4)
        log("D9 all-hit at %.1f%% of 8 TB/s = %.1f%% of its two-burst ceiling (%.2f us, %.1f%%)"
            % (100 * result["roofline"]["frac"], 100 * result["roofline"]["frac_of_burst_ceiling"], two, 100 * two_frac))
    if prefill_T:
        result["prefill"] = bench_prefill(wl, QWEN_PREFILL, args.prefill_chunks)
    if not args.no_cpu:
        result["cpu_baseline"] = bench_cpu(cfg, wl.logits_host, P, period)
    wl.close()
    del wl, ctx
    torch.cuda.empty_cache()
    if args.workload == "qwen" and not args.no_extra:
        result["dsv4_decode"] = bench_dsv4_legs(prime_us=args.prime_us)
        ceil = result.get("peaks", {}).get("hbm_burst", {})
        hit = result["dsv4_decode"].get("roofline_all_hit")
        if hit and "gate_up_mxfp4_dsv4" in ceil:
            two = ceil["gate_up_mxfp4_dsv4"]["us_median"] + ceil["down_mxfp4_dsv4"]["us_median"]
            two_frac = hit["bytes_per_launch"] / (two * 1e-6) / 1e9 / HBM_PEAK_GBS
            hit["burst_ceiling"] = {"two_dependent_bursts": {"us": round(two, 3), "frac": round(two_frac, 4)},
                                    "one_burst": ceil["d9_layer_step_mxfp4_dsv4"]}
            hit["frac_of_burst_ceiling"] = round(hit["frac"] / two_frac, 4)
            log("dsv4 D9 all-hit at %.1f%% of 8 TB/s = %.1f%% of its two-burst ceiling (%.2f us, %.1f%%)"
                % (100 * hit["frac"], 100 * hit["frac_of_burst_ceiling"], two, 100 * two_frac))
        result["cache_ctl_stress"] = bench_cache_ctl_alone()
        result["stress_legs"] = bench_stress_legs()
        if args.cold_start_gb > 0:
            result["cold_start"] = bench_cold_start(cfg, args.cold_start_gb)
    print(json.dumps(result), flush=True)


def bench_dsv4_legs(ratios=((300, 1000), (1000, 1000)), warm=32, steps=64, timing_steps=16, prime_us=0):
    """The DeepSeek-V4-Flash-shaped MXFP4 decode (43 layers, top-6 of 256, H 4096, I 2048, 2752
    slots = 25%, p = 0.6) at BP:BH 300:1000 (most misses on the host branch) and 1000:1000 (every
    miss filled, no host branch): tok/s of graph replays from a cold cache after `warm` steps, and
    the D9 roofline of an eager kernel pass; plus the all-hit D9 roofline. The host pool holds 4
    pool layers (layer l reads pool layer l mod 4), drawn as one layer and copied: the bytes per
    fill and per host-side expert are those of the full bank."""
    import torch
    from gen.configs import DSV4_DECODE
    cfg = DSV4_DECODE
    n_inputs = warm + steps + timing_steps
    wl = DecodeWorkload(cfg, 4, 1, n_inputs)
    wl.prime_us = prime_us
    out = {"workload": "DeepSeek-V4-Flash-shaped MXFP4 decode, batch 1, 43 layers, 2752 slots (25%), "
                       "60% step-to-step routing overlap, 4 pinned pool layers", "legs": {}}
    for bp, bh in ratios:
        wl.ctx.set_bandwidth(bp, bh)
        wl.ctx.rebuild(wl.budget_bp)
        wl.capture()
        for s in range(warm):
            wl.step(s)
        ms, st = wl.timed(warm, steps)
        kt, st2 = wl.kernel_pass(range(warm + steps, n_inputs))
        leg = {"tok_s": round(1e3 / ms, 3), "ms_per_step": round(ms, 4), "steps": steps, "after_warm_steps": warm,
               "miss_rate": round(st["misses"] / max(st["hits"] + st["misses"], 1), 4),
               "fills_per_step": round(st["fills"] / steps, 3), "host_per_step": round(st["host"] / steps, 3),
               "host_branch": wl.ctx.stats()["host_branch"],
               "roofline": wl.d9(kt, st2, "workload BP:BH %d:%d" % (bp, bh))}
        if leg["host_branch"]:
            leg["roofline"]["note"] = ("the down GEMV's duration includes its wait for the host branch's partial "
                                       "sums: not an HBM figure")
        log("dsv4 BP:BH %d:%d: %.2f tok/s, miss rate %.3f, fills/step %.2f, host/step %.2f"
            % (bp, bh, leg["tok_s"], leg["miss_rate"], leg["fills_per_step"], leg["host_per_step"]))
        out["legs"]["%d:%d" % (bp, bh)] = leg
    wl.ctx.set_bandwidth(1000, 1000)
    out["roofline_all_hit"] = wl.all_hit(0)
    wl.close()
    del wl
    torch.cuda.empty_cache()
    return out


def bench_stress_legs(ps=(0.0, 0.3, 0.6, 0.9), Ts=(1, 16), warm=8, steps=24, rec_steps=384, rec_at=(128, 256)):
    """The stress shapes (DeepSeek-V4-Flash layers, MXFP4, 4096 slots, K = 64, BP:BH 1000:1000) in
    a short form of their two sweeps: tok/s and miss rate against step-to-step routing overlap p at
    batch 1 and 16, and the batch-1 miss rate by 32-step window across cache_rebuild 40% -> 15% ->
    40%. The host pool holds 4 pool layers (layer l reads pool layer l mod 4), drawn as one layer
    and copied: the bytes per fill are those of the full bank."""
    import torch
    from gen.configs import STRESS
    cfg = STRESS
    wl = DecodeWorkload(cfg, 4, 1, 4)
    out = {"workload": "stress shapes: DeepSeek-V4-Flash layers (43, top-6 of 256, MXFP4), 4096 slots, "
                       "K = 64, BP:BH 1000:1000, 4 pinned pool layers",
           "locality_sweep": bench_locality_sweep(wl.ctx, cfg, ps=ps, Ts=Ts, warm=warm, steps=steps),
           "rebuild_recovery": bench_rebuild_recovery(wl.ctx, cfg, steps=rec_steps, at=rec_at)}
    wl.close()
    torch.cuda.empty_cache()
    return out


def bench_cache_ctl_alone():
    """The fused cache-control step alone on the stress shapes: batch 16, top-6 of 256 experts per
    layer, 43 layers, 4096 slots, K = 64 (cache control reads no expert bytes, so the context holds
    tiny 64 x 64 experts)."""
    import gen
    import expert_cached_decode_amd as EC
    from gen.configs import BF16, STRESS
    cfg = STRESS.with_(H=64, I=64, wdtype=BF16)
    pool = EC.PinnedBuffer(cfg.L * cfg.E * cfg.expert_bytes)
    gen.fill_pool_ptr(cfg, pool.ptr, 0, cfg.L, layer_period=1)
    ctx = EC.Context(cfg.L, cfg.E, cfg.k, cfg.H, cfg.I, cfg.wdtype, max_tokens=cfg.T, cache_slots=cfg.slots,
                     victim_k=cfg.K, bp=cfg.bp, bh=cfg.bh, host_pool=pool, host_threads=2)
    out = bench_cache_ctl(ctx, cfg)
    ctx.close()
    pool.close()
    return out


def bench_burst_ceilings(sizes, buf_gib=8, reps=100):
    """HBM read ceiling of one-shot bursts of the given byte counts (ec_hbm_read_probe): each burst reads
    distinct memory of an 8 GiB buffer (never resident in the 256 MB last-level cache), timed by an event
    pair its own dispatch stamps; median of `reps`. Bursts queued back to back behind a primer (as the
    primed kernel pass runs the decode kernels), and, for reference, each on an idle queue."""
    import torch
    import expert_cached_decode_amd as EC
    buf = torch.ones(buf_gib << 30, dtype=torch.uint8, device="cuda")
    out = {}
    for name, b in sizes.items():
        med, best, got = EC.binding.hbm_read_probe(buf, b, reps, queued=True)
        imed, _, _ = EC.binding.hbm_read_probe(buf, b, reps, queued=False)
        out[name] = {"bytes": int(got), "us_median": round(med, 3), "us_best": round(best, 3),
                     "GBs": round(got / (med * 1e-6) / 1e9, 1), "frac": round(got / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "idle_queue_us_median": round(imed, 3)}
        log("HBM burst ceiling %s: %.1f MB in %.2f us (median of %d, queued) -> %.0f GB/s, %.1f%% of 8 TB/s; "
            "%.2f us from an idle queue" % (name, got / 1e6, med, reps, out[name]["GBs"], 100 * out[name]["frac"], imed))
    del buf
    torch.cuda.empty_cache()
    return out


def bench_peaks(copy_bytes=1 << 30, reps=8, n=8192):
    """Measured device peaks next to the spec figures (reference points for the rooflines, timed
    with library kernels): an HBM device-to-device copy over 4 rotating 1 GiB buffer pairs (8 GiB
    of distinct memory, far above the 256 MB MALL), counted as read + write bytes; and a bf16
    n x n x n GEMM through torch.matmul (hipBLASLt)."""
    import torch
    srcs = [torch.empty(copy_bytes, dtype=torch.uint8, device="cuda") for _ in range(4)]
    dsts = [torch.empty(copy_bytes, dtype=torch.uint8, device="cuda") for _ in range(4)]
    for i in range(4):
        dsts[i].copy_(srcs[i])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for r in range(reps):
        dsts[r % 4].copy_(srcs[r % 4])
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * copy_bytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del srcs, dsts
    a = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        c = torch.matmul(a, b)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        c = torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    tflops = 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    out = {"hbm_copy_GBs": round(copy_gbs, 1), "hbm_spec_GBs": HBM_PEAK_GBS,
           "bf16_gemm_TFLOPs": round(tflops, 1), "bf16_spec_TFLOPs": 2500.0,
           "method": "copy: read + write bytes over 4 x 1 GiB buffer pairs; gemm: torch.matmul %d^3 bf16" % n}
    log("peaks: HBM copy %.0f GB/s (spec %.0f); bf16 GEMM %.0f TFLOP/s (spec 2500)"
        % (copy_gbs, HBM_PEAK_GBS, tflops))
    return out


def token_bound(cfg, st, steps, bp_mbps, bh_mbps, tok_s):
    """Per-token bound of the decode: per layer step, the cache-side experts streamed from HBM at
    8 TB/s plus the larger of the fills over the host link (measured BP) and the host-list experts
    on the host branch (measured BH). The larger-of is taken over the run's totals, which is exact
    when one of the two terms is zero throughout (every miss filled, or none) and otherwise a lower
    bound of the per-layer sum."""
    se = cfg.expert_bytes
    hbm = (st["hits"] + st["fills"]) * se / (HBM_PEAK_GBS * 1e9) / steps
    link = st["fills"] * se / (bp_mbps * 1e6) / steps if bp_mbps > 0 else 0.0
    host = st["host"] * se / (bh_mbps * 1e6) / steps if bh_mbps > 0 else 0.0
    ms = 1e3 * (hbm + max(link, host))
    return {"ms_per_step": round(ms, 4), "tok_s": round(1e3 * cfg.T / ms, 2) if ms > 0 else None,
            "frac": round(tok_s / (1e3 * cfg.T / ms), 4) if ms > 0 else None,
            "terms_ms": {"hbm": round(1e3 * hbm, 4), "link": round(1e3 * link, 4), "host": round(1e3 * host, 4)},
            "link_GBs": round(bp_mbps / 1e3, 2), "host_GBs": round(bh_mbps / 1e3, 2), "hbm_GBs": HBM_PEAK_GBS}


def bench_measured_split(wl, steps):
    """Extra run: the same decode continued with the measured BP and BH applied (the pages split the
    misses by the two measured bandwidths); the graph is captured again for the new split."""
    cfg = wl.cfg
    bp, bh = wl.ctx.calibrate_bandwidth(min(32, cfg.E // 4), apply=True)
    wl.capture()
    for i in range(16):
        wl.step(i)
    t0 = time.perf_counter()
    ms, st = wl.timed(16, steps)
    dt = time.perf_counter() - t0
    out = {"bp_mbps": bp, "bh_mbps": bh, "steps": steps, "tok_s": round(1e3 * cfg.T / ms, 3),
           "tok_s_wall": round(steps * cfg.T / dt, 3),
           "miss_rate": round(st["misses"] / max(st["hits"] + st["misses"], 1), 4),
           "fills_per_step": round(st["fills"] / steps, 3), "host_per_step": round(st["host"] / steps, 3)}
    out["token_bound"] = token_bound(cfg, st, steps, bp, bh, out["tok_s"])
    # the host's view of the same steps: time per host job (doorbell seen to sums published) and
    # per handoff of the decode loop (sums published to the next layer step's doorbell)
    jobs, gaps = max(st["host_jobs"], 1), max(st["host_gaps"], 1)
    host_bytes = st["host"] * cfg.expert_bytes
    out["host_side"] = {"jobs": st["host_jobs"], "us_per_job": round(st["host_busy_us"] / jobs, 2),
                        "experts_per_job": round(st["host"] / jobs, 3),
                        "GBs_while_busy": round(host_bytes / max(st["host_busy_us"], 1e-9) / 1e3, 1),
                        "handoffs": st["host_gaps"], "us_per_handoff": round(st["host_gap_us"] / gaps, 2),
                        "us_per_layer_step": round(1e3 * ms / cfg.L, 2)}
    log("measured split BP:BH %d:%d: %.2f tok/s, fills/step %.2f, host/step %.2f; per-token bound %.2f tok/s"
        % (bp, bh, out["tok_s"], out["fills_per_step"], out["host_per_step"], out["token_bound"]["tok_s"]))
    hs = out["host_side"]
    log("measured split, host side: %.1f us per job (%.2f experts, %.0f GB/s while busy), %.1f us per handoff, "
        "%.1f us per layer step" % (hs["us_per_job"], hs["experts_per_job"], hs["GBs_while_busy"],
                                     hs["us_per_handoff"], hs["us_per_layer_step"]))
    return out


def bench_cold_start(cfg, gb):
    """Fast start: write the first layers of the expert bank (about `gb` GB) as a bank file,
    then time reading it with parallel direct I/O into freshly pinned host memory (the final
    host-pool layout, no repacking); the rate is extrapolated to the whole bank."""
    import shutil
    import tempfile
    import gen
    import expert_cached_decode_amd as EC
    layer_bytes = cfg.E * cfg.expert_bytes
    P = max(1, min(cfg.L, int(gb * 1e9 // layer_bytes)))
    shape = EC.make_shape(cfg.L, cfg.E, cfg.k, cfg.H, cfg.I, cfg.wdtype)
    src = np.empty(P * layer_bytes, np.uint8)
    gen.fill_pool_ptr(cfg, src.ctypes.data, 0, P)
    d = tempfile.mkdtemp(prefix="ecbank_", dir=os.environ.get("TMPDIR", "/tmp"))
    try:
        path = os.path.join(d, "bank.ecb")
        t0 = time.perf_counter()
        EC.bank_write(path, shape, P, src.ctypes.data, src.nbytes)
        t_write = time.perf_counter() - t0
        pinned = EC.PinnedBuffer(src.nbytes)
        sec, direct = EC.bank_read(path, shape, P, pinned.ptr, pinned.nbytes, threads=16)
        ok = bool(np.array_equal(pinned.numpy()[::4096], src[::4096]) and
                  np.array_equal(pinned.numpy()[-1 << 20:], src[-1 << 20:]))
        pinned.close()
    finally:
        shutil.rmtree(d, ignore_errors=True)
    rate = src.nbytes / sec / 1e9
    full = cfg.L * layer_bytes
    out = {"bytes": int(src.nbytes), "layers": P, "read_s": round(sec, 3), "read_GBs": round(rate, 2),
           "direct_io": direct, "threads": 16, "write_s": round(t_write, 2), "verified": ok,
           "full_bank_bytes": int(full), "full_bank_read_s_extrapolated": round(full / 1e9 / rate, 2)}
    log("cold start: %.2f GB bank file read in %.2f s (%.2f GB/s, direct I/O %s); the %.1f GB bank would take %.1f s"
        % (src.nbytes / 1e9, sec, rate, direct, full / 1e9, out["full_bank_read_s_extrapolated"]))
    return out


def bench_rebuild_recovery(ctx, cfg, steps=768, window=32, at=(256, 512), budgets=(4000, 1500, 4000)):
    """Elastic budget at batch 1: a cold cache of 40% of all experts, cache_rebuild to 15% at step
    256 and back to 40% at step 512 (each cold, at a safe point between tokens); miss rate per
    window of steps, tok/s per phase and each rebuild's latency. One graph per phase (a rebuild
    changes the epoch, so the graph is captured again)."""
    import torch
    import gen
    import expert_cached_decode_amd as EC
    L, E, H = cfg.L, cfg.E, cfg.H
    c = cfg.with_(T=1)
    lg = torch.from_numpy(gen.decode_logits(c, steps=steps)).cuda()
    xs = torch.from_numpy(np.stack([np.stack([gen.decode_x(c, s, l) for l in range(L)])
                                    for s in range(4)]).view(np.int16)).cuda()
    x_stage = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
    lg_stage = torch.empty((L, 1, E), dtype=torch.float32, device="cuda")
    outs = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
    bounds = [0] + list(at) + [steps]
    windows, phases = [], []
    for ph in range(len(bounds) - 1):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        C = ctx.rebuild(budgets[ph])
        torch.cuda.synchronize()
        rb_ms = (time.perf_counter() - t0) * 1e3
        graph, side = torch.cuda.CUDAGraph(), torch.cuda.Stream()
        with torch.cuda.graph(graph, stream=side):
            for l in range(L):
                EC.moe_decode_layer(ctx, l, x_stage[l], lg_stage[l], 1, outs[l], side)
        torch.cuda.synchronize()
        ctx.stats(reset=True)
        busy = 0.0
        for w0 in range(bounds[ph], bounds[ph + 1], window):
            w1 = min(w0 + window, bounds[ph + 1])
            t0 = time.perf_counter()
            for i in range(w0, w1):
                x_stage.copy_(xs[i % 4]); lg_stage.copy_(lg[i])
                graph.replay()
            torch.cuda.synchronize()
            busy += time.perf_counter() - t0
            st = ctx.stats(reset=True)
            windows.append({"steps": [w0, w1], "slots": C,
                            "miss_rate": round(st["misses"] / max(st["hits"] + st["misses"], 1), 4)})
        n = bounds[ph + 1] - bounds[ph]
        phases.append({"budget_bp": budgets[ph], "slots": C, "rebuild_ms": round(rb_ms, 3),
                       "tok_s": round(n / busy, 2), "steps": n})
        log("rebuild recovery: %d slots from step %d (rebuild %.2f ms): %.2f tok/s; miss rate by window %s"
            % (C, bounds[ph], rb_ms, n / busy,
               " ".join("%.3f" % w["miss_rate"] for w in windows if bounds[ph] <= w["steps"][0] < bounds[ph + 1])))
        del graph
    ctx.rebuild(budgets[0])
    return {"window": window, "phases": phases, "windows": windows}


def bench_locality_sweep(ctx, cfg, ps=(0.0, 0.3, 0.6, 0.9), Ts=(1, 16), warm=16, steps=48):
    """tok/s and miss rate against step-to-step routing overlap p at batch 1 and 16 (cold cache at
    each point through cache_rebuild to the configured slot count, one graph per point)."""
    import torch
    import gen
    import expert_cached_decode_amd as EC
    L, E, H = cfg.L, cfg.E, cfg.H
    budget = -(-cfg.slots * 10000 // (L * E))  # smallest budget giving at least cfg.slots slots
    if budget * L * E // 10000 > cfg.slots:
        budget -= 1
    out = []
    for T in Ts:
        assert 1 <= T <= cfg.T
        x_stage = torch.empty((L, T, H), dtype=torch.int16, device="cuda")
        lg_stage = torch.empty((L, T, E), dtype=torch.float32, device="cuda")
        outs = torch.empty((L, T, H), dtype=torch.int16, device="cuda")
        for p in ps:
            c = cfg.with_(T=T, p=p)
            lg = torch.from_numpy(gen.decode_logits(c, steps=warm + steps)).cuda()
            xs = torch.from_numpy(np.stack([np.stack([gen.decode_x(c, s, l) for l in range(L)])
                                            for s in range(4)]).view(np.int16)).cuda()
            ctx.rebuild(budget)
            graph, side = torch.cuda.CUDAGraph(), torch.cuda.Stream()
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=side):
                for l in range(L):
                    EC.moe_decode_layer(ctx, l, x_stage[l], lg_stage[l], T, outs[l], side)
            torch.cuda.synchronize()

            def step(i):
                x_stage.copy_(xs[i % 4]); lg_stage.copy_(lg[i])
                graph.replay()

            for i in range(warm):
                step(i)
            torch.cuda.synchronize()
            ctx.stats(reset=True)
            t0 = time.perf_counter()
            for i in range(warm, warm + steps):
                step(i)
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            st = ctx.stats(reset=True)
            r = {"T": T, "p": p, "tok_s": round(steps * T / dt, 2),
                 "miss_rate": round(st["misses"] / max(st["hits"] + st["misses"], 1), 4),
                 "unique_per_layer_step": round((st["hits"] + st["misses"]) / (steps * L), 2),
                 "fills_per_step": round(st["fills"] / steps, 2), "host_per_step": round(st["host"] / steps, 2)}
            log("locality sweep T=%d p=%.1f: %.2f tok/s, miss rate %.3f, %.1f unique experts per layer step"
                % (T, p, r["tok_s"], r["miss_rate"], r["unique_per_layer_step"]))
            out.append(r)
            del graph
    ctx.rebuild(budget)
    return out


def bench_cache_ctl(ctx, cfg, calls=10000, batch=100):
    """The fused cache-control step alone (expert_cache_step on given ids): T tokens x k experts,
    ids drawn per call from the workload's routing, C slots, K victim candidates; per-call time from
    events around batches of calls, median over the batches."""
    import torch
    import gen
    import expert_cached_decode_amd as EC
    T, L = cfg.T, cfg.L
    lg = gen.decode_logits(cfg, steps=64)
    ids = torch.from_numpy(np.stack([route_top_k(lg[s, l], cfg.k) for s in range(64) for l in range(L)])).cuda()
    n = ids.shape[0]
    stream = torch.cuda.current_stream()
    for i in range(200):
        EC.expert_cache_step(ctx, i % L, ids[i % n], T, stream)
    torch.cuda.synchronize()
    times = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for b in range(calls // batch):
        e0.record()
        for i in range(batch):
            j = b * batch + i
            EC.expert_cache_step(ctx, j % L, ids[j % n], T, stream)
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / batch)
    out = {"calls": calls, "us_per_call_median": round(float(np.median(times)), 3),
           "us_per_call_min": round(float(np.min(times)), 3), "T": T, "k": cfg.k, "slots": cfg.slots, "K": cfg.K}
    log("cache control alone (T=%d, k=%d, C=%d, K=%d): %.2f us per call (median of %d batches of %d)"
        % (T, cfg.k, cfg.slots, cfg.K, out["us_per_call_median"], calls // batch, batch))
    return out


def route_top_k(logits, k):
    """Routed ids [T, k] by (logit desc, id asc) (input preparation for the control-step timing)."""
    order = np.lexsort((np.broadcast_to(np.arange(logits.shape[-1]), logits.shape), -logits), axis=-1)
    return order[:, :k].astype(np.int32)


def bench_rebuild(ctx, cfg):
    """cache_rebuild latency at a safe point: 40% -> 15% -> 40% of all experts."""
    import torch
    from gen.configs import budget_slots
    out = {}
    for bp in (1500, 4000):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        C = ctx.rebuild(bp)
        out["to_%d_bp_ms" % bp] = round((time.perf_counter() - t0) * 1e3, 3)
        out["slots_%d_bp" % bp] = C
    assert out["slots_4000_bp"] == budget_slots(cfg.L, cfg.E, 4000)
    log("cache_rebuild: %s" % out)
    return out


def bench_prefill(wl, pcfg, chunks, link_layers=8):
    """Prefill seconds per 8192-token chunk (median of `chunks` steady-state chunks, full-layer
    double buffering on), the double-buffer-off ablation, and the host-link bound: raw pinned H2D
    copies of whole layers (1.61 GB each) into one device buffer, both the best single layer copy
    and `link_layers` distinct layers back to back (the sustained rate, the bound used)."""
    import torch
    import gen
    import expert_cached_decode_amd as EC
    cfg, ctx = wl.cfg, wl.ctx
    T = pcfg.T
    lb = cfg.E * cfg.expert_bytes
    dst = torch.empty(lb, dtype=torch.uint8, device="cuda")
    best = 1e9
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        EC.binding.memcpy_async(dst.data_ptr(), wl.pool.ptr, lb)
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b))
    sustained = 1e9
    for _ in range(2):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for l in range(link_layers):
            EC.binding.memcpy_async(dst.data_ptr(), wl.pool.ptr + (l % cfg.L) * lb, lb)
        b.record()
        torch.cuda.synchronize()
        sustained = min(sustained, a.elapsed_time(b))
    del dst
    link_single = lb / (best * 1e-3) / 1e9
    link_gbs = link_layers * lb / (sustained * 1e-3) / 1e9
    xs = torch.empty((cfg.L, T, cfg.H), dtype=torch.int16, device="cuda")
    lgs = torch.empty((cfg.L, T, cfg.E), dtype=torch.float32, device="cuda")
    for l in range(cfg.L):
        xs[l].copy_(torch.from_numpy(gen.prefill_x(pcfg, l).view(np.int16)))
        lgs[l].copy_(torch.from_numpy(gen.prefill_logits(pcfg, l)))
    out = torch.empty((T, cfg.H), dtype=torch.int16, device="cuda")
    compute = torch.cuda.current_stream()

    def chunk():
        for l in range(cfg.L):
            EC.moe_prefill_layer(ctx, l, xs[l], lgs[l], T, out, compute, ctx.copy_stream)

    times = []
    ctx.set_prefill_overlap(True)
    for c in range(chunks + 1):  # the first chunk starts from empty buffers: not counted
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        chunk()
        b.record()
        torch.cuda.synchronize()
        if c > 0:
            times.append(a.elapsed_time(b) / 1e3)
    torch.cuda.synchronize()
    ctx.set_prefill_overlap(False)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    chunk()
    b.record()
    torch.cuda.synchronize()
    t_off = a.elapsed_time(b) / 1e3
    ctx.set_prefill_overlap(True)
    # compute alone: layer 0 again and again once its buffer holds it (no upload on the path)
    EC.moe_prefill_layer(ctx, 0, xs[0], lgs[0], T, out, compute, ctx.copy_stream)
    torch.cuda.synchronize()
    reps = 10
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        EC.moe_prefill_layer(ctx, 0, xs[0], lgs[0], T, out, compute, ctx.copy_stream)
    b.record()
    torch.cuda.synchronize()
    compute_ms = a.elapsed_time(b) / reps
    del xs, lgs, out
    s_chunk = float(np.median(times))
    bound = cfg.L * lb / (link_gbs * 1e9)
    log("prefill: %.3f s per 8192-token chunk (double buffer off: %.3f s); raw copies of the same bytes take %.3f s "
        "at %.1f GB/s sustained over %d layers (single layer copy %.1f GB/s); compute alone %.3f ms per layer"
        % (s_chunk, t_off, bound, link_gbs, link_layers, link_single, compute_ms))
    return {"s_per_chunk": round(s_chunk, 4), "tokens": T, "layers": cfg.L, "chunks_timed": len(times),
            "bytes_per_chunk": cfg.L * lb, "link_GBs_sustained": round(link_gbs, 2),
            "link_GBs_single_layer": round(link_single, 2), "link_layers_timed": link_layers,
            "link_copy_s": round(bound, 4), "ratio_to_link_copy": round(s_chunk / bound, 4),
            "chunk_link_GBs": round(cfg.L * lb / s_chunk / 1e9, 2),
            "s_per_chunk_no_double_buffer": round(t_off, 4), "tok_s": round(T / s_chunk, 1),
            "compute_ms_per_layer": round(compute_ms, 4)}


def bench_cpu(cfg, logits, P, period, budget_s=12.0, cache_bytes=6 << 30):
    """The CPU oracle (fp64 plain-loop MoE + literal LRU simulator) on a bounded sample of the same
    workload: steps until about `budget_s` of oracle compute. Drawing the experts' weights is input
    preparation (untimed); drawn experts are kept in a bounded LRU, since consecutive steps share
    most of their experts."""
    from collections import OrderedDict
    import gen
    from oracle import moe
    from oracle.lru_sim import LRUSim
    from oracle.route import route
    cores = len(os.sched_getaffinity(0))
    sim = LRUSim(cfg.L, cfg.E, cfg.slots, cfg.K, cfg.bp, cfg.bh)
    t_moe = t_lru = 0.0
    steps = 0
    drawn = OrderedDict()
    held = 0

    def expert(layer, e):
        nonlocal held
        key = (layer, e)
        if key in drawn:
            drawn.move_to_end(key)
            return drawn[key]
        m = gen.expert_logical(cfg, layer, e)
        drawn[key] = m
        held += sum(sum(a.nbytes for a in v) if isinstance(v, tuple) else v.nbytes for v in m.values())
        while held > cache_bytes and len(drawn) > 1:
            _, old = drawn.popitem(last=False)
            held -= sum(sum(a.nbytes for a in v) if isinstance(v, tuple) else v.nbytes for v in old.values())
        return m

    while (t_moe + t_lru < budget_s or steps == 0) and steps < len(logits):
        s = steps
        for l in range(cfg.L):
            lg = logits[s, l]                                   # [T, E]
            xw = gen.decode_x(cfg, s, l)
            x = (xw.astype(np.float64) if cfg.wdtype == 0 else gen.bf16_to_f32(xw).astype(np.float64))
            ids, _ = route(lg, cfg.k)
            src_l = (l % P) % period if period else l % P  # the layer whose draws the pool holds
            mats = {e: expert(src_l, e) for row in ids for e in row}  # input preparation, untimed
            t0 = time.time()
            sim.step(l, ids)
            t1 = time.time()
            moe.moe_tokens(cfg.wdtype, x, lg, cfg.k, mats.__getitem__)
            t2 = time.time()
            t_lru += t1 - t0
            t_moe += t2 - t1
        steps += 1
    sec = t_moe + t_lru
    log("cpu oracle: %d steps x %d layers in %.2f s of compute (%.2f s LRU sim) on %d cores"
        % (steps, cfg.L, sec, t_lru, cores))
    return {"value": round(steps * cfg.T / sec, 4), "unit": "tok/s", "cores": cores, "kind": "oracle",
            "sample": "first %d decode steps (batch %d) x %d layers of the same workload (fp64 C MoE layer with "
                      "OpenMP over rows, routing and literal LRU simulator in Python; weight generation not timed)"
                      % (steps, cfg.T, cfg.L),
            "lru_sim_s": round(t_lru, 3), "moe_s": round(t_moe, 3)}


if __name__ == "__main__":
    main()
