"""ctypes binding of libexpert_cached_decode.so.

Argument marshalling only: every step of the MoE layer runs in the library's
HIP kernels (or its host threads for the host branch). PyTorch provides device
memory, pinned host memory and streams. The functions keep the C names
(moe_route, expert_cache_step, moe_decode_layer, moe_prefill_layer,
cache_rebuild); see include/ec_api.h for argument meaning and layouts.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libexpert_cached_decode.so")

c_i32, c_u32, c_u64, c_vp = ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p

EC_DT_F32, EC_DT_BF16, EC_DT_MXFP4 = 0, 1, 2
CNT_U, CNT_H, CNT_M, CNT_Q, CNT_HOST, CNT_GPU = range(6)


class ECError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("ec status %d: %s" % (status, msg))
        self.status = status


class ec_shape(ctypes.Structure):
    _fields_ = [("layers", c_i32), ("experts", c_i32), ("top_k", c_i32), ("hidden", c_i32), ("inter", c_i32),
                ("wdtype", c_i32)]


class ec_layout_info(ctypes.Structure):
    _fields_ = [("expert_bytes", c_u64), ("layer_bytes", c_u64), ("gate_off", c_u64), ("up_off", c_u64),
                ("down_off", c_u64), ("gate_scale_off", c_u64), ("up_scale_off", c_u64),
                ("down_scale_off", c_u64)]


class ec_config(ctypes.Structure):
    _fields_ = [("shape", ec_shape), ("max_tokens", c_i32), ("cache_slots", c_i32), ("victim_k", c_i32),
                ("bp_mbps", c_u32), ("bh_mbps", c_u32), ("host_threads", c_i32), ("prefill_max_tokens", c_i32),
                ("pool_layers", c_i32), ("reserved", c_i32 * 3)]


class ec_step_view(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in ("uniq", "counts", "pos", "cls", "slot", "fills", "victims", "evicted",
                                    "host_list", "rewritten")]


class ec_stats(ctypes.Structure):
    _fields_ = [("steps", c_u64), ("hits", c_u64), ("misses", c_u64), ("fills", c_u64), ("host", c_u64),
                ("evictions", c_u64), ("device_error", c_i32), ("slots", c_i32), ("clock", c_u64),
                ("host_only", c_i32), ("host_branch", c_i32), ("host_jobs", c_u64), ("host_busy_us", ctypes.c_double),
                ("host_gaps", c_u64), ("host_gap_us", ctypes.c_double)]


_lib = None
EXPORTS = ["ec_strerror", "ec_last_error", "ec_layout", "ec_workspace_size", "ec_create", "ec_destroy",
           "ec_set_bandwidth", "moe_route", "expert_cache_step", "moe_decode_layer", "moe_prefill_layer",
           "ec_set_prefill_overlap", "cache_rebuild", "ec_epoch", "ec_get_stats", "ec_debug_state",
           "ec_kernel_timing", "ec_kernel_time", "ec_calibrate_bandwidth", "moe_gate_logits",
           "moe_decode_block", "ec_bank_write", "ec_bank_read", "ec_last_step", "ec_rebuild_slots",
           "moe_decode_layer_static", "ec_hbm_read_probe", "ec_queue_delay", "ec_host_branch_test_hooks"]
KERNEL_KINDS = {"ctl": 0, "fill": 1, "gate_up": 2, "down": 3}


def lib():
    """Load the HIP library (raises if it has not been built: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libexpert_cached_decode.so is not built (run __graft_entry__.build() or "
                               "python expert_cached_decode_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.ec_strerror.restype = ctypes.c_char_p
        L.ec_strerror.argtypes = [c_i32]
        L.ec_last_error.restype = ctypes.c_char_p
        L.ec_last_error.argtypes = [c_vp]
        L.ec_layout.argtypes = [P(ec_shape), P(ec_layout_info)]
        L.ec_workspace_size.argtypes = [P(ec_config), P(c_u64), P(c_u64)]
        L.ec_create.argtypes = [P(ec_config), c_vp, c_u64, c_vp, c_u64, c_vp, c_u64, c_vp, c_u64, P(c_vp)]
        L.ec_destroy.argtypes = [c_vp]
        L.ec_set_bandwidth.argtypes = [c_vp, c_u32, c_u32, c_vp]
        L.moe_route.argtypes = [c_vp, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]
        L.expert_cache_step.argtypes = [c_vp, c_i32, c_vp, c_i32, P(ec_step_view), c_vp]
        L.ec_last_step.argtypes = [c_vp, P(ec_step_view)]
        L.moe_decode_layer.argtypes = [c_vp, c_i32, c_vp, c_vp, c_i32, c_vp, c_vp]
        L.moe_decode_layer_static.argtypes = [c_vp, c_i32, c_vp, c_vp, c_i32, c_vp, c_vp]
        L.moe_prefill_layer.argtypes = [c_vp, c_i32, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp]
        L.ec_set_prefill_overlap.argtypes = [c_vp, c_i32]
        L.cache_rebuild.argtypes = [c_vp, c_i32, c_vp, c_u64]
        L.ec_rebuild_slots.argtypes = [c_vp, c_i32, P(c_i32), P(c_u64)]
        L.ec_epoch.restype = c_u64
        L.ec_epoch.argtypes = [c_vp]
        L.ec_get_stats.argtypes = [c_vp, P(ec_stats), c_i32]
        L.ec_debug_state.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp]
        L.ec_kernel_timing.argtypes = [c_vp, c_i32]
        L.ec_kernel_time.argtypes = [c_vp, c_i32, ctypes.POINTER(ctypes.c_double), P(c_u64), c_i32]
        L.ec_hbm_read_probe.argtypes = [c_vp, c_u64, c_u64, c_i32, c_i32, c_vp, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_double), P(c_u64)]
        L.ec_queue_delay.argtypes = [c_vp, ctypes.c_uint32]
        L.ec_host_branch_test_hooks.argtypes = [c_vp, c_i32, ctypes.c_uint32]
        L.ec_calibrate_bandwidth.argtypes = [c_vp, c_i32, c_i32, P(ctypes.c_uint32), P(ctypes.c_uint32)]
        L.moe_gate_logits.argtypes = [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp]
        L.moe_decode_block.argtypes = [c_vp, c_i32, c_vp, c_vp, c_i32, c_vp, c_vp]
        L.ec_bank_write.argtypes = [ctypes.c_char_p, P(ec_shape), c_i32, c_vp, c_u64]
        L.ec_bank_read.argtypes = [ctypes.c_char_p, P(ec_shape), c_i32, c_vp, c_u64, c_i32, P(c_i32),
                                   ctypes.POINTER(ctypes.c_double)]
        for f in EXPORTS:
            getattr(L, f).restype = getattr(L, f).restype or c_i32
        L.ec_strerror.restype = ctypes.c_char_p
        L.ec_last_error.restype = ctypes.c_char_p
        L.ec_epoch.restype = c_u64
        _lib = L
    return _lib


def check(status, ctx=None):
    if status != 0:
        msg = lib().ec_last_error(ctx)
        raise ECError(status, (msg or b"").decode() or lib().ec_strerror(status).decode())
    return status


def make_shape(L, E, k, H, I, wdtype):
    return ec_shape(L, E, k, H, I, wdtype)


def layout(shape):
    out = ec_layout_info()
    check(lib().ec_layout(ctypes.byref(shape), ctypes.byref(out)))
    return out


def workspace_size(cfg):
    d, p = c_u64(), c_u64()
    check(lib().ec_workspace_size(ctypes.byref(cfg), ctypes.byref(d), ctypes.byref(p)))
    return d.value, p.value


# ---- pinned host memory (plumbing) ------------------------------------------------
class PinnedBuffer:
    """Pinned, device-accessible host memory from hipHostMalloc (freed on close)."""

    def __init__(self, nbytes):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipHostMalloc.argtypes = [ctypes.POINTER(c_vp), ctypes.c_size_t, ctypes.c_uint]
        self._hip.hipHostFree.argtypes = [c_vp]
        p = c_vp()
        rc = self._hip.hipHostMalloc(ctypes.byref(p), max(int(nbytes), 1), 0)
        if rc != 0 or not p.value:
            self._hip.hipGetLastError()  # the failure is reported here, not by a later HIP call
            raise MemoryError("hipHostMalloc(%d) failed with %d" % (nbytes, rc))
        self.ptr = p.value
        self.nbytes = int(nbytes)

    def numpy(self):
        import numpy as np
        return np.ctypeslib.as_array(ctypes.cast(self.ptr, ctypes.POINTER(ctypes.c_uint8)), shape=(self.nbytes,))

    def close(self):
        if self.ptr:
            self._hip.hipHostFree(c_vp(self.ptr))
            self.ptr = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t):
    return None if t is None else (t if isinstance(t, int) else t.data_ptr())


# ---- entry points with the C names --------------------------------------------------
def moe_route(logits, T, E, k, ids, w, stream=None):
    check(lib().moe_route(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _stream(stream)))


def expert_cache_step(ctx, layer, ids, T, stream=None):
    v = ec_step_view()
    check(lib().expert_cache_step(ctx.handle, layer, _ptr(ids), T, ctypes.byref(v), _stream(stream)), ctx.handle)
    return v


def last_step(ctx):
    """Device views of the step buffers the last step call on ctx wrote (ec_last_step)."""
    v = ec_step_view()
    check(lib().ec_last_step(ctx.handle, ctypes.byref(v)), ctx.handle)
    return v


def moe_decode_layer(ctx, layer, x, logits, T, out, stream=None):
    check(lib().moe_decode_layer(ctx.handle, layer, _ptr(x), _ptr(logits), T, _ptr(out), _stream(stream)),
          ctx.handle)


def moe_decode_layer_static(ctx, layer, x, logits, T, out, stream=None):
    """moe_decode_layer with the step buffers in the library's static device scratch (allocates nothing)."""
    check(lib().moe_decode_layer_static(ctx.handle, layer, _ptr(x), _ptr(logits), T, _ptr(out), _stream(stream)),
          ctx.handle)


def bank_write(path, shape, pool_layers, ptr, nbytes):
    """Write an expert-bank file (no GPU involved)."""
    check(lib().ec_bank_write(os.fsencode(path), ctypes.byref(shape), pool_layers, c_vp(ptr), nbytes))


def bank_read(path, shape, pool_layers, ptr, nbytes, threads=0):
    """Fill host memory at ptr from an expert-bank file; returns (seconds, mode) with mode 1 direct
    I/O into ptr, 2 direct I/O through bounce buffers, 0 buffered."""
    sec, direct = ctypes.c_double(), c_i32()
    check(lib().ec_bank_read(os.fsencode(path), ctypes.byref(shape), pool_layers, c_vp(ptr), nbytes, threads,
                             ctypes.byref(direct), ctypes.byref(sec)))
    return sec.value, int(direct.value)


def moe_gate_logits(w_router, x, x_dtype, T, E, H, logits, stream=None):
    check(lib().moe_gate_logits(_ptr(w_router), _ptr(x), x_dtype, T, E, H, _ptr(logits), _stream(stream)))


def moe_decode_block(ctx, layer, x, w_router, T, out, stream=None):
    check(lib().moe_decode_block(ctx.handle, layer, _ptr(x), _ptr(w_router), T, _ptr(out), _stream(stream)),
          ctx.handle)


def moe_prefill_layer(ctx, layer, x, logits, T, out, compute_stream=None, copy_stream=None):
    if copy_stream is None:
        copy_stream = ctx.copy_stream
    check(lib().moe_prefill_layer(ctx.handle, layer, _ptr(x), _ptr(logits), T, _ptr(out), _stream(compute_stream),
                                  _stream(copy_stream)), ctx.handle)


def cache_rebuild(ctx, budget_bp, new_slot_pool=None):
    return ctx.rebuild(budget_bp, new_slot_pool)


class Context:
    """An expert-cache context with torch-owned device and pinned workspaces.

    host_pool: a PinnedBuffer (or any pinned pointer + size) holding the
    [L][E][expert_bytes] expert bank. slot_pool: a torch uint8 CUDA tensor of
    at least cache_slots * expert_bytes bytes (allocated here when None).
    """

    def __init__(self, L, E, k, H, I, wdtype, max_tokens, cache_slots, victim_k=0, bp=1000, bh=1000,
                 host_pool=None, host_pool_bytes=None, slot_pool=None, host_threads=0, prefill_max_tokens=0,
                 pool_layers=0):
        import torch
        self.shape = make_shape(L, E, k, H, I, wdtype)
        self.layout = layout(self.shape)
        self.cfg = ec_config(self.shape, max_tokens, cache_slots, victim_k, bp, bh, host_threads,
                             prefill_max_tokens, pool_layers)
        dev_b, pin_b = workspace_size(self.cfg)
        self.dev_ws = torch.empty(dev_b, dtype=torch.uint8, device="cuda")
        self.pin_ws = PinnedBuffer(pin_b)
        if slot_pool is None:
            slot_pool = torch.empty(max(cache_slots * self.layout.expert_bytes, 1), dtype=torch.uint8, device="cuda")
        self.slot_pool = slot_pool
        self.host_pool = host_pool
        hp_ptr = host_pool.ptr if isinstance(host_pool, PinnedBuffer) else int(host_pool)
        hp_bytes = host_pool.nbytes if isinstance(host_pool, PinnedBuffer) else int(host_pool_bytes)
        h = c_vp()
        torch.cuda.synchronize()
        check(lib().ec_create(ctypes.byref(self.cfg), self.dev_ws.data_ptr(), dev_b, self.pin_ws.ptr, pin_b, hp_ptr,
                              hp_bytes, slot_pool.data_ptr(), slot_pool.numel(), ctypes.byref(h)))
        self.handle = h.value
        self.copy_stream = torch.cuda.Stream() if prefill_max_tokens else None

    def set_bandwidth(self, bp, bh, stream=None):
        check(lib().ec_set_bandwidth(self.handle, bp, bh, _stream(stream)), self.handle)

    def calibrate_bandwidth(self, probe_experts=8, apply=True):
        """Measure (BP, BH) in MB/s on this machine; apply them when `apply`."""
        bp, bh = ctypes.c_uint32(), ctypes.c_uint32()
        check(lib().ec_calibrate_bandwidth(self.handle, probe_experts, 1 if apply else 0, ctypes.byref(bp),
                                           ctypes.byref(bh)), self.handle)
        return bp.value, bh.value

    def set_prefill_overlap(self, on):
        check(lib().ec_set_prefill_overlap(self.handle, 1 if on else 0), self.handle)

    def rebuild_slots(self, budget_bp):
        """(C, slot-pool bytes) that cache_rebuild chooses for budget_bp (ec_rebuild_slots)."""
        C, need = c_i32(), c_u64()
        check(lib().ec_rebuild_slots(self.handle, budget_bp, ctypes.byref(C), ctypes.byref(need)), self.handle)
        return C.value, need.value

    def rebuild(self, budget_bp, new_slot_pool=None):
        """cache_rebuild; returns the slot count the library chose (read back from its stats)."""
        import torch
        _, need = self.rebuild_slots(budget_bp)
        if new_slot_pool is None:
            if self.slot_pool.numel() >= need:
                new_slot_pool = self.slot_pool
            else:
                new_slot_pool = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        check(lib().cache_rebuild(self.handle, budget_bp, new_slot_pool.data_ptr(), new_slot_pool.numel()),
              self.handle)
        self.slot_pool = new_slot_pool
        return self.stats()["slots"]

    def kernel_timing(self, on):
        check(lib().ec_kernel_timing(self.handle, 1 if on else 0), self.handle)

    def kernel_time(self, kind, reset=False):
        """(total ms, launches) of one kernel kind ('ctl', 'fill', 'gate_up', 'down')."""
        ms, n = ctypes.c_double(), c_u64()
        check(lib().ec_kernel_time(self.handle, KERNEL_KINDS[kind], ctypes.byref(ms), ctypes.byref(n),
                                   1 if reset else 0), self.handle)
        return ms.value, n.value

    def host_branch_test_hooks(self, pause_host, wait_polls=0):
        """Test support: pause the host branch and/or bound the GPU's wait for it
        (ec_host_branch_test_hooks)."""
        check(lib().ec_host_branch_test_hooks(self.handle, 1 if pause_host else 0, int(wait_polls)), self.handle)

    def epoch(self):
        return lib().ec_epoch(self.handle)

    def stats(self, reset=False, allow_bad_ids=False):
        """Totals since creation (or the last reset). Raises ECError on a device error (a host-branch
        timeout, or a host-side pair in a step without the host branch), except that with
        allow_bad_ids the bad-expert-id bit alone is returned in device_error."""
        s = ec_stats()
        st = lib().ec_get_stats(self.handle, ctypes.byref(s), 1 if reset else 0)
        out = {f: getattr(s, f) for f, _ in ec_stats._fields_}
        if st != 0 and not (st == -7 and allow_bad_ids and out["device_error"] == 1):
            check(st, self.handle)
        return out

    def debug_state(self):
        import numpy as np
        LE = self.shape.layers * self.shape.experts
        C = self.stats(allow_bad_ids=True)["slots"]
        resid = np.empty(LE, np.int32)
        sk = np.empty(max(C, 1), np.int32)
        lru = np.empty(max(C, 1), np.uint64)
        clk = np.empty(1, np.uint64)
        check(lib().ec_debug_state(self.handle, resid.ctypes.data, sk.ctypes.data, lru.ctypes.data,
                                   clk.ctypes.data), self.handle)
        return resid, sk[:C], lru[:C], int(clk[0])

    def close(self):
        if getattr(self, "handle", None):
            lib().ec_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def hbm_read_probe(buf, burst_bytes, reps=100, queued=True, stream=None):
    """(median us, best us, bytes per burst) of one-shot HBM read bursts over a device tensor
    (ec_hbm_read_probe): queued behind a primer and run back to back, or each on an idle queue."""
    med, best, got = ctypes.c_double(), ctypes.c_double(), c_u64()
    check(lib().ec_hbm_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), burst_bytes, reps,
                                  1 if queued else 0, _stream(stream), ctypes.byref(med), ctypes.byref(best),
                                  ctypes.byref(got)))
    return med.value, best.value, got.value


def queue_delay(us, stream=None):
    """Hold `stream` for about `us` microseconds (ec_queue_delay), so that launches queued behind it
    run back to back."""
    check(lib().ec_queue_delay(_stream(stream), int(us)))


def memcpy_async(dst, src, nbytes, stream=None):
    """hipMemcpyAsync (default kind) between raw pointers on `stream` (plumbing for callers/tests)."""
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.argtypes = [c_vp, c_vp, ctypes.c_size_t, ctypes.c_int, c_vp]
    rc = hip.hipMemcpyAsync(c_vp(_ptr(dst)), c_vp(_ptr(src)), int(nbytes), 4, c_vp(_stream(stream)))
    if rc != 0:
        raise RuntimeError("hipMemcpyAsync failed with %d" % rc)
