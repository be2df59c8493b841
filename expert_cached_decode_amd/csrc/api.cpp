// C ABI of libexpert_cached_decode.so: context, workspace carving, argument
// checks and the enqueue order of each MoE layer step.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <algorithm>
#include <sched.h>
#include <thread>
#include <mutex>
#include <atomic>
#include <chrono>
#include <cstring>
#include <string>
#include <vector>

#include "ec_internal.h"
#include "bank_io.h"
#include "host_experts.h"
#include "prefill.h"

using namespace ec;

namespace {

thread_local std::string g_err; // last error of calls that have no context

uint64_t mailbox_ints(int n) { return 8 + 3ull * n + (4 - (3ull * n) % 4) % 4; }

constexpr int kDone = 32; // doorbell word the host writes (own 128-byte line)

} // namespace

struct ec_ctx {
    ec_config cfg{};
    ec_layout_info lay{};
    int L = 0, E = 0, k = 0, H = 0, I = 0, wdt = 0, Tmax = 0, Umax = 0, K = 0, C = 0, nmax = 0;
    int P = 0; // layers held by the host pool (layer l reads pool layer l % P)
    uint32_t bp = 0, bh = 1;
    bool host_branch = false;
    bool host_only = false;  // host pool not device-accessible: no fills, every miss on the host
    uint32_t* probe_sink = nullptr; // never written (link probe of the BP calibration)
    uint64_t epoch = 1;
    const uint8_t* host_pool = nullptr;     // host address
    const uint8_t* host_pool_dev = nullptr; // device address of the same memory
    uint64_t host_pool_bytes = 0;
    uint8_t* slot_pool = nullptr;
    uint64_t slot_pool_bytes = 0;
    DevState st{};
    StepBufs sb{};
    float* act = nullptr;
    // moe_decode_layer_static: the same step buffers laid over the library's static device scratch
    int device = 0;
    void* static_base = nullptr;  // device address of the scratch array on this context's device
    uint64_t static_bytes = 0;    // bytes of it this context's step buffers take
    std::string static_err;       // why the static variant is unavailable (empty when it is)
    StepBufs static_sb{};
    float* static_act = nullptr;
    StepBufs last_sb{};           // the buffers of the last step call (ec_last_step)
    float* gate_logits = nullptr; // [T_max][E] router logits of moe_decode_block
    // host branch: pinned mailbox, partial sums and doorbell, with their device-visible addresses
    int32_t* mb_pinned = nullptr;
    float* y_host_pinned = nullptr;
    uint32_t* doorbell = nullptr; // [0] mailbox sequence (GPU writes), [kDone] finished sequence (host writes)
    int32_t* mb_dev = nullptr;
    float* y_host_dev = nullptr;
    uint32_t* doorbell_dev = nullptr;
    hipStream_t side = nullptr;
    HostPool* pool = nullptr;
    std::mutex pool_mu;           // one host job at a time (poller, calibration)
    std::thread poller;
    // host-branch timing (guarded by pool_mu): jobs, time from the doorbell seen to the partial
    // sums published, and the handoff gaps between a job's publication and the next doorbell
    uint64_t host_jobs = 0, host_gaps = 0;
    double host_busy_us = 0, host_gap_us = 0;
    // test support for the host branch's failure path (ec_host_branch_test_hooks)
    std::atomic<bool> host_paused{false};
    uint32_t host_wait_polls = kHostWaitPolls;
    std::atomic<bool> stop{false};
    std::vector<float> host_act;
    HostJob job{};
    PrefillState pf{};
    int prefill_overlap = 1;
    // kernel timing (measurement support)
    struct Timer {
        std::vector<hipEvent_t> ev; // pairs: 2i start, 2i+1 end
        int used = 0;
        double total_ms = 0;
        uint64_t launches = 0;
    };
    bool timing = false;
    Timer timers[4];
    std::string err;
};

static constexpr int kTimerPairs = 1024;

static void host_branch_poll(ec_ctx* x);

// Host-branch threads by default (the polling thread works in the pool): the CPUs this process
// may run on less four (the caller's launch thread and slack for the rest of the process: the
// workers spin between jobs, and a pool that oversubscribes the CPUs loses most of its rate),
// 1 to 32. Measured on a 16-CPU host: 12 threads ran the measured-split decode 3% faster than 14.
static int default_host_threads() {
    cpu_set_t set;
    int n = 0;
    if (sched_getaffinity(0, sizeof(set), &set) == 0) n = CPU_COUNT(&set);
    if (n <= 0) n = (int)std::thread::hardware_concurrency();
    return std::max(1, std::min(32, n > 4 ? n - 4 : 1));
}

static void timers_free(ec_ctx* x);

static hipError_t timer_drain(ec_ctx::Timer& t) {
    for (int i = 0; i < t.used; ++i) {
        hipError_t e = hipEventSynchronize(t.ev[2 * i + 1]);
        if (e != hipSuccess) return e;
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, t.ev[2 * i], t.ev[2 * i + 1]);
        if (e != hipSuccess) return e;
        t.total_ms += ms;
        t.launches++;
    }
    t.used = 0;
    return hipSuccess;
}

// returns the event pair to bracket the next launch of a kernel kind (nullptr when timing is off)
static hipEvent_t* timer_next(ec_ctx* x, int kind) {
    if (!x->timing) return nullptr;
    ec_ctx::Timer& t = x->timers[kind];
    if (t.used == kTimerPairs && timer_drain(t) != hipSuccess) return nullptr;
    return &t.ev[2 * t.used++];
}

static ec_status fail(ec_ctx* ctx, ec_status s, const std::string& msg) {
    if (ctx) ctx->err = msg;
    g_err = msg;
    return s;
}

#define HIPCHK(ctx, call)                                                                      \
    do {                                                                                       \
        hipError_t e_ = (call);                                                                \
        if (e_ != hipSuccess)                                                                  \
            return fail(ctx, EC_EHIP, std::string(#call) + ": " + hipGetErrorString(e_));      \
    } while (0)

static ec_status check_shape(const ec_shape* s) {
    if (!s) return fail(nullptr, EC_EINVAL, "shape is NULL");
    if (s->layers < 1 || s->experts < 1 || s->experts > kMaxExperts)
        return fail(nullptr, EC_ESHAPE, "need layers >= 1 and 1 <= experts <= 4096");
    if (s->top_k < 1 || s->top_k > kMaxTopK || s->top_k > s->experts)
        return fail(nullptr, EC_ESHAPE, "need 1 <= top_k <= min(32, experts)");
    if (s->wdtype < EC_DT_F32 || s->wdtype > EC_DT_MXFP4) return fail(nullptr, EC_EUNSUP, "unknown wdtype");
    // a weight row of the decode GEMV is at most 8 KiB (f32 2048, bf16 4096, MXFP4 8192 elements)
    const int maxdim = s->wdtype == EC_DT_F32 ? 2048 : s->wdtype == EC_DT_BF16 ? 4096 : 8192;
    if (s->hidden < 64 || s->inter < 64 || s->hidden % 64 || s->inter % 64 || s->hidden > maxdim ||
        s->inter > maxdim)
        return fail(nullptr, EC_ESHAPE, "hidden and inter must be multiples of 64 within the dtype's limit");
    return EC_OK;
}

extern "C" {

const char* ec_strerror(ec_status s) {
    switch (s) {
    case EC_OK: return "ok";
    case EC_EINVAL: return "invalid argument";
    case EC_ESHAPE: return "unsupported or inconsistent shape";
    case EC_ENOSPC: return "caller buffer too small";
    case EC_EHIP: return "HIP runtime error";
    case EC_ESTATE: return "invalid state";
    case EC_EUNSUP: return "unsupported dtype or device";
    case EC_EDEVICE: return "device-side check failed";
    default: return "unknown status";
    }
}

const char* ec_last_error(const ec_ctx* ctx) { return ctx ? ctx->err.c_str() : g_err.c_str(); }

ec_status ec_layout(const ec_shape* s, ec_layout_info* o) {
    ec_status st = check_shape(s);
    if (st) return st;
    if (!o) return fail(nullptr, EC_EINVAL, "out is NULL");
    const uint64_t n = (uint64_t)s->hidden * s->inter;
    std::memset(o, 0, sizeof(*o));
    if (s->wdtype == EC_DT_MXFP4) {
        o->gate_off = 0; o->up_off = n / 2; o->down_off = n;
        o->gate_scale_off = 3 * n / 2; o->up_scale_off = 3 * n / 2 + n / 32; o->down_scale_off = 3 * n / 2 + 2 * n / 32;
        o->expert_bytes = 3 * n / 2 + 3 * n / 32;
    } else {
        const uint64_t es = s->wdtype == EC_DT_F32 ? 4 : 2;
        o->gate_off = 0; o->up_off = n * es; o->down_off = 2 * n * es;
        o->expert_bytes = 3 * n * es;
    }
    o->layer_bytes = o->expert_bytes * (uint64_t)s->experts;
    return EC_OK;
}

static ec_status check_config(const ec_config* c) {
    if (!c) return fail(nullptr, EC_EINVAL, "config is NULL");
    ec_status st = check_shape(&c->shape);
    if (st) return st;
    const auto& s = c->shape;
    if (c->max_tokens < 1 || c->max_tokens > 64 || c->max_tokens * s.top_k > kMaxPairs)
        return fail(nullptr, EC_ESHAPE, "need 1 <= max_tokens <= 64 and max_tokens * top_k <= 1024");
    if (c->cache_slots < 0 || (int64_t)c->cache_slots > (int64_t)s.layers * s.experts)
        return fail(nullptr, EC_EINVAL, "cache_slots must be in [0, layers * experts]");
    if (c->victim_k < 0 || c->victim_k > kMaxK) return fail(nullptr, EC_EINVAL, "victim_k must be in [0, 64]");
    if (c->bh_mbps < 1) return fail(nullptr, EC_EINVAL, "BH must be >= 1");
    if (c->host_threads < 0 || c->host_threads > 256) return fail(nullptr, EC_EINVAL, "host_threads in [0, 256]");
    if (c->prefill_max_tokens < 0 || c->prefill_max_tokens > (1 << 20))
        return fail(nullptr, EC_EINVAL, "prefill_max_tokens in [0, 2^20]");
    if (c->pool_layers < 0 || c->pool_layers > s.layers)
        return fail(nullptr, EC_EINVAL, "pool_layers must be in [0, layers]");
    if (c->prefill_max_tokens > 0 && s.wdtype == EC_DT_F32)
        return fail(nullptr, EC_EUNSUP, "prefill needs bf16 or MXFP4 expert weights");
    return EC_OK;
}

// The per-step buffers of a decode step (route, cache control, GEMV activations), carved from d.
static void carve_step(const ec_ctx* x, Carve& d, StepBufs& sb, float*& act) {
    const int n = x->nmax, U = x->Umax;
    sb.ids = d.take<int32_t>(n);
    sb.w = d.take<float>(n);
    sb.uniq = d.take<int32_t>(U);
    sb.counts = d.take<int32_t>(CNT_N);
    sb.pos = d.take<int32_t>(n);
    sb.cls = d.take<int32_t>(U);
    sb.slot = d.take<int32_t>(U);
    sb.fills = d.take<int32_t>(kMaxK);
    sb.victims = d.take<int32_t>(kMaxK);
    sb.evicted = d.take<int32_t>(kMaxK);
    sb.host_list = d.take<int32_t>(U);
    sb.rewritten = d.take<int32_t>(n);
    sb.gpu_desc = d.take<int4>(U);
    sb.tok_pairs = d.take<int32_t>(n);
    act = d.take<float>((uint64_t)n * x->I);
}

// Carve the device and pinned workspaces (base pointers may be NULL for sizing).
static void carve(ec_ctx* x, uint8_t* dev, uint8_t* pin, uint64_t* dev_bytes, uint64_t* pin_bytes) {
    const int LE = x->L * x->E;
    Carve d(dev);
    x->st.resid = d.take<int32_t>(LE);
    x->st.slot_key = d.take<int32_t>(LE);
    x->st.slot_lru = d.take<uint64_t>(LE);
    // the LRU clock, BP/BH, the mailbox sequences and the per-layer stats share one block, so
    // that the one-token control kernel reaches them from one pointer: clock at +0, bw[2] at +8,
    // hseq at +16, hseen at +20, stats [L][ST_N] from +32
    uint64_t* words = d.take<uint64_t>(4 + (uint64_t)x->L * ST_N);
    x->st.clock = words;
    x->st.bw = words ? reinterpret_cast<uint32_t*>(words + 1) : nullptr;
    x->st.hseq = words ? reinterpret_cast<uint32_t*>(words + 2) : nullptr;
    x->st.hseen = words ? reinterpret_cast<uint32_t*>(words + 2) + 1 : nullptr;
    x->st.stats = words ? reinterpret_cast<unsigned long long*>(words + 4) : nullptr;
    x->st.err = d.take<int32_t>(1);
    x->probe_sink = d.take<uint32_t>(4);
    const int n = x->nmax;
    carve_step(x, d, x->sb, x->act);
    x->gate_logits = d.take<float>((uint64_t)x->Tmax * x->E);
    const uint64_t xbytes = (uint64_t)x->Tmax * x->H * (x->wdt == EC_DT_F32 ? 4 : 2);
    const uint64_t mb_bytes = mailbox_ints(n) * 4 + xbytes;
    prefill_carve(x->pf, d, x->cfg.prefill_max_tokens, x->E, x->k, x->H, x->I, x->lay.layer_bytes);
    *dev_bytes = (d.off + 255) & ~255ull;
    Carve p(pin);
    x->doorbell = p.take<uint32_t>(2 * kDone);
    x->mb_pinned = p.take<int32_t>((mb_bytes + 3) / 4);
    x->y_host_pinned = p.take<float>((uint64_t)n * x->H);
    *pin_bytes = (p.off + 255) & ~255ull;
}

static void init_dims(ec_ctx* x, const ec_config* c) {
    x->cfg = *c;
    ec_layout(&c->shape, &x->lay);
    x->L = c->shape.layers; x->E = c->shape.experts; x->k = c->shape.top_k;
    x->H = c->shape.hidden; x->I = c->shape.inter; x->wdt = c->shape.wdtype;
    x->Tmax = c->max_tokens;
    x->nmax = c->max_tokens * x->k;
    x->Umax = x->nmax < x->E ? x->nmax : x->E;
    x->K = c->victim_k ? c->victim_k : (x->Umax < kMaxK ? x->Umax : kMaxK);
    x->C = c->cache_slots;
    x->P = c->pool_layers ? c->pool_layers : x->L;
    x->bp = c->bp_mbps; x->bh = c->bh_mbps;
}

static bool needs_host_branch(const ec_ctx* x) {
    // q = min(m, floor(m*BP/BH), K, C - h) equals m for every step iff BP >= BH, K >= U_max and C >= U_max
    return x->host_only || !(x->bp >= x->bh && x->K >= x->Umax && x->C >= x->Umax);
}

// BP as the device sees it: without a device-accessible host pool nothing can be
// filled, so the fill count is pinned to 0 (q = floor(m * 0 / BH)).
static uint32_t device_bp(const ec_ctx* x, uint32_t bp) { return x->host_only ? 0u : bp; }

ec_status ec_workspace_size(const ec_config* c, uint64_t* dev_bytes, uint64_t* pinned_bytes) {
    ec_status st = check_config(c);
    if (st) return st;
    if (!dev_bytes || !pinned_bytes) return fail(nullptr, EC_EINVAL, "NULL output");
    ec_ctx tmp;
    init_dims(&tmp, c);
    carve(&tmp, nullptr, nullptr, dev_bytes, pinned_bytes);
    return EC_OK;
}

ec_status ec_create(const ec_config* c, void* dev_ws, uint64_t dev_ws_bytes, void* pinned_ws,
                    uint64_t pinned_ws_bytes, const void* host_pool, uint64_t host_pool_bytes, void* slot_pool,
                    uint64_t slot_pool_bytes, ec_ctx** out) {
    ec_status st = check_config(c);
    if (st) return st;
    if (!out || !dev_ws || !pinned_ws || !host_pool) return fail(nullptr, EC_EINVAL, "NULL argument");
    if (((uintptr_t)dev_ws & 255) || ((uintptr_t)pinned_ws & 255))
        return fail(nullptr, EC_EINVAL, "workspaces must be 256-byte aligned");
    (void)hipGetLastError(); // an error left by an earlier, unrelated HIP call is not this call's
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return fail(nullptr, EC_EHIP, "no HIP device");
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(nullptr, EC_EUNSUP, std::string("needs gfx950, found ") + prop.gcnArchName);
    ec_ctx* x = new ec_ctx();
    init_dims(x, c);
    uint64_t need_dev = 0, need_pin = 0;
    carve(x, nullptr, nullptr, &need_dev, &need_pin);
    if (dev_ws_bytes < need_dev || pinned_ws_bytes < need_pin) {
        delete x;
        return fail(nullptr, EC_ENOSPC, "workspace too small");
    }
    if (host_pool_bytes < x->lay.layer_bytes * x->P) {
        delete x;
        return fail(nullptr, EC_ENOSPC, "host pool smaller than pool_layers * experts * expert_bytes");
    }
    if ((uint64_t)x->C * x->lay.expert_bytes > slot_pool_bytes || (x->C > 0 && !slot_pool)) {
        delete x;
        return fail(nullptr, EC_ENOSPC, "slot pool smaller than cache_slots * expert_bytes");
    }
    carve(x, (uint8_t*)dev_ws, (uint8_t*)pinned_ws, &need_dev, &need_pin);
    x->last_sb = x->sb;
    x->device = dev;
    {
        // the static variant's step buffers: the same layout over the library's device scratch
        Carve sz(nullptr);
        StepBufs tmp{};
        float* tmp_act = nullptr;
        carve_step(x, sz, tmp, tmp_act);
        x->static_bytes = (sz.off + 255) & ~255ull;
        hipError_t e = hipSuccess;
        void* base = static_scratch_ptr(dev, &e);
        if (!base) {
            (void)hipGetLastError();
            x->static_err = std::string("static device scratch unavailable: ") + hipGetErrorString(e);
        } else if (x->static_bytes > kStaticScratchBytes) {
            x->static_err = "the step buffers of this context need " + std::to_string(x->static_bytes) +
                            " bytes; the static device scratch holds " + std::to_string(kStaticScratchBytes);
        } else {
            x->static_base = base;
            Carve sc((uint8_t*)base);
            carve_step(x, sc, x->static_sb, x->static_act);
        }
    }
    void* ws_dev = nullptr;
    if (hipHostGetDevicePointer(&ws_dev, pinned_ws, 0) != hipSuccess || !ws_dev) {
        (void)hipGetLastError();
        delete x;
        return fail(nullptr, EC_EINVAL, "pinned_ws must be pinned, device-accessible memory (hipHostMalloc)");
    }
    {
        auto dev_of = [&](const void* hp) {
            return (uint8_t*)ws_dev + ((const uint8_t*)hp - (const uint8_t*)pinned_ws);
        };
        x->mb_dev = (int32_t*)dev_of(x->mb_pinned);
        x->y_host_dev = (float*)dev_of(x->y_host_pinned);
        x->doorbell_dev = (uint32_t*)dev_of(x->doorbell);
        std::memset(x->doorbell, 0, 2 * kDone * sizeof(uint32_t));
    }
    void* pdev = nullptr;
    if (hipHostGetDevicePointer(&pdev, const_cast<void*>(host_pool), 0) != hipSuccess || !pdev) {
        // ordinary (pageable) memory, e.g. when pinning the bank failed: run host-only
        (void)hipGetLastError();
        pdev = nullptr;
        x->host_only = true;
    }
    x->host_pool = (const uint8_t*)host_pool;
    x->host_pool_dev = (const uint8_t*)pdev;
    x->host_pool_bytes = host_pool_bytes;
    x->slot_pool = (uint8_t*)slot_pool;
    x->slot_pool_bytes = slot_pool_bytes;
    x->host_branch = needs_host_branch(x);
    if (hipStreamCreateWithFlags(&x->side, hipStreamNonBlocking) != hipSuccess) {
        delete x;
        return fail(nullptr, EC_EHIP, "stream creation failed");
    }
    if (prefill_init(x->pf) != hipSuccess) {
        delete x;
        return fail(nullptr, EC_EHIP, "prefill event creation failed");
    }
    // initial device state: cold cache, clock 0, zero stats / flags / counters
    hipStream_t s = x->side;
    launch_fill_i32((int32_t*)x->st.clock, 0, 2, s);
    launch_fill_i32(x->st.err, 0, 1, s);
    launch_fill_i32((int32_t*)x->st.stats, 0, 2ll * x->L * ST_N, s);
    launch_fill_i32((int32_t*)x->sb.gpu_desc, 0, 4ll * x->Umax, s);
    launch_fill_i32(x->sb.counts, 0, CNT_N, s);
    launch_fill_i32((int32_t*)x->st.hseq, 0, 1, s);
    launch_fill_i32((int32_t*)x->st.hseen, 0, 1, s);
    launch_reset_cache(x->st, x->L, x->E, x->C, s);
    launch_set_bw(x->st.bw, device_bp(x, x->bp), x->bh, s);
    prefill_reset_device(x->pf, s);
    hipError_t e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) {
        std::string m = std::string("initialisation failed: ") + hipGetErrorString(e);
        delete x;
        return fail(nullptr, EC_EHIP, m);
    }
    x->pool = host_pool_create(c->host_threads ? c->host_threads : default_host_threads());
    x->host_act.resize((size_t)x->nmax * x->I);
    x->poller = std::thread(host_branch_poll, x);
    *out = x;
    return EC_OK;
}

ec_status ec_destroy(ec_ctx* x) {
    if (!x) return fail(nullptr, EC_EINVAL, "ctx is NULL");
    (void)hipDeviceSynchronize();
    x->stop.store(true);
    if (x->poller.joinable()) x->poller.join();
    if (x->pool) host_pool_destroy(x->pool);
    timers_free(x);
    prefill_destroy(x->pf);
    if (x->side) (void)hipStreamDestroy(x->side);
    delete x;
    return EC_OK;
}

ec_status ec_set_bandwidth(ec_ctx* x, uint32_t bp, uint32_t bh, void* stream) {
    if (!x) return fail(nullptr, EC_EINVAL, "ctx is NULL");
    if (bh < 1) return fail(x, EC_EINVAL, "BH must be >= 1");
    launch_set_bw(x->st.bw, device_bp(x, bp), bh, (hipStream_t)stream);
    HIPCHK(x, hipGetLastError());
    x->bp = bp;
    x->bh = bh;
    const bool hb = needs_host_branch(x);
    if (hb != x->host_branch) { x->host_branch = hb; x->epoch++; }
    return EC_OK;
}

ec_status moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* ids, float* w, void* stream) {
    if (T < 0 || E < 1 || E > kMaxExperts || k < 1 || k > kMaxTopK || k > E)
        return fail(nullptr, EC_EINVAL, "need T >= 0, 1 <= E <= 4096, 1 <= k <= min(32, E)");
    if (T == 0) return EC_OK;
    if (!logits || !ids || !w) return fail(nullptr, EC_EINVAL, "NULL pointer");
    launch_route(logits, T, E, k, ids, w, (hipStream_t)stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(nullptr, EC_EHIP, hipGetErrorString(e));
    return EC_OK;
}

static CtlArgs ctl_args(ec_ctx* x, int layer, int T) {
    CtlArgs a{};
    a.st = x->st;
    a.sb = x->sb;
    a.layer = layer; a.E = x->E; a.k = x->k; a.T = T; a.C = x->C; a.K = x->K;
    return a;
}

static void fill_view(ec_ctx* x, ec_step_view* v) {
    if (!v) return;
    const StepBufs& b = x->last_sb;
    v->uniq = b.uniq; v->counts = b.counts; v->pos = b.pos; v->cls = b.cls;
    v->slot = b.slot; v->fills = b.fills; v->victims = b.victims; v->evicted = b.evicted;
    v->host_list = b.host_list; v->rewritten = b.rewritten;
}

ec_status expert_cache_step(ec_ctx* x, int32_t layer, const int32_t* ids, int32_t T, ec_step_view* out,
                            void* stream) {
    if (!x) return fail(nullptr, EC_EINVAL, "ctx is NULL");
    if (layer < 0 || layer >= x->L) return fail(x, EC_EINVAL, "layer out of range");
    if (T < 1 || T > x->Tmax) return fail(x, EC_EINVAL, "need 1 <= T <= max_tokens");
    if (!ids) return fail(x, EC_EINVAL, "ids is NULL");
    CtlArgs a = ctl_args(x, layer, T);
    a.ids_in = ids;
    launch_ctl(a, (hipStream_t)stream);
    HIPCHK(x, hipGetLastError());
    x->last_sb = x->sb;
    fill_view(x, out);
    return EC_OK;
}

ec_status ec_last_step(const ec_ctx* x, ec_step_view* out) {
    if (!x || !out) return fail(nullptr, EC_EINVAL, "ctx and out must be non-NULL");
    fill_view(const_cast<ec_ctx*>(x), out);
    return EC_OK;
}

// Host branch ("Bandwidth-adaptive execution": misses left to the host are computed
// there in place). The cache-control kernel writes a mailbox into pinned memory and
// rings the doorbell with a new sequence number; this thread polls the doorbell,
// computes the host-list experts from the host pool, writes their partial sums into
// pinned memory and publishes the finished sequence number, which the down GEMV
// waits for before merging. No runtime callbacks or copies are on the step's path,
// so a captured step is kernels only.
static void host_branch_run(ec_ctx* x) {
    const int32_t* mb = x->mb_pinned;
    const int T = mb[6], layer = mb[7], nhost = mb[CNT_HOST];
    const int n = T * x->k;
    HostJob& j = x->job;
    j.n_experts = nhost;
    for (int h = 0; h < nhost; ++h)
        j.expert_base[h] = x->host_pool + ((uint64_t)(layer % x->P) * x->E + mb[CNT_N + h]) * x->lay.expert_bytes;
    j.rewritten = mb + CNT_N + n;
    j.T = T; j.k = x->k; j.H = x->H; j.I = x->I; j.wdtype = x->wdt;
    j.x = mb + mailbox_ints(n);
    j.y = x->y_host_pinned;
    j.act = x->host_act.data();
    host_pool_run(x->pool, j);
}

static inline void cpu_relax() { __builtin_ia32_pause(); }

static void host_branch_poll(ec_ctx* x) {
    using clk = std::chrono::steady_clock;
    uint32_t last = 0;
    auto active = clk::now();
    bool have_done = false;
    while (!x->stop.load(std::memory_order_relaxed)) {
        const uint32_t sq = __atomic_load_n(&x->doorbell[0], __ATOMIC_ACQUIRE);
        if (sq != last && !x->host_paused.load(std::memory_order_acquire)) {
            const auto t0 = clk::now();
            {
                std::lock_guard<std::mutex> lk(x->pool_mu);
                host_branch_run(x);
                __atomic_store_n(&x->doorbell[kDone], sq, __ATOMIC_RELEASE);
                const auto t1 = clk::now();
                x->host_jobs++;
                x->host_busy_us += std::chrono::duration<double, std::micro>(t1 - t0).count();
                // a doorbell within 1 ms of the previous publication: a handoff of the decode loop
                // (the GPU saw the sums, finished the layer step and rang for the next one)
                const double gap = std::chrono::duration<double, std::micro>(t0 - active).count();
                if (have_done && gap < 1000.0) { x->host_gaps++; x->host_gap_us += gap; }
                active = t1;
            }
            have_done = true;
            last = sq;
            continue;
        }
        // spin while steps are arriving (a few pauses between reads of the doorbell line, which
        // stays in this core's cache until the GPU writes it), back off when idle
        if (std::chrono::steady_clock::now() - active < std::chrono::milliseconds(20)) {
            for (int i = 0; i < 4; ++i) cpu_relax();
        } else {
            std::this_thread::sleep_for(std::chrono::microseconds(50));
        }
    }
}

static ec_status decode_layer(ec_ctx* x, int32_t layer, const void* xin, const float* logits, int32_t T, void* out,
                              hipStream_t s, int residual, const StepBufs& sb, float* act);

ec_status moe_decode_layer(ec_ctx* x, int32_t layer, const void* xin, const float* logits, int32_t T, void* out,
                           void* stream) {
    if (!x) return fail(nullptr, EC_EINVAL, "ctx is NULL");
    if (layer < 0 || layer >= x->L) return fail(x, EC_EINVAL, "layer out of range");
    if (T < 1 || T > x->Tmax) return fail(x, EC_EINVAL, "need 1 <= T <= max_tokens");
    if (!xin || !logits || !out) return fail(x, EC_EINVAL, "NULL pointer");
    return decode_layer(x, layer, xin, logits, T, out, (hipStream_t)stream, 0, x->sb, x->act);
}

ec_status moe_decode_layer_static(ec_ctx* x, int32_t layer, const void* xin, const float* logits, int32_t T, void* out,
                                  void* stream) {
    if (!x) return fail(nullptr, EC_EINVAL, "ctx is NULL");
    if (layer < 0 || layer >= x->L) return fail(x, EC_EINVAL, "layer out of range");
    if (T < 1 || T > x->Tmax) return fail(x, EC_EINVAL, "need 1 <= T <= max_tokens");
    if (!xin || !logits || !out) return fail(x, EC_EINVAL, "NULL pointer");
    if (!x->static_base) return fail(x, x->static_bytes > kStaticScratchBytes ? EC_ENOSPC : EC_EHIP, x->static_err);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != x->device)
        return fail(x, EC_ESTATE, "the current device is not the context's device");
    hipStream_t s = (hipStream_t)stream;
    static_scratch_clear_once(x->device, x->static_base, s);
    HIPCHK(x, hipGetLastError());
    return decode_layer(x, layer, xin, logits, T, out, s, 0, x->static_sb, x->static_act);
}

ec_status moe_gate_logits(const void* w_router, const void* xin, int32_t x_dtype, int32_t T, int32_t E, int32_t H,
                          float* logits, void* stream) {
    if (!w_router || !xin || !logits) return fail(nullptr, EC_EINVAL, "NULL pointer");
    if (x_dtype != EC_DT_F32 && x_dtype != EC_DT_BF16) return fail(nullptr, EC_EINVAL, "x_dtype must be f32 or bf16");
    const int maxh = x_dtype == EC_DT_F32 ? 2048 : 4096;
    if (T < 0 || E < 1 || E > kMaxExperts || H < 64 || H % 64 || H > maxh)
        return fail(nullptr, EC_EINVAL, "need T >= 0, 1 <= E <= 4096, H a multiple of 64 within the dtype's limit");
    launch_gate(w_router, xin, x_dtype == EC_DT_F32, T, E, H, logits, (hipStream_t)stream);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? EC_OK : fail(nullptr, EC_EHIP, hipGetErrorString(e));
}

ec_status moe_decode_block(ec_ctx* x, int32_t layer, const void* xin, const void* w_router, int32_t T, void* out,
                           void* stream) {
    if (!x) return fail(nullptr, EC_EINVAL, "ctx is NULL");
    if (layer < 0 || layer >= x->L) return fail(x, EC_EINVAL, "layer out of range");
    if (T < 1 || T > x->Tmax) return fail(x, EC_EINVAL, "need 1 <= T <= max_tokens");
    if (!xin || !w_router || !out) return fail(x, EC_EINVAL, "NULL pointer");
    if (out == xin) return fail(x, EC_EINVAL, "out must not alias x");
    hipStream_t s = (hipStream_t)stream;
    launch_gate(w_router, xin, x->wdt == EC_DT_F32, T, x->E, x->H, x->gate_logits, s);
    HIPCHK(x, hipGetLastError());
    return decode_layer(x, layer, xin, x->gate_logits, T, out, s, 1, x->sb, x->act);
}

static ec_status decode_layer(ec_ctx* x, int32_t layer, const void* xin, const float* logits, int32_t T, void* out,
                              hipStream_t s, int residual, const StepBufs& sb, float* act) {
    const uint64_t xbytes = (uint64_t)T * x->H * (x->wdt == EC_DT_F32 ? 4 : 2);
    CtlArgs a = ctl_args(x, layer, T);
    a.sb = sb;
    a.logits = logits;
    a.x = xin;
    a.x_bytes = (int32_t)xbytes;
    a.host_branch = x->host_branch ? 1 : 0;
    a.sb.mailbox = x->mb_dev;
    a.doorbell = x->doorbell_dev;
    // with kernel timing on, each kernel stamps its timer pair from its own dispatch
    launch_ctl(a, s, timer_next(x, 0));
    HIPCHK(x, hipGetLastError());
    x->last_sb = sb;
    DecodeArgs d{};
    d.pool = x->host_pool_dev; d.slots = x->slot_pool; d.counts = sb.counts; d.fills = sb.fills;
    d.victims = sb.victims; d.gpu_desc = sb.gpu_desc;
    d.tok_pairs = sb.tok_pairs; d.rewritten = sb.rewritten; d.w = sb.w;
    d.x = xin; d.act = act; d.y_host = x->y_host_dev;
    d.out = out; d.expert_bytes = x->lay.expert_bytes;
    d.layer = layer % x->P; d.E = x->E; d.k = x->k; d.T = T; d.H = x->H; d.I = x->I; d.wdtype = x->wdt; d.U_max = x->Umax;
    d.host_pairs = x->host_branch ? 1 : 0;
    d.host_done = x->doorbell_dev + kDone; d.hseq = x->st.hseq; d.hseen = x->st.hseen; d.err = x->st.err;
    d.residual = residual;
    d.wait_polls = x->host_wait_polls;
    if (x->C > 0 && !x->host_only) launch_fill(d, x->K, s, timer_next(x, 1));
    launch_gu(d, s, timer_next(x, 2));
    HIPCHK(x, hipGetLastError());
    launch_down(d, s, timer_next(x, 3));
    HIPCHK(x, hipGetLastError());
    return EC_OK;
}

static void timers_free(ec_ctx* x) {
    for (auto& t : x->timers) {
        for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
        t.ev.clear();
        t.used = 0;
    }
}

ec_status ec_kernel_timing(ec_ctx* x, int32_t on) {
    if (!x) return fail(nullptr, EC_EINVAL, "ctx is NULL");
    if (on && !x->timing) {
        for (auto& t : x->timers) {
            t.ev.resize(2 * kTimerPairs);
            for (auto& e : t.ev) HIPCHK(x, hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
            t.used = 0; t.total_ms = 0; t.launches = 0;
        }
        x->timing = true;
    } else if (!on && x->timing) {
        HIPCHK(x, hipDeviceSynchronize());
        for (auto& t : x->timers) HIPCHK(x, timer_drain(t));
        timers_free(x);
        x->timing = false;
    }
    return EC_OK;
}

ec_status ec_kernel_time(ec_ctx* x, int32_t kind, double* total_ms, uint64_t* launches, int32_t reset) {
    if (!x || kind < 0 || kind > 3 || !total_ms || !launches) return fail(x, EC_EINVAL, "bad argument");
    ec_ctx::Timer& t = x->timers[kind];
    if (x->timing) HIPCHK(x, timer_drain(t));
    *total_ms = t.total_ms;
    *launches = t.launches;
    if (reset) { t.total_ms = 0; t.launches = 0; }
    return EC_OK;
}

static hipError_t wall_clock_khz(int* khz) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev);
    if (e == hipSuccess && *khz <= 0) e = hipErrorInvalidValue;
    return e;
}

ec_status ec_queue_delay(void* stream, uint32_t us) {
    if (us > 1000000) return fail(nullptr, EC_EINVAL, "need us <= 1000000");
    int khz = 0;
    hipError_t e = wall_clock_khz(&khz);
    if (e == hipSuccess) {
        launch_queue_delay((uint64_t)us * (uint64_t)khz / 1000u, (hipStream_t)stream);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return fail(nullptr, EC_EHIP, std::string("queue delay: ") + hipGetErrorString(e));
    return EC_OK;
}

ec_status ec_hbm_read_probe(const void* dev_buf, uint64_t buf_bytes, uint64_t burst_bytes, int32_t reps, int32_t queued,
                            void* stream, double* median_us, double* best_us, uint64_t* bytes_read) {
    if (!dev_buf || reps < 1 || reps > 1000) return fail(nullptr, EC_EINVAL, "need a buffer and 1 <= reps <= 1000");
    if (burst_bytes < (1u << 20) || burst_bytes > buf_bytes / 4)
        return fail(nullptr, EC_EINVAL, "need 1 MiB <= burst_bytes <= buf_bytes / 4");
    hipStream_t s = (hipStream_t)stream;
    const int n = reps + 8; // 8 untimed bursts first
    std::vector<hipEvent_t> ev;
    hipError_t e = hipSuccess;
    for (int i = 0; i < 2 * n && e == hipSuccess; ++i) {
        hipEvent_t v;
        e = hipEventCreate(&v);
        if (e == hipSuccess) ev.push_back(v);
    }
    uint64_t off = 0, got = 0;
    const uint64_t stride = (burst_bytes + (1ull << 20)) & ~((1ull << 20) - 1); // distinct, 1 MiB aligned
    if (queued && e == hipSuccess) {
        // the host queues every burst while the primer holds the stream (about 25 us per launch)
        int khz = 0;
        e = wall_clock_khz(&khz);
        if (e == hipSuccess) {
            launch_queue_delay((2000ull + 25ull * n) * (uint64_t)khz / 1000u, s);
            e = hipGetLastError();
        }
    }
    for (int r = 0; r < n && e == hipSuccess; ++r) {
        if (off + stride > buf_bytes) off = 0;
        got = launch_hbm_burst((const uint8_t*)dev_buf + off, burst_bytes, s, &ev[2 * r]);
        e = hipGetLastError();
        if (e == hipSuccess && !queued) e = hipEventSynchronize(ev[2 * r + 1]);
        off += stride;
    }
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    std::vector<float> ms;
    for (int r = 8; r < n && e == hipSuccess; ++r) {
        float t = 0.f;
        e = hipEventElapsedTime(&t, ev[2 * r], ev[2 * r + 1]);
        ms.push_back(t);
    }
    for (hipEvent_t v : ev) (void)hipEventDestroy(v);
    if (e != hipSuccess) return fail(nullptr, EC_EHIP, std::string("hbm probe: ") + hipGetErrorString(e));
    std::sort(ms.begin(), ms.end());
    if (median_us) *median_us = 1e3 * ms[ms.size() / 2];
    if (best_us) *best_us = 1e3 * ms[0];
    if (bytes_read) *bytes_read = got;
    return EC_OK;
}

ec_status ec_host_branch_test_hooks(ec_ctx* x, int32_t pause_host, uint32_t wait_polls) {
    if (!x) return fail(nullptr, EC_EINVAL, "ctx is NULL");
    x->host_wait_polls = wait_polls ? wait_polls : kHostWaitPolls;
    x->host_paused.store(pause_host != 0, std::memory_order_release);
    return EC_OK;
}

ec_status ec_set_prefill_overlap(ec_ctx* x, int32_t on) {
    if (!x) return fail(nullptr, EC_EINVAL, "ctx is NULL");
    x->prefill_overlap = on ? 1 : 0;
    return EC_OK;
}

ec_status moe_prefill_layer(ec_ctx* x, int32_t layer, const void* xin, const float* logits, int32_t T, void* out,
                            void* compute_stream, void* copy_stream) {
    if (!x) return fail(nullptr, EC_EINVAL, "ctx is NULL");
    if (x->cfg.prefill_max_tokens <= 0) return fail(x, EC_ESTATE, "context created without prefill buffers");
    if (layer < 0 || layer >= x->L) return fail(x, EC_EINVAL, "layer out of range");
    if (T < 1 || T > x->cfg.prefill_max_tokens) return fail(x, EC_EINVAL, "need 1 <= T <= prefill_max_tokens");
    if (!xin || !logits || !out) return fail(x, EC_EINVAL, "NULL pointer");
    PrefillCall c{};
    c.host_pool = x->host_pool;
    c.P = x->P;
    c.layer = layer; c.L = x->L; c.E = x->E; c.k = x->k; c.H = x->H; c.I = x->I; c.T = T; c.wdtype = x->wdt;
    c.layer_bytes = x->lay.layer_bytes; c.expert_bytes = x->lay.expert_bytes;
    c.x = xin; c.logits = logits; c.out = out;
    c.compute = (hipStream_t)compute_stream; c.copy = (hipStream_t)copy_stream;
    c.overlap = x->prefill_overlap;
    hipError_t e = prefill_layer(x->pf, c);
    if (e != hipSuccess) return fail(x, EC_EHIP, std::string("prefill: ") + hipGetErrorString(e));
    return EC_OK;
}

ec_status cache_rebuild(ec_ctx* x, int32_t budget_bp, void* new_slot_pool, uint64_t bytes) {
    if (!x) return fail(nullptr, EC_EINVAL, "ctx is NULL");
    int32_t C = 0;
    uint64_t need = 0;
    if (ec_rebuild_slots(x, budget_bp, &C, &need)) return fail(x, EC_EINVAL, "budget_bp must be in [0, 10000]");
    if (need > bytes || (C > 0 && !new_slot_pool))
        return fail(x, EC_ENOSPC, "new slot pool smaller than C * expert_bytes");
    HIPCHK(x, hipDeviceSynchronize()); // safe point: nothing of this context in flight
    x->C = C;
    x->slot_pool = (uint8_t*)new_slot_pool;
    x->slot_pool_bytes = bytes;
    launch_reset_cache(x->st, x->L, x->E, x->C, x->side);
    HIPCHK(x, hipStreamSynchronize(x->side));
    HIPCHK(x, hipGetLastError());
    x->host_branch = needs_host_branch(x);
    x->epoch++;
    return EC_OK;
}

ec_status ec_calibrate_bandwidth(ec_ctx* x, int32_t probe_experts, int32_t apply, uint32_t* bp_out,
                                 uint32_t* bh_out) {
    if (!x) return fail(nullptr, EC_EINVAL, "ctx is NULL");
    constexpr int kReps = 3; // timed passes after one warm-up; every pass reads different experts
    if (probe_experts < 1 || probe_experts * (kReps + 1) > x->E)
        return fail(x, EC_EINVAL, "need 1 <= probe_experts <= experts / 4");
    HIPCHK(x, hipDeviceSynchronize()); // safe point
    const uint64_t eb = x->lay.expert_bytes, bytes = (uint64_t)probe_experts * eb;
    // BP: the fill path's source side, experts of pool layer 0 read over the link
    double bp = 0.0;
    if (!x->host_only) {
        hipEvent_t e0, e1;
        HIPCHK(x, hipEventCreate(&e0));
        if (hipEventCreate(&e1) != hipSuccess) {
            (void)hipEventDestroy(e0);
            return fail(x, EC_EHIP, "event creation failed");
        }
        double best_ms = 1e30;
        hipError_t e = hipSuccess;
        for (int r = 0; r <= kReps && e == hipSuccess; ++r) { // pass 0 warms the mapping up
            const uint8_t* src = x->host_pool_dev + (uint64_t)r * bytes; // experts [r n, (r+1) n) of layer 0
            e = hipEventRecord(e0, x->side);
            if (e == hipSuccess) { launch_link_probe(src, bytes, x->probe_sink, x->side); e = hipGetLastError(); }
            if (e == hipSuccess) e = hipEventRecord(e1, x->side);
            if (e == hipSuccess) e = hipEventSynchronize(e1);
            float ms = 0.f;
            if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
            if (e == hipSuccess && r > 0 && ms > 0.f && ms < best_ms) best_ms = ms;
        }
        (void)hipEventDestroy(e0);
        (void)hipEventDestroy(e1);
        if (e != hipSuccess) return fail(x, EC_EHIP, std::string("link probe: ") + hipGetErrorString(e));
        bp = bytes / (best_ms * 1e-3) / 1e6;
    }
    // BH: the host branch itself on experts of the last pool layer (each pass on experts
    // not read before, so they come from memory, not from the host's caches), zero input
    double bh = 0.0;
    {
        // a pass runs the host branch on probe_experts experts, as host jobs of at most
        // max_tokens * top_k experts (the most one step can hand over), one token per expert
        HostJob j{};
        const int per = std::min(probe_experts, x->nmax);
        const uint8_t* layer_base = x->host_pool + (uint64_t)(x->P - 1) * x->lay.layer_bytes;
        std::vector<int32_t> rw(per);
        for (int i = 0; i < per; ++i) rw[i] = -(1 + i);
        std::vector<uint8_t> xz((size_t)per * x->H * 4, 0);
        std::vector<float> ysink((size_t)per * x->H);
        j.rewritten = rw.data(); j.T = per; j.k = 1; j.H = x->H; j.I = x->I; j.wdtype = x->wdt;
        j.x = xz.data(); j.y = ysink.data(); j.act = x->host_act.data();
        double best_s = 1e30;
        std::lock_guard<std::mutex> lk(x->pool_mu);
        for (int r = 0; r <= kReps; ++r) {
            const auto t0 = std::chrono::steady_clock::now();
            for (int done = 0; done < probe_experts; done += per) {
                j.n_experts = std::min(per, probe_experts - done);
                for (int i = 0; i < j.n_experts; ++i)
                    j.expert_base[i] = layer_base + (uint64_t)(x->E - 1 - r * probe_experts - done - i) * eb;
                host_pool_run(x->pool, j);
            }
            const double sec = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
            if (r > 0 && sec > 0.0 && sec < best_s) best_s = sec;
        }
        bh = bytes / best_s / 1e6;
    }
    const uint32_t bpi = (uint32_t)std::min(bp, 4.0e9), bhi = (uint32_t)std::max(1.0, std::min(bh, 4.0e9));
    if (bp_out) *bp_out = bpi;
    if (bh_out) *bh_out = bhi;
    if (apply) {
        ec_status st = ec_set_bandwidth(x, bpi, bhi, x->side);
        if (st) return st;
        HIPCHK(x, hipStreamSynchronize(x->side));
    }
    return EC_OK;
}

static ec_status bank_args(const ec_shape* shape, int32_t pool_layers, uint64_t* expert_bytes, uint64_t* bank_bytes,
                           int32_t dims[6]) {
    ec_status st = check_shape(shape);
    if (st) return st;
    if (pool_layers < 1 || pool_layers > shape->layers)
        return fail(nullptr, EC_EINVAL, "need 1 <= pool_layers <= layers");
    ec_layout_info lay;
    ec_layout(shape, &lay);
    *expert_bytes = lay.expert_bytes;
    *bank_bytes = lay.layer_bytes * (uint64_t)pool_layers;
    dims[0] = shape->layers; dims[1] = shape->experts; dims[2] = shape->top_k;
    dims[3] = shape->hidden; dims[4] = shape->inter; dims[5] = shape->wdtype;
    return EC_OK;
}

ec_status ec_bank_write(const char* path, const ec_shape* shape, int32_t pool_layers, const void* bank, uint64_t bytes) {
    if (!path || !bank) return fail(nullptr, EC_EINVAL, "NULL argument");
    uint64_t eb = 0, need = 0;
    int32_t dims[6];
    ec_status st = bank_args(shape, pool_layers, &eb, &need, dims);
    if (st) return st;
    if (bytes < need) return fail(nullptr, EC_ENOSPC, "bank smaller than pool_layers * experts * expert_bytes");
    std::string err;
    if (bank_write(path, dims, pool_layers, eb, bank, need, &err) != 0) return fail(nullptr, EC_EINVAL, err);
    return EC_OK;
}

ec_status ec_bank_read(const char* path, const ec_shape* shape, int32_t pool_layers, void* dst, uint64_t dst_bytes,
                       int32_t threads, int32_t* direct_io, double* seconds) {
    if (!path || !dst) return fail(nullptr, EC_EINVAL, "NULL argument");
    uint64_t eb = 0, need = 0;
    int32_t dims[6];
    ec_status st = bank_args(shape, pool_layers, &eb, &need, dims);
    if (st) return st;
    if (dst_bytes < need) return fail(nullptr, EC_ENOSPC, "destination smaller than the bank");
    std::string err;
    int direct = 0;
    const int r = bank_read(path, dims, pool_layers, eb, dst, need, threads > 0 ? threads : 16, &direct, seconds, &err);
    if (r == -2) return fail(nullptr, EC_ESHAPE, err);
    if (r != 0) return fail(nullptr, EC_EINVAL, err);
    if (direct_io) *direct_io = direct;
    return EC_OK;
}

uint64_t ec_epoch(const ec_ctx* x) { return x ? x->epoch : 0; }

ec_status ec_get_stats(ec_ctx* x, ec_stats* o, int32_t reset) {
    if (!x || !o) return fail(x, EC_EINVAL, "NULL argument");
    HIPCHK(x, hipDeviceSynchronize());
    std::vector<unsigned long long> st((size_t)x->L * ST_N);
    HIPCHK(x, hipMemcpy(st.data(), x->st.stats, st.size() * 8, hipMemcpyDeviceToHost));
    int32_t err = 0;
    uint64_t clk = 0;
    HIPCHK(x, hipMemcpy(&err, x->st.err, 4, hipMemcpyDeviceToHost));
    HIPCHK(x, hipMemcpy(&clk, x->st.clock, 8, hipMemcpyDeviceToHost));
    std::memset(o, 0, sizeof(*o));
    for (int l = 0; l < x->L; ++l) {
        const unsigned long long* s = st.data() + (size_t)l * ST_N;
        o->steps += s[ST_STEPS]; o->hits += s[ST_HITS]; o->misses += s[ST_MISSES];
        o->fills += s[ST_FILLS]; o->host += s[ST_HOST]; o->evictions += s[ST_EVICT];
    }
    o->device_error = err;
    o->slots = x->C;
    o->clock = clk;
    o->host_only = x->host_only ? 1 : 0;
    o->host_branch = x->host_branch ? 1 : 0;
    {
        std::lock_guard<std::mutex> lk(x->pool_mu);
        o->host_jobs = x->host_jobs;
        o->host_busy_us = x->host_busy_us;
        o->host_gaps = x->host_gaps;
        o->host_gap_us = x->host_gap_us;
        if (reset) { x->host_jobs = 0; x->host_busy_us = 0; x->host_gaps = 0; x->host_gap_us = 0; }
    }
    if (reset) {
        launch_fill_i32((int32_t*)x->st.stats, 0, 2ll * x->L * ST_N, x->side);
        HIPCHK(x, hipStreamSynchronize(x->side));
    }
    if (err & 2) return fail(x, EC_EDEVICE, "the host branch did not deliver its partial sums in time");
    if (err & 4)
        return fail(x, EC_EDEVICE, "a host-side expert reached a step compiled without the host branch "
                                   "(a graph replayed after the epoch changed)");
    return err ? fail(x, EC_EDEVICE, "an expert id outside [0, E) was passed to expert_cache_step") : EC_OK;
}

ec_status ec_rebuild_slots(const ec_ctx* x, int32_t budget_bp, int32_t* slots, uint64_t* slot_pool_bytes) {
    if (!x) return fail(nullptr, EC_EINVAL, "ctx is NULL");
    if (budget_bp < 0 || budget_bp > 10000) return fail(nullptr, EC_EINVAL, "budget_bp must be in [0, 10000]");
    const int64_t C = ((int64_t)budget_bp * x->L * x->E) / 10000;
    if (slots) *slots = (int32_t)C;
    if (slot_pool_bytes) *slot_pool_bytes = (uint64_t)C * x->lay.expert_bytes;
    return EC_OK;
}

ec_status ec_debug_state(ec_ctx* x, int32_t* resid, int32_t* slot_key, uint64_t* slot_lru, uint64_t* clock) {
    if (!x) return fail(nullptr, EC_EINVAL, "ctx is NULL");
    HIPCHK(x, hipDeviceSynchronize());
    const uint64_t LE = (uint64_t)x->L * x->E;
    if (resid) HIPCHK(x, hipMemcpy(resid, x->st.resid, LE * 4, hipMemcpyDeviceToHost));
    if (slot_key) HIPCHK(x, hipMemcpy(slot_key, x->st.slot_key, (uint64_t)x->C * 4, hipMemcpyDeviceToHost));
    if (slot_lru) HIPCHK(x, hipMemcpy(slot_lru, x->st.slot_lru, (uint64_t)x->C * 8, hipMemcpyDeviceToHost));
    if (clock) HIPCHK(x, hipMemcpy(clock, x->st.clock, 8, hipMemcpyDeviceToHost));
    return EC_OK;
}

} // extern "C"
