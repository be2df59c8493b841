// Internal definitions shared by the HIP kernels and the host runtime of
// libexpert_cached_decode.so (never exported).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ec_api.h"

namespace ec {

// Bump allocator over a caller-owned workspace (NULL base: sizing only).
struct Carve {
    uint8_t* base;
    uint64_t off = 0;
    explicit Carve(uint8_t* b) : base(b) {}
    template <class T> T* take(uint64_t count) {
        off = (off + 255) & ~255ull;
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += count * sizeof(T);
        return p;
    }
};

// Kernel timing (measurement only): a launcher given an event pair sets it for the one kernel it
// launches, which then stamps the pair from its own dispatch (start and end of the kernel itself,
// no marker commands around it); without a pair the launch is the plain one.
inline thread_local const hipEvent_t* t_launch_ev = nullptr;
struct LaunchEvents {
    explicit LaunchEvents(const hipEvent_t* ev) { t_launch_ev = ev; }
    ~LaunchEvents() { t_launch_ev = nullptr; }
};
#define EC_LAUNCH(KER, GRID, BLK, SH, S, ...)                                                          \
    do {                                                                                                \
        if (::ec::t_launch_ev)                                                                          \
            hipExtLaunchKernelGGL(KER, GRID, BLK, SH, S, ::ec::t_launch_ev[0], ::ec::t_launch_ev[1], 0u,  \
                                  __VA_ARGS__);                                                         \
        else                                                                                            \
            hipLaunchKernelGGL(KER, GRID, BLK, SH, S, __VA_ARGS__);                                     \
    } while (0)

constexpr int kMaxPairs = 1024;   // T_max * k
constexpr int kMaxExperts = 4096; // E
constexpr int kMaxTopK = 32;
constexpr int kMaxK = 64;         // victim candidates per step (one wave)

// counts[] layout
enum { CNT_U = 0, CNT_H = 1, CNT_M = 2, CNT_Q = 3, CNT_HOST = 4, CNT_GPU = 5, CNT_N = 8 };
// per-layer stats layout (u64)
enum { ST_STEPS = 0, ST_HITS, ST_MISSES, ST_FILLS, ST_HOST, ST_EVICT, ST_N = 8 };
enum { CLS_HIT = 0, CLS_FILL = 1, CLS_HOST = 2 };

constexpr uint64_t kLruTouched = 1ull << 63; // LRU key of a slot touched at clock c, rank r:
                                             // 2^63 | (c + 1) << 16 | r; empty slot s: s

// Device-resident cache state (persistent across steps).
struct DevState {
    int32_t* resid;    // [L*E] slot or -1
    int32_t* slot_key; // [L*E] (only the first C used) l*E+e or -1
    uint64_t* slot_lru;// [L*E] LRU key
    uint64_t* clock;   // [1]; clock, bw, hseq, hseen and stats share one block: bw = clock + 1 (as
                       // two u32), hseq = clock + 2 (as u32), hseen right after hseq, stats = clock + 4
    uint32_t* bw;      // [2] BP, BH
    int32_t* err;      // [1] device error flags (bit 0 bad expert id, bit 1 host branch timeout)
    unsigned long long* stats; // [L][ST_N]
    uint32_t* hseq;    // [1] sequence number of the last mailbox handed to the host branch
    uint32_t* hseen;   // [1] last finished sequence as relayed on the device
};

// Per-step work buffers (fixed shape, reused by every layer).
struct StepBufs {
    int32_t* ids;       // [T_max*k]
    float* w;           // [T_max*k]
    int32_t* uniq;      // [U_max]
    int32_t* counts;    // [CNT_N]
    int32_t* pos;       // [T_max*k]
    int32_t* cls;       // [U_max]
    int32_t* slot;      // [U_max]
    int32_t* fills;     // [kMaxK]
    int32_t* victims;   // [kMaxK]
    int32_t* evicted;   // [kMaxK]
    int32_t* host_list; // [U_max]
    int32_t* rewritten; // [T_max*k]
    int4* gpu_desc;     // [U_max] cache-side experts in uniq order: {slot, first entry in tok_pairs,
                        //          number of pairs, first pair}
    int32_t* tok_pairs; // [T_max*k] pair index t*k+j, grouped by unique expert, ascending inside
    int32_t* mailbox;   // pinned host mailbox (device-visible address) read by the host branch
                        // (layout in host code)
};

struct CtlArgs {
    DevState st;
    StepBufs sb;
    const float* logits; // fused routing when non-null
    const int32_t* ids_in; // routed ids [T*k] when logits is null
    const void* x;       // layer input, copied into the mailbox when host_branch
    int32_t x_bytes;     // bytes of x (T*H*elem)
    int32_t layer, E, k, T, C, K;
    int32_t host_branch; // 1: hand steps with host-list experts to the host branch
    uint32_t* doorbell;  // pinned (device-visible): [0] sequence of the last mailbox written
};

// The library's static device scratch (static_scratch.hip): the per-step buffers and activations of
// moe_decode_layer_static. 4 MiB per device.
constexpr uint64_t kStaticScratchBytes = 4ull << 20;
void* static_scratch_ptr(int device, hipError_t* err);
void static_scratch_clear_once(int device, void* ptr, hipStream_t s);

// Launchers (defined in the .hip files).
void launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s);
void launch_ctl(const CtlArgs& a, hipStream_t s, const hipEvent_t* ev = nullptr);
void launch_set_bw(uint32_t* bw, uint32_t bp, uint32_t bh, hipStream_t s);
void launch_reset_cache(DevState st, int L, int E, int C, hipStream_t s);
void launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s);

struct DecodeArgs {
    const uint8_t* pool;   // device pointer of the pinned host pool
    uint8_t* slots;        // slot pool
    const int32_t* counts;
    const int32_t* fills;
    const int32_t* victims;
    const int4* gpu_desc;
    const int32_t* tok_pairs;
    const int32_t* rewritten;
    const float* w;
    const void* x;
    float* act;            // [T_max*k][I] SwiGLU activations of cache-side pairs
    const float* y_host;   // [T_max][H][k] host partials, pinned (device-visible address)
    void* out;
    uint64_t expert_bytes;
    int32_t layer, E, k, T, H, I, wdtype, U_max; // layer: the host-pool layer the fills read
    int32_t host_pairs; // 1 when the step can have host-side pairs (the host branch is on)
    const uint32_t* host_done; // pinned (device-visible): sequence of the last mailbox the host finished
    const uint32_t* hseq;      // device: sequence of this step's mailbox
    uint32_t* hseen;           // device: last finished sequence, relayed by block 0 of the down GEMV
    int32_t* err;              // device error flags
    int32_t residual;          // 1: out = x + merged output (chained MoE block)
    uint32_t wait_polls;       // bound on the down GEMV's polls for the host's partial sums
};
constexpr uint32_t kHostWaitPolls = 1u << 22; // default wait bound (seconds of polling)
void launch_fill(const DecodeArgs& a, int K, hipStream_t s, const hipEvent_t* ev = nullptr);
void launch_link_probe(const uint8_t* src_dev, uint64_t bytes, uint32_t* sink, hipStream_t s);
uint64_t launch_hbm_burst(const uint8_t* base, uint64_t bytes, hipStream_t s, const hipEvent_t* ev);
void launch_queue_delay(uint64_t ticks, hipStream_t s);
void launch_gate(const void* wr, const void* x, bool f32, int T, int E, int H, float* logits, hipStream_t s);
void launch_gu(const DecodeArgs& a, hipStream_t s, const hipEvent_t* ev = nullptr);
void launch_down(const DecodeArgs& a, hipStream_t s, const hipEvent_t* ev = nullptr);

} // namespace ec
