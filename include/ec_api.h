/*
 * expert_cached_decode: one MoE layer step with a GPU expert cache (C ABI).
 *
 * The operations follow the FreeToken edge-MoE serving write-up
 * (theainews.cc, "FreeToken: Efficient Edge-Native MoE Serving with
 * Bandwidth-Adaptive Execution"):
 *   - "Design: three mechanisms": the full expert pool lives in host memory
 *     and is the source of truth; leftover GPU memory is one elastic expert
 *     cache shared by all MoE layers.
 *   - "1. Bandwidth-adaptive execution": prefill uploads each layer's full
 *     expert set into one of two buffers while the GPU computes on the other;
 *     decode splits the step's cache misses between GPU fills and host-side
 *     compute with q* ~ m * BP / BH, and merges both sides' partial sums
 *     exactly.
 *   - "2. Semantic-aware caching": a shared LRU expert cache captures routing
 *     locality across tokens.
 *   - "3. Elastic edge resource management": the GPU cache is rebuilt for a
 *     new memory budget at safe points, without reloading the host pool.
 *   - "Implementation notes": all routing-dependent control runs on the GPU
 *     in one kernel (dedup, classify against the residency table, fill count,
 *     K least-recently-used victims in one scan, logical id -> slot rewrite),
 *     with fixed-shape work buffers and device-resident counts so that a
 *     decode step can be captured in a graph together with its host branch.
 *
 * Conventions
 *   - Every entry point returns an ec_status (0 = EC_OK, < 0 = error). On an
 *     error nothing has been enqueued; ec_last_error(ctx) gives a message.
 *   - "dev" pointers are HIP device memory, "pinned" pointers are host memory
 *     from hipHostMalloc (device-accessible), "host" pointers are ordinary host
 *     memory. `stream` arguments are hipStream_t values passed as void*.
 *   - The caller owns every buffer passed in and keeps it alive until
 *     ec_destroy (or, for slot pools replaced by cache_rebuild, until the
 *     rebuild returns). The library allocates no device or pinned memory; the
 *     context owns host-heap state, HIP events and its host worker threads.
 *   - Asynchronous device-side errors set bits of a device flag that
 *     ec_get_stats reports (ec_stats.device_error) and turns into EC_EDEVICE:
 *       bit 0: an expert id outside [0, E) reached the cache control (the step
 *              is skipped);
 *       bit 1: the host branch did not publish a step's partial sums within
 *              the down GEMV's bounded wait (that step's output is wrong);
 *       bit 2: a host-side pair reached a step launched without the host
 *              branch, i.e. a graph captured before ec_epoch() changed was
 *              replayed (the pair is skipped, the output is wrong).
 *     No device error faults or hangs the GPU. HIP runtime errors are EC_EHIP.
 *   - One context is driven from one host thread at a time.
 *
 * Graph capture: moe_route, expert_cache_step, moe_decode_layer and
 * ec_set_bandwidth neither synchronise nor allocate nor read device memory on
 * the host, so a decode step can be captured into a hipGraph and replayed;
 * the token count T is fixed by the capture. moe_prefill_layer and
 * cache_rebuild are eager (not capturable). ec_epoch() changes whenever a
 * captured graph must be re-captured (cache_rebuild, or a bandwidth change
 * that switches the host branch on or off).
 */
#ifndef EC_API_H
#define EC_API_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ec_status;
#define EC_OK 0
#define EC_EINVAL (-1)  /* bad argument */
#define EC_ESHAPE (-2)  /* unsupported or inconsistent shape */
#define EC_ENOSPC (-3)  /* caller buffer too small */
#define EC_EHIP (-4)    /* HIP runtime error */
#define EC_ESTATE (-5)  /* call not valid in the current state */
#define EC_EUNSUP (-6)  /* dtype or device not supported (needs gfx950) */
#define EC_EDEVICE (-7) /* a device-side check failed (device error bits below) */

/* expert weight dtypes */
#define EC_DT_F32 0
#define EC_DT_BF16 1
#define EC_DT_MXFP4 2 /* OCP MX: FP4 E2M1 elements, one E8M0 scale per 32 */

/* Shape of the MoE stack: hidden and inter are multiples of 64 and at most
 * 2048 (f32), 4096 (bf16) or 8192 (MXFP4); experts <= 4096; top_k <= 32. */
typedef struct ec_shape {
    int32_t layers;  /* L: MoE layers sharing the cache */
    int32_t experts; /* E: routed experts per layer */
    int32_t top_k;   /* k: experts per token */
    int32_t hidden;  /* H */
    int32_t inter;   /* I: expert intermediate size */
    int32_t wdtype;  /* EC_DT_* */
} ec_shape;

/* Expert-bank byte layout ("expert bank": layer x expert are the leading
 * dimensions). The host pool is [L][E][expert_bytes]; a cache slot holds one
 * expert in the same layout. Logical matrices: gate [I][H], up [I][H],
 * down [H][I], each row-major; the contraction dimension is the row.
 * f32 / bf16: gate, up, down stored back to back as elements.
 * MXFP4: codes of gate, up, down (two per byte along the row, even element in
 * the low nibble), then the E8M0 scale bytes of gate, up, down (one per 32
 * consecutive row elements). Offsets are in bytes from the expert start. */
typedef struct ec_layout_info {
    uint64_t expert_bytes;
    uint64_t layer_bytes; /* E * expert_bytes */
    uint64_t gate_off, up_off, down_off;
    uint64_t gate_scale_off, up_scale_off, down_scale_off; /* MXFP4 only, else 0 */
} ec_layout_info;

typedef struct ec_config {
    ec_shape shape;
    int32_t max_tokens;    /* T_max for decode steps (1..64, T_max * k <= 1024) */
    int32_t cache_slots;   /* C at creation (0..L*E) */
    int32_t victim_k;      /* K victim candidates per step (1..64); 0 = min(64, U_max) */
    uint32_t bp_mbps;      /* BP: expert transfer bandwidth (integer, any unit) */
    uint32_t bh_mbps;      /* BH: host expert processing bandwidth (>= 1, same unit) */
    int32_t host_threads;  /* host branch threads (the polling thread included); 0 = the CPUs the
                              process may run on less 4 (1..32) */
    int32_t prefill_max_tokens; /* 0 = no prefill; else T_max for moe_prefill_layer */
    int32_t pool_layers;   /* layers the host pool holds (0 = L). With P < L, layer l reads its
                              experts from pool layer l mod P: the bytes moved per fill, host
                              expert or prefill upload are unchanged, only the distinct host
                              memory shrinks (for hosts that cannot pin all L layers). */
    int32_t reserved[3];
} ec_config;

/* Device views returned by expert_cache_step (pointers into the context's
 * device workspace; valid until the next step call on the context).
 * U_max = min(E, T_max*k). */
typedef struct ec_step_view {
    int32_t* uniq;      /* [U_max] routed experts of the step, ascending id */
    int32_t* counts;    /* [8]: U, h, m, q, n_host, n_gpu, (reserved) x2 */
    int32_t* pos;       /* [T*k] index of each routed (t, j) into uniq */
    int32_t* cls;       /* [U_max] 0 hit, 1 fill, 2 host */
    int32_t* slot;      /* [U_max] cache slot, or -(1 + host-list index) */
    int32_t* fills;     /* [K] expert ids filled, in fill order */
    int32_t* victims;   /* [K] victim slots, oldest first (first q used) */
    int32_t* evicted;   /* [K] key l*E+e evicted from each victim, or -1 */
    int32_t* host_list; /* [U_max] experts computed on the host, ascending id */
    int32_t* rewritten; /* [T*k] slot, or -(1 + host-list index) */
} ec_step_view;

typedef struct ec_stats {
    uint64_t steps, hits, misses, fills, host, evictions; /* totals over layers */
    int32_t device_error; /* device error bits (see Conventions): 1 bad expert id, 2 host-branch
                             timeout, 4 host-side pair in a step without the host branch */
    int32_t slots;        /* current C */
    uint64_t clock;       /* LRU clock: expert_cache_step calls so far */
    int32_t host_only;    /* 1: the host pool is not device-accessible (see ec_create) */
    int32_t host_branch;  /* 1: decode steps are launched with the host branch (some step can
                             have host-side experts: BP < BH, K or C below U_max, or host-only
                             mode); 0: every routed expert is cache-side */
    /* host branch, measured on the host: jobs run; their total time from the doorbell seen to
     * the partial sums published; and the handoffs of the decode loop (a doorbell within 1 ms
     * of the previous publication: the GPU saw the sums, finished the layer step and rang for
     * the next one), their count and total time */
    uint64_t host_jobs;
    double host_busy_us;
    uint64_t host_gaps;
    double host_gap_us;
} ec_stats;

typedef struct ec_ctx ec_ctx;

const char* ec_strerror(ec_status s);
const char* ec_last_error(const ec_ctx* ctx);

/* Byte layout of one expert for `shape`. EC_ESHAPE on unsupported shapes. */
ec_status ec_layout(const ec_shape* shape, ec_layout_info* out);

/* Sizes of the device and pinned workspaces ec_create needs for `cfg`. */
ec_status ec_workspace_size(const ec_config* cfg, uint64_t* dev_bytes, uint64_t* pinned_bytes);

/* Create a context on the current HIP device (must be gfx950).
 *   dev_ws     : dev, >= dev_bytes from ec_workspace_size, 256-byte aligned
 *   pinned_ws  : pinned, >= pinned_bytes
 *   host_pool  : [P][E][expert_bytes] expert bank (source of truth),
 *                P = pool_layers (or L); pinned (device-accessible). Ordinary
 *                pageable memory (a host where pinning the bank failed) is
 *                accepted and selects host-only mode: the device sees BP = 0,
 *                so q = 0 and every miss is computed on the host threads
 *                ("Implementation notes": platforms that cannot pin or DMA
 *                fall back to a CPU MoE backend); prefill uploads still work,
 *                through staged copies. ec_stats.host_only reports the mode.
 *   slot_pool  : dev, >= cache_slots * expert_bytes (may be NULL if C = 0)
 * The cache starts cold (every slot empty), the LRU clock at 0. Enqueues its
 * initialisation on the null stream and waits for it. */
ec_status ec_create(const ec_config* cfg, void* dev_ws, uint64_t dev_ws_bytes, void* pinned_ws,
                    uint64_t pinned_ws_bytes, const void* host_pool, uint64_t host_pool_bytes,
                    void* slot_pool, uint64_t slot_pool_bytes, ec_ctx** out);
ec_status ec_destroy(ec_ctx* ctx);

/* Set BP and BH (BH >= 1) used by the fill count q = min(m, floor(m*BP/BH),
 * K, C - h) ("Bandwidth-adaptive execution"). Writes device-resident values
 * on `stream` (capturable). Bumps the epoch when the host branch is switched
 * on or off. */
ec_status ec_set_bandwidth(ec_ctx* ctx, uint32_t bp, uint32_t bh, void* stream);

/* Measure BP and BH on this machine at a safe point ("Bandwidth-adaptive
 * execution": the split follows the two measured bandwidths; "Elastic edge
 * resource management": resources change at run time, so this may be
 * repeated at later safe points). Synchronises the device; not capturable.
 *   BP: bytes/s the fill path moves over the host link, timed by reading
 *       probe_experts experts of pool layer 0 from the pinned pool with the
 *       fill kernel's access pattern (read only: no slot is touched);
 *       0 in host-only mode.
 *   BH: bytes/s of expert weights the host branch's worker threads turn into
 *       partial sums, timed by running that branch on probe_experts experts
 *       of the last pool layer (zero input).
 * One warm-up and three timed passes each, every pass on experts not read
 * before; the best timed pass counts. Results in MB/s (10^6 bytes/s) in
 * *bp_mbps and *bh_mbps (either may be NULL). apply != 0 also sets them as
 * ec_set_bandwidth would (BH at least 1).
 * A pass hands the host branch probe_experts experts in jobs of at most
 * max_tokens * top_k. 1 <= probe_experts <= experts / 4. */
ec_status ec_calibrate_bandwidth(ec_ctx* ctx, int32_t probe_experts, int32_t apply, uint32_t* bp_mbps,
                                 uint32_t* bh_mbps);

/* Router top-k ("Why personal MoE is hard": k of E routed experts per token).
 *   logits : dev f32 [T][E], finite values
 *   ids    : dev i32 [T][k], experts by (logit desc, id asc)
 *   w      : dev f32 [T][k], softmax over the k selected logits
 * 1 <= k <= min(E, 32), E <= 4096, T >= 0 (T = 0 enqueues nothing). */
ec_status moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* ids, float* w,
                    void* stream);

/* Fused cache control for one layer of one decode step ("Implementation
 * notes"): dedup the routed ids, classify each unique expert against the
 * residency table shared by all layers, fill count q (above), the K
 * least-recently-used untouched slots in one scan (empty slots first, in
 * slot order), assignment of the first q misses (ascending id) to the oldest
 * victims, residency/LRU update, host list of the other m - q misses
 * (residency unchanged), and rewrite of each (t, j) to its slot or to
 * -(1 + host index). The clock advances by one; inside the step recency
 * follows ascending expert id.
 *   ids : dev i32 [T][k], each in [0, E) (else the step is skipped and the
 *         device error flag set); 1 <= T <= T_max.
 *   out : host struct receiving device pointers (may be NULL).
 * Moves no expert bytes. */
ec_status expert_cache_step(ec_ctx* ctx, int32_t layer, const int32_t* ids, int32_t T,
                            ec_step_view* out, void* stream);

/* The step buffers written by the most recent expert_cache_step,
 * moe_decode_layer or moe_decode_block call on the context (the decisions of
 * the fused routing path included), as device pointers: the same pointers
 * expert_cache_step returns. Valid until the next step call; read them after
 * that step's stream work has completed. Enqueues nothing, does not sync.
 *   out : host struct receiving the pointers (non-NULL).
 * EC_EINVAL for a NULL ctx or out. */
ec_status ec_last_step(const ec_ctx* ctx, ec_step_view* out);

/* One decode MoE layer ("Bandwidth-adaptive execution", decode):
 * route -> cache control -> fill of the q victims from the host pool ->
 * SwiGLU of the cache-side experts from HBM, and of the host-list experts
 * on host threads reading the host pool -> exact merge
 *   out[t] = sum_j w[t,j] * W_down (silu(W_gate x_t) * (W_up x_t))
 * summed over j = 0..k-1 in order.
 *   x      : dev [T][H], f32 when wdtype is EC_DT_F32, else bf16
 *   logits : dev f32 [T][E]
 *   out    : dev [T][H], same dtype as x
 * 1 <= T <= T_max. Capturable. */
ec_status moe_decode_layer(ec_ctx* ctx, int32_t layer, const void* x, const float* logits, int32_t T,
                           void* out, void* stream);

/* moe_decode_layer for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, results and kernels; the per-step buffers (routing, cache
 * decisions, activations) live in the library's static device scratch instead
 * of the context's workspace: one 4 MiB array per GPU, set up by ec_create
 * and kept until the process ends. The call allocates nothing.
 * ec_last_step then returns pointers into that scratch.
 * EC_ENOSPC when this context's step buffers need more than the scratch holds
 * (max_tokens * top_k * inter activations and the decision buffers); EC_ESTATE
 * when the current device is not the context's. All calls on one GPU share the
 * array, which keeps the last call's contents: calls that can overlap on one
 * GPU (other contexts, other streams) race and must be serialised by the
 * caller. */
ec_status moe_decode_layer_static(ec_ctx* ctx, int32_t layer, const void* x, const float* logits, int32_t T,
                                  void* out, void* stream);

/* Router logits, the step before top-k ("Why personal MoE is hard": a router
 * scores the E experts of a layer for each token):
 *   logits[t][e] = sum_h w_router[e][h] * x[t][h], fp32 accumulation.
 *   w_router : dev [E][H], row-major, x_dtype (EC_DT_F32 or EC_DT_BF16)
 *   x        : dev [T][H], x_dtype
 *   logits   : dev f32 [T][E]
 * H a multiple of 64, at most 2048 (f32) or 4096 (bf16); 1 <= E <= 4096;
 * T >= 0 (T = 0 enqueues nothing). Capturable. */
ec_status moe_gate_logits(const void* w_router, const void* x, int32_t x_dtype, int32_t T, int32_t E, int32_t H,
                          float* logits, void* stream);

/* One MoE block of a chained decode: logits = w_router x (moe_gate_logits
 * into the context's workspace), moe_decode_layer on them, and the residual:
 *   out[t] = x[t] + sum_j w[t,j] f_e(t,j)(x[t]), rounded once to x's dtype,
 * so out is the next layer's input and routing follows the data ("Semantic-
 * aware caching": the cache sees the locality of real routing).
 *   w_router : dev [E][H] in x's dtype (f32 when wdtype is EC_DT_F32, else bf16)
 *   x, out   : dev [T][H], distinct buffers
 * 1 <= T <= T_max. Capturable. */
ec_status moe_decode_block(ec_ctx* ctx, int32_t layer, const void* x, const void* w_router, int32_t T, void* out,
                           void* stream);

/* One prefill MoE layer ("Bandwidth-adaptive execution", prefill: full-layer
 * double buffering). Ensures the layer's whole expert set is in one of two
 * device buffers (uploading it on `copy_stream` if it is not), makes
 * `compute_stream` wait for it, then starts the upload of layer + 1 into the
 * other buffer on `copy_stream` (once that buffer's previous user is done)
 * and computes route -> group by expert -> grouped SwiGLU GEMM (bf16 MFMA) ->
 * exact merge on `compute_stream`. Reads and changes nothing of the decode
 * cache.
 *   x : dev bf16 [T][H]; logits : dev f32 [T][E]; out : dev bf16 [T][H]
 *   1 <= T <= prefill_max_tokens. Eager (not capturable). */
ec_status moe_prefill_layer(ec_ctx* ctx, int32_t layer, const void* x, const float* logits, int32_t T,
                            void* out, void* compute_stream, void* copy_stream);

/* Switch prefill double buffering on (1, default) or off (0: each layer is
 * uploaded and then computed, with no overlap). */
ec_status ec_set_prefill_overlap(ec_ctx* ctx, int32_t on);

/* Rebuild the GPU cache for a new budget at a safe point ("Elastic edge
 * resource management"): waits until no work of the context is in flight,
 * then C = floor(budget_bp * L * E / 10000) slots, all empty (cold); the
 * host pool is not touched and the LRU clock continues.
 *   budget_bp     : 0..10000 (basis points of all L*E experts)
 *   new_slot_pool : dev, >= C * expert_bytes (may equal the old pool; NULL
 *                   only when C = 0)
 * Bumps the epoch. */
ec_status cache_rebuild(ec_ctx* ctx, int32_t budget_bp, void* new_slot_pool, uint64_t bytes);

/* The slot count C = floor(budget_bp * L * E / 10000) that cache_rebuild
 * would choose for budget_bp, and the slot-pool bytes it needs (C *
 * expert_bytes), so that a caller can size the new pool; either output may be
 * NULL. After a rebuild, ec_get_stats reports the C in use (ec_stats.slots).
 * EC_EINVAL for a NULL ctx or a budget outside 0..10000. */
ec_status ec_rebuild_slots(const ec_ctx* ctx, int32_t budget_bp, int32_t* slots, uint64_t* slot_pool_bytes);

/* Expert-bank files ("Implementation notes": weights stored ahead of time in the
 * runtime's expert-bank layout are loaded without discovery or repacking, with
 * parallel direct I/O of aligned blocks; "Elastic edge resource management":
 * reading straight into the final host layout keeps the cold start short).
 * A file is a 4096-byte header (magic "ECBANK01", version, shape, pool layers,
 * expert and bank byte counts, header checksum) followed by the
 * [P][E][expert_bytes] bank, padded to a multiple of 4096 bytes.
 * Neither call touches the GPU.
 *
 * ec_bank_write: writes `bank` (host memory, >= P * E * expert_bytes bytes)
 *   to `path` and syncs it to storage.
 * ec_bank_read: fills `dst` (host memory, typically the pinned pool later
 *   given to ec_create) from a file written for the same shape and P
 *   (EC_ESHAPE otherwise), with `threads` readers (0 = 16) over 32 MiB
 *   chunks. *direct_io (may be NULL) tells how: 1 O_DIRECT straight into dst
 *   (dst 4096-byte aligned and its pages accept direct transfers), 2 O_DIRECT
 *   into per-reader aligned bounce buffers copied to dst (e.g. pinned memory
 *   from the GPU driver, which refuses direct transfers), 0 buffered reads
 *   (no O_DIRECT on the file system). *seconds (may be NULL) is the wall
 *   time. EC_EINVAL on I/O errors or a truncated file. */
ec_status ec_bank_write(const char* path, const ec_shape* shape, int32_t pool_layers, const void* bank, uint64_t bytes);
ec_status ec_bank_read(const char* path, const ec_shape* shape, int32_t pool_layers, void* dst, uint64_t dst_bytes,
                       int32_t threads, int32_t* direct_io, double* seconds);

/* Changes whenever captured graphs of this context must be re-captured. */
uint64_t ec_epoch(const ec_ctx* ctx);

/* Synchronises the device; totals since creation (or the last reset). */
ec_status ec_get_stats(ec_ctx* ctx, ec_stats* out, int32_t reset);

/* Synchronises the device and copies the cache state to host buffers (any
 * may be NULL): resid [L*E] (slot or -1), slot_key [C] (l*E+e or -1),
 * slot_lru [C] (LRU key: empty slot s -> s; else 2^63 | (clock+1) << 16 |
 * rank), clock [1]. */
ec_status ec_debug_state(ec_ctx* ctx, int32_t* resid, int32_t* slot_key, uint64_t* slot_lru,
                         uint64_t* clock);

/* Kernel timing (measurement support). While on, each kernel moe_decode_layer
 * launches stamps a HIP event pair from its own dispatch on the caller's
 * stream (start and end of the kernel itself; the step is then not
 * capturable). Switching on allocates the events; off frees them. Kinds:
 * 0 cache control (route + control), 1 fill, 2 gate/up GEMV, 3 down GEMV +
 * exact merge. */
ec_status ec_kernel_timing(ec_ctx* ctx, int32_t on);

/* Sum of event-measured durations (ms) and number of launches of one kernel
 * kind since timing was switched on (or last reset). Synchronises. */
ec_status ec_kernel_time(ec_ctx* ctx, int32_t kind, double* total_ms, uint64_t* launches, int32_t reset);

/* Test support for the host branch's failure path. pause_host != 0: the host
 * stops answering doorbells (the mailbox waits) until called again with 0.
 * wait_polls bounds how often the down GEMV polls for the host's partial sums
 * in launches made after this call (0: the default 4194304, seconds of
 * polling; a graph captured earlier keeps the bound it was captured with).
 * With a paused host and a small bound, a step with host-side experts ends
 * without their partial sums (its output is then wrong) and sets device error
 * bit 2, which ec_get_stats reports as EC_EDEVICE: the failure path runs
 * without any wait that could last. EC_EINVAL on a NULL ctx. */
ec_status ec_host_branch_test_hooks(ec_ctx* ctx, int32_t pause_host, uint32_t wait_polls);

/* Queue primer (measurement support): enqueues on `stream` one small kernel
 * that holds it for about `us` microseconds of the device's constant-rate
 * real-time clock, then ends. Launches the host queues behind it meet a busy
 * queue, so each kernel of a timed pass starts right behind its predecessor (as
 * in a graph replay) instead of waking an idle queue; without a primer a pass
 * whose kernels are shorter than the host's per-launch cost times each kernel
 * from an idle queue. Asynchronous. EC_EINVAL unless us <= 1000000. */
ec_status ec_queue_delay(void* stream, uint32_t us);

/* HBM read ceiling of a one-shot burst (measurement support, beside the
 * kernel timing): launches that each issue every load of `burst_bytes` at once
 * (32 KiB per workgroup, 16-byte nontemporal loads, the data discarded), the
 * shape of the decode GEMVs' per-layer weight stream. Successive bursts read
 * distinct 1 MiB-aligned regions of `dev_buf` (dev, `buf_bytes`; give it far
 * more than the 256 MB last-level cache so that no burst is served from it).
 * `reps` timed bursts follow 8 untimed ones; each is timed by an event pair its
 * own dispatch stamps on `stream`. `queued` != 0: all bursts are queued behind a
 * primer (ec_queue_delay) and run back to back; 0: each burst is launched on an
 * idle queue and waited for. Outputs (any may be NULL): median and best
 * microseconds per burst, and the bytes one burst reads (burst_bytes rounded
 * down to 32 KiB). Synchronises; nothing is written to dev_buf.
 * EC_EINVAL unless 1 MiB <= burst_bytes <= buf_bytes / 4 and 1 <= reps <= 1000. */
ec_status ec_hbm_read_probe(const void* dev_buf, uint64_t buf_bytes, uint64_t burst_bytes, int32_t reps, int32_t queued,
                            void* stream, double* median_us, double* best_us, uint64_t* bytes_read);

#ifdef __cplusplus
}
#endif
#endif
