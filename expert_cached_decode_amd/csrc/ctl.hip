// Routing and the fused cache-control kernel for gfx950 (wave64).
//
// FreeToken edge-MoE write-up, "Implementation notes": all routing-dependent
// control of a decode step runs on the GPU in one kernel (dedup of the routed
// experts, classification against a residency table shared by all layers,
// the bandwidth-derived fill count, a single scan that finds the K least
// recently used candidate slots, and the rewrite of logical routing ids to
// cache slots), writing fixed-shape buffers plus device-resident counts.
//
// The control work is tiny and latency-bound, so it runs in ONE workgroup (4
// wavefronts when the step has at most 256 routed pairs, else 16): top-k with
// DPP wave reductions (one token: a 64-logit segment per wavefront, then one
// ranking pass over their candidates), bitmap dedup and prefix popcounts in LDS,
// ballot/popcount block scans for the miss and cache-side lists, and the
// victims from the slot table read once into registers (issued before the
// routing, whose latency it then hides), selected in one pass whose cost does
// not grow with the number of misses (select_victims).
#include "ec_internal.h"

namespace ec {

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Order-preserving 32-bit key of a finite logit (larger logit, larger key; -0 equals +0;
// every finite value maps above 0).
__device__ __forceinline__ uint32_t value_key(float v) {
    uint32_t u = __float_as_uint(v + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The logit a value_key came from (-0 comes back as +0).
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Wave-wide float sum through DPP row shifts and row broadcasts (lane 63 total, read back).
__device__ __forceinline__ float wave_sum_f(float v) {
#define EC_DPP_ADDF(CTRL, RMASK) \
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, RMASK, 0xf, false))
    EC_DPP_ADDF(0x111, 0xf);
    EC_DPP_ADDF(0x112, 0xf);
    EC_DPP_ADDF(0x114, 0xf);
    EC_DPP_ADDF(0x118, 0xf);
    EC_DPP_ADDF(0x142, 0xa);
    EC_DPP_ADDF(0x143, 0xc);
#undef EC_DPP_ADDF
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Wave-wide maximum of a 32-bit value through DPP row shifts and row broadcasts.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#define EC_DPP_MAX32(CTRL, RMASK)                                                                  \
    {                                                                                              \
        const uint32_t o = __builtin_amdgcn_update_dpp(0u, v, CTRL, RMASK, 0xf, false);            \
        v = o > v ? o : v;                                                                         \
    }
    EC_DPP_MAX32(0x111, 0xf)
    EC_DPP_MAX32(0x112, 0xf)
    EC_DPP_MAX32(0x114, 0xf)
    EC_DPP_MAX32(0x118, 0xf)
    EC_DPP_MAX32(0x142, 0xa)
    EC_DPP_MAX32(0x143, 0xc)
#undef EC_DPP_MAX32
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Inclusive wave-wide prefix sum through the same DPP row shifts and row broadcasts.
__device__ __forceinline__ int wave_incl_scan(int v) {
#define EC_DPP_ADDI(CTRL, RMASK) v += __builtin_amdgcn_update_dpp(0, v, CTRL, RMASK, 0xf, false)
    EC_DPP_ADDI(0x111, 0xf);
    EC_DPP_ADDI(0x112, 0xf);
    EC_DPP_ADDI(0x114, 0xf);
    EC_DPP_ADDI(0x118, 0xf);
    EC_DPP_ADDI(0x142, 0xa);
    EC_DPP_ADDI(0x143, 0xc);
#undef EC_DPP_ADDI
    return v;
}

// A row of up to 512 logits in registers, eight per lane (element lane + 64 i). The loads are
// unconditional (index clamped into the row) so all eight are in flight together.
__device__ __forceinline__ void load_row512(const float* row, int E, float* v) {
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int e = lane + 64 * i;
        v[i] = row[e < E ? e : E - 1];
    }
}

// Top-k of one row of E logits by one wavefront: ids by (logit desc, id asc),
// weights = softmax over the selected logits. ids/w may be global; lds_ids /
// lds_w (optional) receive copies. Rows of up to 512 logits are held in
// registers so the k selection rounds touch memory once; with use_rv the row
// is rv, preloaded by load_row512, else it is read here.
__device__ __forceinline__ void wave_topk(const float* row, int E, int k, int32_t* ids, float* w,
                                          int32_t* lds_ids, float* lds_w, const float (&rv)[8], bool use_rv) {
    const int lane = lane_id();
    float sel_v = 0.f;
    int sel_i = 0;
    if (E <= 512) {
        float v[8];
        if (use_rv) {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = rv[i];
        } else {
            load_row512(row, E, v);
        }
        // 32-bit order keys of the logits (0 marks a taken or absent element); each round takes
        // the wave maximum and then the lowest expert id holding it (ballots in id order)
        uint32_t key[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = lane + 64 * i;
            key[i] = e < E ? value_key(v[i]) : 0u;
        }
        for (int j = 0; j < k; ++j) {
            uint32_t b = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) b = key[i] > b ? key[i] : b;
            const uint32_t M = wave_max_u32(b);
            // wave-uniform: the first register (lowest id block) whose ballot holds the maximum
            int e = 0;
#pragma unroll
            for (int i = 7; i >= 0; --i) {
                const uint64_t bl = __ballot(key[i] == M);
                if (bl) e = 64 * i + __ffsll((unsigned long long)bl) - 1;
            }
            const bool mine = (e & 63) == lane;
#pragma unroll
            for (int i = 0; i < 8; ++i) key[i] = (mine && i == (e >> 6)) ? 0u : key[i];
            if (lane == j) { sel_i = e; sel_v = key_value(M); }
        }
    } else {
        uint64_t chosen = 0; // bit i: element lane + 64 i already selected
        for (int j = 0; j < k; ++j) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
            for (int i = 0, e = lane; e < E; ++i, e += 64) {
                if ((chosen >> i) & 1) continue;
                float v = row[e];
                if (v > bv || (v == bv && e < bi)) { bv = v; bi = e; }
            }
            for (int off = 32; off > 0; off >>= 1) {
                float ov = __shfl_xor(bv, off);
                int oi = __shfl_xor(bi, off);
                if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
            }
            if ((bi & 63) == lane) chosen |= 1ull << (bi >> 6);
            if (lane == j) { sel_v = bv; sel_i = bi; }
        }
    }
    const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sel_v), 0));
    float ex = lane < k ? expf(sel_v - top) : 0.f;
    const float s = wave_sum_f(ex);
    if (lane < k) {
        ids[lane] = sel_i;
        w[lane] = ex / s;
        if (lds_ids) { lds_ids[lane] = sel_i; lds_w[lane] = ex / s; }
    }
}

__global__ __launch_bounds__(256) void route_kernel(const float* logits, int T, int E, int k, int32_t* ids,
                                                    float* w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float none[8] = {};
    wave_topk(logits + (int64_t)t * E, E, k, ids + (int64_t)t * k, w + (int64_t)t * k, nullptr, nullptr, none,
              false);
}

// Butterfly maximum / minimum over the 16 lanes of a DPP row: quad swaps, then the half-row and
// row mirrors; every lane of the row ends with the result.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
#define EC_ROW_MAX(CTRL) { const uint32_t o = __builtin_amdgcn_update_dpp(v, v, CTRL, 0xf, 0xf, false); v = o > v ? o : v; }
    EC_ROW_MAX(0xB1) EC_ROW_MAX(0x4E) EC_ROW_MAX(0x141) EC_ROW_MAX(0x140)
#undef EC_ROW_MAX
    return v;
}
__device__ __forceinline__ int row_min_i32(int v) {
#define EC_ROW_MIN(CTRL) { const int o = __builtin_amdgcn_update_dpp(v, v, CTRL, 0xf, 0xf, false); v = o < v ? o : v; }
    EC_ROW_MIN(0xB1) EC_ROW_MIN(0x4E) EC_ROW_MIN(0x141) EC_ROW_MIN(0x140)
#undef EC_ROW_MIN
    return v;
}

// Top-k of four tokens at once per wavefront (E <= 256, k <= 16): DPP row r holds token t0 + r, its
// lane l the logits 16 i + l (i < 16; lv, loaded by the caller). Each round takes the row maximum and
// then the lowest id holding it (the smallest 16 i + l); lane j of the row records the j-th. The
// weights are the softmax over the selected logits summed in wave_topk's order (row shifts, the
// total at the row's last lane), so they are bit-identical to it.
__device__ __forceinline__ void rows_topk(const float (&lv)[16], int T, int E, int k, int t0, int32_t* ids,
                                          float* w, int32_t* lds_ids, float* lds_w) {
    const int lane = lane_id(), l = lane & 15;
    const int t = t0 + (lane >> 4);
    const bool tv = t < T;
    uint32_t key[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) key[i] = (tv && 16 * i + l < E) ? value_key(lv[i]) : 0u;
    uint32_t sel_k = 0u;
    int sel_i = 0;
    for (int j = 0; j < k; ++j) {
        uint32_t b = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) b = key[i] > b ? key[i] : b;
        const uint32_t M = row_max_u32(b);
        int best = 1 << 20;
#pragma unroll
        for (int i = 15; i >= 0; --i) best = (M != 0u && key[i] == M) ? 16 * i + l : best;
        const int e = row_min_i32(best);
        const bool mine = e < (1 << 20) && (e & 15) == l;
#pragma unroll
        for (int i = 0; i < 16; ++i) key[i] = (mine && i == (e >> 4)) ? 0u : key[i];
        if (l == j) { sel_k = M; sel_i = e; }
    }
    const float sel_v = l < k ? key_value(sel_k) : 0.f;
    const float top = __int_as_float(__builtin_amdgcn_ds_bpermute((lane & 48) * 4, __float_as_int(sel_v)));
    float ex = l < k ? expf(sel_v - top) : 0.f;
#define EC_DPP_ADDF(CTRL) ex += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ex), CTRL, 0xf, 0xf, false))
    EC_DPP_ADDF(0x111);
    EC_DPP_ADDF(0x112);
    EC_DPP_ADDF(0x114);
    EC_DPP_ADDF(0x118);
#undef EC_DPP_ADDF
    const float sum = __int_as_float(__builtin_amdgcn_ds_bpermute(((lane & 48) | 15) * 4, __float_as_int(ex)));
    const float ex0 = l < k ? expf(sel_v - top) : 0.f;
    if (tv && l < k) {
        const float wj = ex0 / sum;
        ids[t * k + l] = sel_i;
        w[t * k + l] = wj;
        lds_ids[t * k + l] = sel_i;
        lds_w[t * k + l] = wj;
    }
}

// Top-k of one token's E <= 64 * (NT / 64) logits by the whole block: wavefront w takes the
// top-k of logits 64w .. 64w + 63 (one per lane: k rounds of a DPP wave maximum and one ballot,
// lowest lane = lowest id on ties), then wavefront 0 ranks the wavefronts' candidates by (logit
// desc, id asc) in one pass. The weights are the softmax over the selected logits, computed
// lane by lane exactly as in wave_topk. v is this thread's logit (element 64 wave + lane).
template <int NT>
__device__ __forceinline__ void block_topk1(float v, int E, int k, int32_t* ids, float* w, int32_t* lds_ids,
                                            float* lds_w, uint32_t* s_ck, int32_t* s_ci) {
    constexpr int kWaves = NT / 64;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    uint32_t key = 64 * wave + lane < E ? value_key(v) : 0u;
    uint32_t ck = 0u;
    int ci = -1;
    for (int j = 0; j < k; ++j) {
        const uint32_t M = wave_max_u32(key);
        const uint64_t bl = M ? __ballot(key == M) : 0ull;
        if (bl) {
            const int wl = __ffsll((unsigned long long)bl) - 1;
            if (lane == wl) key = 0u;
            if (lane == j) { ck = M; ci = 64 * wave + wl; }
        }
    }
    if (lane < k) { s_ck[wave * k + lane] = ck; s_ci[wave * k + lane] = ci; }
    __syncthreads();
    if (wave == 0) {
        const int nc = kWaves * k;
        const uint32_t mk = lane < nc ? s_ck[lane] : 0u;
        const uint32_t mi = lane < nc ? (uint32_t)s_ci[lane] : ~0u;
        int rank = 0; // candidates are read from this wavefront's registers, one lane at a time
#pragma unroll 4
        for (int c = 0; c < nc; ++c) {
            const uint32_t ok = (uint32_t)__builtin_amdgcn_readlane((int)mk, c);
            const uint32_t oi = (uint32_t)__builtin_amdgcn_readlane((int)mi, c);
            rank += (ok > mk || (ok == mk && oi < mi)) ? 1 : 0;
        }
        if (mk && rank < k) { lds_ids[rank] = (int)mi; lds_w[rank] = key_value(mk); }
    }
    __syncthreads();
    if (wave == 0) {
        const float sel_v = lane < k ? lds_w[lane] : 0.f;
        const int sel_i = lane < k ? lds_ids[lane] : 0;
        const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sel_v), 0));
        const float ex = lane < k ? expf(sel_v - top) : 0.f;
        const float sum = wave_sum_f(ex);
        if (lane < k) {
            ids[lane] = sel_i;
            w[lane] = ex / sum;
            lds_w[lane] = ex / sum;
        }
    }
}

// Wave-wide minimum of a 64-bit key through DPP row shifts and row broadcasts.
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#define EC_DPP_MIN_STEP(CTRL, RMASK)                                                               \
    {                                                                                              \
        const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);                                 \
        const uint32_t olo = __builtin_amdgcn_update_dpp(lo, lo, CTRL, RMASK, 0xf, false);         \
        const uint32_t ohi = __builtin_amdgcn_update_dpp(hi, hi, CTRL, RMASK, 0xf, false);         \
        const uint64_t o = ((uint64_t)ohi << 32) | olo;                                            \
        v = o < v ? o : v;                                                                         \
    }
    EC_DPP_MIN_STEP(0x111, 0xf)
    EC_DPP_MIN_STEP(0x112, 0xf)
    EC_DPP_MIN_STEP(0x114, 0xf)
    EC_DPP_MIN_STEP(0x118, 0xf)
    EC_DPP_MIN_STEP(0x142, 0xa)
    EC_DPP_MIN_STEP(0x143, 0xc)
#undef EC_DPP_MIN_STEP
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// ---------------------------------------------------------------------------
// K-LRU victims in one pass over the slot table ("Implementation notes": one scan yields the K
// least-recently-used candidates, whatever the number of misses). The victims are the q smallest
// LRU keys of the untouched slots (keys are unique; excluded slots carry ~0). The block does not
// take q rounds of a minimum; instead:
//   1. every thread takes the minimum of its keys;
//   2. the q-th smallest of those thread minima, mu, is found by sorting each wavefront's minima
//      (a bitonic network across the lanes) and merging the sorted lists in one wavefront. Exactly
//      q threads hold a key <= mu, so at least q keys are <= mu and every thread whose minimum is
//      above mu holds none of them;
//   3. the keys <= mu (the candidates: at most q times the keys per thread, usually little more
//      than q) are collected in LDS, and each candidate's rank is the number of smaller
//      candidates: rank r < q makes it victim r, oldest first.
// The cost is a few block barriers and work proportional to the table and to the candidates, not
// to q. Should the candidates not fit in LDS (only with slot tables beyond the registers), a
// bisection over key values first narrows mu to the exact q-th smallest key.

// The value of lane (lane ^ m), for a mask m known at compile time once the callers' loops are
// unrolled, without an LDS round trip (the whole wavefront must be active):
//   m = 1, 2: one DPP quad permutation ([1,0,3,2], [2,3,0,1]);
//   m = 4: the quad reversal (lane ^ 3) and then the half-row mirror (lane ^ 7);
//   m = 8: the half-row mirror (lane ^ 7) and then the row mirror (lane ^ 15);
//   m = 16, 32: v_permlane16_swap / v_permlane32_swap of the value with itself leaves the other
//     half's copy in one of the two results: lanes whose bit m is clear take the second.
// Other masks go through ds_bpermute.
__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int m) {
    switch (m) {
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
    case 4: return (uint32_t)__builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp((int)v, 0x1B, 0xF, 0xF, false), 0x141, 0xF,
                                                      0xF, false);
    case 8: return (uint32_t)__builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false), 0x140, 0xF,
                                                      0xF, false);
    case 16: {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane_id() & 16) ? r[0] : r[1];
    }
    case 32: {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane_id() & 32) ? r[0] : r[1];
    }
    default: return (uint32_t)__shfl_xor((int)v, m);
    }
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    const uint32_t lo = shfl_xor_u32((uint32_t)v, m), hi = shfl_xor_u32((uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

// One key per lane sorted ascending in lane order (bitonic network, 21 compare-exchange steps).
__device__ __forceinline__ uint64_t wave_sort_u64(uint64_t v) {
    const int lane = lane_id();
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint64_t o = shfl_xor_u64(v, j);
            const bool keep_min = ((lane & j) == 0) == ((lane & k) == 0);
            v = keep_min ? (o < v ? o : v) : (o > v ? o : v);
        }
    return v;
}

// The 64 smallest of two ascending lane-ordered lists, ascending: the elementwise minimum of a and
// b reversed is bitonic and holds exactly them; one bitonic merge sorts it.
__device__ __forceinline__ uint64_t merge_lower64(uint64_t a, uint64_t b) {
    const int lane = lane_id();
    const uint32_t blo = (uint32_t)__shfl((int)(uint32_t)b, 63 - lane), bhi = (uint32_t)__shfl((int)(uint32_t)(b >> 32), 63 - lane);
    const uint64_t br = ((uint64_t)bhi << 32) | blo;
    uint64_t v = a < br ? a : br;
#pragma unroll
    for (int j = 32; j > 0; j >>= 1) {
        const uint64_t o = shfl_xor_u64(v, j);
        v = (lane & j) == 0 ? (o < v ? o : v) : (o > v ? o : v);
    }
    return v;
}

// LDS of the victim selection (kept in the kernel's static shared memory). With SR register keys per
// thread, at most q * SR <= 64 * SR keys are candidates (see above).
template <int NT, int SR>
struct VictimLds {
    static constexpr int kCand = 64 * SR;
    uint64_t sel[NT / 64][64]; // each wavefront's sorted thread minima
    uint64_t key[kCand];
    int32_t slot[kCand];
    int32_t occ[kCand];
    uint64_t mu;
    int32_t ncand;
    int32_t part[NT / 64];
};

// Slot keys beyond the registers (tables larger than NT * SR): slot s with its exclusion applied.
struct MemSlots {
    const uint64_t* lru;
    const int32_t* key;
    const uint32_t* hit_bits; // LDS bitmap of the layer's experts hit in this step
    int layer, E, first;      // slots [first, C) are read from memory
};

__device__ __forceinline__ uint64_t excluded_slot(uint64_t key, int occ, int s, int C, int l, int E,
                                                  const uint32_t* hit_bits);

__device__ __forceinline__ uint64_t mem_key(const MemSlots& m, int s, int& occ) {
    occ = m.key[s];
    return excluded_slot(m.lru[s], occ, 0, 1, m.layer, m.E, m.hit_bits);
}

// The LRU key of slot s as a victim candidate: ~0 (never chosen) when s is past C or its occupant
// (key l * E + e) is an expert of this layer routed in this step (bit e of hit_bits). Written
// without branches: the LDS read is always made (index clamped) and the key selected.
__device__ __forceinline__ uint64_t excluded_slot(uint64_t key, int occ, int s, int C, int l, int E,
                                                  const uint32_t* hit_bits) {
    const uint32_t e = (uint32_t)(occ - l * E);
    const uint32_t ec = e < (uint32_t)E ? e : 0u;
    const bool hit = e < (uint32_t)E && ((hit_bits[ec >> 5] >> (ec & 31)) & 1u);
    return (s >= C || hit) ? ~0ull : key;
}

// Victims 0..q-1 into vslot / vocc (LDS), oldest first. pk / po: the thread's SR register keys
// (slot tid + NT p; excluded ones ~0) and occupants; mem: slots from mem.first on, when C is larger.
// Called by all NT threads with the same q >= 1 (at most 64); ends with a block barrier.
template <int NT, int SR, bool MEM>
__device__ void select_victims(const uint64_t (&pk)[SR], const int (&po)[SR], int q, int C, const MemSlots& mem,
                               VictimLds<NT, SR>& L, int32_t* vslot, int32_t* vocc) {
    constexpr int kW = NT / 64;
    constexpr int kVictimCand = VictimLds<NT, SR>::kCand;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    // 1. the thread's minimum key
    uint64_t tmin = ~0ull;
#pragma unroll
    for (int p = 0; p < SR; ++p) tmin = pk[p] < tmin ? pk[p] : tmin;
    if constexpr (MEM) {
        for (int s = mem.first + tid; s < C; s += NT) {
            int occ;
            const uint64_t k = mem_key(mem, s, occ);
            tmin = k < tmin ? k : tmin;
        }
    }
    // 2. mu = the q-th smallest thread minimum
    L.sel[wave][lane] = wave_sort_u64(tmin);
    __syncthreads();
    if (wave == 0) {
        uint64_t best = L.sel[0][lane];
#pragma unroll
        for (int w2 = 1; w2 < kW; ++w2) best = merge_lower64(best, L.sel[w2][lane]);
        const uint32_t mlo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)best, q - 1);
        const uint32_t mhi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(best >> 32), q - 1);
        if (lane == 0) { L.mu = ((uint64_t)mhi << 32) | mlo; L.ncand = 0; }
    }
    __syncthreads();
    uint64_t mu = L.mu;
    // 3. candidates (keys <= mu, never an excluded one) in LDS; ranks among them
    auto count_le = [&](uint64_t x) { // block-wide number of keys <= x (excluded keys never count)
        int c = 0;
#pragma unroll
        for (int p = 0; p < SR; ++p) c += (pk[p] <= x && pk[p] != ~0ull) ? 1 : 0;
        if constexpr (MEM) {
            for (int s = mem.first + tid; s < C; s += NT) {
                int occ;
                const uint64_t k = mem_key(mem, s, occ);
                c += (k <= x && k != ~0ull) ? 1 : 0;
            }
        }
        c = (int)wave_sum_f((float)c); // exact: counts stay far below 2^24
        __syncthreads();
        if (lane == 0) L.part[wave] = c;
        __syncthreads();
        int tot = 0;
#pragma unroll
        for (int w2 = 0; w2 < kW; ++w2) tot += L.part[w2];
        return tot;
    };
    if constexpr (MEM) {
        // candidates that would not fit: bisect to the exact q-th smallest key (count == q)
        if (count_le(mu) > kVictimCand) {
            uint64_t lo = 0, hi = mu; // count_le(hi) >= q
            while (lo < hi) {
                const uint64_t mid = lo + (hi - lo) / 2;
                if (count_le(mid) >= q) hi = mid; else lo = mid + 1;
            }
            mu = lo;
        }
    }
#pragma unroll
    for (int p = 0; p < SR; ++p) {
        if (pk[p] <= mu && pk[p] != ~0ull) {
            const int i = atomicAdd(&L.ncand, 1);
            if (i < kVictimCand) { L.key[i] = pk[p]; L.slot[i] = tid + NT * p; L.occ[i] = po[p]; }
        }
    }
    if constexpr (MEM) {
        for (int s = mem.first + tid; s < C; s += NT) {
            int occ;
            const uint64_t k = mem_key(mem, s, occ);
            if (k <= mu && k != ~0ull) {
                const int i = atomicAdd(&L.ncand, 1);
                if (i < kVictimCand) { L.key[i] = k; L.slot[i] = s; L.occ[i] = occ; }
            }
        }
    }
    __syncthreads();
    const int nc = min(L.ncand, kVictimCand);
    for (int i = tid; i < nc; i += NT) {
        const uint64_t k = L.key[i];
        int r = 0;
        for (int j = 0; j < nc; ++j) r += L.key[j] < k ? 1 : 0;
        if (r < q) { vslot[r] = L.slot[i]; vocc[r] = L.occ[i]; }
    }
    __syncthreads();
}

// Exclusive block scan of a flag (ballot + popcount; NT threads).
template <int NT>
__device__ int block_scan_flag(bool f, int* s_wtot, int* total) {
    constexpr int kCtlWaves = NT / 64;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const uint64_t b = __ballot(f);
    if (lane == 0) s_wtot[wave] = __popcll(b);
    __syncthreads();
    int wpre = 0, tot = 0;
    for (int w2 = 0; w2 < kCtlWaves; ++w2) {
        const int c = s_wtot[w2];
        wpre += w2 < wave ? c : 0;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return wpre + __popcll(b & ((1ull << lane) - 1ull));
}

// Exclusive block scan of flag f plus the block-wide count of a second flag e (one pair
// of barriers for both).
template <int NT>
__device__ int block_scan_flag2(bool f, bool e, int* s_wtot, int* total_f, int* total_e) {
    constexpr int kCtlWaves = NT / 64;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const uint64_t bf = __ballot(f), be = __ballot(e);
    if (lane == 0) { s_wtot[wave] = __popcll(bf); s_wtot[kCtlWaves + wave] = __popcll(be); }
    __syncthreads();
    int wpre = 0, tf = 0, te = 0;
    for (int w2 = 0; w2 < kCtlWaves; ++w2) {
        const int c = s_wtot[w2];
        wpre += w2 < wave ? c : 0;
        tf += c;
        te += s_wtot[kCtlWaves + w2];
    }
    __syncthreads();
    *total_f = tf;
    *total_e = te;
    return wpre + __popcll(bf & ((1ull << lane) - 1ull));
}

// Exclusive block scan of one int per thread (NT threads).
template <int NT>
__device__ int block_scan(int v, int* s_wtot, int* total) {
    constexpr int kCtlWaves = NT / 64;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v);
    if (lane == 63) s_wtot[wave] = incl;
    __syncthreads();
    int wpre = 0, tot = 0;
    for (int w2 = 0; w2 < kCtlWaves; ++w2) {
        int c = s_wtot[w2];
        wpre += w2 < wave ? c : 0;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return wpre + incl - v;
}

// NT threads (256 when T*k <= 256: one wavefront per SIMD keeps the VALU cost of
// this latency-bound kernel low; 1024 otherwise). Each thread holds SR entries
// of the slot table in registers (slots tid + NT p): 5120 slots; larger tables
// are re-read from memory in the victim rounds. The leading scalar arguments (the
// pointers and sizes of the up-front loads; resid_l is the layer's residency row)
// are preloaded into SGPRs at dispatch.
template <int NT>
__global__ __launch_bounds__(NT) void ctl_kernel(const float* logits, const int32_t* ids_in, const int32_t* resid_l,
                                                 const uint64_t* slot_lru, const int32_t* slot_key, int E, int k, int T,
                                                 int C, CtlArgs a) {
    constexpr int kCtlThreads = NT;
    constexpr int kCtlWaves = NT / 64;
    constexpr int kSlotRegs = 5120 / NT;
    __shared__ int32_t s_ids[kMaxPairs];
    __shared__ float s_w[kMaxPairs];
    __shared__ int32_t s_pos[kMaxPairs];
    __shared__ uint32_t s_bits[kMaxExperts / 32];
    __shared__ int32_t s_wpre[kMaxExperts / 32];
    __shared__ int32_t s_uniq[kMaxPairs];
    __shared__ int32_t s_slot[kMaxPairs];
    __shared__ int32_t s_off[kMaxPairs + 1];
    __shared__ int32_t s_first[kMaxPairs];
    __shared__ int32_t s_g[kMaxPairs];
    __shared__ VictimLds<NT, kSlotRegs> s_vl;
    __shared__ int32_t s_vslot[kMaxK];
    __shared__ int32_t s_vocc[kMaxK];
    __shared__ int32_t s_wtot[2 * kCtlWaves];
    __shared__ int32_t s_misc[4];
    __shared__ int32_t s_res[512];
    __shared__ uint32_t s_emask[512]; // fused routing, T <= 32: bit t set when token t routes to expert e
    __shared__ uint32_t s_ck[64];
    __shared__ int32_t s_ci[64];

    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int l = a.layer;
    const int n = T * k;
    const int nwords = (E + 31) >> 5;
    const uint64_t clk = *a.st.clock;

    // 0. loads issued up front, in the order they are needed: the routing rows of the first
    //    tokens (one per wavefront) and then the slot table for the victim scan (LRU key +
    //    occupant of each slot; nothing before the victim rounds changes it), whose latency the
    //    routing and dedup then hide
    //    (one token with E <= 64 per wavefront: each wavefront holds a 64-logit segment), then
    //    the layer's residency row (E <= 512; staged through LDS after the routing)
    const bool seg = logits && T == 1 && E <= 64 * kCtlWaves && kCtlWaves * k <= 64;
    // several tokens with E <= 256, k <= 16: four per wavefront, one per DPP row (rows_topk);
    // else one per wavefront from a row of up to 512 logits held in registers (wave_topk)
    const bool rows = logits && !seg && T > 1 && E <= 256 && k <= 16;
    const bool pre = logits && !seg && !rows && E <= 512 && wave < T;
    // with fused routing a token's k ids are distinct, so a pair's rank among the earlier pairs of
    // its expert is the number of earlier tokens routed to that expert (token masks in LDS)
    const bool tmask = logits && T <= 32 && E <= 512;
    // The first routing rows, as 16 unconditional loads per lane (index clamped; a valid dummy
    // word when neither form applies): rows: logits 16 i + (lane & 15) of token 4 wave + lane / 16;
    // pre: logits lane + 64 i (i < 8) of token wave.
    float rl[16];
    {
        const int tr = rows ? min(4 * wave + (lane >> 4), T - 1) : wave;
        const float* base = (rows || pre) ? logits + (int64_t)tr * E : reinterpret_cast<const float*>(resid_l);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int e = rows ? 16 * i + (lane & 15) : pre ? lane + 64 * (i & 7) : 0;
            rl[i] = base[(rows || pre) ? (e < E ? e : E - 1) : 0];
        }
    }
    float rv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) rv[i] = rl[i];
    // One unconditional load per thread for the segment's logit or, without logits, for the
    // thread's routed id (n <= NT: the launch picks NT >= T * k); otherwise it reads a word that
    // is always valid. Unconditional loads keep the wait counts static, so no use of an early
    // load waits for the loads issued after it.
    const int seg_e = 64 * wave + lane;
    const uint32_t* in_p = seg ? reinterpret_cast<const uint32_t*>(logits) + (seg_e < E ? seg_e : E - 1)
                           : (!logits && n > 0) ? reinterpret_cast<const uint32_t*>(ids_in) + (tid < n ? tid : 0)
                                                  : reinterpret_cast<const uint32_t*>(resid_l);
    const uint32_t in_v = *in_p;
    const float segv = __uint_as_float(in_v);
    constexpr int kResRegs = (512 + NT - 1) / NT;
    const bool rrow = E <= 512;
    int rres[kResRegs];
#pragma unroll
    for (int p = 0; p < kResRegs; ++p) {
        const int e = tid + NT * p;
        rres[p] = resid_l[e < E ? e : E - 1];
    }
    uint64_t pk[kSlotRegs];
    int po[kSlotRegs];
    // (every load is unconditional, its index clamped into the table, so that the first use of
    // the routing row waits for that row alone and not for the whole table)
#pragma unroll
    for (int p = 0; p < kSlotRegs; ++p) {
        const int s = tid + kCtlThreads * p;
        pk[p] = slot_lru[s < C ? s : 0];
        po[p] = slot_key[s < C ? s : 0];
    }
    __builtin_amdgcn_sched_barrier(0);

    // 1. routing (fused) or routed ids from the caller
    if (seg) {
        block_topk1<NT>(segv, E, k, a.sb.ids, a.sb.w, s_ids, s_w, s_ck, s_ci);
    } else if (rows) {
        for (int t0 = 4 * wave; t0 < T; t0 += 4 * kCtlWaves) {
            if (t0 != 4 * wave) { // later groups of four tokens (more than 4 per wavefront)
                const int tr = min(t0 + (lane >> 4), T - 1);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int e = 16 * i + (lane & 15);
                    rl[i] = logits[(int64_t)tr * E + (e < E ? e : E - 1)];
                }
            }
            rows_topk(rl, T, E, k, t0, a.sb.ids, a.sb.w, s_ids, s_w);
        }
    } else if (logits) {
        for (int t = wave; t < T; t += kCtlWaves)
            wave_topk(logits + (int64_t)t * E, E, k, a.sb.ids + t * k, a.sb.w + t * k, s_ids + t * k,
                      s_w + t * k, rv, pre && t == wave);
    } else if (tid < n) {
        s_ids[tid] = (int32_t)in_v;
    }
    for (int wd = tid; wd < nwords; wd += kCtlThreads) s_bits[wd] = 0;
    if (tmask)
        for (int e = tid; e < E; e += kCtlThreads) s_emask[e] = 0u;
    if (tid == 0) s_misc[0] = 0;
    if (rrow) {
#pragma unroll
        for (int p = 0; p < kResRegs; ++p)
            if (tid + NT * p < E) s_res[tid + NT * p] = rres[p];
    }
    __syncthreads();

    // 2. dedup: bitmap of routed experts, ranks by prefix popcount; the residency of every
    //    routed expert is looked up now (from the staged row, else from memory, kept per pair)
    constexpr int kPairRegs = kMaxPairs / NT;
    int res_p[kPairRegs];
#pragma unroll
    for (int c = 0; c < kPairRegs; ++c) {
        const int i = tid + kCtlThreads * c;
        const int id = i < n ? s_ids[i] : -1;
        res_p[c] = (id >= 0 && id < E) ? (rrow ? s_res[id] : resid_l[id]) : -1;
    }
    for (int i = tid; i < n; i += kCtlThreads) {
        int id = s_ids[i];
        if (id < 0 || id >= E) s_misc[0] = 1;
        else {
            atomicOr(&s_bits[id >> 5], 1u << (id & 31));
            if (tmask) atomicOr(&s_emask[id], 1u << (i / k));
        }
    }
    __syncthreads();
    if (s_misc[0]) { // invalid expert id: flag it, do nothing else
        if (tid == 0) atomicOr(a.st.err, 1);
        if (tid < CNT_N) a.sb.counts[tid] = 0;
        return;
    }
    if (wave == 0) {
        int w0 = 2 * lane, w1 = 2 * lane + 1;
        int c0 = w0 < nwords ? __popc(s_bits[w0]) : 0;
        int c1 = w1 < nwords ? __popc(s_bits[w1]) : 0;
        const int v = c0 + c1, incl = wave_incl_scan(v);
        if (w0 < nwords) s_wpre[w0] = incl - v;
        if (w1 < nwords) s_wpre[w1] = incl - v + c0;
        if (lane == 63) s_misc[1] = incl;
    }
    __syncthreads();
    const int U = s_misc[1];
    for (int wd = tid; wd < nwords; wd += kCtlThreads) {
        uint32_t bits = s_bits[wd];
        int r = s_wpre[wd];
        while (bits) {
            int b = __ffs(bits) - 1;
            s_uniq[r++] = wd * 32 + b;
            bits &= bits - 1;
        }
    }
#pragma unroll
    for (int c = 0; c < kPairRegs; ++c) {
        const int i = tid + kCtlThreads * c;
        if (i < n) {
            const int id = s_ids[i];
            const int ps = s_wpre[id >> 5] + __popc(s_bits[id >> 5] & ((1u << (id & 31)) - 1u));
            s_pos[i] = ps;
            s_slot[ps] = res_p[c]; // residency by unique index (equal for repeated ids)
        }
    }
    __syncthreads();

    // 3. residency of the unique experts
    const int r = tid;
    const bool valid = r < U;
    const int u = valid ? s_uniq[r] : 0;
    const int sl = valid ? s_slot[r] : -1;

    // 4. classify, fill count q = min(m, floor(m*BP/BH), K, C - h)
    const bool miss = valid && sl < 0;
    int m;
    const int midx = block_scan_flag<NT>(miss, s_wtot, &m);
    const int h = U - m;
    const uint32_t bp = a.st.bw[0], bh = a.st.bw[1];
    int64_t qq = bh ? (int64_t)(((uint64_t)m * bp) / bh) : 0;
    qq = min(qq, (int64_t)m);
    qq = min(qq, (int64_t)a.K);
    qq = min(qq, (int64_t)(C - h));
    const int q = qq > 0 ? (int)qq : 0;

    // 4b. with host-side experts, the mailbox is published and the doorbell rung here, before the
    //     victim selection: the host's work needs only the host list, the host-side pairs'
    //     rewritten ids, the weights and x, all known now. Mailbox in pinned host memory:
    //     [counts 8][host_list n][rewritten n][w n][x bytes], n = T*k; cache-side pairs read 0 there
    //     (the host computes the pairs with negative ids only). Every writer makes its stores
    //     visible system-wide before the block barrier, then one thread publishes the sequence.
    //     s_slot holds the unique experts' early ids meanwhile (each thread has read its residency
    //     above; step 6 overwrites them with the final slots).
    if (a.host_branch && m - q > 0) {
        int32_t* mb = a.sb.mailbox;
        const bool host_r = miss && midx >= q;
        if (valid) s_slot[r] = host_r ? -(1 + midx - q) : 0;
        if (host_r) mb[CNT_N + (midx - q)] = u;
        if (tid == 0) {
            mb[CNT_U] = U; mb[CNT_H] = h; mb[CNT_M] = m; mb[CNT_Q] = q; mb[CNT_HOST] = m - q;
            mb[CNT_GPU] = U - (m - q); mb[6] = T; mb[7] = l;
        }
        __syncthreads();
        for (int i = tid; i < n; i += kCtlThreads) {
            mb[CNT_N + n + i] = s_slot[s_pos[i]];
            reinterpret_cast<float*>(mb)[CNT_N + 2 * n + i] = s_w[i];
        }
        const uint4* xs = reinterpret_cast<const uint4*>(a.x);
        uint4* xd = reinterpret_cast<uint4*>(mb + CNT_N + 3 * n + ((4 - (3 * n) % 4) % 4));
        for (int i = tid; i < a.x_bytes / 16; i += kCtlThreads) xd[i] = xs[i];
        __threadfence_system(); // each thread's mailbox stores are complete before the barrier
        __syncthreads();
        if (tid == 0) {
            const uint32_t sq = *a.st.hseq + 1;
            *a.st.hseq = sq;
            __hip_atomic_store(a.doorbell, sq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }

    // 5. victims: the q oldest slots not hit in this step (empty slots first, in slot order),
    //    in one pass over the slot table read above (select_victims); slots past C and slots
    //    hit in this step are not candidates
    if (q > 0) {
#pragma unroll
        for (int p = 0; p < kSlotRegs; ++p) pk[p] = excluded_slot(pk[p], po[p], tid + kCtlThreads * p, C, l, E, s_bits);
        const MemSlots mem{slot_lru, slot_key, s_bits, l, E, kCtlThreads * kSlotRegs};
        if (C > kCtlThreads * kSlotRegs) select_victims<NT, kSlotRegs, true>(pk, po, q, C, mem, s_vl, s_vslot, s_vocc);
        else select_victims<NT, kSlotRegs, false>(pk, po, q, C, mem, s_vl, s_vslot, s_vocc);
    }
    if (tid < a.K) a.sb.victims[tid] = tid < q ? s_vslot[tid] : -1;
    if (tid < a.K && tid >= q) { a.sb.fills[tid] = -1; a.sb.evicted[tid] = -1; }

    // 6. assign fills to victims (oldest first), host list, LRU update
    int cls = CLS_HIT, slot_r = sl, ev = 0;
    if (valid) {
        if (miss) {
            if (midx < q) {
                const int v = s_vslot[midx];
                const int old = s_vocc[midx];
                a.sb.evicted[midx] = old;
                if (old >= 0) { a.st.resid[old] = -1; ev = 1; }
                a.st.slot_key[v] = l * E + u;
                a.st.resid[(int64_t)l * E + u] = v;
                a.sb.fills[midx] = u;
                cls = CLS_FILL;
                slot_r = v;
            } else {
                const int hidx = midx - q;
                a.sb.host_list[hidx] = u;
                cls = CLS_HOST;
                slot_r = -(1 + hidx);
            }
        }
        if (cls != CLS_HOST) a.st.slot_lru[slot_r] = kLruTouched | ((clk + 1) << 16) | (uint64_t)r;
        s_slot[r] = slot_r;
        a.sb.uniq[r] = u;
        a.sb.cls[r] = cls;
        a.sb.slot[r] = slot_r;
    }
    int n_gpu, n_ev;
    const int g = block_scan_flag2<NT>(valid && cls != CLS_HOST, ev != 0, s_wtot, &n_gpu, &n_ev);
    if (valid) s_g[r] = cls != CLS_HOST ? g : -1;

    // 7. rewrite (t, j) -> slot or -(1 + host index); pair lists per unique expert
    int cnt, off;
    if (U == n) { // every unique expert has one pair (e.g. one token: its k ids are distinct)
        for (int i = tid; i < n; i += kCtlThreads) {
            const int pr = s_pos[i];
            a.sb.rewritten[i] = s_slot[pr];
            a.sb.pos[i] = pr;
            a.sb.tok_pairs[pr] = i;
            s_first[pr] = i;
        }
        __syncthreads();
        cnt = valid ? 1 : 0;
        off = r;
    } else {
        if (tid <= U) s_off[tid] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kCtlThreads) {
            a.sb.rewritten[i] = s_slot[s_pos[i]];
            a.sb.pos[i] = s_pos[i];
            atomicAdd(&s_off[s_pos[i]], 1);
        }
        __syncthreads();
        int ntot;
        cnt = valid ? s_off[r] : 0;
        off = block_scan<NT>(cnt, s_wtot, &ntot);
        if (valid) s_off[r] = off;
        __syncthreads();
        for (int i = tid; i < n; i += kCtlThreads) {
            const int pr = s_pos[i];
            int within = 0;
            if (tmask) {
                within = __popc(s_emask[s_ids[i]] & ((1u << (i / k)) - 1u));
            } else {
                for (int i2 = 0; i2 < i; ++i2) within += (s_pos[i2] == pr);
            }
            a.sb.tok_pairs[s_off[pr] + within] = i;
            if (within == 0) s_first[pr] = i;
        }
        __syncthreads();
    }
    // work descriptor of each cache-side expert: slot, first entry in tok_pairs, pair count, first pair
    if (valid && s_g[r] >= 0) a.sb.gpu_desc[s_g[r]] = make_int4(slot_r, off, cnt, s_first[r]);

    // 8. counts, stats, clock (the mailbox went out after step 4)
    if (tid == 0) {
        int32_t* c = a.sb.counts;
        c[CNT_U] = U; c[CNT_H] = h; c[CNT_M] = m; c[CNT_Q] = q; c[CNT_HOST] = m - q; c[CNT_GPU] = n_gpu;
        c[6] = 0; c[7] = 0;
        unsigned long long* st = a.st.stats + (int64_t)l * ST_N;
        st[ST_STEPS] += 1; st[ST_HITS] += h; st[ST_MISSES] += m; st[ST_FILLS] += q;
        st[ST_HOST] += m - q; st[ST_EVICT] += n_ev;
        *a.st.clock = clk + 1;
    }
}

// The control step of one token (fused routing, E <= 256, k <= 16, C <= 5120: the batch-1
// decode step). Same outputs and state updates as ctl_kernel, with fewer block barriers
// and no dependent global loads: the token-level work (routing stage 2 and softmax, dedup,
// classification, the fill count, assignment, rewrite, outputs and the mailbox) runs in
// wavefront 0 with register permutes (lane r holds unique expert r, lane j routed pair j),
// and all four wavefronts meet only for the routing candidates and for the victim scan over
// the slot table. Everything read from memory (logits, the layer's residency row, the slot
// table, the layer's stats row, the clock, BP/BH, the mailbox sequence) is loaded up front.
// SR: slot-table entries per thread (C <= 256 SR). The leading scalar arguments (what the
// up-front loads need) are preloaded into SGPRs at dispatch, so those loads do not wait for a
// fetch of the argument block; `words` is the state block holding the clock, BP/BH, the mailbox
// sequence and the per-layer stats (clock at +0, bw at +8, hseq at +16, stats from +32), read
// and updated through it.
template <int SR>
__global__ __launch_bounds__(256) void ctl1_kernel(const float* logits, const int32_t* resid, const uint64_t* slot_lru,
                                                   const int32_t* slot_key, int E, int k, int l, int C,
                                                   uint64_t* words, CtlArgs a) {
    constexpr int NT = 256, kWaves = NT / 64, kSlotRegs = SR;
    __shared__ uint32_t s_ck[64];
    __shared__ int32_t s_ci[64];
    __shared__ int32_t s_res[256];
    __shared__ uint32_t s_bits[8];
    __shared__ VictimLds<NT, kSlotRegs> s_vl;
    __shared__ int32_t s_vslot[kMaxK];
    __shared__ int32_t s_vocc[kMaxK];
    __shared__ int32_t s_q;

    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const uint64_t lt = (1ull << lane) - 1ull;

    // 0. loads, all unconditional (indices clamped), in the order they are needed
    const int ec = tid < E ? tid : E - 1;
    const float lv = logits[ec];                          // logit of expert tid
    const int rres = resid[(int64_t)l * E + ec];          // residency of expert tid
    // the state words before the slot table: the fill count and the mailbox (steps 4 and 4b)
    // need them, the slot table only the victim scan after them (loads complete in order)
    const uint64_t clk = words[0];
    const uint32_t bp = reinterpret_cast<const uint32_t*>(words + 1)[0];
    const uint32_t bh = reinterpret_cast<const uint32_t*>(words + 1)[1];
    const uint32_t hs = reinterpret_cast<const uint32_t*>(words + 2)[0];
    unsigned long long* stats = reinterpret_cast<unsigned long long*>(words + 4);
    const unsigned long long st_v = stats[(int64_t)l * ST_N + (lane < ST_N ? lane : 0)];
    uint64_t pk[kSlotRegs];
    int po[kSlotRegs];
#pragma unroll
    for (int p = 0; p < kSlotRegs; ++p) {
        const int s = tid + NT * p;
        pk[p] = slot_lru[s < C ? s : 0];
        po[p] = slot_key[s < C ? s : 0];
    }
    // output pointers of the argument block, fetched now (the empty asm keeps the compiler from
    // sinking their loads past the first routing stage, where the block barrier would wait for them)
    asm volatile("" ::"s"(a.sb.ids), "s"(a.sb.w), "s"(a.sb.uniq), "s"(a.sb.counts), "s"(a.sb.pos), "s"(a.sb.cls),
                 "s"(a.sb.slot), "s"(a.sb.fills), "s"(a.x), "s"(a.x_bytes));
    __builtin_amdgcn_sched_barrier(0);

    // 1. routing, stage 1: the top-k of this wavefront's 64 logits (ties: lowest id)
    uint32_t key = tid < E ? value_key(lv) : 0u;
    uint32_t ck = 0u;
    int ci = -1;
    for (int j = 0; j < k; ++j) {
        const uint32_t M = wave_max_u32(key);
        const uint64_t bl = M ? __ballot(key == M) : 0ull;
        if (bl) {
            const int wl = __ffsll((unsigned long long)bl) - 1;
            if (lane == wl) key = 0u;
            if (lane == j) { ck = M; ci = 64 * wave + wl; }
        }
    }
    if (lane < k) { s_ck[wave * k + lane] = ck; s_ci[wave * k + lane] = ci; }
    if (tid < E) s_res[tid] = rres;
    if (tid < 8) s_bits[tid] = 0u;
    __syncthreads();

    // wavefront 0: per routed pair j (lane j < k) and per unique expert r (lane r < U = k)
    int sel_i = 0, pos = 0, u = 0, pr = 0, sl = -1, midx = 0, m = 0, h = 0;
    float wj = 0.f;
    bool valid = false, miss = false;
    if (wave == 0) {
        // routing, stage 2: k rounds of a DPP wave maximum over the candidates (lane c holds
        // candidate c; at least k are present since E >= k). Candidates sit in lane order of
        // (wavefront, selection round), so among equal logits the lowest lane holds the lowest
        // id. Lane j takes the j-th; the weights are the softmax over the k selected logits,
        // computed lane by lane as in wave_topk.
        const int nc = kWaves * k;
        uint32_t ck2 = lane < nc ? s_ck[lane] : 0u;
        const int ci2 = lane < nc ? s_ci[lane] : -1;
        uint32_t sel_k = 0u;
        for (int j = 0; j < k; ++j) {
            const uint32_t M = wave_max_u32(ck2);
            const int wl = __ffsll((unsigned long long)__ballot(ck2 == M)) - 1;
            const int idw = __builtin_amdgcn_readlane(ci2, wl);
            if (lane == wl) ck2 = 0u;
            if (lane == j) { sel_k = M; sel_i = idw; }
        }
        const float sel_v = lane < k ? key_value(sel_k) : 0.f;
        const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sel_v), 0));
        const float ex = lane < k ? expf(sel_v - top) : 0.f;
        const float sum = wave_sum_f(ex);
        wj = ex / sum;
        if (lane < k) { a.sb.ids[lane] = sel_i; a.sb.w[lane] = wj; }

        // 2. dedup: the k ids of one token are distinct; a pair's unique index is the number
        //    of routed ids below its own
        for (int j2 = 0; j2 < k; ++j2)
            pos += (uint32_t)__builtin_amdgcn_readlane(sel_i, j2) < (uint32_t)sel_i ? 1 : 0;
        if (lane >= k) pos = lane;
        u = __builtin_amdgcn_ds_permute(pos * 4, sel_i);
        pr = __builtin_amdgcn_ds_permute(pos * 4, lane);
        valid = lane < k;

        // 3. residency of the unique experts; 4. classify, q = min(m, floor(m*BP/BH), K, C - h)
        sl = valid ? s_res[u] : -1;
        if (valid) atomicOr(&s_bits[u >> 5], 1u << (u & 31));
        miss = valid && sl < 0;
        const uint64_t bm = __ballot(miss);
        m = __popcll(bm);
        h = k - m;
        midx = __popcll(bm & lt);
        // min(m, floor(m*BP/BH)) for m <= 16 without a division: the number of i in 1..m
        // with i*BH <= m*BP
        const bool qi = bh != 0u && lane >= 1 && lane <= m && (uint64_t)lane * bh <= (uint64_t)m * bp;
        int qq = __popcll(__ballot(qi));
        qq = min(qq, a.K);
        qq = min(qq, C - h);
        if (lane == 0) s_q = qq > 0 ? qq : 0;

        // 4b. the host list is fixed once q is (the misses past the first q, in unique order):
        //     the mailbox is published and the doorbell rung here, before victim selection, so
        //     the host starts on its experts while the GPU finishes the step, fills and streams.
        //     Mailbox in pinned host memory: [counts 8][host_list n][rewritten n][w n][x bytes],
        //     n = k; rewritten holds -(1 + host index) for host-side pairs (0 for the others,
        //     whose slots the host does not use); the wavefront's stores are made visible
        //     system-wide before lane 0 rings.
        const int q0 = qq > 0 ? qq : 0;
        if (a.host_branch && m - q0 > 0) {
            const int n = k;
            int32_t* mb = a.sb.mailbox;
            if (lane == 0) {
                mb[CNT_U] = k; mb[CNT_H] = h; mb[CNT_M] = m; mb[CNT_Q] = q0; mb[CNT_HOST] = m - q0;
                mb[CNT_GPU] = k - (m - q0); mb[6] = 1; mb[7] = l;
            }
            const bool host_r = valid && miss && midx >= q0;
            if (host_r) mb[CNT_N + (midx - q0)] = u;
            const int hv = host_r ? -(1 + midx - q0) : 0;
            const int rwh = __builtin_amdgcn_ds_bpermute(pos * 4, hv);
            if (lane < n) {
                mb[CNT_N + n + lane] = rwh;
                reinterpret_cast<float*>(mb)[CNT_N + 2 * n + lane] = wj;
            }
            const uint4* xs = reinterpret_cast<const uint4*>(a.x);
            uint4* xd = reinterpret_cast<uint4*>(mb + CNT_N + 3 * n + ((4 - (3 * n) % 4) % 4));
            for (int i = lane; i < a.x_bytes / 16; i += 64) xd[i] = xs[i];
            __threadfence_system(); // the mailbox's stores are complete before the doorbell is
            if (lane == 0) {
                reinterpret_cast<uint32_t*>(words + 2)[0] = hs + 1;
                __hip_atomic_store(a.doorbell, hs + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            }
        }
    }
    __syncthreads();
    const int q = s_q;

    // 5. victims in one pass over the slot table held in registers (select_victims)
    if (q > 0) {
#pragma unroll
        for (int p = 0; p < kSlotRegs; ++p) pk[p] = excluded_slot(pk[p], po[p], tid + NT * p, C, l, E, s_bits);
        const MemSlots none{nullptr, nullptr, nullptr, 0, 0, C};
        select_victims<NT, kSlotRegs, false>(pk, po, q, C, none, s_vl, s_vslot, s_vocc);
    }
    if (wave != 0) return;

    if (lane < a.K) {
        a.sb.victims[lane] = lane < q ? s_vslot[lane] : -1;
        if (lane >= q) { a.sb.fills[lane] = -1; a.sb.evicted[lane] = -1; }
    }
    // 6. assign fills to victims (oldest first), host list, LRU update (lane r: unique expert r)
    int cls = CLS_HIT, slot_r = sl, ev = 0;
    if (valid) {
        if (miss) {
            if (midx < q) {
                const int v = s_vslot[midx];
                const int old = s_vocc[midx];
                a.sb.evicted[midx] = old;
                if (old >= 0) { a.st.resid[old] = -1; ev = 1; }
                a.st.slot_key[v] = l * E + u;
                a.st.resid[(int64_t)l * E + u] = v;
                a.sb.fills[midx] = u;
                cls = CLS_FILL;
                slot_r = v;
            } else {
                const int hidx = midx - q;
                a.sb.host_list[hidx] = u;
                cls = CLS_HOST;
                slot_r = -(1 + hidx);
            }
        }
        if (cls != CLS_HOST) a.st.slot_lru[slot_r] = kLruTouched | ((clk + 1) << 16) | (uint64_t)lane;
        a.sb.uniq[lane] = u;
        a.sb.cls[lane] = cls;
        a.sb.slot[lane] = slot_r;
    }
    const uint64_t bg = __ballot(valid && cls != CLS_HOST);
    const int n_gpu = __popcll(bg), g = __popcll(bg & lt);
    const int n_ev = __popcll(__ballot(ev != 0));

    // 7. rewrite pair j -> the slot of its unique expert, or -(1 + host index); one pair per
    //    unique expert: tok_pairs[r] = its pair, descriptor {slot, r, 1, pair}
    const int rw = __builtin_amdgcn_ds_bpermute(pos * 4, slot_r);
    if (lane < k) { a.sb.rewritten[lane] = rw; a.sb.pos[lane] = pos; }
    if (valid) a.sb.tok_pairs[lane] = pr;
    if (valid && cls != CLS_HOST) a.sb.gpu_desc[g] = make_int4(slot_r, lane, 1, pr);

    // 8. counts, stats, clock (the mailbox went out after step 4)
    if (lane == 0) {
        int32_t* c = a.sb.counts;
        c[CNT_U] = k; c[CNT_H] = h; c[CNT_M] = m; c[CNT_Q] = q; c[CNT_HOST] = m - q; c[CNT_GPU] = n_gpu;
        c[6] = 0; c[7] = 0;
        words[0] = clk + 1;
    }
    if (lane <= ST_EVICT) {
        const unsigned long long d = lane == ST_STEPS ? 1ull : lane == ST_HITS ? (unsigned long long)h
                                   : lane == ST_MISSES ? (unsigned long long)m : lane == ST_FILLS ? (unsigned long long)q
                                   : lane == ST_HOST ? (unsigned long long)(m - q) : (unsigned long long)n_ev;
        stats[(int64_t)l * ST_N + lane] = st_v + d;
    }
}

__global__ void set_bw_kernel(uint32_t* bw, uint32_t bp, uint32_t bh) {
    if (threadIdx.x == 0) { bw[0] = bp; bw[1] = bh; }
}

__global__ void reset_cache_kernel(DevState st, int LE, int C) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < LE; i += gridDim.x * blockDim.x) {
        st.resid[i] = -1;
        st.slot_key[i] = -1;
        st.slot_lru[i] = (uint64_t)i; // empty slot s: key s
    }
    (void)C;
}

__global__ void fill_i32_kernel(int32_t* p, int32_t v, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

void launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s) {
    if (T <= 0) return;
    hipLaunchKernelGGL(route_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, ids, w);
}

void launch_ctl(const CtlArgs& a, hipStream_t s, const hipEvent_t* ev) {
    const LaunchEvents le(ev);
    if (a.logits && a.T == 1 && a.E <= 256 && a.k <= 16 && a.C <= 5120) {
#define EC_C1(SR) EC_LAUNCH(ctl1_kernel<SR>, dim3(1), dim3(256), 0, s, a.logits, (const int32_t*)a.st.resid, \
                         (const uint64_t*)a.st.slot_lru, (const int32_t*)a.st.slot_key, a.E, a.k, a.layer, a.C, \
                         a.st.clock, a)
        if (a.C <= 2048) EC_C1(8);
        else if (a.C <= 3072) EC_C1(12);
        else if (a.C <= 4096) EC_C1(16);
        else EC_C1(20);
#undef EC_C1
    } else {
        const int32_t* resid_l = a.st.resid + (int64_t)a.layer * a.E;
#define EC_CG(NT) EC_LAUNCH(ctl_kernel<NT>, dim3(1), dim3(NT), 0, s, a.logits, a.ids_in, resid_l, \
                            (const uint64_t*)a.st.slot_lru, (const int32_t*)a.st.slot_key, a.E, a.k, a.T, a.C, a)
        if (a.T * a.k <= 256) EC_CG(256);
        else EC_CG(1024);
#undef EC_CG
    }
}

void launch_set_bw(uint32_t* bw, uint32_t bp, uint32_t bh, hipStream_t s) {
    hipLaunchKernelGGL(set_bw_kernel, dim3(1), dim3(64), 0, s, bw, bp, bh);
}

void launch_reset_cache(DevState st, int L, int E, int C, hipStream_t s) {
    int LE = L * E;
    hipLaunchKernelGGL(reset_cache_kernel, dim3((LE + 255) / 256), dim3(256), 0, s, st, LE, C);
}

void launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s) {
    if (n <= 0) return;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, v, n);
}

} // namespace ec
