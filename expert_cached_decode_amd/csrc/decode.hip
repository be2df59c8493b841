// Decode-side expert kernels for gfx950: fill of victim slots from the pinned
// host pool, and the grouped SwiGLU GEMV over cache-side experts with the
// exact merge of cache-side and host-side partial sums.
//
// FreeToken edge-MoE write-up, "Bandwidth-adaptive execution" (decode): filled
// experts enter the cache and are computed on the GPU; misses left to the
// host are computed there in place; each side produces partial sums that are
// merged exactly. Batch-1 decode streams every cache-side expert once from
// HBM, so these kernels are bandwidth kernels: one wavefront per weight row,
// 16-byte coalesced loads, the activation slice of each lane kept in
// registers, and several rows in flight per wavefront.
#include "ec_internal.h"

namespace ec {

typedef float f2v __attribute__((ext_vector_type(2)));

constexpr int kGuWaves = 4;     // 256 threads
constexpr int kGuRowsPerWave = 1;
constexpr int kGuRows = kGuWaves * kGuRowsPerWave;

__device__ __forceinline__ float wave_sum(float v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// 2^(e - 127) for an E8M0 byte (e = 255 is never produced by a valid bank)
__device__ __forceinline__ float e8m0_scale(uint32_t e) {
    return e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streamed weight chunk: read once per step, so it is loaded non-temporally.
__device__ __forceinline__ uint4 load_stream(const uint8_t* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Elements covered by one 16-byte chunk of a weight row.
template <int WDT> struct Fmt;
template <> struct Fmt<EC_DT_F32> { static constexpr int EPC = 4; };
template <> struct Fmt<EC_DT_BF16> { static constexpr int EPC = 8; };
template <> struct Fmt<EC_DT_MXFP4> { static constexpr int EPC = 32; };

template <int WDT> __device__ __forceinline__ int row_bytes(int n) {
    return WDT == EC_DT_F32 ? n * 4 : WDT == EC_DT_BF16 ? n * 2 : n / 2;
}

// Load EPC activation values (elements c*EPC ...) as float.
// act_bf16: x is bf16 (decode input) else float32.
template <int EPC>
__device__ __forceinline__ void load_vec(const void* base, int64_t elem0, bool is_bf16, float* v) {
    if (is_bf16) {
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem0);
#pragma unroll
        for (int q = 0; q < EPC / 8; ++q) {
            uint4 u = p[q];
            v[q * 8 + 0] = bf16_lo(u.x); v[q * 8 + 1] = bf16_hi(u.x);
            v[q * 8 + 2] = bf16_lo(u.y); v[q * 8 + 3] = bf16_hi(u.y);
            v[q * 8 + 4] = bf16_lo(u.z); v[q * 8 + 5] = bf16_hi(u.z);
            v[q * 8 + 6] = bf16_lo(u.w); v[q * 8 + 7] = bf16_hi(u.w);
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem0);
#pragma unroll
        for (int q = 0; q < EPC / 4; ++q) {
            float4 f = p[q];
            v[q * 4 + 0] = f.x; v[q * 4 + 1] = f.y; v[q * 4 + 2] = f.z; v[q * 4 + 3] = f.w;
        }
    }
}

// dot of one 16-byte weight chunk with EPC activations (scale: MXFP4 block scale byte)
template <int WDT>
__device__ __forceinline__ float chunk_dot(uint4 wv, uint32_t scale, const float* v, float acc) {
    if constexpr (WDT == EC_DT_F32) {
        acc = fmaf(__uint_as_float(wv.x), v[0], acc);
        acc = fmaf(__uint_as_float(wv.y), v[1], acc);
        acc = fmaf(__uint_as_float(wv.z), v[2], acc);
        acc = fmaf(__uint_as_float(wv.w), v[3], acc);
    } else if constexpr (WDT == EC_DT_BF16) {
        acc = fmaf(bf16_lo(wv.x), v[0], acc); acc = fmaf(bf16_hi(wv.x), v[1], acc);
        acc = fmaf(bf16_lo(wv.y), v[2], acc); acc = fmaf(bf16_hi(wv.y), v[3], acc);
        acc = fmaf(bf16_lo(wv.z), v[4], acc); acc = fmaf(bf16_hi(wv.z), v[5], acc);
        acc = fmaf(bf16_lo(wv.w), v[6], acc); acc = fmaf(bf16_hi(wv.w), v[7], acc);
    } else {
        const float sc = e8m0_scale(scale);
        const uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // byte b of the word holds elements 2b (low nibble) and 2b + 1 (high nibble)
            f2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(words[q], sc, 0);
            f2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(words[q], sc, 1);
            f2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(words[q], sc, 2);
            f2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(words[q], sc, 3);
            acc = fmaf(p0.x, v[q * 8 + 0], acc); acc = fmaf(p0.y, v[q * 8 + 1], acc);
            acc = fmaf(p1.x, v[q * 8 + 2], acc); acc = fmaf(p1.y, v[q * 8 + 3], acc);
            acc = fmaf(p2.x, v[q * 8 + 4], acc); acc = fmaf(p2.y, v[q * 8 + 5], acc);
            acc = fmaf(p3.x, v[q * 8 + 6], acc); acc = fmaf(p3.y, v[q * 8 + 7], acc);
        }
    }
    return acc;
}

// ---------------------------------------------------------------------------
// Fill: copy the q filled experts from the pinned host pool (read over the
// host link by the GPU itself: the slot addresses are decided on the device)
// into their victim slots. Grid: K x chunks; blocks past q exit.
constexpr uint64_t kFillChunk = 256 * 1024;

__global__ __launch_bounds__(256) void fill_kernel(DecodeArgs a, int chunks) {
    const int i = blockIdx.x / chunks, c = blockIdx.x % chunks;
    if (i >= a.counts[CNT_Q]) return;
    const int f = a.fills[i], v = a.victims[i];
    const uint64_t n16 = a.expert_bytes / 16;
    const uint4* src = reinterpret_cast<const uint4*>(a.pool + ((uint64_t)a.layer * a.E + f) * a.expert_bytes);
    uint4* dst = reinterpret_cast<uint4*>(a.slots + (uint64_t)v * a.expert_bytes);
    const uint64_t b0 = (uint64_t)c * (kFillChunk / 16);
    uint64_t b1 = b0 + kFillChunk / 16;
    if (b1 > n16) b1 = n16;
    uint64_t idx = b0 + threadIdx.x;
    for (; idx + 768 < b1; idx += 1024) {
        uint4 r0 = src[idx], r1 = src[idx + 256], r2 = src[idx + 512], r3 = src[idx + 768];
        dst[idx] = r0; dst[idx + 256] = r1; dst[idx + 512] = r2; dst[idx + 768] = r3;
    }
    for (; idx < b1; idx += 256) dst[idx] = src[idx];
}

// ---------------------------------------------------------------------------
// Gate/up GEMV: for each cache-side expert g and each token routed to it,
// act[pair][i] = silu(W_gate[i] . x) * (W_up[i] . x), one wavefront per row
// pair, kGuRowsPerWave row pairs in flight per wavefront. Grid: U_max x
// (I / kGuRows); blocks past the step's cache-side count exit.
template <int WDT, int NCH, bool T1>
__global__ __launch_bounds__(256) void gu_kernel(DecodeArgs a, int chunks) {
    constexpr int EPC = Fmt<WDT>::EPC;
    const int g = blockIdx.x / chunks, ch = blockIdx.x % chunks;
    const int n_gpu = a.counts[CNT_GPU];
    const int4 d = a.gpu_desc[g];
    if (g >= n_gpu) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H, I = a.I;
    const int rb = row_bytes<WDT>(H), n16 = rb >> 4;
    const uint8_t* base = a.slots + (uint64_t)d.x * a.expert_bytes;
    const uint8_t* gate = base;
    const uint8_t* up = base + (uint64_t)I * rb;
    const uint8_t* gsc = base + 3ull * I * rb;             // MXFP4 scale rows (H/32 bytes each)
    const uint8_t* usc = gsc + (uint64_t)I * (H / 32);
    const int row0 = ch * kGuRows + wave * kGuRowsPerWave;
    const bool xbf16 = WDT != EC_DT_F32;

    const int np = T1 ? 1 : d.z; // batch 1: one token per expert
    for (int pi = 0; pi < np; ++pi) {
        const int pair = pi == 0 ? d.w : a.tok_pairs[d.y + pi];
        const int t = T1 ? 0 : pair / a.k;
        uint4 wg[kGuRowsPerWave][NCH], wu[kGuRowsPerWave][NCH];
        uint32_t sg[kGuRowsPerWave][NCH], su[kGuRowsPerWave][NCH];
#pragma unroll
        for (int rr = 0; rr < kGuRowsPerWave; ++rr) {
            const int row = row0 + rr;
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const int c = lane + 64 * j;
                if (row < I && c < n16) {
                    wg[rr][j] = load_stream(gate + (uint64_t)row * rb + 16ull * c);
                    wu[rr][j] = load_stream(up + (uint64_t)row * rb + 16ull * c);
                    if (WDT == EC_DT_MXFP4) {
                        sg[rr][j] = gsc[(uint64_t)row * (H / 32) + c];
                        su[rr][j] = usc[(uint64_t)row * (H / 32) + c];
                    }
                }
            }
        }
        float xv[NCH][EPC];
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int c = lane + 64 * j;
            if (c < n16) load_vec<EPC>(a.x, (int64_t)t * H + (int64_t)c * EPC, xbf16, xv[j]);
        }
#pragma unroll
        for (int rr = 0; rr < kGuRowsPerWave; ++rr) {
            const int row = row0 + rr;
            float accg = 0.f, accu = 0.f;
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const int c = lane + 64 * j;
                if (row < I && c < n16) {
                    accg = chunk_dot<WDT>(wg[rr][j], WDT == EC_DT_MXFP4 ? sg[rr][j] : 0u, xv[j], accg);
                    accu = chunk_dot<WDT>(wu[rr][j], WDT == EC_DT_MXFP4 ? su[rr][j] : 0u, xv[j], accu);
                }
            }
            accg = wave_sum(accg);
            accu = wave_sum(accu);
            if (lane == 0 && row < I) {
                const float sv = accg / (1.f + expf(-accg));
                a.act[(int64_t)pair * I + row] = sv * accu;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Down GEMV + exact merge. One wavefront owns one output row h: for every token
// t it computes y[t,j][h] = W_down,e(t,j)[h] . act[t,j] for the cache-side
// pairs (the rows of up to 8 experts in flight at once, activation slices in
// registers) and merges out[t][h] = sum_j w[t,j] y[t,j][h] in j order, taking
// host-side pairs' partial sums from y_host. No LDS and no cross-block
// communication; a block is 4 rows. T1: batch-1 specialisation (no token
// loop); HOST: the step may have host-side pairs (else every pair is cache-side).
template <int WDT, int NCH, bool HOST>
__device__ __forceinline__ float down_group(const DecodeArgs& a, int t, int j0, int row, int lane) {
    constexpr int EPC = Fmt<WDT>::EPC;
    constexpr int G = 128 / (NCH * EPC) >= 8 ? 8 : (128 / (NCH * EPC) >= 1 ? 128 / (NCH * EPC) : 1);
    const int H = a.H, I = a.I, k = a.k, last = t * k + k - 1;
    const int rbi = row_bytes<WDT>(I), n16 = rbi >> 4;
    const uint64_t down_off = 2ull * I * row_bytes<WDT>(H) + (uint64_t)row * rbi;
    const uint64_t dsc_off = 3ull * I * row_bytes<WDT>(H) + 2ull * I * (H / 32) + (uint64_t)row * (I / 32);
    int rw[G], pr[G];
    float wt[G];
#pragma unroll
    for (int jj = 0; jj < G; ++jj) { // pairs past k repeat the last pair with weight 0
        pr[jj] = min(t * k + j0 + jj, last);
        rw[jj] = a.rewritten[pr[jj]];
        wt[jj] = a.w[pr[jj]];
        if (j0 + jj >= k) wt[jj] = 0.f;
    }
    // weight rows; a host-side pair reads a dummy row of the activation buffer
    // (always allocated, larger than one weight row) and is discarded below, so
    // every load of the group is issued back to back
    uint4 wd[G][NCH];
    uint32_t sd[G][NCH];
#pragma unroll
    for (int jj = 0; jj < G; ++jj) {
        const uint8_t* base = a.slots + (uint64_t)(HOST && rw[jj] < 0 ? 0 : rw[jj]) * a.expert_bytes;
        const uint8_t* rowp = base + down_off;
        const uint8_t* scp = base + dsc_off;
        if (HOST && rw[jj] < 0) rowp = scp = reinterpret_cast<const uint8_t*>(a.act);
#pragma unroll
        for (int q = 0; q < NCH; ++q) {
            const int c = lane + 64 * q;
            if (c < n16) {
                wd[jj][q] = load_stream(rowp + 16ull * c);
                if (WDT == EC_DT_MXFP4) sd[jj][q] = scp[c];
            }
        }
    }
    float av[G][NCH][EPC];
#pragma unroll
    for (int jj = 0; jj < G; ++jj)
#pragma unroll
        for (int q = 0; q < NCH; ++q) {
            const int c = lane + 64 * q;
            if (c < n16) load_vec<EPC>(a.act, (int64_t)pr[jj] * I + (int64_t)c * EPC, false, av[jj][q]);
        }
    float acc = 0.f;
#pragma unroll
    for (int jj = 0; jj < G; ++jj) {
        float part = 0.f;
#pragma unroll
        for (int q = 0; q < NCH; ++q)
            if (lane + 64 * q < n16)
                part = chunk_dot<WDT>(wd[jj][q], WDT == EC_DT_MXFP4 ? sd[jj][q] : 0u, av[jj][q], part);
        float y = wave_sum(part);
        if (HOST) {
            const float yh = a.y_host[(int64_t)pr[jj] * H + row];
            y = rw[jj] >= 0 ? y : yh;
        }
        acc = fmaf(wt[jj], y, acc);
    }
    return acc;
}

template <int WDT, int NCH, bool T1, bool HOST>
__global__ __launch_bounds__(256) void down_kernel(DecodeArgs a) {
    constexpr int EPC = Fmt<WDT>::EPC;
    constexpr int G = 128 / (NCH * EPC) >= 8 ? 8 : (128 / (NCH * EPC) >= 1 ? 128 / (NCH * EPC) : 1);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x * 4 + wave;
    if (row >= a.H) return;
    auto token = [&](int t) {
        float acc = down_group<WDT, NCH, HOST>(a, t, 0, row, lane);
        for (int j0 = G; j0 < a.k; j0 += G) acc += down_group<WDT, NCH, HOST>(a, t, j0, row, lane);
        if (lane == 0) {
            if (WDT == EC_DT_F32) reinterpret_cast<float*>(a.out)[(int64_t)t * a.H + row] = acc;
            else reinterpret_cast<uint16_t*>(a.out)[(int64_t)t * a.H + row] = f32_to_bf16(acc);
        }
    };
    if (T1) token(0);
    else for (int t = 0; t < a.T; ++t) token(t);
}

void launch_fill(const DecodeArgs& a, int K, hipStream_t s) {
    const int chunks = (int)((a.expert_bytes + kFillChunk - 1) / kFillChunk);
    hipLaunchKernelGGL(fill_kernel, dim3(K * chunks), dim3(256), 0, s, a, chunks);
}

template <int WDT> static int nch_for(int n) {
    const int rb = WDT == EC_DT_F32 ? n * 4 : WDT == EC_DT_BF16 ? n * 2 : n / 2;
    return (rb + 1023) / 1024;
}

#define EC_DISPATCH_NCH(KERNEL, WDT, NCH, GRID, ...)                                              \
    switch (NCH) {                                                                                \
    case 1: hipLaunchKernelGGL((KERNEL<WDT, 1>), GRID, dim3(256), 0, s, __VA_ARGS__); break;      \
    case 2: hipLaunchKernelGGL((KERNEL<WDT, 2>), GRID, dim3(256), 0, s, __VA_ARGS__); break;      \
    case 3: case 4: hipLaunchKernelGGL((KERNEL<WDT, 4>), GRID, dim3(256), 0, s, __VA_ARGS__); break; \
    default: hipLaunchKernelGGL((KERNEL<WDT, 8>), GRID, dim3(256), 0, s, __VA_ARGS__); break;     \
    }

void launch_gu(const DecodeArgs& a, hipStream_t s) {
    const int chunks = (a.I + kGuRows - 1) / kGuRows;
    const dim3 grid(a.U_max * chunks);
#define EC_GU(WDT, NCH)                                                                            \
    do {                                                                                           \
        if (a.T == 1) hipLaunchKernelGGL((gu_kernel<WDT, NCH, true>), grid, dim3(256), 0, s, a, chunks); \
        else hipLaunchKernelGGL((gu_kernel<WDT, NCH, false>), grid, dim3(256), 0, s, a, chunks);  \
    } while (0)
#define EC_GU_NCH(WDT, N)                                                                          \
    switch (N) {                                                                                   \
    case 1: EC_GU(WDT, 1); break;                                                                  \
    case 2: EC_GU(WDT, 2); break;                                                                  \
    case 3: case 4: EC_GU(WDT, 4); break;                                                          \
    default: EC_GU(WDT, 8); break;                                                                 \
    }
    if (a.wdtype == EC_DT_F32) { EC_GU_NCH(EC_DT_F32, nch_for<EC_DT_F32>(a.H)) }
    else if (a.wdtype == EC_DT_BF16) { EC_GU_NCH(EC_DT_BF16, nch_for<EC_DT_BF16>(a.H)) }
    else { EC_GU_NCH(EC_DT_MXFP4, nch_for<EC_DT_MXFP4>(a.H)) }
#undef EC_GU_NCH
#undef EC_GU
}

void launch_down(const DecodeArgs& a, hipStream_t s) {
    const dim3 grid((a.H + 3) / 4);
#define EC_DOWN(WDT, NCH)                                                                          \
    do {                                                                                           \
        if (a.T == 1 && !a.host_pairs) hipLaunchKernelGGL((down_kernel<WDT, NCH, true, false>), grid, dim3(256), 0, s, a); \
        else if (a.T == 1) hipLaunchKernelGGL((down_kernel<WDT, NCH, true, true>), grid, dim3(256), 0, s, a); \
        else hipLaunchKernelGGL((down_kernel<WDT, NCH, false, true>), grid, dim3(256), 0, s, a);  \
    } while (0)
#define EC_DOWN_NCH(WDT, N)                                                                        \
    switch (N) {                                                                                   \
    case 1: EC_DOWN(WDT, 1); break;                                                                \
    case 2: EC_DOWN(WDT, 2); break;                                                                \
    case 3: case 4: EC_DOWN(WDT, 4); break;                                                        \
    default: EC_DOWN(WDT, 8); break;                                                               \
    }
    if (a.wdtype == EC_DT_F32) { EC_DOWN_NCH(EC_DT_F32, nch_for<EC_DT_F32>(a.I)) }
    else if (a.wdtype == EC_DT_BF16) { EC_DOWN_NCH(EC_DT_BF16, nch_for<EC_DT_BF16>(a.I)) }
    else { EC_DOWN_NCH(EC_DT_MXFP4, nch_for<EC_DT_MXFP4>(a.I)) }
#undef EC_DOWN_NCH
#undef EC_DOWN
}

} // namespace ec
