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

// Wave-wide sum through DPP row shifts and row broadcasts (fixed order; the
// result is returned to every lane).
__device__ __forceinline__ float wave_sum_dpp(float v) {
#define EC_DPP_ADD_STEP(CTRL, RMASK)                                                                   \
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, RMASK, 0xf, false));
    EC_DPP_ADD_STEP(0x111, 0xf) // row_shr:1
    EC_DPP_ADD_STEP(0x112, 0xf) // row_shr:2
    EC_DPP_ADD_STEP(0x114, 0xf) // row_shr:4
    EC_DPP_ADD_STEP(0x118, 0xf) // row_shr:8 -> lane 15 of each row holds the row sum
    EC_DPP_ADD_STEP(0x142, 0xa) // row_bcast:15 into rows 1 and 3
    EC_DPP_ADD_STEP(0x143, 0xc) // row_bcast:31 into rows 2 and 3 -> lane 63 holds the sum
#undef EC_DPP_ADD_STEP
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Add a * (down^T chunk) into the lane's output slice. MXFP4 chunks are decoded
// unscaled (the per-output scale of the 32-unit group is applied at the end).
template <int WDT>
__device__ __forceinline__ void chunk_axpy(uint4 wv, float a, float* y) {
    if constexpr (WDT == EC_DT_F32) {
        y[0] = fmaf(a, __uint_as_float(wv.x), y[0]); y[1] = fmaf(a, __uint_as_float(wv.y), y[1]);
        y[2] = fmaf(a, __uint_as_float(wv.z), y[2]); y[3] = fmaf(a, __uint_as_float(wv.w), y[3]);
    } else if constexpr (WDT == EC_DT_BF16) {
        y[0] = fmaf(a, bf16_lo(wv.x), y[0]); y[1] = fmaf(a, bf16_hi(wv.x), y[1]);
        y[2] = fmaf(a, bf16_lo(wv.y), y[2]); y[3] = fmaf(a, bf16_hi(wv.y), y[3]);
        y[4] = fmaf(a, bf16_lo(wv.z), y[4]); y[5] = fmaf(a, bf16_hi(wv.z), y[5]);
        y[6] = fmaf(a, bf16_lo(wv.w), y[6]); y[7] = fmaf(a, bf16_hi(wv.w), y[7]);
    } else {
        const uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(words[q], 1.0f, 0);
            f2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(words[q], 1.0f, 1);
            f2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(words[q], 1.0f, 2);
            f2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(words[q], 1.0f, 3);
            y[q * 8 + 0] = fmaf(a, p0.x, y[q * 8 + 0]); y[q * 8 + 1] = fmaf(a, p0.y, y[q * 8 + 1]);
            y[q * 8 + 2] = fmaf(a, p1.x, y[q * 8 + 2]); y[q * 8 + 3] = fmaf(a, p1.y, y[q * 8 + 3]);
            y[q * 8 + 4] = fmaf(a, p2.x, y[q * 8 + 4]); y[q * 8 + 5] = fmaf(a, p2.y, y[q * 8 + 5]);
            y[q * 8 + 6] = fmaf(a, p3.x, y[q * 8 + 6]); y[q * 8 + 7] = fmaf(a, p3.y, y[q * 8 + 7]);
        }
    }
}

// ---------------------------------------------------------------------------
// Expert GEMV (fused gate/up/down): block (g, c) takes cache-side expert g and
// the R intermediate units [c R, (c+1) R). Each unit i is one row of gate, one
// of up and one of down^T (each H elements, in that order of the bank), so a
// wavefront streams 3 rows per unit: a_i = silu(gate_i . x) * (up_i . x), then
// y += a_i * downT_i over its slice of the H outputs. The block's partial y
// (summed over its waves in a fixed order) goes to part[pair][c][:]; the merge
// kernel adds the R-unit partials and merges the experts of each token.
constexpr int kGvWaves = 4;

template <int WDT, int NCH, int UPW>
__global__ __launch_bounds__(kGvWaves * 64) void gemv_kernel(DecodeArgs a, int chunks) {
    constexpr int EPC = Fmt<WDT>::EPC;
    extern __shared__ float s_y[]; // [kGvWaves][H]
    const int g = blockIdx.x / chunks, ch = blockIdx.x % chunks;
    const int n_gpu = a.counts[CNT_GPU];
    const int4 d = a.gpu_desc[g];
    if (g >= n_gpu) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H, I = a.I, R = a.units_per_block;
    const int rb = row_bytes<WDT>(H), n16 = rb >> 4;
    const uint8_t* base = a.slots + (uint64_t)d.x * a.expert_bytes;
    const uint8_t* gate = base;
    const uint8_t* up = base + (uint64_t)I * rb;
    const uint8_t* down = base + 2ull * I * rb;
    const uint8_t* gsc = base + 3ull * I * rb;               // MXFP4: [I][H/32]
    const uint8_t* usc = gsc + (uint64_t)I * (H / 32);        //        [I][H/32]
    const uint8_t* dsc = gsc + 2ull * I * (H / 32);           //        [I/32][H]
    const int u0 = ch * R;
    const int per_wave = R / kGvWaves;
    const bool xbf16 = WDT != EC_DT_F32;

    for (int pi = 0; pi < d.z; ++pi) {
        const int pair = pi == 0 ? d.w : a.tok_pairs[d.y + pi];
        const int t = pair / a.k;
        float xv[NCH][EPC], y[NCH][EPC];
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int c = lane + 64 * j;
            if (c < n16) load_vec<EPC>(a.x, (int64_t)t * H + (int64_t)c * EPC, xbf16, xv[j]);
#pragma unroll
            for (int q = 0; q < EPC; ++q) y[j][q] = 0.f;
        }
        for (int ub = 0; ub < per_wave; ub += UPW) {
            uint4 wg[UPW][NCH], wu[UPW][NCH], wd[UPW][NCH];
            uint32_t sg[UPW][NCH], su[UPW][NCH];
#pragma unroll
            for (int uu = 0; uu < UPW; ++uu) {
                const int i = u0 + wave * per_wave + ub + uu;
#pragma unroll
                for (int j = 0; j < NCH; ++j) {
                    const int c = lane + 64 * j;
                    if (c < n16) {
                        wg[uu][j] = reinterpret_cast<const uint4*>(gate + (uint64_t)i * rb)[c];
                        wu[uu][j] = reinterpret_cast<const uint4*>(up + (uint64_t)i * rb)[c];
                        wd[uu][j] = reinterpret_cast<const uint4*>(down + (uint64_t)i * rb)[c];
                        if (WDT == EC_DT_MXFP4) {
                            sg[uu][j] = gsc[(uint64_t)i * (H / 32) + c];
                            su[uu][j] = usc[(uint64_t)i * (H / 32) + c];
                        }
                    }
                }
            }
#pragma unroll
            for (int uu = 0; uu < UPW; ++uu) {
                float ag = 0.f, au = 0.f;
#pragma unroll
                for (int j = 0; j < NCH; ++j) {
                    const int c = lane + 64 * j;
                    if (c < n16) {
                        ag = chunk_dot<WDT>(wg[uu][j], WDT == EC_DT_MXFP4 ? sg[uu][j] : 0u, xv[j], ag);
                        au = chunk_dot<WDT>(wu[uu][j], WDT == EC_DT_MXFP4 ? su[uu][j] : 0u, xv[j], au);
                    }
                }
                ag = wave_sum_dpp(ag);
                au = wave_sum_dpp(au);
                const float av = ag / (1.f + expf(-ag)) * au;
#pragma unroll
                for (int j = 0; j < NCH; ++j)
                    if (lane + 64 * j < n16) chunk_axpy<WDT>(wd[uu][j], av, y[j]);
            }
        }
        if (WDT == EC_DT_MXFP4) { // apply the down scales of the wave's 32-unit group
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const int c = lane + 64 * j;
                if (c < n16) {
                    const uint8_t* sp = dsc + (uint64_t)((u0 + wave * per_wave) / 32) * H + (uint64_t)c * EPC;
#pragma unroll
                    for (int q = 0; q < EPC; ++q) y[j][q] *= e8m0_scale(sp[q]);
                }
            }
        }
        // block sum over waves in a fixed order
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int c = lane + 64 * j;
            if (c < n16)
#pragma unroll
                for (int q = 0; q < EPC; ++q) s_y[wave * H + c * EPC + q] = y[j][q];
        }
        __syncthreads();
        float* dst = a.part + ((int64_t)pair * chunks + ch) * H;
        for (int h = threadIdx.x; h < H; h += kGvWaves * 64) {
            float v = s_y[h];
#pragma unroll
            for (int w2 = 1; w2 < kGvWaves; ++w2) v += s_y[w2 * H + h];
            dst[h] = v;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Exact merge: out[t][h] = sum_j w[t,j] * y[t,j][h], j in order, where y of a
// cache-side pair is the fixed-order sum of its R-unit partials and y of a
// host-side pair is the host partial sum. Block: 64 outputs of one token; wave w
// sums the partials c = w, w + 4, ...; wave 0 combines.
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a, int chunks) {
    __shared__ float s_r[4][kMaxTopK][64];
    const int t = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.x * 64 + lane, H = a.H, k = a.k;
    if (h < H) {
        for (int j = 0; j < k; ++j) {
            const int pair = t * k + j;
            float v = 0.f;
            if (a.rewritten[pair] >= 0) {
                const float* p = a.part + (int64_t)pair * chunks * H + h;
                for (int c = wave; c < chunks; c += 4) v += p[(int64_t)c * H];
            }
            s_r[wave][j][lane] = v;
        }
    }
    __syncthreads();
    if (wave != 0 || h >= H) return;
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
        const int pair = t * k + j;
        const float y = a.rewritten[pair] >= 0 ? ((s_r[0][j][lane] + s_r[1][j][lane]) + s_r[2][j][lane]) + s_r[3][j][lane]
                                               : a.y_host[(int64_t)pair * H + h];
        acc = fmaf(a.w[pair], y, acc);
    }
    if (a.wdtype == EC_DT_F32) reinterpret_cast<float*>(a.out)[(int64_t)t * H + h] = acc;
    else reinterpret_cast<uint16_t*>(a.out)[(int64_t)t * H + h] = f32_to_bf16(acc);
}

void launch_fill(const DecodeArgs& a, int K, hipStream_t s) {
    const int chunks = (int)((a.expert_bytes + kFillChunk - 1) / kFillChunk);
    hipLaunchKernelGGL(fill_kernel, dim3(K * chunks), dim3(256), 0, s, a, chunks);
}

template <int WDT> static int nch_for(int n) {
    const int rb = WDT == EC_DT_F32 ? n * 4 : WDT == EC_DT_BF16 ? n * 2 : n / 2;
    return (rb + 1023) / 1024;
}

// Units per block: 16 (32 for MXFP4, one scale group of the down projection);
// doubled while a pair would have more than 64 partials. MXFP4 keeps every
// wavefront's units inside one 32-unit scale group (R / 4 divides 32).
int gemv_units_per_block(int wdtype, int I) {
    int R = wdtype == EC_DT_MXFP4 ? 32 : 16;
    while (I / R > 64 && R < 128 && I % (2 * R) == 0) R *= 2; // R always divides I (a multiple of 64)
    return R;
}

void launch_gemv(const DecodeArgs& a, hipStream_t s) {
    const int chunks = a.I / a.units_per_block;
    const dim3 grid(a.U_max * chunks);
    const size_t shm = (size_t)kGvWaves * a.H * 4;
#define EC_GEMV(WDT, NCH) hipLaunchKernelGGL((gemv_kernel<WDT, NCH, 2>), grid, dim3(kGvWaves * 64), shm, s, a, chunks)
#define EC_GEMV_NCH(WDT, N)                                                                        \
    switch (N) {                                                                                   \
    case 1: EC_GEMV(WDT, 1); break;                                                                \
    case 2: EC_GEMV(WDT, 2); break;                                                                \
    case 3: case 4: EC_GEMV(WDT, 4); break;                                                        \
    default: EC_GEMV(WDT, 8); break;                                                               \
    }
    if (a.wdtype == EC_DT_F32) { EC_GEMV_NCH(EC_DT_F32, nch_for<EC_DT_F32>(a.H)) }
    else if (a.wdtype == EC_DT_BF16) { EC_GEMV_NCH(EC_DT_BF16, nch_for<EC_DT_BF16>(a.H)) }
    else { EC_GEMV_NCH(EC_DT_MXFP4, nch_for<EC_DT_MXFP4>(a.H)) }
#undef EC_GEMV_NCH
#undef EC_GEMV
}

void launch_merge(const DecodeArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(merge_kernel, dim3((a.H + 63) / 64, a.T), dim3(256), 0, s, a, a.I / a.units_per_block);
}

} // namespace ec
