// Prefill MoE layer for gfx950.
//
// FreeToken edge-MoE write-up, "Bandwidth-adaptive execution" (prefill):
// because the routing union of a long prompt covers almost every expert of a
// layer, nothing is fetched on demand; instead, while the GPU computes layer
// l from one buffer, a dedicated transfer stream loads the complete expert
// set of layer l+1 into the other buffer, and the buffers swap roles. The
// mechanism attribution reports the result as transfer-bound (one pass of the
// expert pool over the host link per prompt chunk).
//
// Compute per layer: route every token (top-k, softmax over the selected k),
// a stable counting sort of the (token, j) pairs by expert, a grouped
// SwiGLU GEMM on bf16 matrix cores (v_mfma_f32_16x16x32_bf16; 128x64 block
// tiles, gate and up sharing the A tile), a grouped down-projection GEMM
// (128x128 tiles where H allows), and the exact merge out[t] = sum_j w[t,j]
// y[t,j] in j order.
#include "prefill.h"

namespace ec {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f2v __attribute__((ext_vector_type(2)));
// 16-byte chunk in flight between global memory and LDS (a native vector type, so that the
// prefetch arrays stay in registers; arrays of uint4 were placed in private memory)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BK = 64, LDSP = BK; // LDS row pitch in bf16 elements (rows are swizzled, not padded)
constexpr int CPR = BK / 8;           // 16-byte chunks per tile row
constexpr int AQ = BM * BK / 8 / 256; // 16-byte chunks per thread of an A tile
static_assert(AQ * 256 * 8 == BM * BK, "tile chunks per thread");
// N tile width: 64 for the gate/up GEMM (two weight tiles share the A tile), 128 for the down
// GEMM where N allows (one weight tile, so the same registers and LDS as gate/up's two)
template <int BN> struct BTile { static constexpr int Q = BN * BK / 8 / 256; }; // 16-byte chunks per thread

void launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s);

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ---- grouping ---------------------------------------------------------------
// A stable counting sort of the n = T k pairs by expert, in segments of kSeg pairs (one
// wavefront each): per-segment counts, a scan down each expert's column of segments (which
// also gives the counts), and a placement pass in which each wavefront ranks its pairs among
// the pairs of the same expert in pair order. Every expert's rows then list its pairs in
// ascending pair index.
constexpr int kSeg = 512;

__global__ __launch_bounds__(64) void seg_count_kernel(const int32_t* ids, int n, int E, int32_t* segc) {
    extern __shared__ int32_t s_h[]; // [E]
    const int lane = threadIdx.x, sg = blockIdx.x;
    for (int e = lane; e < E; e += 64) s_h[e] = 0;
    __syncthreads();
    const int i1 = min(n, (sg + 1) * kSeg);
    for (int i = sg * kSeg + lane; i < i1; i += 64) atomicAdd(&s_h[ids[i]], 1);
    __syncthreads();
    for (int e = lane; e < E; e += 64) segc[(int64_t)sg * E + e] = s_h[e];
}

// cnt[e] = pairs routed to e; segc[s][e] becomes the number of those in segments before s.
// One wavefront per expert: 64 segments at a time, an inclusive wave prefix sum by lane shuffles.
__global__ __launch_bounds__(64) void seg_scan_kernel(int32_t* segc, int nseg, int E, int32_t* cnt) {
    const int e = blockIdx.x, lane = threadIdx.x;
    int run = 0;
    for (int s0 = 0; s0 < nseg; s0 += 64) {
        const int sg = s0 + lane;
        const int c = sg < nseg ? segc[(int64_t)sg * E + e] : 0;
        int v = c; // inclusive scan over the wavefront
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(v, o);
            if (lane >= o) v += u;
        }
        if (sg < nseg) segc[(int64_t)sg * E + e] = run + v - c;
        run += __shfl(v, 63);
    }
    if (lane == 0) cnt[e] = run;
}

// off[e] = rows before expert e; toff[e] = BM-row tiles before expert e
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* cnt, int E, int32_t* off, int32_t* toff) {
    __shared__ int s_w[16][2];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    int c[4], tl[4], sc = 0, st = 0;
    for (int q = 0; q < 4; ++q) {
        int e = t * 4 + q;
        c[q] = e < E ? cnt[e] : 0;
        tl[q] = (c[q] + BM - 1) / BM;
        sc += c[q];
        st += tl[q];
    }
    int ic = sc, it = st;
    for (int o = 1; o < 64; o <<= 1) {
        int a = __shfl_up(ic, o), b = __shfl_up(it, o);
        if (lane >= o) { ic += a; it += b; }
    }
    if (lane == 63) { s_w[wave][0] = ic; s_w[wave][1] = it; }
    __syncthreads();
    int pc = 0, pt = 0, tc = 0, tt = 0;
    for (int w2 = 0; w2 < 16; ++w2) {
        if (w2 < wave) { pc += s_w[w2][0]; pt += s_w[w2][1]; }
        tc += s_w[w2][0];
        tt += s_w[w2][1];
    }
    int rc = pc + ic - sc, rt = pt + it - st;
    for (int q = 0; q < 4; ++q) {
        int e = t * 4 + q;
        if (e < E) { off[e] = rc; toff[e] = rt; }
        rc += c[q];
        rt += tl[q];
    }
    if (t == 0) { off[E] = tc; toff[E] = tt; }
}

// Pair i of segment s routed to expert e goes to row off[e] + (pairs of e in earlier segments)
// + (pairs of e before i in s). The wavefront takes its segment 64 pairs at a time: lanes holding
// the same expert find each other with one ballot per bit of the expert id, each lane's rank among
// them is a popcount, and the group's lowest lane then advances the expert's next row in LDS.
__global__ __launch_bounds__(64) void seg_place_kernel(const int32_t* ids, int n, int E, const int32_t* segc,
                                                        const int32_t* off, int32_t* perm) {
    extern __shared__ int32_t s_run[]; // [E] next row of each expert
    const int lane = threadIdx.x, sg = blockIdx.x;
    for (int e = lane; e < E; e += 64) s_run[e] = off[e] + segc[(int64_t)sg * E + e];
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t below = (1ull << lane) - 1ull;
    const int i1 = min(n, (sg + 1) * kSeg);
    for (int i0 = sg * kSeg; i0 < i1; i0 += 64) {
        __syncthreads(); // the previous round's updates (and the initial rows) are visible
        const int i = i0 + lane;
        const bool v = i < i1;
        const int e = v ? ids[i] : 0;
        uint64_t m = __ballot(v); // lanes with this lane's expert
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t bb = __ballot(bit);
            m &= bit ? bb : ~bb;
        }
        const int row = v ? s_run[e] + __popcll(m & below) : 0;
        __syncthreads(); // every lane has read its expert's row before the leaders advance it
        if (v) {
            perm[row] = i;
            if ((m & below) == 0) s_run[e] += __popcll(m);
        }
    }
}

// ---- grouped GEMM -------------------------------------------------------------
// Expert e of tile tt (toff[e] <= tt < toff[e+1]).
__device__ __forceinline__ int tile_expert(const int32_t* toff, int E, int tt) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (toff[mid] <= tt) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// B tile rows [n0, n0+BN) x cols [k0, k0+BK) of a [N][K] weight matrix, as BQ
// 16-byte chunks per thread (bf16 source), or decoded from MXFP4.
template <int WDT, int BQ>
__device__ __forceinline__ void load_b(const uint8_t* W, const uint8_t* Ws, int K, int n0, int k0, u32x4 (&r)[BQ]) {
#pragma unroll
    for (int q = 0; q < BQ; ++q) {
        const int c = threadIdx.x + 256 * q, row = c / CPR, col = (c % CPR) * 8;
        if constexpr (WDT == EC_DT_BF16) {
            r[q] = *reinterpret_cast<const u32x4*>(W + ((uint64_t)(n0 + row) * K + k0 + col) * 2);
        } else {
            // 8 MXFP4 elements (4 bytes) -> 8 bf16, exact (E2M1 x 2^(s-127) fits bf16)
            const uint32_t codes = *reinterpret_cast<const uint32_t*>(W + ((uint64_t)(n0 + row) * K + k0 + col) / 2);
            const uint32_t se = Ws[(uint64_t)(n0 + row) * (K / 32) + (k0 + col) / 32];
            const float sc = se ? __uint_as_float(se << 23) : __uint_as_float(0x00400000u);
            f2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, sc, 0);
            f2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, sc, 1);
            f2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, sc, 2);
            f2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, sc, 3);
            r[q].x = (__float_as_uint(p0.x) >> 16) | (__float_as_uint(p0.y) & 0xffff0000u);
            r[q].y = (__float_as_uint(p1.x) >> 16) | (__float_as_uint(p1.y) & 0xffff0000u);
            r[q].z = (__float_as_uint(p2.x) >> 16) | (__float_as_uint(p2.y) & 0xffff0000u);
            r[q].w = (__float_as_uint(p3.x) >> 16) | (__float_as_uint(p3.y) & 0xffff0000u);
        }
    }
}

// LDS tiles: row r keeps its 16-byte chunk c at chunk position c ^ ((r / 2) mod CPR). A row is
// 128 bytes, so two consecutive rows fill the 64 banks once (tile stores: two rows per 16 lanes,
// no conflict), and the 16 rows a fragment read touches at one chunk land on 16 distinct groups
// of four banks.
__device__ __forceinline__ int lds_swz(int row, int col) { return row * LDSP + (((col >> 3) ^ ((row >> 1) & (CPR - 1))) << 3); }

template <int NQ>
__device__ __forceinline__ void store_lds(uint16_t* lds, const u32x4 (&r)[NQ]) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int c = threadIdx.x + 256 * q, row = c / CPR, col = (c % CPR) * 8;
        *reinterpret_cast<u32x4*>(lds + lds_swz(row, col)) = r[q];
    }
}

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* lds, int row, int col) {
    uint4 u = *reinterpret_cast<const uint4*>(lds + lds_swz(row, col));
    return __builtin_bit_cast(bf16x8, u);
}

struct GemmArgs {
    const uint8_t* wbuf;   // full-layer expert buffer
    uint64_t expert_bytes;
    uint64_t off_a, off_b, off_sa, off_sb; // byte offsets of the B matrices (and MXFP4 scales) in an expert
    const uint16_t* x;     // GEMM1: [T][H] bf16 tokens
    const uint16_t* act_in;// GEMM2: [rows][I] bf16
    uint16_t* act_out;     // GEMM1 output
    float* y;              // GEMM2 output [pairs][H]
    const int32_t* cnt;
    const int32_t* off;
    const int32_t* toff;
    const int32_t* perm;
    int E, k, H, I;
};

// GEMM1: act[g][n] = silu(X_g . Wg[n]) * (X_g . Wu[n]) for grouped rows g of expert e.
// GEMM2: y[perm[g]][n] = act[g] . Wd[n].
// At most 168 registers (three wavefronts per SIMD): measured about 8% faster per bf16 layer than
// the 180-184 the compiler otherwise takes (two per SIMD), with no spills
template <int WDT, bool FIRST, int BN>
__global__ __launch_bounds__(256, 3) void grouped_gemm_kernel(GemmArgs a) {
    constexpr int NB = FIRST ? 2 : 1;
    constexpr int BQ = BTile<BN>::Q;
    // one LDS block: the A tile and the NB weight tiles during the K loop; afterwards the down
    // GEMM stages its fp32 output tile there, half a tile at a time
    constexpr int kTileElems = (BM + NB * BN) * LDSP, kOutElems = FIRST ? 0 : (BM / 2) * (BN + 4) * 2;
    __shared__ __align__(16) uint16_t s_tiles[kTileElems > kOutElems ? kTileElems : kOutElems];
    uint16_t* const sA = s_tiles;
    uint16_t (*const sB)[BN * LDSP] = reinterpret_cast<uint16_t (*)[BN * LDSP]>(s_tiles + BM * LDSP);
    // Block b -> (M tile, N tile). The work items (expert e, N tile n, M tile m of e) are ordered
    // e, then n, then m, and cut into eight contiguous ranges, one per XCD (workgroups are dealt
    // to the XCDs in turn, b mod 8). An XCD thus runs the M tiles of one (expert, N tile) back to
    // back, so the weight tile is fetched from HBM once and served to its other M tiles by that
    // XCD's L2, and the N tiles of one expert follow one another, so its A rows (gathered tokens
    // or activations) stay in that L2 too.
    const int NT = (FIRST ? a.I : a.H) / BN;
    const int total = a.toff[a.E] * NT;   // (M tile, N tile) items of this call
    const int per = (total + 7) >> 3;     // items per XCD
    const int bi = blockIdx.x >> 3;
    const int item = (blockIdx.x & 7) * per + bi;
    if (bi >= per || item >= total) return;
    const int e = tile_expert(a.toff, a.E, item / NT); // toff[e] * NT <= item < toff[e + 1] * NT
    const int mts = a.toff[e + 1] - a.toff[e];          // M tiles of expert e
    const int r = item - a.toff[e] * NT;
    const int mt = r % mts;
    const int rows = a.cnt[e] - mt * BM;  // valid rows in this tile (>= 1)
    const int g0 = a.off[e] + mt * BM;    // first grouped row
    const int n0 = (r / mts) * BN;
    const int K = FIRST ? a.H : a.I;
    const uint8_t* ebase = a.wbuf + (uint64_t)e * a.expert_bytes;
    const uint8_t* Wm[2] = {ebase + a.off_a, ebase + a.off_b};
    const uint8_t* Ws[2] = {ebase + a.off_sa, ebase + a.off_sb};

    // A rows this thread loads (AQ chunks), clamped to a valid row
    const uint16_t* arow[AQ];
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
        const int c = threadIdx.x + 256 * q, row = c / CPR;
        const int rr = row < rows ? row : 0;
        if (FIRST) arow[q] = a.x + (uint64_t)(a.perm[g0 + rr] / a.k) * a.H;
        else arow[q] = a.act_in + (uint64_t)(g0 + rr) * a.I;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
    // wavefront (wm, wn) owns rows wm * BM/2 .. + BM/2 (MI 16-row fragments) and columns
    // wn * BN/2 .. + BN/2 (NJ 16-column fragments)
    constexpr int MI = BM / 32;
    constexpr int NJ = BN / 32;
    f32x4 acc[NB][MI][NJ];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[b][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 ra[AQ], rb[NB][BQ];
    auto gload = [&](int k0) {
#pragma unroll
        for (int q = 0; q < AQ; ++q) {
            const int c = threadIdx.x + 256 * q, col = (c % CPR) * 8;
            ra[q] = *reinterpret_cast<const u32x4*>(arow[q] + k0 + col);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) load_b<WDT>(Wm[b], Ws[b], K, n0, k0, rb[b]);
    };
    gload(0);
    for (int k0 = 0; k0 < K; k0 += BK) {
        __syncthreads();
        store_lds(sA, ra);
#pragma unroll
        for (int b = 0; b < NB; ++b) store_lds(sB[b], rb[b]);
        __syncthreads();
        if (k0 + BK < K) gload(k0 + BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            const int kc = kk + (lane >> 4) * 8;
            bf16x8 fa[MI];
#pragma unroll
            for (int i = 0; i < MI; ++i) fa[i] = lds_frag(sA, wm * (BM / 2) + i * 16 + (lane & 15), kc);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    bf16x8 fb = lds_frag(sB[b], wn * (BN / 2) + j * 16 + (lane & 15), kc);
#pragma unroll
                    for (int i = 0; i < MI; ++i)
                        acc[b][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb, acc[b][i][j], 0, 0, 0);
                }
        }
    }
    // epilogue: lane holds D[(lane/16)*4 + q][lane%16] of each 16x16 tile
    if constexpr (FIRST) {
        // (staging these bf16 stores through LDS as well measured no faster: 67 MB per layer)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int tr = wm * (BM / 2) + i * 16 + (lane >> 4) * 4 + q; // row in the tile
                    const int n = n0 + wn * (BN / 2) + j * 16 + (lane & 15);
                    if (tr >= rows) continue;
                    const float gv = acc[0][i][j][q], uv = acc[1][i][j][q];
                    a.act_out[(uint64_t)(g0 + tr) * a.I + n] = f32_to_bf16_rne(gv / (1.f + expf(-gv)) * uv);
                }
    } else {
        // The fp32 outputs go through LDS, one half of the tile's rows at a time (the wavefronts
        // with wm = half write theirs), and leave as whole-row segments of 16 bytes per lane, so
        // each scattered output row y[perm[g]] is written in full 128-byte lines.
        constexpr int CP = BN + 4; // row pitch in floats: rows 4 apart start 16 banks apart
        static_assert((BM / 2) * CP * 2 <= kOutElems, "output half-tile fits the tile LDS");
        constexpr int LPR = BN / 4; // lanes per output row (16 bytes each)
        float* const sC = reinterpret_cast<float*>(s_tiles);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            __syncthreads(); // the K loop's (or the previous half's) reads of this LDS are done
            if (wm == half)
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            sC[(i * 16 + (lane >> 4) * 4 + q) * CP + wn * (BN / 2) + j * 16 + (lane & 15)] =
                                acc[0][i][j][q];
            __syncthreads();
#pragma unroll
            for (int rr = threadIdx.x / LPR; rr < BM / 2; rr += 256 / LPR) {
                const int tr = half * (BM / 2) + rr, c4 = (threadIdx.x % LPR) * 4;
                if (tr < rows)
                    *reinterpret_cast<f32x4*>(a.y + (uint64_t)a.perm[g0 + tr] * a.H + n0 + c4) =
                        *reinterpret_cast<const f32x4*>(sC + rr * CP + c4);
            }
        }
    }
}

// out[t][h] = sum_j w[t,j] * y[t*k+j][h], j in order; four adjacent outputs per thread (H is a
// multiple of 64), so each thread has its k 16-byte loads in flight at once
__global__ __launch_bounds__(256) void combine_kernel(const float* y, const float* w, int k, int H, uint16_t* out) {
    const int t = blockIdx.x, h = (blockIdx.y * 256 + threadIdx.x) * 4;
    if (h >= H) return;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int j = 0; j < k; ++j) {
        const float wj = w[t * k + j];
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y + ((uint64_t)t * k + j) * H + h));
        a0 = fmaf(wj, v[0], a0);
        a1 = fmaf(wj, v[1], a1);
        a2 = fmaf(wj, v[2], a2);
        a3 = fmaf(wj, v[3], a3);
    }
    const uint32_t lo = (uint32_t)f32_to_bf16_rne(a0) | ((uint32_t)f32_to_bf16_rne(a1) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_rne(a2) | ((uint32_t)f32_to_bf16_rne(a3) << 16);
    *reinterpret_cast<uint2*>(out + (uint64_t)t * H + h) = make_uint2(lo, hi);
}

// ---- host orchestration --------------------------------------------------------
void prefill_carve(PrefillState& p, Carve& d, int Tp, int E, int k, int H, int I, uint64_t layer_bytes) {
    p.Tp = Tp;
    if (Tp <= 0) return;
    const uint64_t n = (uint64_t)Tp * k;
    p.buf[0] = d.take<uint8_t>(layer_bytes);
    p.buf[1] = d.take<uint8_t>(layer_bytes);
    p.ids = d.take<int32_t>(n);
    p.w = d.take<float>(n);
    p.cnt = d.take<int32_t>(E);
    p.segc = d.take<int32_t>((n + kSeg - 1) / kSeg * (uint64_t)E);
    p.off = d.take<int32_t>(E + 1);
    p.toff = d.take<int32_t>(E + 1);
    p.perm = d.take<int32_t>(n);
    p.act = d.take<uint16_t>(n * I);
    p.y = d.take<float>(n * H);
}

hipError_t prefill_init(PrefillState& p) {
    for (int b = 0; b < 2; ++b) {
        hipError_t e = hipEventCreateWithFlags(&p.loaded[b], hipEventDisableTiming);
        if (e != hipSuccess) return e;
        e = hipEventCreateWithFlags(&p.done[b], hipEventDisableTiming);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

void prefill_reset_device(PrefillState& p, hipStream_t s) { (void)p; (void)s; }

void prefill_destroy(PrefillState& p) {
    for (int b = 0; b < 2; ++b) {
        if (p.loaded[b]) (void)hipEventDestroy(p.loaded[b]);
        if (p.done[b]) (void)hipEventDestroy(p.done[b]);
    }
}

static hipError_t upload(PrefillState& p, const PrefillCall& c, int b, int layer) {
    hipError_t e;
    if (p.used[b] && (e = hipStreamWaitEvent(c.copy, p.done[b], 0)) != hipSuccess) return e;
    e = hipMemcpyAsync(p.buf[b], c.host_pool + (uint64_t)(layer % c.P) * c.layer_bytes, c.layer_bytes,
                       hipMemcpyHostToDevice, c.copy);
    if (e != hipSuccess) return e;
    p.buf_layer[b] = layer;
    return hipEventRecord(p.loaded[b], c.copy);
}

hipError_t prefill_layer(PrefillState& p, const PrefillCall& c) {
    hipError_t e;
    // the buffer holding (or about to hold) this layer
    int b;
    if (c.overlap) {
        b = p.buf_layer[0] == c.layer ? 0 : p.buf_layer[1] == c.layer ? 1 : -1;
        if (b < 0) {
            b = 1 - p.last;
            if ((e = upload(p, c, b, c.layer)) != hipSuccess) return e;
        }
    } else { // one buffer: each upload waits for the previous layer's compute
        b = 0;
        if (p.buf_layer[0] != c.layer && (e = upload(p, c, 0, c.layer)) != hipSuccess) return e;
    }
    if ((e = hipStreamWaitEvent(c.compute, p.loaded[b], 0)) != hipSuccess) return e;
    if (c.overlap) { // full-layer prefetch of the next layer into the other buffer
        const int nl = (c.layer + 1) % c.L, nb = 1 - b;
        if (p.buf_layer[nb] != nl && nl != c.layer)
            if ((e = upload(p, c, nb, nl)) != hipSuccess) return e;
    }
    const int n = c.T * c.k;
    hipStream_t s = c.compute;
    launch_route(c.logits, c.T, c.E, c.k, p.ids, p.w, s);
    const int nseg = (n + kSeg - 1) / kSeg;
    const size_t hist_lds = (size_t)c.E * sizeof(int32_t);
    hipLaunchKernelGGL(seg_count_kernel, dim3(nseg), dim3(64), hist_lds, s, p.ids, n, c.E, p.segc);
    hipLaunchKernelGGL(seg_scan_kernel, dim3(c.E), dim3(64), 0, s, p.segc, nseg, c.E, p.cnt);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, p.cnt, c.E, p.off, p.toff);
    hipLaunchKernelGGL(seg_place_kernel, dim3(nseg), dim3(64), hist_lds, s, p.ids, n, c.E, p.segc, p.off, p.perm);
    GemmArgs g{};
    g.wbuf = p.buf[b];
    g.expert_bytes = c.expert_bytes;
    const uint64_t hi = (uint64_t)c.H * c.I;
    if (c.wdtype == EC_DT_MXFP4) {
        g.off_a = 0; g.off_b = hi / 2; g.off_sa = 3 * hi / 2; g.off_sb = 3 * hi / 2 + hi / 32;
    } else {
        g.off_a = 0; g.off_b = hi * 2;
    }
    g.x = (const uint16_t*)c.x;
    g.act_out = p.act;
    g.act_in = p.act;
    g.y = p.y;
    g.cnt = p.cnt; g.off = p.off; g.toff = p.toff; g.perm = p.perm;
    g.E = c.E; g.k = c.k; g.H = c.H; g.I = c.I;
    // 1-D grids: eight ranges (one per XCD) of at most ceil(max_tiles * NT / 8) items each (see the
    // kernel's mapping); blocks past the call's items exit
    const int64_t max_tiles = (n + BM - 1) / BM + c.E;
    auto grid = [&](int N, int bn) { return dim3((unsigned)(8 * ((max_tiles * (N / bn) + 7) / 8))); };
    if (c.wdtype == EC_DT_MXFP4)
        hipLaunchKernelGGL((grouped_gemm_kernel<EC_DT_MXFP4, true, 64>), grid(c.I, 64), dim3(256), 0, s, g);
    else
        hipLaunchKernelGGL((grouped_gemm_kernel<EC_DT_BF16, true, 64>), grid(c.I, 64), dim3(256), 0, s, g);
    GemmArgs g2 = g;
    const bool wide = c.H % 128 == 0;
    if (c.wdtype == EC_DT_MXFP4) {
        g2.off_a = hi; g2.off_sa = 3 * hi / 2 + 2 * hi / 32;
        if (wide) hipLaunchKernelGGL((grouped_gemm_kernel<EC_DT_MXFP4, false, 128>), grid(c.H, 128), dim3(256), 0, s, g2);
        else hipLaunchKernelGGL((grouped_gemm_kernel<EC_DT_MXFP4, false, 64>), grid(c.H, 64), dim3(256), 0, s, g2);
    } else {
        g2.off_a = 4 * hi;
        if (wide) hipLaunchKernelGGL((grouped_gemm_kernel<EC_DT_BF16, false, 128>), grid(c.H, 128), dim3(256), 0, s, g2);
        else hipLaunchKernelGGL((grouped_gemm_kernel<EC_DT_BF16, false, 64>), grid(c.H, 64), dim3(256), 0, s, g2);
    }
    hipLaunchKernelGGL(combine_kernel, dim3(c.T, (c.H + 1023) / 1024), dim3(256), 0, s, p.y, p.w, c.k, c.H,
                       (uint16_t*)c.out);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipEventRecord(p.done[b], s)) != hipSuccess) return e;
    p.used[b] = true;
    p.last = b;
    return hipSuccess;
}

} // namespace ec
