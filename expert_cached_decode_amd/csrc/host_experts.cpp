// Host branch of the decode step: SwiGLU experts computed on host cores,
// reading the expert bank in host memory.
//
// FreeToken edge-MoE write-up, "Bandwidth-adaptive execution" (decode): the
// misses not filled into the GPU cache are executed directly on the CPU,
// leaving residency unchanged; host and GPU partial sums are merged exactly.
// Work is split over worker threads by (expert, block of rows): the gate/up
// rows of every host-list expert (activations of every token routed to it),
// then the down rows, each expert's down rows as soon as its own gate/up rows
// are done (no barrier across experts), so each weight byte is read from host
// memory once per step.
// bf16 and MXFP4 rows use the host's AVX-512 bf16 dot unit when it has one
// (the SwiGLU activations are then rounded to bf16, as on the GPU), else AVX2.
#include "host_experts.h"

#include <immintrin.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

namespace ec {

namespace {

inline float bf16f(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// FP4 E2M1 magnitudes (OCP MX v1.0), signed by bit 3.
const float kE2M1[16] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f,
                         -0.f, -0.5f, -1.f, -1.5f, -2.f, -3.f, -4.f, -6.f};

inline float e8m0(uint8_t e) {
    uint32_t u = e ? (uint32_t)e << 23 : 0x00400000u;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// dot(row, v) over n elements; row in the bank's format (MXFP4: codes + scale row)
float dot_row(int wdt, const uint8_t* row, const uint8_t* srow, const float* v, int n) {
    float acc[16] = {0};
    if (wdt == 0) {
        const float* w = reinterpret_cast<const float*>(row);
        for (int i = 0; i < n; i += 16)
            for (int q = 0; q < 16; ++q) acc[q] += w[i + q] * v[i + q];
    } else if (wdt == 1) {
        const uint16_t* w = reinterpret_cast<const uint16_t*>(row);
        for (int i = 0; i < n; i += 16)
            for (int q = 0; q < 16; ++q) acc[q] += bf16f(w[i + q]) * v[i + q];
    } else {
        // 32 codes per block: nibbles in element order (low nibble = even element), looked up
        // eight at a time in the E2M1 magnitude table with the sign bit applied separately,
        // times the activations, then the block sum times its E8M0 scale
        const __m256 lut = _mm256_loadu_ps(kE2M1);
        const __m256i seven = _mm256_set1_epi32(7), eight = _mm256_set1_epi32(8);
        const __m128i lo_mask = _mm_set1_epi8(0x0f);
        __m256 tot = _mm256_setzero_ps();
        for (int b = 0; b < n / 32; ++b) {
            const __m128i raw = _mm_loadu_si128(reinterpret_cast<const __m128i*>(row + b * 16));
            const __m128i lo = _mm_and_si128(raw, lo_mask), hi = _mm_and_si128(_mm_srli_epi16(raw, 4), lo_mask);
            const __m128i e0 = _mm_unpacklo_epi8(lo, hi), e1 = _mm_unpackhi_epi8(lo, hi); // elements 0..15, 16..31
            const float* vb = v + b * 32;
            __m256 blk = _mm256_setzero_ps();
            const __m128i parts[4] = {e0, _mm_srli_si128(e0, 8), e1, _mm_srli_si128(e1, 8)};
            for (int g = 0; g < 4; ++g) {
                const __m256i idx = _mm256_cvtepu8_epi32(parts[g]);
                __m256 w = _mm256_permutevar8x32_ps(lut, _mm256_and_si256(idx, seven));
                const __m256i sgn = _mm256_slli_epi32(_mm256_and_si256(idx, eight), 28);
                w = _mm256_xor_ps(w, _mm256_castsi256_ps(sgn));
                blk = _mm256_fmadd_ps(w, _mm256_loadu_ps(vb + 8 * g), blk);
            }
            tot = _mm256_fmadd_ps(blk, _mm256_set1_ps(e8m0(srow[b])), tot);
        }
        alignas(32) float t8[8];
        _mm256_store_ps(t8, tot);
        for (int q = 0; q < 8; ++q) acc[q] += t8[q];
    }
    float s = 0.f;
    for (int q = 0; q < 16; ++q) s += acc[q];
    return s;
}

// ---- AVX-512 BF16 path (the host's bf16 dot-product unit), chosen at run time ----
#define EC_BF16_TARGET __attribute__((target("avx512f,avx512bw,avx512vl,avx512bf16")))

bool host_has_bf16_dot() {
#ifdef EC_HOST_NO_BF16_DOT // test builds that exercise the AVX2 path on a host with the bf16 unit
    return false;
#else
    static const bool ok = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
                           __builtin_cpu_supports("avx512bf16");
    return ok;
#endif
}

// dot of n bf16 weights with n bf16 activations (n a multiple of 64); products exact in fp32
EC_BF16_TARGET float dot_bf16_bf16(const uint16_t* w, const uint16_t* x, int n) {
    __m512 a0 = _mm512_setzero_ps(), a1 = _mm512_setzero_ps();
    for (int i = 0; i < n; i += 64) {
        a0 = _mm512_dpbf16_ps(a0, (__m512bh)_mm512_loadu_si512(w + i), (__m512bh)_mm512_loadu_si512(x + i));
        a1 = _mm512_dpbf16_ps(a1, (__m512bh)_mm512_loadu_si512(w + i + 32),
                              (__m512bh)_mm512_loadu_si512(x + i + 32));
    }
    return _mm512_reduce_add_ps(_mm512_add_ps(a0, a1));
}

// bf16 bit patterns of the 16 E2M1 codes (bit 3 the sign), OCP MX v1.0
alignas(64) const uint16_t kE2M1Bf16[32] = {0x0000, 0x3F00, 0x3F80, 0x3FC0, 0x4000, 0x4040, 0x4080, 0x40C0,
                                            0x8000, 0xBF00, 0xBF80, 0xBFC0, 0xC000, 0xC040, 0xC080, 0xC0C0};

// MXFP4 row (codes + E8M0 scales) with n bf16 activations: each 32-code block becomes 32 bf16
// weights by table lookup, its scale 2^(s-127) added to their exponent fields (exact while the
// results stay normal: 2 <= s <= 252, checked by the caller), then the bf16 dot unit
EC_BF16_TARGET float dot_mx_bf16(const uint8_t* codes, const uint8_t* sc, const uint16_t* x, int n) {
    const __m512i lut = _mm512_load_si512(kE2M1Bf16);
    const __m128i lo_mask = _mm_set1_epi8(0x0f);
    __m512 acc = _mm512_setzero_ps();
    for (int b = 0; b < n / 32; ++b) {
        const __m128i raw = _mm_loadu_si128(reinterpret_cast<const __m128i*>(codes + 16 * b));
        const __m128i lo = _mm_and_si128(raw, lo_mask), hi = _mm_and_si128(_mm_srli_epi16(raw, 4), lo_mask);
        const __m256i el = _mm256_set_m128i(_mm_unpackhi_epi8(lo, hi), _mm_unpacklo_epi8(lo, hi));
        __m512i w = _mm512_permutexvar_epi16(_mm512_cvtepu8_epi16(el), lut);
        const __mmask32 nz = _mm512_test_epi16_mask(w, _mm512_set1_epi16(0x7fff));
        w = _mm512_mask_add_epi16(w, nz, w, _mm512_set1_epi16((int16_t)(((int)sc[b] - 127) * 128)));
        acc = _mm512_dpbf16_ps(acc, (__m512bh)w, (__m512bh)_mm512_loadu_si512(x + 32 * b));
    }
    return _mm512_reduce_add_ps(acc);
}

bool scales_in_range(const uint8_t* sc, int nblocks) {
    for (int b = 0; b < nblocks; ++b)
        if (sc[b] < 2 || sc[b] > 252) return false;
    return true;
}

inline uint16_t bf16_rne(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// dot of a weight row with activations held both as f32 (v) and as bf16 (vb, or null)
inline float dot_row_any(int wdt, const uint8_t* row, const uint8_t* srow, const float* v, const uint16_t* vb,
                         int n) {
    if (vb && wdt == 1) return dot_bf16_bf16(reinterpret_cast<const uint16_t*>(row), vb, n);
    if (vb && wdt == 2 && scales_in_range(srow, n / 32)) return dot_mx_bf16(row, srow, vb, n);
    return dot_row(wdt, row, srow, v, n);
}

} // namespace

struct HostPool {
    std::vector<std::thread> threads;
    std::mutex mu;
    std::condition_variable cv;
    std::atomic<uint64_t> generation{0}; // bumped (under mu) for every job
    std::atomic<bool> stop{false};
    const HostJob* job = nullptr;
    // phase bookkeeping
    std::vector<int> task_expert, task_r0;   // phase-1 and phase-2 task tables
    std::vector<std::vector<int>> pairs_of;  // host index -> pairs
    std::vector<float> xf;                   // [T][H] activations widened to f32
    std::vector<uint16_t> act_b;             // [T*k][I] SwiGLU activations rounded to bf16 (bf16 dot path)
    bool bf16dot = false;                    // bf16/MXFP4 weights on a host with the bf16 dot unit
    int n1 = 0, n2 = 0;
    std::atomic<int> next1{0}, next2{0}, arrived{0};
    // per host-list expert: its gate/up tasks not yet finished (a down task of the expert waits
    // for zero; the tasks it waits for have all been claimed, so the wait ends)
    std::unique_ptr<std::atomic<int>[]> left1{new std::atomic<int>[1024]};
    int nworkers = 0;
    // Rows per task, gate/up and down alike: the power of two (8 to 256) giving at most 512 KiB of
    // gate + up weight codes per task. Measured on a 16-core host with 14 workers at a fixed 300:1000 split:
    // 64 rows best for bf16 rows of 2048 (about 2% over 32 and 128), 128 for MXFP4 rows of 4096
    // (12% over 32); 8-row tasks lost 20-35%.
    int rows = 32;
    static int task_rows(uint64_t row_bytes_h) {
        int r = 8;
        while (r < 256 && 4ull * r * row_bytes_h <= (512ull << 10)) r *= 2;
        return r;
    }

    void work() {
        const HostJob& j = *job;
        const int H = j.H, I = j.I;
        const uint64_t rbH = j.wdtype == 0 ? H * 4ull : j.wdtype == 1 ? H * 2ull : H / 2;
        const uint64_t rbI = j.wdtype == 0 ? I * 4ull : j.wdtype == 1 ? I * 2ull : I / 2;
        // phase 1: gate/up rows -> act
        for (int t; (t = next1.fetch_add(1)) < n1;) {
            const int e = task_expert[t], r0 = task_r0[t];
            const uint8_t* base = j.expert_base[e];
            const uint8_t* gsc = base + 3ull * I * rbH;
            const uint8_t* usc = gsc + (uint64_t)I * (H / 32);
            for (int i = r0; i < r0 + rows && i < I; ++i) {
                const uint8_t* g = base + i * rbH;
                const uint8_t* u = base + (uint64_t)I * rbH + i * rbH;
                for (int p : pairs_of[e]) {
                    const float* xv = xf.data() + (uint64_t)(p / j.k) * H;
                    const uint16_t* xb = bf16dot ? reinterpret_cast<const uint16_t*>(j.x) + (uint64_t)(p / j.k) * H
                                                 : nullptr;
                    float gv = dot_row_any(j.wdtype, g, gsc + (uint64_t)i * (H / 32), xv, xb, H);
                    float uv = dot_row_any(j.wdtype, u, usc + (uint64_t)i * (H / 32), xv, xb, H);
                    const float hv = gv / (1.f + std::exp(-gv)) * uv;
                    j.act[(uint64_t)p * I + i] = hv;
                    if (bf16dot) act_b[(uint64_t)p * I + i] = bf16_rne(hv);
                }
            }
            left1[e].fetch_sub(1, std::memory_order_release);
        }
        // phase 2: down rows -> y, each task once its expert's activations are complete
        for (int t; (t = next2.fetch_add(1)) < n2;) {
            const int e = task_expert[n1 + t], r0 = task_r0[n1 + t];
            while (left1[e].load(std::memory_order_acquire) > 0) _mm_pause();
            const uint8_t* base = j.expert_base[e];
            const uint8_t* d = base + 2ull * I * rbH;
            const uint8_t* dsc = base + 3ull * I * rbH + 2ull * I * (H / 32);
            for (int h = r0; h < r0 + rows && h < H; ++h)
                for (int p : pairs_of[e])
                    j.y[((uint64_t)(p / j.k) * H + h) * j.k + p % j.k] =
                        dot_row_any(j.wdtype, d + h * rbI, dsc + (uint64_t)h * (I / 32), j.act + (uint64_t)p * I,
                                    bf16dot ? act_b.data() + (uint64_t)p * I : nullptr, I);
        }
    }

    // After a job a worker spins for kSpin on the generation counter before it sleeps on the
    // condition variable: during decode the next layer's job arrives well within that, so the
    // workers start it without a wake-up; an idle context still sleeps.
    static constexpr std::chrono::microseconds kSpin{2000};
    void loop() {
        uint64_t seen = 0;
        for (;;) {
            const auto t0 = std::chrono::steady_clock::now();
            bool woke = false;
            for (uint32_t i = 0;; ++i) {
                if (stop.load(std::memory_order_acquire)) return;
                if (generation.load(std::memory_order_acquire) != seen) { woke = true; break; }
                _mm_pause();
                if ((i & 255) == 255 && std::chrono::steady_clock::now() - t0 > kSpin) break;
            }
            if (!woke) {
                std::unique_lock<std::mutex> lk(mu);
                cv.wait(lk, [&] { return stop.load() || generation.load() != seen; });
                if (stop.load()) return;
            }
            seen = generation.load(std::memory_order_acquire);
            work();
            arrived.fetch_add(1, std::memory_order_release);
        }
    }
};

HostPool* host_pool_create(int threads) {
    HostPool* p = new HostPool();
    p->nworkers = threads > 1 ? threads - 1 : 0; // the calling thread works too
    for (int i = 0; i < p->nworkers; ++i) p->threads.emplace_back([p] { p->loop(); });
    return p;
}

void host_pool_destroy(HostPool* p) {
    {
        std::lock_guard<std::mutex> lk(p->mu);
        p->stop.store(true, std::memory_order_release);
    }
    p->cv.notify_all();
    for (auto& t : p->threads) t.join();
    delete p;
}

void host_pool_run(HostPool* p, const HostJob& j) {
    if (j.n_experts <= 0) return;
    p->job = &j;
    p->pairs_of.assign(j.n_experts, {});
    for (int i = 0; i < j.T * j.k; ++i)
        if (j.rewritten[i] < 0) {
            int h = -j.rewritten[i] - 1;
            if (h < j.n_experts) p->pairs_of[h].push_back(i);
        }
    // bf16 and MXFP4 weights meet bf16 activations in the bf16 dot unit when the host has one:
    // x is bf16 already, the SwiGLU activations are rounded to bf16 as on the GPU
    p->bf16dot = j.wdtype != 0 && host_has_bf16_dot();
    if (p->bf16dot) p->act_b.resize((size_t)j.T * j.k * j.I);
    p->xf.resize((size_t)j.T * j.H);
    for (size_t i = 0; i < p->xf.size(); ++i)
        p->xf[i] = j.wdtype == 0 ? reinterpret_cast<const float*>(j.x)[i]
                                 : bf16f(reinterpret_cast<const uint16_t*>(j.x)[i]);
    p->rows = HostPool::task_rows(j.wdtype == 0 ? j.H * 4ull : j.wdtype == 1 ? j.H * 2ull : j.H / 2ull);
    p->task_expert.clear();
    p->task_r0.clear();
    for (int e = 0; e < j.n_experts; ++e)
        for (int r = 0; r < j.I; r += p->rows) { p->task_expert.push_back(e); p->task_r0.push_back(r); }
    p->n1 = (int)p->task_expert.size();
    for (int e = 0; e < j.n_experts; ++e)
        for (int r = 0; r < j.H; r += p->rows) { p->task_expert.push_back(e); p->task_r0.push_back(r); }
    p->n2 = (int)p->task_expert.size() - p->n1;
    const int per_expert = (j.I + p->rows - 1) / p->rows;
    for (int e = 0; e < j.n_experts; ++e) p->left1[e].store(per_expert, std::memory_order_relaxed);
    p->next1 = 0; p->next2 = 0; p->arrived = 0;
    {
        std::lock_guard<std::mutex> lk(p->mu);
        p->generation.fetch_add(1, std::memory_order_release);
    }
    p->cv.notify_all();
    p->work();
    while (p->arrived.load(std::memory_order_acquire) < p->nworkers) std::this_thread::yield();
    p->job = nullptr;
}

} // namespace ec
