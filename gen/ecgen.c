/*
 * Seeded synthetic inputs for the MoE expert-cache workloads.
 *
 * This file draws numbers and packs them into the byte layouts the library
 * consumes. It holds none of the layer's arithmetic (no routing, no SwiGLU,
 * no cache policy, no dequantisation): both the GPU path and the CPU oracle
 * take their inputs from here, and nothing else is shared between them.
 *
 * Random source: the splitmix64 generator (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014). Every stream is
 * addressed by a key derived from (seed, tag, a, b, c), and element i of a
 * stream is the i-th splitmix64 output for that key, so any slice of any
 * tensor can be regenerated on its own. Normals come from the Box-Muller
 * transform on the two 32-bit halves of one output.
 *
 * Workload structure follows the edge-MoE serving write-up (FreeToken,
 * "Why personal MoE is hard" and "Semantic-aware caching"): decode routing
 * has step-to-step expert overlap p, prefill routing covers almost every
 * expert.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ull

static inline uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* i-th output of the splitmix64 stream whose state starts at `key`. */
static inline uint64_t stream_u64(uint64_t key, uint64_t i) {
    return sm64_mix(key + (i + 1) * GOLDEN);
}

uint64_t ecg_key(uint64_t seed, uint64_t tag, uint64_t a, uint64_t b, uint64_t c) {
    uint64_t h = sm64_mix(seed + GOLDEN);
    h = sm64_mix(h ^ (tag + 1) * GOLDEN);
    h = sm64_mix(h ^ (a + 1) * 0xD1B54A32D192ED03ull);
    h = sm64_mix(h ^ (b + 1) * 0x8CB92BA72F3D8DD7ull);
    h = sm64_mix(h ^ (c + 1) * 0xABC98388FB8FAC03ull);
    return h;
}

static inline double u01_open(uint64_t h) { /* (0,1) from the high half */
    return ((double)(h >> 32) + 0.5) * (1.0 / 4294967296.0);
}

/* Box-Muller normal (continuous values; used where ties must be avoided). */
static inline double normal_bm(uint64_t key, uint64_t i) {
    uint64_t h = stream_u64(key, i);
    double u1 = u01_open(h);
    double u2 = (double)(h & 0xffffffffull) * (1.0 / 4294967296.0);
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

/* Fast normal for bulk tensors: each splitmix64 output gives four 16-bit
 * uniforms j, each mapped to the normal quantile z_j = Phi^-1((j + 1/2) / 65536)
 * (a 16-bit inverse-CDF table; |z| <= 4.33). Element i uses 16-bit lane i % 4
 * of output i / 4. */
static double g_qtab[65536];
static pthread_once_t g_qtab_once = PTHREAD_ONCE_INIT;

static double inv_norm_cdf(double p) {
    /* Rational start (Acklam) refined by two Halley steps on erfc. */
    static const double a[] = {-3.969683028665376e+01, 2.209460984245205e+02, -2.759285104469687e+02,
                               1.383577518672690e+02, -3.066479806614716e+01, 2.506628277459239e+00};
    static const double b[] = {-5.447609879822406e+01, 1.615858368580409e+02, -1.556989798598866e+02,
                               6.680131188771972e+01, -1.328068155288572e+01};
    static const double c[] = {-7.784894002430293e-03, -3.223964580411365e-01, -2.400758277161838e+00,
                               -2.549732539343734e+00, 4.374664141464968e+00, 2.938163982698783e+00};
    static const double d[] = {7.784695709041462e-03, 3.224671290700398e-01, 2.445134137142996e+00,
                               3.754408661907416e+00};
    double q, r, x;
    if (p < 0.02425) {
        q = sqrt(-2 * log(p));
        x = (((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
            ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1);
    } else if (p <= 1 - 0.02425) {
        q = p - 0.5;
        r = q * q;
        x = (((((a[0] * r + a[1]) * r + a[2]) * r + a[3]) * r + a[4]) * r + a[5]) * q /
            (((((b[0] * r + b[1]) * r + b[2]) * r + b[3]) * r + b[4]) * r + 1);
    } else {
        q = sqrt(-2 * log(1 - p));
        x = -(((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
            ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1);
    }
    for (int it = 0; it < 2; ++it) {
        double e = 0.5 * erfc(-x / sqrt(2.0)) - p;
        double u = e * sqrt(2 * 3.14159265358979323846) * exp(x * x / 2);
        x = x - u / (1 + x * u / 2);
    }
    return x;
}

static void qtab_init(void) {
    for (int j = 0; j < 65536; ++j) g_qtab[j] = inv_norm_cdf((j + 0.5) / 65536.0);
}

static inline void qtab_ready(void) { pthread_once(&g_qtab_once, qtab_init); }

static inline double normal_at(uint64_t key, uint64_t i) {
    uint64_t h = stream_u64(key, i >> 2);
    return g_qtab[(h >> (16 * (i & 3))) & 0xffff];
}

/* Uniform integer in [0, n) from one stream output (n << 2^32, bias < 2^-32*n). */
static inline uint32_t below(uint64_t key, uint64_t i, uint32_t n) {
    return (uint32_t)(((stream_u64(key, i) >> 32) * (uint64_t)n) >> 32);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* ---- tensor tags ---------------------------------------------------------- */
enum { TAG_GATE = 0, TAG_UP = 1, TAG_DOWN = 2, TAG_LOGIT = 10, TAG_X = 11, TAG_PLOGIT = 12,
       TAG_PX = 13, TAG_VEC = 14, TAG_ROUTER = 15 };
enum { DT_F32 = 0, DT_BF16 = 1, DT_MXFP4 = 2 };

/* Fill n normals N(0, sigma) of stream (seed, tag, a, b, c), starting at index i0. */
void ecg_normals_f64(uint64_t seed, uint64_t tag, uint64_t a, uint64_t b, uint64_t c,
                     uint64_t i0, int64_t n, double sigma, double* out) {
    qtab_ready();
    uint64_t key = ecg_key(seed, tag, a, b, c);
    for (int64_t i = 0; i < n; ++i) out[i] = sigma * normal_at(key, i0 + (uint64_t)i);
}

void ecg_normals_f32(uint64_t seed, uint64_t tag, uint64_t a, uint64_t b, uint64_t c,
                     int64_t n, double sigma, float* out) {
    qtab_ready();
    uint64_t key = ecg_key(seed, tag, a, b, c);
    #pragma omp parallel for schedule(static) if (n > 65536)
    for (int64_t i = 0; i < n; ++i) out[i] = (float)(sigma * normal_at(key, (uint64_t)i));
}

void ecg_normals_bf16(uint64_t seed, uint64_t tag, uint64_t a, uint64_t b, uint64_t c,
                      int64_t n, double sigma, uint16_t* out) {
    qtab_ready();
    uint64_t key = ecg_key(seed, tag, a, b, c);
    #pragma omp parallel for schedule(static) if (n > 65536)
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne((float)(sigma * normal_at(key, (uint64_t)i)));
}

/* ---- MXFP4 quantisation of a drawn weight matrix ---------------------------
 * OCP Microscaling (MX) v1.0: 32-element blocks along the contraction
 * dimension share one E8M0 exponent; elements are FP4 E2M1 codes (bit 3 sign,
 * magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 for codes 0..7). Shared exponent
 * s = floor(log2(amax)) - 2 (the OCP conversion rule with emax_elem = 2),
 * code = round-to-nearest-even(w / 2^s) on the E2M1 grid, saturating at 6. */
static inline uint8_t e2m1_rne_mag(double a) {
    /* thresholds are the midpoints of the grid; ties go to the even code */
    return (uint8_t)((a > 0.25) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) +
                     (a > 5.0));
}

/* One row of `cols` weights (cols % 32 == 0): codes[cols] (one code per byte,
 * unpacked) and scales[cols/32] (E8M0 bytes). */
static void quant_row_mxfp4(const double* w, int cols, uint8_t* codes, uint8_t* scales) {
    for (int b = 0; b < cols / 32; ++b) {
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) { double a = fabs(w[b * 32 + i]); amax = a > amax ? a : amax; }
        int s = 0;
        if (amax > 0.0) { int ex; frexp(amax, &ex); s = (ex - 1) - 2; }
        int e8 = s + 127;
        if (e8 < 0) e8 = 0;
        if (e8 > 254) e8 = 254;
        s = e8 - 127;
        scales[b] = (uint8_t)e8;
        double inv = ldexp(1.0, -s);
        for (int i = 0; i < 32; ++i) {
            double v = w[b * 32 + i] * inv;
            uint8_t mag = e2m1_rne_mag(fabs(v));
            codes[b * 32 + i] = (uint8_t)(mag | ((v < 0.0 && mag != 0) ? 8u : 0u));
        }
    }
}

/* cols draws (cols % 4 == 0) of stream `key` starting at element base (base % 4 == 0). */
static inline void draw_row(uint64_t key, uint64_t base, int cols, double sigma, double* w) {
    for (int c = 0; c < cols; c += 4) {
        uint64_t h = stream_u64(key, (base + (uint64_t)c) >> 2);
        w[c + 0] = sigma * g_qtab[h & 0xffff];
        w[c + 1] = sigma * g_qtab[(h >> 16) & 0xffff];
        w[c + 2] = sigma * g_qtab[(h >> 32) & 0xffff];
        w[c + 3] = sigma * g_qtab[(h >> 48) & 0xffff];
    }
}

/* ---- logical expert matrices ----------------------------------------------
 * Logical orientation: gate and up are [I][H] (row i = intermediate unit i),
 * down is [H][I]; the contraction dimension is the row (last) dimension.
 * Element (r, c) of tensor `tag` of expert (layer, expert) is element
 * r*cols + c of stream (seed, tag, layer, expert, 0). */
static void matrix_dims(int tag, int H, int I, int* rows, int* cols) {
    if (tag == TAG_DOWN) { *rows = H; *cols = I; } else { *rows = I; *cols = H; }
}

/* f32 (dtype 0) or bf16 (dtype 1) logical matrix. out: float* or uint16_t*. */
void ecg_expert_matrix(uint64_t seed, int dtype, int layer, int expert, int tag, int H, int I,
                       double sigma, void* out) {
    int rows, cols;
    matrix_dims(tag, H, I, &rows, &cols);
    int64_t n = (int64_t)rows * cols;
    if (dtype == DT_F32) ecg_normals_f32(seed, tag, layer, expert, 0, n, sigma, (float*)out);
    else ecg_normals_bf16(seed, tag, layer, expert, 0, n, sigma, (uint16_t*)out);
}

/* MXFP4 logical matrix: codes[rows][cols] unpacked, scales[rows][cols/32]. */
void ecg_expert_matrix_mxfp4(uint64_t seed, int layer, int expert, int tag, int H, int I,
                             double sigma, uint8_t* codes, uint8_t* scales) {
    qtab_ready();
    int rows, cols;
    matrix_dims(tag, H, I, &rows, &cols);
    uint64_t key = ecg_key(seed, tag, layer, expert, 0);
    #pragma omp parallel if ((int64_t)rows * cols > 65536)
    {
        double* w = (double*)malloc(sizeof(double) * cols);
        #pragma omp for schedule(static)
        for (int r = 0; r < rows; ++r) {
            draw_row(key, (uint64_t)r * cols, cols, sigma, w);
            quant_row_mxfp4(w, cols, codes + (int64_t)r * cols, scales + (int64_t)r * (cols / 32));
        }
        free(w);
    }
}

/* ---- packed expert bank -----------------------------------------------------
 * Byte layout of one expert (the library's expert-bank format):
 *   f32 / bf16 : [gate I*H][up I*H][down H*I] elements, each matrix row-major
 *                in its logical orientation.
 *   MXFP4      : [gate codes I*H/2][up codes I*H/2][down codes H*I/2]
 *                [gate scales I*H/32][up scales I*H/32][down scales H*I/32]
 *                codes packed two per byte along the row, even element in
 *                the low nibble; scales one byte per 32-element row block.
 * The pool is [L][E][expert bytes]. */
uint64_t ecg_expert_bytes(int dtype, int H, int I) {
    uint64_t n = (uint64_t)H * I;
    if (dtype == DT_F32) return 3 * n * 4;
    if (dtype == DT_BF16) return 3 * n * 2;
    return 3 * (n / 2) + 3 * (n / 32);
}

static void pack_expert(uint64_t seed, int dtype, int layer, int expert, int H, int I, double sigma,
                        uint8_t* dst) {
    uint64_t n = (uint64_t)H * I;
    int maxc = H > I ? H : I;
    double* w = (double*)malloc(sizeof(double) * maxc);
    uint8_t* codes = (uint8_t*)malloc(maxc);
    for (int tag = 0; tag < 3; ++tag) {
        int rows, cols;
        matrix_dims(tag, H, I, &rows, &cols);
        uint64_t key = ecg_key(seed, tag, layer, expert, 0);
        for (int r = 0; r < rows; ++r) {
            draw_row(key, (uint64_t)r * cols, cols, sigma, w);
            if (dtype == DT_F32) {
                float* o = (float*)(dst + tag * n * 4) + (uint64_t)r * cols;
                for (int c = 0; c < cols; ++c) o[c] = (float)w[c];
            } else if (dtype == DT_BF16) {
                uint16_t* o = (uint16_t*)(dst + tag * n * 2) + (uint64_t)r * cols;
                for (int c = 0; c < cols; ++c) o[c] = f32_to_bf16_rne((float)w[c]);
            } else {
                uint8_t* prow = dst + tag * (n / 2) + (uint64_t)r * (cols / 2);
                uint8_t* ps = dst + 3 * (n / 2) + tag * (n / 32) + (uint64_t)r * (cols / 32);
                quant_row_mxfp4(w, cols, codes, ps);
                for (int c = 0; c < cols; c += 2) prow[c / 2] = (uint8_t)(codes[c] | (codes[c + 1] << 4));
            }
        }
    }
    free(codes);
    free(w);
}

/* Pack experts of layers [l0, l1) into dst, which points at layer l0 of the
 * pool. Layer l of the pool is drawn as layer (l % layer_period) when
 * layer_period > 0 (aliasing keeps every byte distinct in memory but lets a
 * big pool be drawn once per period). */
void ecg_fill_pool(uint64_t seed, int dtype, int E, int H, int I, double sigma, int l0, int l1,
                   int layer_period, uint8_t* dst) {
    qtab_ready();
    uint64_t se = ecg_expert_bytes(dtype, H, I);
    uint64_t lbytes = se * (uint64_t)E;
    /* layers to draw: all of them, or (with aliasing) the first occurrence of each period slot */
    int64_t total = (int64_t)(l1 - l0) * E;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < total; ++j) {
        int l = l0 + (int)(j / E), e = (int)(j % E);
        if (layer_period > 0 && l >= l0 + layer_period) continue;
        int ls = layer_period > 0 ? l % layer_period : l;
        pack_expert(seed, dtype, ls, e, H, I, sigma, dst + (uint64_t)j * se);
    }
    if (layer_period > 0) {
        /* copy drawn layers into the aliased ones, in 64 MiB pieces */
        const uint64_t piece = 64ull << 20;
        int64_t nl = l1 - l0 - layer_period;
        if (nl > 0) {
            int64_t per = (int64_t)((lbytes + piece - 1) / piece);
            #pragma omp parallel for schedule(dynamic, 1)
            for (int64_t j = 0; j < nl * per; ++j) {
                int64_t li = layer_period + j / per;
                uint64_t off = (uint64_t)(j % per) * piece;
                uint64_t len = lbytes - off < piece ? lbytes - off : piece;
                int64_t src_i = li % layer_period; /* same residue mod the period, already drawn */
                memcpy(dst + (uint64_t)li * lbytes + off, dst + (uint64_t)src_i * lbytes + off, len);
            }
        }
    }
}

/* ---- decode routing logits with step-to-step overlap ----------------------
 * For each (layer, token) sequence over steps: keep n ~ Binomial(k, p)
 * experts picked at random from the previous step's chosen set, draw the
 * other k - n uniformly from the experts outside that set, then draw E
 * N(0,1) values and place the k largest on the chosen experts (random
 * order) and the rest on the others (random order). Step 0 chooses k
 * experts uniformly. logits: [steps][L][T][E] float32. */
static int cmp_desc(const void* a, const void* b) {
    double x = *(const double*)a, y = *(const double*)b;
    return (x < y) - (x > y);
}

void ecg_decode_logits(uint64_t seed, int steps, int L, int T, int E, int k, double p, float* logits) {
    #pragma omp parallel for schedule(dynamic, 1)
    for (int lt = 0; lt < L * T; ++lt) {
        int l = lt / T, t = lt % T;
        int* prev = (int*)malloc(sizeof(int) * k);
        int* cur = (int*)malloc(sizeof(int) * k);
        int* perm = (int*)malloc(sizeof(int) * E);
        char* mark = (char*)malloc(E);
        double* v = (double*)malloc(sizeof(double) * E);
        for (int s = 0; s < steps; ++s) {
            uint64_t key = ecg_key(seed, TAG_LOGIT, (uint64_t)l, (uint64_t)t, (uint64_t)s);
            uint64_t c = 0;
            memset(mark, 0, E);
            int n = 0;
            if (s > 0) {
                int keep = 0;
                for (int j = 0; j < k; ++j) keep += (u01_open(stream_u64(key, c++)) < p);
                /* the fresh draws come from the E - k experts outside the previous set: when fewer
                   remain than k - keep, the shortfall is kept from the previous set instead */
                if (k - keep > E - k) keep = 2 * k - E;
                /* partial Fisher-Yates over the previous set */
                for (int j = 0; j < keep; ++j) {
                    int r = j + (int)below(key, c++, (uint32_t)(k - j));
                    int tmp = prev[j]; prev[j] = prev[r]; prev[r] = tmp;
                    cur[n++] = prev[j];
                }
                for (int j = 0; j < k; ++j) mark[prev[j]] = 1; /* exclude the whole previous set */
            }
            /* uniform draws from the remaining experts (rejection) */
            while (n < k) {
                int e = (int)below(key, c++, (uint32_t)E);
                if (mark[e]) continue;
                mark[e] = 1;
                cur[n++] = e;
            }
            /* values: E normals sorted descending */
            for (int e = 0; e < E; ++e) v[e] = normal_bm(key, 1000000 + (uint64_t)e);
            qsort(v, E, sizeof(double), cmp_desc);
            /* random order of the chosen experts for the top-k values */
            for (int j = k - 1; j > 0; --j) {
                int r = (int)below(key, c++, (uint32_t)(j + 1));
                int tmp = cur[j]; cur[j] = cur[r]; cur[r] = tmp;
            }
            float* out = logits + (((int64_t)s * L + l) * T + t) * E;
            memset(mark, 0, E);
            for (int j = 0; j < k; ++j) { out[cur[j]] = (float)v[j]; mark[cur[j]] = 1; }
            int m = 0;
            for (int e = 0; e < E; ++e) if (!mark[e]) perm[m++] = e;
            for (int j = m - 1; j > 0; --j) {
                int r = (int)below(key, c++, (uint32_t)(j + 1));
                int tmp = perm[j]; perm[j] = perm[r]; perm[r] = tmp;
            }
            for (int j = 0; j < m; ++j) out[perm[j]] = (float)v[k + j];
            memcpy(prev, cur, sizeof(int) * k);
        }
        free(prev); free(cur); free(perm); free(mark); free(v);
    }
}
