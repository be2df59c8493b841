/*
 * Reference MoE expert layer: plain loops, fp64 throughout.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): never linked into the
 * product library.
 *
 * The FreeToken write-up ("Bandwidth-adaptive execution") states that the
 * cache-side and host-side partial sums are merged exactly and that the
 * method adds no algorithmic approximation ("Related work": routing stays
 * exact, the model is unchanged). So the layer output is just the definition
 * of a SwiGLU mixture of experts, with no cache at all:
 *
 *   out[t] = sum_j w[t,j] * f_{e[t,j]}(x_t)
 *   f_e(x) = W_down,e ( silu(W_gate,e x) * (W_up,e x) ),  silu(z) = z / (1 + exp(-z))
 *
 * W_gate and W_up are [I][H], W_down is [H][I] (logical orientation). Weights
 * are widened exactly to fp64: f32 and bf16 values directly; an MXFP4 element
 * is its FP4 E2M1 value times 2^(scale - 127) (OCP Microscaling v1.0: E2M1
 * has 1 sign bit, 2 exponent bits with bias 1 and 1 mantissa bit; E8M0 is an
 * unsigned power-of-two exponent with bias 127). Nothing is rounded between
 * steps.
 *
 * Weight formats (wfmt): 0 = float32, 1 = bf16 bit patterns (uint16),
 * 2 = MXFP4 with one code per byte (unpacked) plus a scale byte per 32
 * consecutive elements of a row.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* FP4 E2M1 code -> value, from the field definition (not a lookup table). */
static double e2m1_value(unsigned code) {
    unsigned sign = (code >> 3) & 1u, exp = (code >> 1) & 3u, man = code & 1u;
    double mag = exp == 0 ? 0.5 * man                      /* subnormal: m * 2^(1-bias) / 2 */
                          : ldexp(1.0 + 0.5 * man, (int)exp - 1);
    return sign ? -mag : mag;
}

static double bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Row r of a [rows][cols] weight matrix in format wfmt, widened exactly to
 * fp64: f32 and bf16 values directly; MXFP4 element c is its E2M1 value times
 * 2^(scale - 127), the scale byte being that of the row's block of 32
 * elements containing c. */
static void widen_row(int wfmt, const void* w, const uint8_t* sc, int cols, int64_t r, double* out) {
    if (wfmt == 0) {
        const float* p = (const float*)w + r * cols;
        for (int c = 0; c < cols; ++c) out[c] = (double)p[c];
    } else if (wfmt == 1) {
        const uint16_t* p = (const uint16_t*)w + r * cols;
        for (int c = 0; c < cols; ++c) out[c] = bf16_value(p[c]);
    } else {
        /* the 16 code values from the field definition; scaling one of them by the block's
         * power of two is exact (at most 2 significant bits, exponent within fp64's range) */
        double val[16];
        for (unsigned code = 0; code < 16; ++code) val[code] = e2m1_value(code);
        const uint8_t* p = (const uint8_t*)w + r * cols;
        for (int c0 = 0; c0 < cols; c0 += 32) {
            const double scale = ldexp(1.0, (int)sc[r * (cols / 32) + c0 / 32] - 127);
            for (int c = c0; c < c0 + 32; ++c) out[c] = val[p[c] & 15u] * scale;
        }
    }
}

void oracle_decode_weights(int wfmt, const void* w, const uint8_t* sc, int rows, int cols, double* out) {
    for (int64_t r = 0; r < rows; ++r) widen_row(wfmt, w, sc, cols, r, out + r * cols);
}

/* y[H] = f_e(x) for one expert and one token. act[I] receives the SwiGLU
 * activation silu(gate x) * (up x) (optional, may be NULL). Each dot product
 * runs over the contraction index in ascending order. */
void oracle_expert(int wfmt, int H, int I, const void* wg, const uint8_t* sg, const void* wu,
                   const uint8_t* su, const void* wd, const uint8_t* sd, const double* x, double* y,
                   double* act_out) {
    double* act = act_out;
    #pragma omp parallel
    {
        double* rg = (double*)malloc(sizeof(double) * (size_t)(H > I ? H : I));
        double* ru = (double*)malloc(sizeof(double) * (size_t)H);
        #pragma omp for schedule(static)
        for (int i = 0; i < I; ++i) {
            widen_row(wfmt, wg, sg, H, i, rg);
            widen_row(wfmt, wu, su, H, i, ru);
            double g = 0.0, u = 0.0;
            for (int h = 0; h < H; ++h) {
                g += rg[h] * x[h];
                u += ru[h] * x[h];
            }
            act[i] = silu(g) * u;
        }
        /* (the implicit barrier of the loop above: every act[i] is written before it is read) */
        #pragma omp for schedule(static)
        for (int h = 0; h < H; ++h) {
            widen_row(wfmt, wd, sd, I, h, rg);
            double s = 0.0;
            for (int i = 0; i < I; ++i) s += rg[i] * act[i];
            y[h] = s;
        }
        free(rg);
        free(ru);
    }
}
