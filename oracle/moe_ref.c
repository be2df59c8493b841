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

/* element (r, c) of a [rows][cols] matrix in format wfmt */
static double weight_at(int wfmt, const void* w, const uint8_t* sc, int cols, int64_t r, int64_t c) {
    int64_t i = r * cols + c;
    if (wfmt == 0) return (double)((const float*)w)[i];
    if (wfmt == 1) return bf16_value(((const uint16_t*)w)[i]);
    double v = e2m1_value(((const uint8_t*)w)[i]);
    int e = (int)sc[r * (cols / 32) + c / 32] - 127;
    return ldexp(v, e);
}

void oracle_decode_weights(int wfmt, const void* w, const uint8_t* sc, int rows, int cols, double* out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) out[r * cols + c] = weight_at(wfmt, w, sc, cols, r, c);
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* y[H] = f_e(x) for one expert and one token. act[I] receives the SwiGLU
 * activation silu(gate x) * (up x) (optional, may be NULL). */
void oracle_expert(int wfmt, int H, int I, const void* wg, const uint8_t* sg, const void* wu,
                   const uint8_t* su, const void* wd, const uint8_t* sd, const double* x, double* y,
                   double* act_out) {
    double* act = act_out;
    #pragma omp parallel for schedule(static)
    for (int i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int h = 0; h < H; ++h) {
            g += weight_at(wfmt, wg, sg, H, i, h) * x[h];
            u += weight_at(wfmt, wu, su, H, i, h) * x[h];
        }
        act[i] = silu(g) * u;
    }
    #pragma omp parallel for schedule(static)
    for (int h = 0; h < H; ++h) {
        double s = 0.0;
        for (int i = 0; i < I; ++i) s += weight_at(wfmt, wd, sd, I, h, i) * act[i];
        y[h] = s;
    }
}
