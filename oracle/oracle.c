/*
 * oracle.c -- plain CPU reference of the per-layer MoE FFN (fp64, per-token loops).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the HIP library or its binding.
 * Shares nothing with the HIP sources.  The operations and the readings they
 * follow are listed in oracle.h; each function below restates its definition.
 *
 * Build: gcc -O3 -fno-fast-math -fno-semantic-interposition -fopenmp -shared -fPIC
 *        -std=c11 oracle.c -o liboracle.so -lm  (ISO C: no floating-point contraction)
 */
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* ---- scalar formats ---------------------------------------------------- */

/* bf16 is the top half of an IEEE binary32; widening is exact. */
double or_bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a double to the nearest bf16 (ties to even), handling subnormals and
 * overflow to infinity.  A bf16 number has 8 significant bits (7 stored); its
 * smallest normal is 2^-126 and its smallest subnormal 2^-133. */
uint16_t or_f64_to_bf16(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int e;
    double m = frexp(a, &e);              /* a = m * 2^e, 0.5 <= m < 1 */
    int bits = 8;                          /* significant bits kept */
    if (e < -125) bits = 8 - (-125 - e);  /* below the normal range */
    double r = nearbyint(ldexp(m, bits)); /* default rounding mode: ties to even */
    double q = ldexp(r, e - bits);
    if (q >= 0x1p128) return sign | 0x7F80;
    float f = (float)q;                    /* exact: q has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (u >> 16));
}

/* e2m1 code c (bit 3 sign, bits 2..1 exponent, bit 0 mantissa) times the
 * e8m0 scale 2^(X-127); X = 255 is NaN.  Exponent field 0 is the subnormal
 * 0.5*m, otherwise 2^(E-1) * (1 + m/2).  OCP Microscaling Formats v1.0. */
double or_mxfp4_value(uint8_t code, uint8_t scale) {
    if (scale == 0xFF) return NAN;
    int s = (code >> 3) & 1, ex = (code >> 1) & 3, m = code & 1;
    double mag = (ex == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, ex - 1);
    double v = ldexp(mag, (int)scale - 127);
    return s ? -v : v;
}

/* e4m3 code c (bit 7 sign, bits 6..3 exponent, bits 2..0 mantissa), the OCP
 * 8-bit floating point "E4M3" encoding: bias 7, no infinities, exponent and
 * mantissa fields all ones is NaN.  Exponent field 0 is the subnormal
 * 2^-6 * m/8, otherwise 2^(E-7) * (1 + m/8).  OCP 8-bit Floating Point
 * Specification (OFP8) v1.0. */
double or_fp8_value(uint8_t code) {
    int s = code >> 7, ex = (code >> 3) & 15, m = code & 7;
    if (ex == 15 && m == 7) return NAN;
    double mag = (ex == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, ex - 7);
    return s ? -mag : mag;
}

/* e2m1 code times an e4m3 block scale: the two element formats above, the
 * code with the neutral e8m0 exponent 127 (a factor of 1). */
double or_nvfp4_value(uint8_t code, uint8_t scale) {
    return or_mxfp4_value(code, 127) * or_fp8_value(scale);
}

/* Decode tables: the values of the functions above for every code, filled
 * once when the library is loaded.  They only cache those exact fp64 values
 * (the per-element ldexp calls made the narrow formats some ten times slower
 * than bf16); a pin compares every entry with its function.
 *   g_e2m1[c]  = or_mxfp4_value(c, 127)   (the e2m1 value, scale 2^0)
 *   g_pow2[X]  = 2^(X - 127)              (the e8m0 scale; NaN for X = 255)
 *   g_fp8[c]   = or_fp8_value(c) */
static double g_e2m1[16], g_pow2[256], g_fp8[256];

__attribute__((constructor)) static void or_fill_tables(void) {
    for (int c = 0; c < 16; ++c) g_e2m1[c] = or_mxfp4_value((uint8_t)c, 127);
    for (int X = 0; X < 256; ++X) g_pow2[X] = X == 255 ? NAN : ldexp(1.0, X - 127);
    for (int c = 0; c < 256; ++c) g_fp8[c] = or_fp8_value((uint8_t)c);
}

/* the cached values, for the pins */
double or_table_e2m1(uint8_t code) { return g_e2m1[code & 15]; }
double or_table_pow2(uint8_t X) { return g_pow2[X]; }
double or_table_fp8(uint8_t code) { return g_fp8[code]; }

/* element (row, kk) of a [rows][K] matrix stored in fmt (ts: the tensor scale
 * of an NVFP4 matrix).  MXFP4: e2m1 value times 2^(X-127); NVFP4: e2m1 value
 * times the e4m3 block scale times the tensor scale; FP8: e4m3 value times the
 * matrix scale.  Every product of table values here is exact in fp64. */
static double w_at(const void* base, const uint8_t* sc, const uint8_t* ts, int fmt, int row, int K,
                   int kk) {
    size_t r = (size_t)row;
    if (fmt == OR_F32) return ((const float*)base)[r * K + kk];
    if (fmt == OR_BF16) return or_bf16_to_f64(((const uint16_t*)base)[r * K + kk]);
    if (fmt == OR_FP8) {  /* code times the matrix's fp32 scale (sc points at it) */
        float scale;
        memcpy(&scale, sc, 4);
        return g_fp8[((const uint8_t*)base)[r * K + kk]] * (double)scale;
    }
    uint8_t byte = ((const uint8_t*)base)[r * (K / 2) + kk / 2];
    uint8_t c = (kk & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
    if (fmt == OR_NVFP4) {
        float tensor;
        memcpy(&tensor, ts, 4);
        return g_e2m1[c] * g_fp8[sc[r * (K / 16) + kk / 16]] * (double)tensor;
    }
    return g_e2m1[c] * g_pow2[sc[r * (K / 32) + kk / 32]];
}

static double act_at(const void* x, int fmt, int t, int H, int h) {
    if (fmt == OR_F32) return ((const float*)x)[(size_t)t * H + h];
    return or_bf16_to_f64(((const uint16_t*)x)[(size_t)t * H + h]);
}

/* ---- router --------------------------------------------------------------- */

int or_router_logits(const void* x, const void* wr, int fmt, int T, int H, int E,
                     float* logits) {
    if (fmt != OR_F32 && fmt != OR_BF16) return -1;
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int h = 0; h < H; ++h) s += act_at(x, fmt, t, H, h) * act_at(wr, fmt, e, H, h);
            logits[(size_t)t * E + e] = (float)s;
        }
    return 0;
}

/* The j-th pick is the largest remaining biased logit; among equal values the
 * lower expert id is picked first (IEEE compare, so -0 equals +0).  Gates are
 * the softmax over all E experts restricted to the picks and renormalised,
 * which equals the softmax over the k picked logits. */
int or_route(const float* logits, const float* bias, int T, int E, int k,
             int32_t* ids, float* w) {
    if (k < 1 || k > E) return -1;
    float* lp = (float*)malloc(sizeof(float) * (size_t)E);
    char* taken = (char*)malloc((size_t)E);
    int rc = 0;
    for (int t = 0; t < T && rc == 0; ++t) {
        for (int e = 0; e < E; ++e) {
            float l = logits[(size_t)t * E + e];
            lp[e] = bias ? l + bias[e] : l; /* one binary32 addition */
            if (!isfinite(lp[e])) rc = -2;
            taken[e] = 0;
        }
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || lp[e] > lp[best]) best = e;
            }
            taken[best] = 1;
            ids[(size_t)t * k + j] = best;
        }
        double m = lp[ids[(size_t)t * k]];
        double s = 0.0;
        for (int j = 0; j < k; ++j) s += exp((double)lp[ids[(size_t)t * k + j]] - m);
        for (int j = 0; j < k; ++j)
            w[(size_t)t * k + j] = (float)(exp((double)lp[ids[(size_t)t * k + j]] - m) / s);
    }
    free(lp);
    free(taken);
    return rc;
}

/* ---- alignment ------------------------------------------------------------- */

/* counts[e] = number of (t, j) routed to e; offsets = exclusive prefix sum;
 * perm lists the flat slots f = t*k + j of expert 0, then expert 1, ..., each
 * group in increasing f; inv_perm is its inverse. */
int or_align(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
             int32_t* perm, int32_t* inv_perm) {
    long n = (long)T * k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (long f = 0; f < n; ++f) {
        if (ids[f] < 0 || ids[f] >= E) return -1;
        counts[ids[f]]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    long p = 0;
    for (int e = 0; e < E; ++e)
        for (long f = 0; f < n; ++f)
            if (ids[f] == e) perm[p++] = (int32_t)f;
    for (long q = 0; q < n; ++q) inv_perm[perm[q]] = (int32_t)q;
    return 0;
}

/* ---- expert FFN -------------------------------------------------------------- */

/* SwiGLU expert: g = Wg x, u = Wu x, h = silu(g) * u with silu(z) = z/(1+e^-z),
 * y = Wd h.  Sums in fp64; h optionally rounded to bf16 (the down projection
 * consumes a bf16 activation when weights are bf16 or MXFP4). */
int or_expert_ffn(const or_expert* ex, const double* x, int H, int I, int round_h,
                  double* y) {
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    for (int i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int c = 0; c < H; ++c) {
            g += x[c] * w_at(ex->gate, ex->gate_sc, ex->gate_ts, ex->fmt, i, H, c);
            u += x[c] * w_at(ex->up, ex->up_sc, ex->up_ts, ex->fmt, i, H, c);
        }
        double a = g / (1.0 + exp(-g)) * u;
        h[i] = round_h ? or_bf16_to_f64(or_f64_to_bf16(a)) : a;
    }
    for (int d = 0; d < H; ++d) {
        double s = 0.0;
        for (int i = 0; i < I; ++i) s += h[i] * w_at(ex->down, ex->down_sc, ex->down_ts, ex->fmt, d, I, i);
        y[d] = s;
    }
    free(h);
    return 0;
}

/* ---- whole layer ---------------------------------------------------------------- */

/* out[t] = sum_j w[t,j] * FFN_{ids[t,j]}(x[t]) (+ FFN_shared(x[t])), fp64, one rounding. */
int or_moe_layer(const void* x, int x_fmt, int T, int H, int I, int E, int k,
                 const int32_t* ids, const float* w, const or_expert* experts,
                 const or_expert* shared, int round_h, int out_fmt, void* out,
                 const int32_t* tokens, int n_tokens, int nthreads) {
    if (!tokens && n_tokens != T) return -1;
    int bad = 0;
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
    for (int i = 0; i < n_tokens; ++i) {
        int t = tokens ? tokens[i] : i;
        double* xr = (double*)malloc(sizeof(double) * (size_t)H);
        double* y = (double*)malloc(sizeof(double) * (size_t)H);
        double* acc = (double*)calloc((size_t)H, sizeof(double));
        for (int c = 0; c < H; ++c) xr[c] = act_at(x, x_fmt, t, H, c);
        for (int j = 0; j < k; ++j) {
            int e = ids[(size_t)t * k + j];
            if (e < 0 || e >= E) { bad = 1; continue; }
            or_expert_ffn(&experts[e], xr, H, I, round_h, y);
            double wj = (double)w[(size_t)t * k + j];
            for (int c = 0; c < H; ++c) acc[c] += wj * y[c];
        }
        if (shared) {
            or_expert_ffn(shared, xr, H, I, round_h, y);
            for (int c = 0; c < H; ++c) acc[c] += y[c];
        }
        for (int c = 0; c < H; ++c) {
            if (out_fmt == OR_F32)
                ((float*)out)[(size_t)i * H + c] = (float)acc[c];
            else
                ((uint16_t*)out)[(size_t)i * H + c] = or_f64_to_bf16(acc[c]);
        }
        free(xr);
        free(y);
        free(acc);
    }
    return bad ? -1 : 0;
}

int or_max_threads(void) { return omp_get_max_threads(); }
