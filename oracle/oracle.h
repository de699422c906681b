/*
 * oracle.h -- plain CPU reference of the per-layer MoE FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; it is written from the
 * definitions of the operations, as per-token loops, in fp64.
 *
 * What it computes (one MoE layer, T tokens):
 *   logits  l[t,e]   = sum_h x[t,h] * Wr[e,h]                (fp64 sum, one fp32 rounding)
 *   biased  l'[t,e]  = fl32(l[t,e] + b[e])
 *   top-k   ids[t,j] = j-th largest l'[t,.], ties -> lower expert id
 *   gates   w[t,j]   = exp(l'_j - l'_0) / sum_{i<k} exp(l'_i - l'_0)   (fp64, one fp32 rounding)
 *   align   counts, exclusive offsets, perm = flat slots f = t*k+j sorted stably
 *           by expert, inv_perm[perm[p]] = p
 *   expert  h = silu(x Wg^T) * (x Wu^T),  y = h Wd^T         (fp64; h rounded to bf16
 *           for bf16 / MXFP4 / FP8 weights)
 *   combine out[t] = sum_j w[t,j] * y(t,j) (+ y_shared(t)), fp64, one rounding to the
 *           output format.
 *
 * The pages state only that a few experts run per token and that only the
 * experts needed are brought to the GPU (claypier.com article,
 * "从 MoE「用不到的权重」入手的推理引擎"; chenxutan.com article,
 * "瓶颈为什么是带宽而不是容量").  Routing rule, SwiGLU and combine are the
 * plain readings listed in the design notes.
 *
 * Parity pins: every function here is checked in tests/test_oracle_pins.py
 * against library routines, closed forms, brute force and invariants.
 */
#ifndef FT_ORACLE_H
#define FT_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage formats of a tensor */
enum { OR_F32 = 0, OR_BF16 = 1, OR_MXFP4 = 2, OR_FP8 = 3, OR_NVFP4 = 4 };

/* One expert in logical layout.
 *   OR_F32 / OR_BF16: gate [I][H], up [I][H], down [H][I] row-major.
 *   OR_MXFP4: gate/up codes [I][H/2], down codes [H][I/2] (element 2j in the
 *   low nibble of byte j), e8m0 scales gate_sc/up_sc [I][H/32], down_sc [H][I/32].
 *   OR_FP8: e4m3 codes gate/up [I][H], down [H][I], one byte each; gate_sc,
 *   up_sc, down_sc each point at the matrix's fp32 scale (4 bytes): the weight
 *   is the code's value times that scale.  The pages list FP8 weights without
 *   their scaling (refft.com guide, the format list); one scale per matrix is
 *   the plainest reading.
 *   OR_NVFP4: e2m1 codes as for OR_MXFP4; gate_sc/up_sc [I][H/16], down_sc
 *   [H][I/16] hold one e4m3 scale byte per block of 16 consecutive elements of
 *   a row; gate_ts, up_ts, down_ts each point at the matrix's fp32 tensor
 *   scale.  The weight is e2m1(code) * e4m3(block scale) * tensor scale.  The
 *   pages name NVFP4 without its layout (refft.com guide, the format list);
 *   this is NVIDIA's published NVFP4 definition. */
typedef struct {
    int fmt;
    const void* gate;
    const void* up;
    const void* down;
    const uint8_t* gate_sc;
    const uint8_t* up_sc;
    const uint8_t* down_sc;
    const uint8_t* gate_ts;
    const uint8_t* up_ts;
    const uint8_t* down_ts;
} or_expert;

/* Exact value of one e2m1 code scaled by an e8m0 byte (OCP MX v1.0). */
double or_mxfp4_value(uint8_t code, uint8_t scale);
/* Exact value of one e4m3 code (OCP OFP8 v1.0, the E4M3 encoding; NaN for the
 * two NaN codes). */
double or_fp8_value(uint8_t code);
/* Exact value of one NVFP4 element before its tensor scale: the e2m1 code
 * times its block's e4m3 scale byte. */
double or_nvfp4_value(uint8_t code, uint8_t scale);
/* The cached decode values used per element (filled from the functions above
 * when the library loads): e2m1 value of a code (scale 2^0), the e8m0 scale
 * 2^(X-127) (NaN for 255), the e4m3 value of a code. */
double or_table_e2m1(uint8_t code);
double or_table_pow2(uint8_t X);
double or_table_fp8(uint8_t code);
/* bf16 bits -> double (exact) and double -> bf16 bits (round to nearest even). */
double or_bf16_to_f64(uint16_t b);
uint16_t or_f64_to_bf16(double v);

/* l = x Wr^T (fp64 sums, rounded once to fp32).  x [T][H], wr [E][H], both fmt. */
int or_router_logits(const void* x, const void* wr, int fmt, int T, int H, int E,
                     float* logits);

/* top-k selection and renormalised softmax gates from fp32 logits [T][E].
 * bias may be NULL.  ids [T][k] int32, w [T][k] fp32. */
int or_route(const float* logits, const float* bias, int T, int E, int k,
             int32_t* ids, float* w);

/* counts [E], offsets [E+1], perm [T*k], inv_perm [T*k]. */
int or_align(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
             int32_t* perm, int32_t* inv_perm);

/* One expert FFN on one token row x [H] (fp64): y [H].
 * round_h: 1 rounds h to bf16 before the down projection. */
int or_expert_ffn(const or_expert* ex, const double* x, int H, int I, int round_h,
                  double* y);

/* Whole routed layer after routing: out[t] for the tokens in `tokens`
 * (all T when tokens == NULL; then n_tokens must equal T).
 *   x [T][H] in x_fmt (OR_F32 or OR_BF16); ids/w [T][k];
 *   experts[E]; shared may be NULL;
 *   out [n_tokens][H] in out_fmt (OR_F32 or OR_BF16), row i for tokens[i].
 * nthreads <= 0 uses the OpenMP default. */
int or_moe_layer(const void* x, int x_fmt, int T, int H, int I, int E, int k,
                 const int32_t* ids, const float* w, const or_expert* experts,
                 const or_expert* shared, int round_h, int out_fmt, void* out,
                 const int32_t* tokens, int n_tokens, int nthreads);

/* number of OpenMP threads a parallel region gets */
int or_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif
