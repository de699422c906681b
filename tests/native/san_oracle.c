/* san_oracle.c -- the CPU oracle on small layers of every weight format under
 * AddressSanitizer + UndefinedBehaviorSanitizer, built by
 * tests/test_sanitizers.py: router logits, routing, alignment and the whole
 * layer (with and without the shared expert, all tokens and a subset).  Exits
 * non-zero on a failed call or a non-finite output. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint32_t rng = 12345u;
static uint32_t next(void) { rng = rng * 1664525u + 1013904223u; return rng >> 8; }
static float unit(void) { return (float)(next() % 20001) / 10000.0f - 1.0f; }
static uint16_t bf16(float f) { uint32_t u; memcpy(&u, &f, 4); return (uint16_t)(u >> 16); }

#define REQUIRE(c) do { if (!(c)) { fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

static void* fill_codes(size_t n, int fmt) {
    uint8_t* p = malloc(n);
    for (size_t i = 0; i < n; ++i) {
        uint8_t v = (uint8_t)next();
        if (fmt == OR_FP8 && (v & 0x7F) == 0x7F) v = 0x3F;   /* no NaN codes */
        p[i] = v;
    }
    return p;
}

static int one(int fmt, int shared_on) {
    const int T = 7, H = 64, I = 64, E = 4, k = 2;
    const size_t HI = (size_t)H * I;
    or_expert ex[5];
    void* keep[64];
    int nk = 0;
    float ts = 0.01f;
    for (int e = 0; e < E + 1; ++e) {
        or_expert* x = &ex[e];
        memset(x, 0, sizeof *x);
        x->fmt = fmt;
        if (fmt == OR_F32 || fmt == OR_BF16) {
            size_t es = fmt == OR_F32 ? 4 : 2;
            void* m[3];
            for (int j = 0; j < 3; ++j) {
                m[j] = malloc(HI * es);
                for (size_t i = 0; i < HI; ++i) {
                    float v = unit() * 0.1f;
                    if (es == 4) ((float*)m[j])[i] = v; else ((uint16_t*)m[j])[i] = bf16(v);
                }
                keep[nk++] = m[j];
            }
            x->gate = m[0]; x->up = m[1]; x->down = m[2];
        } else {
            size_t cb = fmt == OR_FP8 ? HI : HI / 2;
            size_t sb = fmt == OR_FP8 ? 4 : fmt == OR_MXFP4 ? HI / 32 : HI / 16;
            void* c[3]; uint8_t* s[3];
            for (int j = 0; j < 3; ++j) {
                c[j] = fill_codes(cb, fmt); keep[nk++] = c[j];
                s[j] = malloc(sb); keep[nk++] = s[j];
                if (fmt == OR_FP8) { float v = 0.002f; memcpy(s[j], &v, 4); }
                else for (size_t i = 0; i < sb; ++i) s[j][i] = fmt == OR_MXFP4 ? (uint8_t)(120 + next() % 6) : (uint8_t)(0x30 + next() % 8);
            }
            x->gate = c[0]; x->up = c[1]; x->down = c[2];
            x->gate_sc = s[0]; x->up_sc = s[1]; x->down_sc = s[2];
            if (fmt == OR_NVFP4) x->gate_ts = x->up_ts = x->down_ts = (const uint8_t*)&ts;
        }
    }
    uint16_t xb[7 * 64], wr[4 * 64];
    for (int i = 0; i < T * H; ++i) xb[i] = bf16(unit());
    for (int i = 0; i < E * H; ++i) wr[i] = bf16(unit() * 0.2f);
    float logits[7 * 4], bias[4] = {0.1f, -0.2f, 0.0f, 0.3f}, w[7 * 2];
    int32_t ids[7 * 2], counts[4], offsets[5], perm[14], inv[14];
    REQUIRE(or_router_logits(xb, wr, OR_BF16, T, H, E, logits) == 0);
    REQUIRE(or_route(logits, bias, T, E, k, ids, w) == 0);
    REQUIRE(or_align(ids, T, k, E, counts, offsets, perm, inv) == 0);
    REQUIRE(offsets[E] == T * k);
    float out[7 * 64];
    REQUIRE(or_moe_layer(xb, OR_BF16, T, H, I, E, k, ids, w, ex, shared_on ? &ex[E] : NULL,
                         fmt != OR_F32, OR_F32, out, NULL, T, 2) == 0);
    for (int i = 0; i < T * H; ++i) REQUIRE(isfinite(out[i]));
    int32_t sub[3] = {6, 0, 3};
    uint16_t outb[3 * 64];
    REQUIRE(or_moe_layer(xb, OR_BF16, T, H, I, E, k, ids, w, ex, shared_on ? &ex[E] : NULL,
                         fmt != OR_F32, OR_BF16, outb, sub, 3, 1) == 0);
    for (int i = 0; i < 3 * H; ++i) REQUIRE(isfinite(or_bf16_to_f64(outb[i])));
    for (int i = 0; i < nk; ++i) free(keep[i]);
    return 0;
}

int main(void) {
    for (int fmt = OR_F32; fmt <= OR_NVFP4; ++fmt)
        for (int sh = 0; sh < 2; ++sh)
            if (one(fmt, sh)) { fprintf(stderr, "format %d shared %d\n", fmt, sh); return 1; }
    for (int c = 0; c < 256; ++c) { (void)or_fp8_value((uint8_t)c); (void)or_table_fp8((uint8_t)c); (void)or_f64_to_bf16(ldexp(1.0, c - 140)); }
    printf("oracle ok\n");
    return 0;
}
