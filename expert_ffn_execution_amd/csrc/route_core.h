// route_core.h -- top-k gating of one token by one wavefront (gfx950); used
// by the top-k kernel (route.hip) and the fused top-k + alignment kernel
// (align.hip).
//
// Top-k rule (pages silent beyond "a few experts per token": claypier.com
// article, "从 MoE「用不到的权重」入手的推理引擎"): the k largest biased
// logits l' = fl32(l + b), equal values ordered by increasing expert id,
// -0.0 equal to +0.0; gates = softmax over the k picks.  Each lane holds
// E/64 keys; a key packs the order-preserving integer image of l' above the
// complemented expert id, so a single 64-bit max picks the largest value and,
// among equal values, the lowest id.  k rounds of a wave max pick the experts
// in order.
#pragma once

#include "common.h"

namespace {

__device__ __forceinline__ uint64_t make_key(float v, int e) {
    if (v == 0.0f) v = 0.0f;  // -0.0 -> +0.0
    uint32_t u = __float_as_uint(v);
    uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint32_t)(~(uint32_t)e);
}
__device__ __forceinline__ float key_value(uint64_t key) {
    uint32_t ord = (uint32_t)(key >> 32);
    uint32_t u = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
    return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, o, 64);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
        uint64_t w = ((uint64_t)hi << 32) | lo;
        v = w > v ? w : v;
    }
    return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Token t's picks and gates: row = its E logits, ids_out / w_out = its k
// slots; ids_copy (may be null) receives the picks too.  NPL = keys per lane
// (E <= 64 * NPL).
template <int NPL>
__device__ __forceinline__ void topk_token(const float* __restrict__ row, const float* __restrict__ bias,
                                           int E, int k, int32_t* __restrict__ ids_out,
                                           float* __restrict__ w_out, int32_t* ids_copy, int lane) {
    uint64_t key[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        int e = lane + 64 * i;
        key[i] = 0;  // below every finite key
        if (e < E) {
            float v = row[e];
            if (bias) v = v + bias[e];
            key[i] = make_key(v, e);
        }
    }
    float pick_v[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) pick_v[i] = 0.0f;
    float v0 = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < NPL; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
        int e = (int)(~(uint32_t)best);
        float v = key_value(best);
        if (j == 0) v0 = v;
        if (lane == (e & 63)) {
#pragma unroll
            for (int i = 0; i < NPL; ++i)
                if (i == (e >> 6)) key[i] = 0;
        }
        if (lane == (j & 63)) {
#pragma unroll
            for (int i = 0; i < NPL; ++i)
                if (i == (j >> 6)) pick_v[i] = v;
            ids_out[j] = e;
            if (ids_copy) ids_copy[j] = e;
        }
    }
    // gates in fp64: w_j = exp(v_j - v_0) / sum_i exp(v_i - v_0)
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
        if (lane + 64 * i < k) s += exp((double)pick_v[i] - (double)v0);
    s = wave_sum_f64(s);
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        int j = lane + 64 * i;
        if (j < k) w_out[j] = (float)(exp((double)pick_v[i] - (double)v0) / s);
    }
}

}  // namespace
