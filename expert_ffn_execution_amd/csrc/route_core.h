// route_core.h -- top-k gating of one token by one wavefront (gfx950); used
// by the top-k kernel (route.hip) and the fused top-k + alignment kernel
// (align.hip).
//
// Top-k rule (pages silent beyond "a few experts per token": claypier.com
// article, "从 MoE「用不到的权重」入手的推理引擎"): the k largest biased
// logits l' = fl32(l + b), equal values ordered by increasing expert id,
// -0.0 equal to +0.0; gates = softmax over the k picks.  Each lane holds
// E/64 keys; a key packs the order-preserving integer image of l' above the
// complemented expert id, so the larger key is the larger value and, among
// equal values, the lower id.  k rounds pick the experts in order.
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
// Wave-wide sum and max, returned uniform.  DPP exchanges inside each row of
// 16 lanes (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror: each pairs lanes across the next larger group), then the four
// row results read as scalars.  (The xor-shuffle form goes through LDS
// permutes, a round trip each, and the top-k's k maxima are a dependent
// chain.)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ double dpp_add_f64(double v, uint64_t o) { return v + __builtin_bit_cast(double, o); }
__device__ __forceinline__ double wave_sum_f64(double v) {
    uint64_t b = __builtin_bit_cast(uint64_t, v);
    v = dpp_add_f64(v, dpp_u64<0xB1>(b));
    b = __builtin_bit_cast(uint64_t, v);
    v = dpp_add_f64(v, dpp_u64<0x4E>(b));
    b = __builtin_bit_cast(uint64_t, v);
    v = dpp_add_f64(v, dpp_u64<0x141>(b));
    b = __builtin_bit_cast(uint64_t, v);
    v = dpp_add_f64(v, dpp_u64<0x140>(b));
    b = __builtin_bit_cast(uint64_t, v);
    return (__builtin_bit_cast(double, lane_u64(b, 0)) + __builtin_bit_cast(double, lane_u64(b, 16))) +
           (__builtin_bit_cast(double, lane_u64(b, 32)) + __builtin_bit_cast(double, lane_u64(b, 48)));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<0xB1>(v));
    v = max(v, dpp_u32<0x4E>(v));
    v = max(v, dpp_u32<0x141>(v));
    v = max(v, dpp_u32<0x140>(v));
    const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
    const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
    return max(a, b);
}

// Token t's picks and gates: row = its E logits, ids_out / w_out = its k
// slots; ids_copy (may be null) receives the picks too.  NPL = keys per lane
// (E <= 64 * NPL).  Each lane first sorts its NPL keys, so a pick compares
// only the lanes' heads: the largest value by one 32-bit wave max, then the
// lowest id among the lanes holding it (the largest complemented id) by
// another; the winning lane drops its head.  (One 64-bit wave max over all
// keys per pick took about 880 cycles a pick on one wavefront.)
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
#pragma unroll
    for (int i = 0; i < NPL; ++i)
#pragma unroll
        for (int j = i + 1; j < NPL; ++j) {
            const uint64_t hi = key[i] > key[j] ? key[i] : key[j];
            const uint64_t lo = key[i] > key[j] ? key[j] : key[i];
            key[i] = hi;
            key[j] = lo;
        }
    uint32_t hv = (uint32_t)(key[0] >> 32), lv = (uint32_t)key[0];
    float pick_v[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) pick_v[i] = 0.0f;
    float v0 = 0.0f;
    for (int j = 0; j < k; ++j) {
        const uint32_t mh = wave_max_u32(hv);
        const uint32_t ml = wave_max_u32(hv == mh ? lv : 0u);
        const int e = (int)(~ml);
        const float v = key_value(((uint64_t)mh << 32) | ml);
        if (j == 0) v0 = v;
        if (lane == (j & 63)) {
#pragma unroll
            for (int i = 0; i < NPL; ++i)
                if (i == (j >> 6)) pick_v[i] = v;
            ids_out[j] = e;
            if (ids_copy) ids_copy[j] = e;
        }
        if (hv == mh && lv == ml) {  // the winning lane drops its head
#pragma unroll
            for (int i = 0; i + 1 < NPL; ++i) key[i] = key[i + 1];
            key[NPL - 1] = 0;
            hv = (uint32_t)(key[0] >> 32);
            lv = (uint32_t)key[0];
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
