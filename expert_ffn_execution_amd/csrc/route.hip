// route.hip -- router logits and top-k gating (gfx950).
//
// Top-k rule (pages silent beyond "a few experts per token": claypier.com
// article, "从 MoE「用不到的权重」入手的推理引擎"): the k largest biased
// logits l' = fl32(l + b), equal values ordered by increasing expert id,
// -0.0 equal to +0.0; gates = softmax over the k picks.
//
// One wavefront per token (route_core.h has the per-token selection).
#include "common.h"
#include "gemm_mfma.h"
#include "route_core.h"

namespace {

template <int NPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                   const float* __restrict__ bias, int T, int E,
                                                   int k, int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (t >= T) return;
    topk_token<NPL>(logits + (size_t)t * E, bias, E, k, ids + (size_t)t * k, w + (size_t)t * k,
                    nullptr, lane);
}

// Router logits for few tokens: one wavefront per (expert, token group of up
// to 8 tokens); lanes split H in 16-byte chunks; the expert's router row is
// read once per group.
template <typename TA>
__global__ __launch_bounds__(256) void logits_stream_kernel(const TA* __restrict__ x,
                                                            const TA* __restrict__ wr, int T,
                                                            int H, int E,
                                                            float* __restrict__ out) {
    constexpr int TG = 8;
    constexpr int EPC = 16 / sizeof(TA);  // elements per 16-byte chunk
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int n_tg = (T + TG - 1) / TG;
    if (gw >= E * n_tg) return;
    const int e = gw / n_tg;
    const int t0 = (gw % n_tg) * TG;
    const int nt = min(TG, T - t0);
    float acc[TG];
#pragma unroll
    for (int r = 0; r < TG; ++r) acc[r] = 0.f;
    const int nch = H / EPC;
    const u32x4_t* wrow = reinterpret_cast<const u32x4_t*>(wr + (size_t)e * H);
    for (int c = lane; c < nch; c += 64) {
        u32x4_t wv = wrow[c];
#pragma unroll
        for (int r = 0; r < TG; ++r) {
            if (r < nt) {
                u32x4_t xv = reinterpret_cast<const u32x4_t*>(x + (size_t)(t0 + r) * H)[c];
                if constexpr (sizeof(TA) == 2) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[r] = dot2_bf16(wv[q], xv[q], acc[r]);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[r] = fmaf(__uint_as_float(wv[q]), __uint_as_float(xv[q]), acc[r]);
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < TG; ++r) {
        float v = wave_sum(acc[r]);
        if (lane == 0 && r < nt) out[(size_t)(t0 + r) * E + e] = v;
    }
}

}  // namespace

namespace ft {

ft_status launch_topk(const float* logits, const float* bias, int T, int E, int k,
                      int32_t* ids, float* w, hipStream_t s) {
    dim3 grid(cdiv(T, 4)), block(256);
    if (E <= 64) topk_kernel<1><<<grid, block, 0, s>>>(logits, bias, T, E, k, ids, w);
    else if (E <= 128) topk_kernel<2><<<grid, block, 0, s>>>(logits, bias, T, E, k, ids, w);
    else if (E <= 256) topk_kernel<4><<<grid, block, 0, s>>>(logits, bias, T, E, k, ids, w);
    else if (E <= 512) topk_kernel<8><<<grid, block, 0, s>>>(logits, bias, T, E, k, ids, w);
    else topk_kernel<16><<<grid, block, 0, s>>>(logits, bias, T, E, k, ids, w);
    FT_LAUNCHED("topk");
    return FT_OK;
}

ft_status launch_router_logits(const void* x, ft_dtype dt, const void* wr, int T, int H, int E,
                               float* out, hipStream_t s) {
    // bf16 with enough tokens: MFMA tiles (fp32 accumulate); otherwise streaming.
    if (dt == FT_BF16 && T > 64) return launch_dense_gemm_f32out(x, wr, T, E, H, out, s);
    int n_tg = cdiv(T, 8);
    dim3 grid(cdiv((long)E * n_tg, 4)), block(256);
    if (dt == FT_BF16)
        logits_stream_kernel<__bf16><<<grid, block, 0, s>>>((const __bf16*)x, (const __bf16*)wr,
                                                            T, H, E, out);
    else
        logits_stream_kernel<float><<<grid, block, 0, s>>>((const float*)x, (const float*)wr, T,
                                                           H, E, out);
    FT_LAUNCHED("router_logits");
    return FT_OK;
}

}  // namespace ft
