// combine.hip -- gate-weighted sum of the expert outputs back to token order.
//
// out[t] = sum_{j<k} w[t][j] * y_perm[inv_perm[t*k + j]] (+ shared row), in
// fp32, j increasing, then one rounding to the output format.  Each thread
// owns 8 consecutive hidden elements of one token and reads the k expert rows
// with 16-byte (bf16) or 32-byte (fp32) loads; no atomics, so the result does
// not depend on scheduling.
#include "common.h"

namespace {

template <typename YT, typename OT>
__global__ __launch_bounds__(256) void combine_kernel(const YT* __restrict__ y,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int T, int k,
                                                      int H, int n_shared, OT* __restrict__ out) {
    const int t = blockIdx.x;
    const int d = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
    if (d >= H) return;
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    auto add_row = [&](size_t row, float wj) {
        const YT* src = y + row * H + d;
        if constexpr (sizeof(YT) == 2) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = fmaf(wj, bf16_bits_to_f32(v[q] & 0xffffu), acc[2 * q]);
                acc[2 * q + 1] = fmaf(wj, bf16_bits_to_f32(v[q] >> 16), acc[2 * q + 1]);
            }
        } else {
            const f32x4_t a = *reinterpret_cast<const f32x4_t*>(src);
            const f32x4_t b = *reinterpret_cast<const f32x4_t*>(src + 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[q] = fmaf(wj, a[q], acc[q]);
                acc[4 + q] = fmaf(wj, b[q], acc[4 + q]);
            }
        }
    };
    for (int j = 0; j < k; ++j) add_row((size_t)inv[(size_t)t * k + j], w[(size_t)t * k + j]);
    if (n_shared) add_row((size_t)T * k + t, 1.0f);
    OT* dst = out + (size_t)t * H + d;
    if constexpr (sizeof(OT) == 2) {
        u32x4_t o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
        *reinterpret_cast<u32x4_t*>(dst) = o;
    } else {
        *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
    }
}

}  // namespace

namespace ft {

ft_status launch_combine(const void* y, ft_dtype y_dt, const int32_t* inv, const float* w, int T,
                         int k, int H, int n_shared, void* out, ft_dtype out_dt, hipStream_t s) {
    dim3 grid((unsigned)T, (unsigned)cdiv(H, 256 * 8)), block(256);
#define FT_C(YT, OT) \
    combine_kernel<YT, OT><<<grid, block, 0, s>>>((const YT*)y, inv, w, T, k, H, n_shared, (OT*)out)
    if (y_dt == FT_BF16) {
        if (out_dt == FT_BF16) FT_C(__bf16, __bf16); else FT_C(__bf16, float);
    } else {
        if (out_dt == FT_BF16) FT_C(float, __bf16); else FT_C(float, float);
    }
#undef FT_C
    FT_LAUNCHED("combine");
    return FT_OK;
}

}  // namespace ft
