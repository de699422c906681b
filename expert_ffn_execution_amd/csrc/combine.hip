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

// y[pos[i]] = rows[i] rounded to the output format (fp32 -> bf16 to nearest
// even, or copied), one block per row, 8 consecutive elements per thread.
template <typename OT>
__global__ __launch_bounds__(256) void scatter_rows_kernel(const float* __restrict__ rows,
                                                           const int64_t* __restrict__ pos, int H,
                                                           OT* __restrict__ y) {
    const int i = blockIdx.x;
    const int d = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
    if (d >= H) return;
    const float* src = rows + (size_t)i * H + d;
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(src);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(src + 4);
    OT* dst = y + (size_t)pos[i] * H + d;
    if constexpr (sizeof(OT) == 2) {
        *reinterpret_cast<u32x4_t*>(dst) =
            u32x4_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                    pack_bf16x2(b[2], b[3])};
    } else {
        *reinterpret_cast<f32x4_t*>(dst) = a;
        *reinterpret_cast<f32x4_t*>(dst + 4) = b;
    }
}

// dst[i] = src[i] for i < n: a few hundred int32 between device memory and
// pinned host memory mapped for the device (one block; an in-stream copy of
// this size costs more than the kernel)
__global__ __launch_bounds__(256) void copy_i32_kernel(const int32_t* __restrict__ src,
                                                       int32_t* __restrict__ dst, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = src[i];
    __threadfence_system();
}

// copy_i32 and then *flag = epoch (pinned host memory mapped for the
// device): the host polls the flag instead of an event
__global__ __launch_bounds__(256) void copy_i32_flag_kernel(const int32_t* __restrict__ src,
                                                            int32_t* __restrict__ dst, int n,
                                                            int32_t* flag, int32_t epoch) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = src[i];
    __threadfence_system();
    __syncthreads();
    if (threadIdx.x == 0) {
        __hip_atomic_store(flag, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

// the expert counts of up to STACK_MAX_LAYERS layers, gathered into one
// host-visible array [n_layers][n], then a flag (as copy_i32_flag_kernel)
struct CountsArg {
    const int32_t* src[ft::STACK_MAX_LAYERS];
};
__global__ __launch_bounds__(256) void copy_counts_flag_kernel(const CountsArg a, int n_layers, int n,
                                                               int32_t* __restrict__ dst, int32_t* flag,
                                                               int32_t epoch) {
    for (int l = 0; l < n_layers; ++l)
        for (int i = threadIdx.x; i < n; i += blockDim.x) dst[(size_t)l * n + i] = a.src[l][i];
    __threadfence_system();
    __syncthreads();
    if (threadIdx.x == 0) {
        __hip_atomic_store(flag, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

// a slot table of up to TABLE_MAX entries carried in the kernel's arguments
struct TableArg {
    int32_t v[ft::TABLE_MAX];
};
__global__ __launch_bounds__(256) void set_table_kernel(const TableArg t, int32_t* __restrict__ dst, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = t.v[i];
}

}  // namespace

namespace ft {

ft_status launch_copy_i32_flag(const int32_t* src, int32_t* dst, int n, int32_t* flag, int32_t epoch,
                               hipStream_t s) {
    copy_i32_flag_kernel<<<1, 256, 0, s>>>(src, dst, n, flag, epoch);
    FT_LAUNCHED("copy_i32_flag");
    return FT_OK;
}

ft_status launch_copy_counts_flag(const int32_t* const* src, int n_layers, int n, int32_t* dst,
                                  int32_t* flag, int32_t epoch, hipStream_t s) {
    if (n_layers < 1 || n_layers > STACK_MAX_LAYERS)
        return set_error(FT_ERR_INVALID_ARG, "%d layers: 1 to %d", n_layers, STACK_MAX_LAYERS);
    CountsArg a{};
    for (int l = 0; l < n_layers; ++l) a.src[l] = src[l];
    copy_counts_flag_kernel<<<1, 256, 0, s>>>(a, n_layers, n, dst, flag, epoch);
    FT_LAUNCHED("copy_counts_flag");
    return FT_OK;
}

ft_status launch_set_table(const int32_t* table, int n, int32_t* dst, hipStream_t s) {
    if (n > TABLE_MAX) return set_error(FT_ERR_INVALID_ARG, "slot table of %d entries > %d", n, TABLE_MAX);
    TableArg t;
    for (int i = 0; i < n; ++i) t.v[i] = table[i];
    set_table_kernel<<<1, 256, 0, s>>>(t, dst, n);
    FT_LAUNCHED("set_table");
    return FT_OK;
}

ft_status launch_copy_i32(const int32_t* src, int32_t* dst, int n, hipStream_t s) {
    copy_i32_kernel<<<1, 256, 0, s>>>(src, dst, n);
    FT_LAUNCHED("copy_i32");
    return FT_OK;
}

ft_status launch_scatter_rows(const float* rows, const int64_t* pos, int n, int H, void* y,
                              ft_dtype y_dt, hipStream_t s) {
    dim3 grid((unsigned)n, (unsigned)cdiv(H, 256 * 8)), block(256);
    if (y_dt == FT_BF16)
        scatter_rows_kernel<__bf16><<<grid, block, 0, s>>>(rows, pos, H, (__bf16*)y);
    else
        scatter_rows_kernel<float><<<grid, block, 0, s>>>(rows, pos, H, (float*)y);
    FT_LAUNCHED("scatter_rows");
    return FT_OK;
}

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
