// common.h -- shared host/device helpers of libftmoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <tuple>
#include <utility>
#include <stdint.h>
#include <stddef.h>

#include "../../include/ftmoe.h"

// ---------------------------------------------------------------------------
// host-side status plumbing
// ---------------------------------------------------------------------------
namespace ft {

ft_status set_error(ft_status st, const char* fmt, ...);
void clear_error();

#define FT_CHECK_ARG(cond, ...)                                        \
    do {                                                               \
        if (!(cond)) return ::ft::set_error(FT_ERR_INVALID_ARG, __VA_ARGS__); \
    } while (0)

#define FT_HIP(call)                                                               \
    do {                                                                           \
        hipError_t e_ = (call);                                                    \
        if (e_ != hipSuccess)                                                      \
            return ::ft::set_error(FT_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
    } while (0)

// launch-error check after <<<>>>
#define FT_LAUNCHED(name)                                                          \
    do {                                                                           \
        hipError_t e_ = hipGetLastError();                                         \
        if (e_ != hipSuccess)                                                      \
            return ::ft::set_error(FT_ERR_HIP, "launch %s: %s", name, hipGetErrorString(e_)); \
    } while (0)

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// largest slot table uploaded through a kernel argument (ft_slot_cache_map)
constexpr int TABLE_MAX = 512;
// layers of one device-table stack pass (their counts travel in one kernel's arguments)
constexpr int STACK_MAX_LAYERS = 64;
inline int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

// profiling hooks: events recorded around selected kernels (see ft_set_profile_events)
enum { PROF_FFN_GEMM1 = 0, PROF_FFN_GEMM2 = 1, PROF_FFN = 2, PROF_ROUTE = 3,
       PROF_ALIGN = 4, PROF_COMBINE = 5, PROF_N = 6 };
void prof_begin(int which, hipStream_t s);
void prof_end(int which, hipStream_t s);
// The gate/up and down stages are one kernel each: their events ride on that
// kernel's dispatch (hipExtLaunchKernel), which timestamps the kernel itself
// and adds no marker packet (a marker between two kernels left the GPU idle
// for 5-9 us).  Null events when the stage is not profiled or the thread
// captures a graph.
struct StageEvents {
    hipEvent_t start, stop;
};
StageEvents prof_stage(int which);

template <typename Tup, size_t... I>
inline void kernel_argv(Tup& t, void** argv, std::index_sequence<I...>) {
    ((argv[I] = (void*)&std::get<I>(t)), ...);
}
// kern<<<grid, block, lds, s>>>(args...), with stage `which`'s events when set
template <typename... P, typename... A>
inline hipError_t launch_timed(int which, void (*kern)(P...), dim3 grid, dim3 block, size_t lds,
                               hipStream_t s, A... args) {
    const StageEvents ev = prof_stage(which);
    if (!ev.start) {
        kern<<<grid, block, lds, s>>>(args...);
        return hipGetLastError();
    }
    std::tuple<P...> t(args...);
    void* argv[sizeof...(P) > 0 ? sizeof...(P) : 1];
    kernel_argv(t, argv, std::index_sequence_for<P...>{});
    const hipError_t e = hipExtLaunchKernel((const void*)kern, grid, block, argv, lds, s, ev.start,
                                            ev.stop, 0);
    return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace ft

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}
// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet)
// Round to nearest even; NaN stays a (quiet) NaN.  Written as a select, not an
// early return: the branch became an exec-mask round trip per value (the bf16
// GEMM epilogues convert up to 256 values per lane: 7.7 -> 5.6 us per tile of
// the 35B-A3B down projection).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t quiet_nan = (u >> 16) | 0x40u;
    return (u & 0x7fffffffu) > 0x7f800000u ? quiet_nan : rounded;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) {
    return __builtin_bit_cast(bf16x2_t, u);
}
// sum of the two bf16 products of a and b, accumulated into c (fp32)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), c, false);
}
// silu(g) * u with the hardware exp2 and reciprocal (about 1 ulp each; the
// result is rounded to bf16 by every caller): e^-g = 2^(-g log2 e)
__device__ __forceinline__ float silu_mul_fast(float g, float u) {
    const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
    return g * u * __builtin_amdgcn_rcpf(1.0f + e);
}
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + expf(-g)) * u;
}

// Sum over the wavefront, returned uniform: DPP exchanges inside each row of
// 16 lanes (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror), then the four row sums read as scalars, added as
// (r0 + r1) + (r2 + r3).  A fixed order, like any other: the result is
// deterministic.  (xor shuffles would go through LDS permutes.)
template <int CTRL>
__device__ __forceinline__ float dpp_sum_step(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float wave_sum(float v) {
    v = dpp_sum_step<0xB1>(v);
    v = dpp_sum_step<0x4E>(v);
    v = dpp_sum_step<0x141>(v);
    v = dpp_sum_step<0x140>(v);
    const int b = __builtin_bit_cast(int, v);
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}
