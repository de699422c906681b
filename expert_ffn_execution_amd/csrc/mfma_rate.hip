// mfma_rate.hip -- issue-rate probe of the matrix-core instructions the expert
// GEMMs use or could use, under identical conditions: the bf16
// v_mfma_f32_32x32x16_bf16 (the shipped tiles) against the block-scaled
// v_mfma_scale_f32_32x32x64_f8f6f4 with fp8 x fp4 operands (what MX-quantised
// activations against MXFP4 weights would run on) and fp4 x fp4.
//
// Every variant runs the same grid (one 256-thread block per CU per wave-slot,
// so 1 or 2 waves per SIMD), the same number of independent accumulator
// chains per wave (8) and operands held in registers, so only the instruction
// differs.  Each point runs twice: a burst of a few milliseconds, and a
// sustained run of about 400 ms, long enough for the chip's power management
// to settle.  The operands are either small integers that every MFMA reuses
// (few bits change) or two sets of random bits (finite bf16 values in
// [2^-7, 2), any fp8 / fp4 codes) that consecutive MFMAs alternate between,
// since the matrix cores' power, and with it the clock the chip can hold,
// depends on how many bits change.  Both sets are made before the loop, so
// the loop holds MFMAs only.  Wave 0 of
// every block reads the shader-clock counter (s_memtime) and the 100 MHz
// constant clock (s_memrealtime) at its start and end; their ratio is the
// average shader clock the block saw.
//
// Output: one JSON object per line.  Exit status 0 when every launch succeeded.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned lcg(unsigned v) { return v * 1664525u + 1013904223u; }

constexpr int CHAINS = 8;
constexpr int THREADS = 256;

enum Kind { BF16 = 0, FP8_FP4 = 1, FP4_FP4 = 2 };

double flop_per_instruction(int kind) { return kind == BF16 ? 2.0 * 32 * 32 * 16 : 2.0 * 32 * 32 * 64; }

template <int KIND, bool RAND>
__global__ __launch_bounds__(THREADS) void issue_kernel(float* sink, unsigned long long* clocks, int iters,
                                                        int seed) {
    unsigned long long t0 = 0, r0 = 0;
    if (threadIdx.x == 0) {
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    f32x16 acc[CHAINS];
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[c][q] = 0.f;
    const int t = threadIdx.x + seed;
    if constexpr (KIND == BF16) {
        bf16x8 a, b;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            a[q] = (__bf16)(float)((t + q) & 3);
            b[q] = (__bf16)(float)((3 * t + q) & 3);
        }
        bf16x8 a2 = a, b2 = b;
        if constexpr (RAND) {
            u32x4 r[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                r[0][q] = lcg(lcg(2u * t + q));
                r[1][q] = lcg(lcg(7u * t + q + 1u));
                r[2][q] = lcg(r[0][q] ^ 0x9e3779b9u);
                r[3][q] = lcg(r[1][q] ^ 0x7f4a7c15u);
            }
            // sign and mantissa random, exponent 0x78..0x7f: finite, in [2^-7, 2)
            a = __builtin_bit_cast(bf16x8, (r[0] & 0x83FF83FFu) | 0x3C003C00u);
            b = __builtin_bit_cast(bf16x8, (r[1] & 0x83FF83FFu) | 0x3C003C00u);
            a2 = __builtin_bit_cast(bf16x8, (r[2] & 0x83FF83FFu) | 0x3C003C00u);
            b2 = __builtin_bit_cast(bf16x8, (r[3] & 0x83FF83FFu) | 0x3C003C00u);
        }
        for (int i = 0; i < iters; ++i)
#pragma unroll
            for (int c = 0; c < CHAINS; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c & 1 ? a2 : a, c & 1 ? b2 : b, acc[c], 0, 0, 0);
    } else {
        // operand formats of the scaled MFMA: 0 = fp8 e4m3, 4 = fp4 e2m1; scale
        // bytes 127 = 2^0
        constexpr int FA = KIND == FP4_FP4 ? 4 : 0, FB = 4;
        i32x8 a, b;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            a[q] = (7 * t + q) & 0x3f3f3f3f;
            b[q] = (5 * t + q) & 0x33333333;
        }
        i32x8 a2 = a, b2 = b;
        if constexpr (RAND) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                a[q] = (int)lcg(lcg(2u * t + q));
                b[q] = (int)lcg(lcg(7u * t + q + 1u));
                a2[q] = (int)lcg((unsigned)a[q] ^ 0x9e3779b9u);
                b2[q] = (int)lcg((unsigned)b[q] ^ 0x7f4a7c15u);
            }
        }
        for (int i = 0; i < iters; ++i)
#pragma unroll
            for (int c = 0; c < CHAINS; ++c)
                acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(c & 1 ? a2 : a, c & 1 ? b2 : b, acc[c],
                                                                         FA, FB, 0, 127, 0, 127);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
#pragma unroll
        for (int q = 0; q < 16; ++q) s += acc[c][q];
    sink[blockIdx.x * THREADS + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        const unsigned long long t1 = __builtin_amdgcn_s_memtime();
        const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
        clocks[2 * blockIdx.x] = t1 - t0;
        clocks[2 * blockIdx.x + 1] = r1 - r0;
    }
}

struct Point {
    double ms, tflops, clock_ghz;
};

#define CHECK(call)                                                                        \
    do {                                                                                   \
        hipError_t e_ = (call);                                                            \
        if (e_ != hipSuccess) {                                                            \
            fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                     \
            exit(1);                                                                       \
        }                                                                                  \
    } while (0)

template <int KIND, bool RAND>
Point run(int blocks, int iters, float* sink, unsigned long long* clocks_dev) {
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    CHECK(hipEventRecord(e0));
    issue_kernel<KIND, RAND><<<blocks, THREADS>>>(sink, clocks_dev, iters, 1);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    std::vector<unsigned long long> clk(2 * (size_t)blocks);
    CHECK(hipMemcpy(clk.data(), clocks_dev, clk.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost));
    double cyc = 0, ref = 0;
    for (int b = 0; b < blocks; ++b) {
        cyc += (double)clk[2 * b];
        ref += (double)clk[2 * b + 1];
    }
    CHECK(hipEventDestroy(e0));
    CHECK(hipEventDestroy(e1));
    const double flops = flop_per_instruction(KIND) * CHAINS * (double)iters * blocks * (THREADS / 64);
    // s_memrealtime ticks at a constant 100 MHz
    return {ms, flops / (ms * 1e-3) / 1e12, ref > 0 ? cyc / ref * 0.1 : 0.0};
}

template <int KIND, bool RAND>
void sweep(const char* name, int ncu, float* sink, unsigned long long* clocks_dev) {
    for (int wps = 1; wps <= 2; ++wps) {
        const int blocks = ncu * wps;  // 256-thread blocks, one per CU per slot: wps waves per SIMD
        run<KIND, RAND>(blocks, 64, sink, clocks_dev);                       // warm-up
        const Point probe = run<KIND, RAND>(blocks, 2000, sink, clocks_dev);  // sizes the runs below
        const double per_iter_ms = probe.ms / 2000.0;
        for (double target_ms : {5.0, 400.0}) {
            const long long it = (long long)(target_ms / per_iter_ms);
            const int iters = (int)(it < 1 ? 1 : (it > 200000000 ? 200000000 : it));
            const Point p = run<KIND, RAND>(blocks, iters, sink, clocks_dev);
            printf("{\"mfma\": \"%s\", \"operands\": \"%s\", \"waves_per_simd\": %d, \"chains\": %d, "
                   "\"ms\": %.3f, \"tflops\": %.1f, \"shader_clock_ghz\": %.3f}\n",
                   name, RAND ? "random" : "fixed", wps, CHAINS, p.ms, p.tflops, p.clock_ghz);
            fflush(stdout);
        }
    }
}

}  // namespace

int main() {
    int ncu = 0;
    CHECK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, 0));
    if (ncu <= 0 || ncu > 1024) {
        fprintf(stderr, "unexpected compute-unit count %d\n", ncu);
        return 1;
    }
    const int max_blocks = 2 * ncu;
    float* sink = nullptr;
    unsigned long long* clocks_dev = nullptr;
    CHECK(hipMalloc(&sink, (size_t)max_blocks * THREADS * sizeof(float)));
    CHECK(hipMalloc(&clocks_dev, (size_t)max_blocks * 2 * sizeof(unsigned long long)));
    printf("{\"compute_units\": %d, \"bf16_flop_per_cycle_per_cu\": %d}\n", ncu, 4 * 1024);
    sweep<BF16, false>("bf16 32x32x16", ncu, sink, clocks_dev);
    sweep<FP8_FP4, false>("scaled fp8 x fp4 32x32x64", ncu, sink, clocks_dev);
    sweep<FP4_FP4, false>("scaled fp4 x fp4 32x32x64", ncu, sink, clocks_dev);
    sweep<BF16, true>("bf16 32x32x16", ncu, sink, clocks_dev);
    sweep<FP8_FP4, true>("scaled fp8 x fp4 32x32x64", ncu, sink, clocks_dev);
    CHECK(hipFree(sink));
    CHECK(hipFree(clocks_dev));
    return 0;
}
