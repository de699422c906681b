// ffn_stream.hip -- expert FFN for few tokens: weight streaming (gfx950).
//
// With a handful of tokens the layer reads every byte of each routed expert's
// weights once and does a few multiply-adds per byte, so the time is the HBM
// read of the active experts (the pages make the same point one level up:
// time goes to moving expert weights, not to arithmetic -- chenxutan.com
// article, "瓶颈为什么是带宽而不是容量").  These kernels therefore stream
// weights with 16-byte loads, every lane of a wavefront reading consecutive
// chunks of one weight row, and keep the routed tokens' activations in LDS.
// They use vector ALU dot products (v_dot2_f32_bf16 for bf16; MXFP4 codes are
// decoded exactly to bf16 first), not MFMA: the work per byte is too small for
// a matrix tile to pay off.
//
// Grid: (active expert j, block of weight rows).  A block finds the j-th
// expert with routed tokens (and a slot) from `offsets` by wave ballots, so
// no host round trip is needed; blocks beyond the active count exit.
#include "common.h"
#include "gemm_mfma.h"

#include <type_traits>

namespace {

// WT: 0 = fp32 weights (fp32 activations), 1 = bf16, 2 = MXFP4 (bf16 activations)
template <int WT> struct W;
template <> struct W<0> { static constexpr int EPC = 4; };   // elements per 16 B chunk
template <> struct W<1> { static constexpr int EPC = 8; };
template <> struct W<2> { static constexpr int EPC = 32; };

// j-th expert (in id order) with rows and a slot; -1 if fewer than j+1.
__device__ int find_active(const int32_t* __restrict__ offsets, const int32_t* __restrict__ slot_of,
                           int E, int j, int lane) {
    int seen = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        bool act = false;
        if (e < E) act = offsets[e + 1] > offsets[e] && (!slot_of || slot_of[e] >= 0);
        const uint64_t m = __ballot(act);
        const int pc = __popcll(m);
        if (j < seen + pc) {
            uint64_t mm = m;
            for (int q = 0; q < j - seen; ++q) mm &= mm - 1;
            return e0 + __builtin_ctzll(mm);
        }
        seen += pc;
    }
    return -1;
}

// Multiply-accumulate one 16-byte weight chunk with the matching activation
// chunk held in LDS.  xs points at the chunk's first element (bf16 or fp32).
template <int WT>
__device__ __forceinline__ float chunk_dot(u32x4_t wv, uint32_t sc, const void* xs, float acc) {
    if constexpr (WT == 0) {
        const f32x4_t xv = *reinterpret_cast<const f32x4_t*>(xs);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = fmaf(__uint_as_float(wv[q]), xv[q], acc);
    } else if constexpr (WT == 1) {
        const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xs);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = dot2_bf16(wv[q], xv[q], acc);
    } else {
        const float s = __uint_as_float(sc << 23);
        const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(xs);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4_t xv = xp[q];
            const uint32_t w = wv[q];
            acc = dot2_bf16(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0)), xv[0], acc);
            acc = dot2_bf16(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1)), xv[1], acc);
            acc = dot2_bf16(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2)), xv[2], acc);
            acc = dot2_bf16(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3)), xv[3], acc);
        }
    }
    return acc;
}

// Weight row `row` of a [N][K] matrix at byte offset `moff` (codes) /
// `soff` (scales) inside the slot: pointer to its 16-byte chunks and scales.
template <int WT>
__device__ __forceinline__ const u32x4_t* row_chunks(const uint8_t* slot, size_t moff, int row,
                                                     int K) {
    constexpr int bytes_per_row_num = WT == 0 ? 4 : (WT == 1 ? 2 : 1);
    const size_t rb = WT == 2 ? (size_t)K / 2 : (size_t)K * bytes_per_row_num;
    return reinterpret_cast<const u32x4_t*>(slot + moff + (size_t)row * rb);
}

// One pass over a weight row: this lane's chunks c = c0 + lane + 64 q, q < 4.
// All loads of a pass are issued together so that a wavefront has 4 (or 8
// for gate + up) 16-byte loads per lane in flight.
template <int WT>
struct RowPass {
    u32x4_t v[4];
    uint32_t s[4];
    __device__ __forceinline__ void load(const u32x4_t* __restrict__ row,
                                         const uint8_t* __restrict__ sc, int c0, int nch,
                                         int lane) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = c0 + 64 * q + lane;
            if (c < nch) {
                v[q] = __builtin_nontemporal_load(row + c);
                if constexpr (WT == 2) s[q] = sc[c];
            }
        }
    }
    template <typename AT>
    __device__ __forceinline__ float dot(const AT* xrow, int c0, int nch, int lane, float acc) const {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = c0 + 64 * q + lane;
            if (c < nch) acc = chunk_dot<WT>(v[q], WT == 2 ? s[q] : 0u, xrow + (size_t)c * W<WT>::EPC, acc);
        }
        return acc;
    }
};

// Wavefront sum: DPP inside each row of 16 lanes, then two cross-row swaps.
#define FT_DPP(v, ctrl) \
    __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xF, 0xF, true))
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += FT_DPP(v, 0xB1);   // quad_perm [1,0,3,2]
    v += FT_DPP(v, 0x4E);   // quad_perm [2,3,0,1]
    v += FT_DPP(v, 0x141);  // row_half_mirror
    v += FT_DPP(v, 0x140);  // row_mirror
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}
#undef FT_DPP

// Activation rows into LDS: row r of the chunk is source row src_row(r).
template <typename AT, typename RowF>
__device__ __forceinline__ void stage_rows(AT* xs, const AT* __restrict__ src, RowF src_row,
                                           int R, int K) {
    const int per_row = K * (int)sizeof(AT) / 16;
    for (int i = threadIdx.x; i < R * per_row; i += blockDim.x) {
        const int r = i / per_row, c = i % per_row;
        reinterpret_cast<u32x4_t*>(xs + (size_t)r * K)[c] =
            reinterpret_cast<const u32x4_t*>(src + (size_t)src_row(r) * K)[c];
    }
}

// ---------------------------------------------------------------------------
// GEMM1 + SwiGLU.  Block: RPB row pairs (gate row i, up row i); wave w takes
// pairs w, w+4, ...  Activations: RMAX token rows at a time in LDS.  The
// first pass of weight loads is issued before the activations are staged.
// ---------------------------------------------------------------------------
template <int WT, int RMAX>
__global__ __launch_bounds__(256) void ffn1_stream_kernel(ft::FfnGeom g, const void* __restrict__ xv,
                                                          const int32_t* __restrict__ perm,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ slot_of,
                                                          int shared_slot, int n_routed_groups,
                                                          int RPB, int RCAP,
                                                          void* __restrict__ hv) {
    using AT = typename std::conditional<WT == 0, float, __bf16>::type;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    AT* xs = reinterpret_cast<AT*>(smem);
    const int NB = g.I / RPB;
    const int j = blockIdx.x / NB, nb = blockIdx.x % NB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int e, slot, p_lo, cnt;
    size_t hrow0;
    if (j < n_routed_groups) {
        e = find_active(offsets, slot_of, g.E, j, lane);
        if (e < 0) return;
        slot = slot_of ? slot_of[e] : e;
        p_lo = offsets[e];
        cnt = offsets[e + 1] - p_lo;
        hrow0 = p_lo;
    } else {
        e = g.E;
        slot = shared_slot;
        p_lo = 0;
        cnt = g.T;
        hrow0 = (size_t)g.T * g.k;
    }
    const bool shared = e == g.E;
    const uint8_t* sl = g.pool + (size_t)slot * g.slot_stride;
    const int K = g.H;
    const int nch = K / W<WT>::EPC;
    const AT* x = reinterpret_cast<const AT*>(xv);
    auto gate_row = [&](int i) { return row_chunks<WT>(sl, g.off[0], i, K); };
    auto up_row = [&](int i) { return row_chunks<WT>(sl, g.off[1], i, K); };
    auto gate_sc = [&](int i) { return WT == 2 ? sl + g.off[3] + (size_t)i * (K / 32) : nullptr; };
    auto up_sc = [&](int i) { return WT == 2 ? sl + g.off[4] + (size_t)i * (K / 32) : nullptr; };

    RowPass<WT> pg, pu;
    for (int r0 = 0; r0 < cnt; r0 += RCAP) {
        const int R = min(RCAP, cnt - r0);
        // first pass of this wave's first row pair, in flight during staging
        int i = nb * RPB + wave;
        pg.load(gate_row(i), gate_sc(i), 0, nch, lane);
        pu.load(up_row(i), up_sc(i), 0, nch, lane);
        __syncthreads();  // previous chunk's readers are done with xs
        stage_rows<AT>(xs, x, [&](int r) { int p = p_lo + r0 + r; return shared ? p : perm[p] / g.k; },
                       R, K);
        __syncthreads();
        for (int ip = wave; ip < RPB; ip += 4) {
            i = nb * RPB + ip;
            float ag[RMAX], au[RMAX];
#pragma unroll
            for (int r = 0; r < RMAX; ++r) ag[r] = au[r] = 0.f;
            for (int c0 = 0; c0 < nch; c0 += 256) {
                if (c0 > 0 || ip != wave) {
                    pg.load(gate_row(i), gate_sc(i), c0, nch, lane);
                    pu.load(up_row(i), up_sc(i), c0, nch, lane);
                }
#pragma unroll
                for (int r = 0; r < RMAX; ++r)
                    if (r < R) {
                        ag[r] = pg.dot(xs + (size_t)r * K, c0, nch, lane, ag[r]);
                        au[r] = pu.dot(xs + (size_t)r * K, c0, nch, lane, au[r]);
                    }
            }
#pragma unroll
            for (int r = 0; r < RMAX; ++r)
                if (r < R) {
                    const float gs = wave_sum_dpp(ag[r]), us = wave_sum_dpp(au[r]);
                    if (lane == r) {
                        const float hval = silu_mul(gs, us);
                        const size_t idx = (hrow0 + r0 + r) * g.I + i;
                        if constexpr (WT == 0) reinterpret_cast<float*>(hv)[idx] = hval;
                        else reinterpret_cast<uint16_t*>(hv)[idx] = (uint16_t)f32_to_bf16_bits(hval);
                    }
                }
        }
    }
}

// ---------------------------------------------------------------------------
// GEMM2: y[p][d] = h[p] . Wd[d].  Block: RPB rows d; h rows in LDS.
// ---------------------------------------------------------------------------
template <int WT, int RMAX, typename OT>
__global__ __launch_bounds__(256) void ffn2_stream_kernel(ft::FfnGeom g, const void* __restrict__ hv,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ slot_of,
                                                          int shared_slot, int n_routed_groups,
                                                          int RPB, int RCAP,
                                                          OT* __restrict__ y) {
    using AT = typename std::conditional<WT == 0, float, __bf16>::type;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    AT* hs = reinterpret_cast<AT*>(smem);
    const int NB = g.H / RPB;
    const int j = blockIdx.x / NB, nb = blockIdx.x % NB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int e, slot, cnt;
    size_t hrow0;
    if (j < n_routed_groups) {
        e = find_active(offsets, slot_of, g.E, j, lane);
        if (e < 0) return;
        slot = slot_of ? slot_of[e] : e;
        hrow0 = offsets[e];
        cnt = offsets[e + 1] - offsets[e];
    } else {
        slot = shared_slot;
        cnt = g.T;
        hrow0 = (size_t)g.T * g.k;
    }
    const uint8_t* sl = g.pool + (size_t)slot * g.slot_stride;
    const int K = g.I;
    const int nch = K / W<WT>::EPC;
    const AT* h = reinterpret_cast<const AT*>(hv);
    auto down_row = [&](int d) { return row_chunks<WT>(sl, g.off[2], d, K); };
    auto down_sc = [&](int d) { return WT == 2 ? sl + g.off[5] + (size_t)d * (K / 32) : nullptr; };

    RowPass<WT> pd;
    for (int r0 = 0; r0 < cnt; r0 += RCAP) {
        const int R = min(RCAP, cnt - r0);
        int d = nb * RPB + wave;
        pd.load(down_row(d), down_sc(d), 0, nch, lane);
        __syncthreads();
        stage_rows<AT>(hs, h, [&](int r) { return (int)(hrow0 + r0 + r); }, R, K);
        __syncthreads();
        for (int dp = wave; dp < RPB; dp += 4) {
            d = nb * RPB + dp;
            float acc[RMAX];
#pragma unroll
            for (int r = 0; r < RMAX; ++r) acc[r] = 0.f;
            for (int c0 = 0; c0 < nch; c0 += 256) {
                if (c0 > 0 || dp != wave) pd.load(down_row(d), down_sc(d), c0, nch, lane);
#pragma unroll
                for (int r = 0; r < RMAX; ++r)
                    if (r < R) acc[r] = pd.dot(hs + (size_t)r * K, c0, nch, lane, acc[r]);
            }
#pragma unroll
            for (int r = 0; r < RMAX; ++r)
                if (r < R) {
                    const float v = wave_sum_dpp(acc[r]);
                    if (lane == r) {
                        const size_t idx = (hrow0 + r0 + r) * g.H + d;
                        if constexpr (sizeof(OT) == 4) reinterpret_cast<float*>(y)[idx] = v;
                        else reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)f32_to_bf16_bits(v);
                    }
                }
        }
    }
}

// rows per block: smallest of {4, 8, 16, 32, 64} keeping the grid <= ~4096 blocks
int pick_rpb(long groups, int n_rows) {
    int rpb = 4;
    while (rpb < 64 && groups * (n_rows / rpb) > 4096 && n_rows % (rpb * 2) == 0) rpb *= 2;
    return rpb;
}

}  // namespace

namespace ft {

ft_status launch_ffn_stream(const FfnGeom& g, const void* x, const int32_t* perm,
                            const int32_t* offsets, const int32_t* slot_of, int shared_slot,
                            void* h, void* y, ft_dtype y_dt, hipStream_t s) {
    const long tk = (long)g.T * g.k;
    const int routed_groups = (int)(tk < g.E ? tk : g.E);
    const int groups = routed_groups + (g.n_shared ? 1 : 0);
    const int rpb1 = pick_rpb(groups, g.I), rpb2 = pick_rpb(groups, g.H);
    dim3 g1((unsigned)groups * (g.I / rpb1)), g2((unsigned)groups * (g.H / rpb2)), blk(256);
    const int big = g.H > 2048 || g.I > 2048;

    prof_begin(PROF_FFN_GEMM1, s);
    // activation rows per pass: at most RMAX, at most T (an expert never gets more than T rows)
#define FT_S1(WT, RM)                                                                         \
    ffn1_stream_kernel<WT, RM><<<g1, blk, (size_t)min(RM, g.T) * g.H * (WT == 0 ? 4 : 2), s>>>( \
        g, x, perm, offsets, slot_of, shared_slot, routed_groups, rpb1, min(RM, g.T), h)
    if (g.w_dt == FT_F32) FT_S1(0, 8);
    else if (g.w_dt == FT_BF16) { if (big) FT_S1(1, 4); else FT_S1(1, 8); }
    else { if (big) FT_S1(2, 4); else FT_S1(2, 8); }
#undef FT_S1
    FT_LAUNCHED("ffn1_stream");
    prof_end(PROF_FFN_GEMM1, s);

    prof_begin(PROF_FFN_GEMM2, s);
#define FT_S2(WT, RM, OT)                                                                     \
    ffn2_stream_kernel<WT, RM, OT><<<g2, blk, (size_t)min(RM, g.T) * g.I * (WT == 0 ? 4 : 2), s>>>( \
        g, h, offsets, slot_of, shared_slot, routed_groups, rpb2, min(RM, g.T), (OT*)y)
    if (g.w_dt == FT_F32) FT_S2(0, 8, float);
    else if (g.w_dt == FT_BF16) {
        if (y_dt == FT_F32) { if (big) FT_S2(1, 4, float); else FT_S2(1, 8, float); }
        else { if (big) FT_S2(1, 4, __bf16); else FT_S2(1, 8, __bf16); }
    } else {
        if (y_dt == FT_F32) { if (big) FT_S2(2, 4, float); else FT_S2(2, 8, float); }
        else { if (big) FT_S2(2, 4, __bf16); else FT_S2(2, 8, __bf16); }
    }
#undef FT_S2
    FT_LAUNCHED("ffn2_stream");
    prof_end(PROF_FFN_GEMM2, s);
    return FT_OK;
}

}  // namespace ft
