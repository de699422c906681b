// gemm_mfma.hip -- MFMA tile kernels of the grouped expert GEMMs (gfx950).
//
// The expert FFN over many tokens is a set of dense contractions, one per
// expert, over the rows routed to it (claypier.com article,
// "从 MoE「用不到的权重」入手的推理引擎": only the experts a token needs are
// computed).  Each 128-row M-tile of an expert's segment of the permutation is
// one entry of a tile list; a block computes a 128 x 128 output tile with
// v_mfma_f32_16x16x32_bf16 and fp32 accumulation, staging 64-wide K slices of
// both operands through LDS (double-buffered: the global loads of slice k+1
// are in flight while slice k feeds the MFMAs).
//
// GEMM1 fuses SwiGLU: the B tile holds 64 gate rows and the same 64 up rows,
// each wavefront owns matching gate/up accumulators, and the epilogue writes
// h = silu(g) * u in bf16.  GEMM2 multiplies h by the down projection.
// MXFP4 weights are decoded exactly to bf16 (e2m1 value times the e8m0 block
// scale) on their way into LDS, so the MFMA loop is the same for both formats.
//
// LDS layout of a 128 x 64 bf16 slice: row r is 128 bytes = 8 chunks of 16
// bytes; chunk c is stored at position c ^ ((r >> 1) & 7) so that the 16 rows
// a fragment read touches fall on distinct banks.
#include "gemm_mfma.h"

namespace {

using ft::TileDesc;
constexpr int BM = ft::GEMM_BM, BN = ft::GEMM_BN, BK = ft::GEMM_BK, NTHR = 256;

__device__ __forceinline__ int lds_idx(int r, int c) {
    return r * BK + ((c ^ ((r >> 1) & 7)) << 3);
}

// 32 e2m1 values (16 code bytes) times 2^(X-127) -> 4 chunks of 8 bf16.
// Element 2j is the low nibble of byte j.
__device__ __forceinline__ void decode_fp4x32(u32x4_t codes, uint32_t X, u32x4_t out[4]) {
    const float sc = __uint_as_float(X << 23);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t w = codes[q];
        out[q][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
        out[q][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
        out[q][2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
        out[q][3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
    }
}

// Staging of one 128 x 64 B slice.  bf16: thread owns rows (tid>>3)+32i, chunk
// tid&7.  MXFP4: thread owns row tid>>1, half tid&1 (32 codes, one scale).
template <int BT>
struct BStage {
    u32x4_t v[4];
    uint32_t sc;
    const uint8_t* src[4];
    const uint8_t* scp;

    // rowptr(r) = byte address of B row r (codes for MXFP4), scrow(r) = its scales
    template <typename RowF, typename ScF>
    __device__ __forceinline__ void init(int tid, RowF rowptr, ScF scrow) {
        if constexpr (BT == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) src[i] = rowptr((tid >> 3) + 32 * i) + (tid & 7) * 16;
        } else {
            src[0] = rowptr(tid >> 1) + (tid & 1) * 16;
            scp = scrow(tid >> 1) + (tid & 1);
        }
    }
    __device__ __forceinline__ void load(int kt) {
        if constexpr (BT == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const u32x4_t*>(src[i] + kt * BK * 2);
        } else {
            v[0] = *reinterpret_cast<const u32x4_t*>(src[0] + kt * (BK / 2));
            sc = scp[kt * (BK / 32)];
        }
    }
    __device__ __forceinline__ void store(__bf16* lds, int tid) const {
        if constexpr (BT == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<u32x4_t*>(lds + lds_idx((tid >> 3) + 32 * i, tid & 7)) = v[i];
        } else {
            u32x4_t d[4];
            decode_fp4x32(v[0], sc, d);
            const int r = tid >> 1, h = (tid & 1) * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x4_t*>(lds + lds_idx(r, h + q)) = d[q];
        }
    }
};

struct AStage {
    u32x4_t v[4];
    const __bf16* src[4];
    __device__ __forceinline__ void load(int kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const u32x4_t*>(src[i] + kt * BK);
    }
    __device__ __forceinline__ void store(__bf16* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4_t*>(lds + lds_idx((tid >> 3) + 32 * i, tid & 7)) = v[i];
    }
};

__device__ __forceinline__ bf16x8_t frag(const __bf16* lds, int r, int c) {
    return *reinterpret_cast<const bf16x8_t*>(lds + lds_idx(r, c));
}
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// GEMM1 + SwiGLU
// ---------------------------------------------------------------------------
template <int BT>
__global__ __launch_bounds__(NTHR, 2) void gemm1_kernel(ft::FfnGeom g, const __bf16* __restrict__ x,
                                                        const int32_t* __restrict__ perm,
                                                        const TileDesc* __restrict__ tiles,
                                                        const int* __restrict__ n_tiles,
                                                        int n_ntiles, __bf16* __restrict__ h) {
    __shared__ __attribute__((aligned(16))) __bf16 As[2][BM * BK];
    __shared__ __attribute__((aligned(16))) __bf16 Bs[2][BN * BK];
    const int ti = blockIdx.x / n_ntiles, nt = blockIdx.x % n_ntiles;
    if (ti >= *n_tiles) return;
    const TileDesc td = tiles[ti];
    const int tid = threadIdx.x, K = g.H, I = g.I;
    const int i0 = nt * (BN / 2);
    const bool shared = td.e == g.E;
    const uint8_t* slot = g.pool + (size_t)td.slot * g.slot_stride;

    AStage as;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int r = min((tid >> 3) + 32 * i, td.rows - 1);
        int p = td.p0 + r;
        int t = shared ? p : perm[p] / g.k;
        as.src[i] = x + (size_t)t * K + (tid & 7) * 8;
    }
    BStage<BT> bs;
    if constexpr (BT == 0) {
        bs.init(tid,
                [&](int r) {
                    return slot + (r < 64 ? g.off[0] : g.off[1]) + (size_t)(i0 + (r & 63)) * K * 2;
                },
                [&](int) { return (const uint8_t*)nullptr; });
    } else {
        bs.init(tid,
                [&](int r) {
                    return slot + (r < 64 ? g.off[0] : g.off[1]) + (size_t)(i0 + (r & 63)) * (K / 2);
                },
                [&](int r) {
                    return slot + (r < 64 ? g.off[3] : g.off[4]) + (size_t)(i0 + (r & 63)) * (K / 32);
                });
    }

    const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    f32x4_t accg[4][2], accu[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) accg[a][b] = accu[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = K / BK;
    as.load(0);
    bs.load(0);
    as.store(As[0], tid);
    bs.store(Bs[0], tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            as.load(kt + 1);
            bs.load(kt + 1);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int ch = ks * 4 + (lane >> 4);
            bf16x8_t a[4], bg[2], bu[2];
#pragma unroll
            for (int m = 0; m < 4; ++m) a[m] = frag(As[cur], wm * 64 + m * 16 + (lane & 15), ch);
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                bg[n] = frag(Bs[cur], wn * 32 + n * 16 + (lane & 15), ch);
                bu[n] = frag(Bs[cur], 64 + wn * 32 + n * 16 + (lane & 15), ch);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    accg[m][n] = mfma16(a[m], bg[n], accg[m][n]);
                    accu[m][n] = mfma16(a[m], bu[n], accu[m][n]);
                }
        }
        if (kt + 1 < nk) {
            as.store(As[cur ^ 1], tid);
            bs.store(Bs[cur ^ 1], tid);
        }
        __syncthreads();
    }

    const size_t hbase = shared ? (size_t)g.T * g.k + td.p0 : (size_t)td.p0;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = wm * 64 + m * 16 + 4 * (lane >> 4) + j;
                const int col = i0 + wn * 32 + n * 16 + (lane & 15);
                if (row < td.rows) {
                    float hv = silu_mul(accg[m][n][j], accu[m][n][j]);
                    reinterpret_cast<uint16_t*>(h)[(hbase + row) * I + col] =
                        (uint16_t)f32_to_bf16_bits(hv);
                }
            }
}

// ---------------------------------------------------------------------------
// plain GEMM: out[row][n] = A[row] . B[n]  (GEMM2 over the tile list, or a
// dense M x N problem for the router logits)
// ---------------------------------------------------------------------------
template <int BT, typename OutT, bool DENSE>
__global__ __launch_bounds__(NTHR, 2) void gemm_plain_kernel(
    ft::FfnGeom g, const __bf16* __restrict__ A, const __bf16* __restrict__ Bdense, int M,
    int N, int K, const TileDesc* __restrict__ tiles, const int* __restrict__ n_tiles,
    int n_ntiles, OutT* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) __bf16 As[2][BM * BK];
    __shared__ __attribute__((aligned(16))) __bf16 Bs[2][BN * BK];
    const int ti = blockIdx.x / n_ntiles, nt = blockIdx.x % n_ntiles;
    TileDesc td;
    if constexpr (DENSE) {
        td.e = 0;
        td.p0 = ti * BM;
        td.rows = min(BM, M - ti * BM);
        td.slot = 0;
    } else {
        if (ti >= *n_tiles) return;
        td = tiles[ti];
    }
    const int tid = threadIdx.x;
    const int n0 = nt * BN;
    const size_t rbase =
        DENSE ? (size_t)td.p0 : (td.e == g.E ? (size_t)g.T * g.k + td.p0 : (size_t)td.p0);

    AStage as;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int r = min((tid >> 3) + 32 * i, td.rows - 1);
        as.src[i] = A + (rbase + r) * K + (tid & 7) * 8;
    }
    BStage<BT> bs;
    if constexpr (DENSE) {
        bs.init(tid,
                [&](int r) {
                    return reinterpret_cast<const uint8_t*>(Bdense + (size_t)min(n0 + r, N - 1) * K);
                },
                [&](int) { return (const uint8_t*)nullptr; });
    } else {
        const uint8_t* slot = g.pool + (size_t)td.slot * g.slot_stride;
        // rows past N (H not a multiple of 128) re-read row N-1; their columns are not stored
        if constexpr (BT == 0)
            bs.init(tid, [&](int r) { return slot + g.off[2] + (size_t)min(n0 + r, N - 1) * K * 2; },
                    [&](int) { return (const uint8_t*)nullptr; });
        else
            bs.init(tid, [&](int r) { return slot + g.off[2] + (size_t)min(n0 + r, N - 1) * (K / 2); },
                    [&](int r) { return slot + g.off[5] + (size_t)min(n0 + r, N - 1) * (K / 32); });
    }

    const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    f32x4_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = K / BK;
    as.load(0);
    bs.load(0);
    as.store(As[0], tid);
    bs.store(Bs[0], tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            as.load(kt + 1);
            bs.load(kt + 1);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int ch = ks * 4 + (lane >> 4);
            bf16x8_t a[4], b[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) a[m] = frag(As[cur], wm * 64 + m * 16 + (lane & 15), ch);
#pragma unroll
            for (int n = 0; n < 4; ++n) b[n] = frag(Bs[cur], wn * 64 + n * 16 + (lane & 15), ch);
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int n = 0; n < 4; ++n) acc[m][n] = mfma16(a[m], b[n], acc[m][n]);
        }
        if (kt + 1 < nk) {
            as.store(As[cur ^ 1], tid);
            bs.store(Bs[cur ^ 1], tid);
        }
        __syncthreads();
    }

#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = wm * 64 + m * 16 + 4 * (lane >> 4) + j;
                const int col = n0 + wn * 64 + n * 16 + (lane & 15);
                if (row < td.rows && col < N) {
                    float v = acc[m][n][j];
                    if constexpr (sizeof(OutT) == 4)
                        reinterpret_cast<float*>(out)[(rbase + row) * N + col] = v;
                    else
                        reinterpret_cast<uint16_t*>(out)[(rbase + row) * N + col] =
                            (uint16_t)f32_to_bf16_bits(v);
                }
            }
}

// ---------------------------------------------------------------------------
// tile list
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ slot_of,
                                                           int E, int T, int n_shared,
                                                           int shared_slot, TileDesc* tiles,
                                                           int* n_tiles, int max_tiles) {
    __shared__ int scan[1024];
    const int e = threadIdx.x;
    int cnt = 0, c = 0, off = 0, slot = -1;
    if (e < E) {
        off = offsets[e];
        c = offsets[e + 1] - off;
        slot = slot_of ? slot_of[e] : e;
        if (slot >= 0 && c > 0) cnt = (c + BM - 1) / BM;
    }
    scan[e] = cnt;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
        int v = e >= o ? scan[e - o] : 0;
        __syncthreads();
        scan[e] += v;
        __syncthreads();
    }
    const int base = scan[e] - cnt, total = scan[1023];
    for (int m = 0; m < cnt; ++m) {
        int idx = base + m;
        if (idx < max_tiles) tiles[idx] = TileDesc{e, off + m * BM, min(BM, c - m * BM), slot};
    }
    int ns = n_shared ? (T + BM - 1) / BM : 0;
    for (int m = e; m < ns; m += 1024) {
        int idx = total + m;
        if (idx < max_tiles) tiles[idx] = TileDesc{E, m * BM, min(BM, T - m * BM), shared_slot};
    }
    if (e == 0) *n_tiles = min(total + ns, max_tiles);
}

}  // namespace

namespace ft {

ft_status launch_build_tiles(const FfnGeom& g, const int32_t* offsets,
                             const int32_t* slot_of_expert, int shared_slot, TileDesc* tiles,
                             int* n_tiles, int max_tiles, hipStream_t s) {
    build_tiles_kernel<<<1, 1024, 0, s>>>(offsets, slot_of_expert, g.E, g.T, g.n_shared,
                                          shared_slot, tiles, n_tiles, max_tiles);
    FT_LAUNCHED("build_tiles");
    return FT_OK;
}

ft_status launch_gemm1_mfma(const FfnGeom& g, const __bf16* x, const int32_t* perm,
                            const TileDesc* tiles, const int* n_tiles, int max_tiles,
                            __bf16* h, hipStream_t s) {
    const int n_ntiles = g.I / (BN / 2);
    dim3 grid((unsigned)max_tiles * n_ntiles), block(NTHR);
    if (g.w_dt == FT_MXFP4)
        gemm1_kernel<1><<<grid, block, 0, s>>>(g, x, perm, tiles, n_tiles, n_ntiles, h);
    else
        gemm1_kernel<0><<<grid, block, 0, s>>>(g, x, perm, tiles, n_tiles, n_ntiles, h);
    FT_LAUNCHED("gemm1_mfma");
    return FT_OK;
}

ft_status launch_gemm2_mfma(const FfnGeom& g, const __bf16* h, const TileDesc* tiles,
                            const int* n_tiles, int max_tiles, void* y, ft_dtype y_dt,
                            hipStream_t s) {
    const int n_ntiles = cdiv(g.H, BN);
    dim3 grid((unsigned)max_tiles * n_ntiles), block(NTHR);
#define FT_G2(BT, OT)                                                                    \
    gemm_plain_kernel<BT, OT, false><<<grid, block, 0, s>>>(g, h, nullptr, 0, g.H, g.I, tiles, \
                                                            n_tiles, n_ntiles, (OT*)y)
    if (g.w_dt == FT_MXFP4) {
        if (y_dt == FT_F32) FT_G2(1, float); else FT_G2(1, __bf16);
    } else {
        if (y_dt == FT_F32) FT_G2(0, float); else FT_G2(0, __bf16);
    }
#undef FT_G2
    FT_LAUNCHED("gemm2_mfma");
    return FT_OK;
}

ft_status launch_dense_gemm_f32out(const void* A, const void* B, int M, int N, int K,
                                   float* out, hipStream_t s) {
    FfnGeom g{};
    const int n_ntiles = cdiv(N, BN);
    dim3 grid((unsigned)cdiv(M, BM) * n_ntiles), block(NTHR);
    gemm_plain_kernel<0, float, true><<<grid, block, 0, s>>>(
        g, (const __bf16*)A, (const __bf16*)B, M, N, K, nullptr, nullptr, n_ntiles, out);
    FT_LAUNCHED("dense_gemm_f32out");
    return FT_OK;
}

}  // namespace ft
