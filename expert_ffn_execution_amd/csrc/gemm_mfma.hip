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

#include <type_traits>

namespace {

using ft::TileDesc;
constexpr int BK = ft::GEMM_BK;

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

__device__ __forceinline__ bf16x8_t frag(const __bf16* lds, int r, int c) {
    return *reinterpret_cast<const bf16x8_t*>(lds + lds_idx(r, c));
}
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_32x32x16_bf16 sustains about twice the rate of the 16x16x32 form
// on gfx950 (measured), so the expert GEMMs use it
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Tile shapes.  A block computes a BM x BN output tile with NW = (BM/WM) x
// (BN/WN) wavefronts, each owning a WM x WN sub-tile of 16 x 16 MFMA tiles
// (fp32 accumulators: WM*WN/64 registers per lane, held in AGPRs for the
// large shape).  LDS holds two stages of BM x 64 (A) and BN x 64 (B) bf16.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int WM_, int WN_, int MINB_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, MINB = MINB_;
    static constexpr int WAVES_N = BN / WN, NW = (BM / WM) * (BN / WN), NT = NW * 64;
    static constexpr int MT = WM / 16, NTL = WN / 16;
    static constexpr int A_CH = BM * 8 / NT;   // 16-byte A chunks per thread per slice
    static constexpr int B_CH = BN * 8 / NT;   // 16-byte bf16 B chunks per thread
    static constexpr int B_MX = BN * 2 / NT;   // (row, half) MXFP4 units per thread
    static constexpr size_t LDS = (size_t)2 * (BM + BN) * BK * 2;
};
// the router logits (N = E is small) use 64 x 64 tiles to spread over more CUs
using RouterTile = TileCfg<64, 64, 32, 32, 4>;

enum { MODE_GATED = 0, MODE_LIST = 1, MODE_DENSE = 2 };

// B staging: 32-bit byte offsets from a block-uniform base (the slot), so
// that the per-thread state is one VGPR per chunk.
template <class C, int BT>
struct BSlice {
    static constexpr int NV = BT == 0 ? C::B_CH : C::B_MX;
    u32x4_t v[NV];
    uint32_t sc[BT == 0 ? 1 : NV];
    const uint8_t* base;
    uint32_t off[NV];
    uint32_t scoff[BT == 0 ? 1 : NV];

    // rowoff(r) = byte offset of B row r (codes for MXFP4), scoff(r) = its scales
    template <typename RowF, typename ScF>
    __device__ __forceinline__ void init(const uint8_t* b, int tid, RowF rowoff, ScF scrow) {
        base = b;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if constexpr (BT == 0) {
                off[i] = rowoff((tid >> 3) + (C::NT / 8) * i) + (tid & 7) * 16;
            } else {
                const int q = tid + C::NT * i;
                off[i] = rowoff(q >> 1) + (q & 1) * 16;
                scoff[i] = scrow(q >> 1) + (q & 1);
            }
        }
    }
    __device__ __forceinline__ void load(int kt) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if constexpr (BT == 0) {
                v[i] = *reinterpret_cast<const u32x4_t*>(base + off[i] + kt * BK * 2);
            } else {
                v[i] = *reinterpret_cast<const u32x4_t*>(base + off[i] + kt * (BK / 2));
                sc[i] = base[scoff[i] + kt * (BK / 32)];
            }
        }
    }
    __device__ __forceinline__ void store(__bf16* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if constexpr (BT == 0) {
                *reinterpret_cast<u32x4_t*>(lds + lds_idx((tid >> 3) + (C::NT / 8) * i, tid & 7)) = v[i];
            } else {
                u32x4_t d[4];
                decode_fp4x32(v[i], sc[i], d);
                const int q = tid + C::NT * i, r = q >> 1, h = (q & 1) * 4;
#pragma unroll
                for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4_t*>(lds + lds_idx(r, h + c)) = d[c];
            }
        }
    }
};

// A staging: 32-bit element offsets of the (gathered) rows from the A base.
template <class C>
struct ASlice {
    u32x4_t v[C::A_CH];
    const __bf16* base;
    uint32_t off[C::A_CH];
    __device__ __forceinline__ void load(int kt) {
#pragma unroll
        for (int i = 0; i < C::A_CH; ++i)
            v[i] = *reinterpret_cast<const u32x4_t*>(base + off[i] + kt * BK);
    }
    __device__ __forceinline__ void store(__bf16* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < C::A_CH; ++i)
            *reinterpret_cast<u32x4_t*>(lds + lds_idx((tid >> 3) + (C::NT / 8) * i, tid & 7)) = v[i];
    }
};

// One kernel for the three contractions:
//   MODE_GATED: h[p][i] = bf16(silu(x_t . Wg_i) * (x_t . Wu_i)) (B tile = BN/2 gate rows
//               followed by the same BN/2 up rows)
//   MODE_LIST:  out[p][n] = A[p] . B_n over the tile list (down projection)
//   MODE_DENSE: out[m][n] = A[m] . B_n for a dense M x N problem (router logits)
template <class C, int MODE, int BT, typename OutT>
__global__ __launch_bounds__(C::NT, C::MINB) void gemm_tile_kernel(
    ft::FfnGeom g, const __bf16* __restrict__ A, const int32_t* __restrict__ perm,
    const __bf16* __restrict__ Bdense, int M, int N, int K, const TileDesc* __restrict__ tiles,
    const int* __restrict__ n_tiles, int n_ntiles, OutT* __restrict__ out) {
    extern __shared__ __attribute__((aligned(16))) __bf16 smem[];
    __bf16* const A0 = smem;
    __bf16* const B0 = smem + 2 * C::BM * BK;
    const int ti = blockIdx.x / n_ntiles, nt = blockIdx.x % n_ntiles;
    TileDesc td;
    if constexpr (MODE == MODE_DENSE) {
        td = TileDesc{0, ti * C::BM, min(C::BM, M - ti * C::BM), 0};
    } else {
        if (ti >= *n_tiles) return;
        td = tiles[ti];
    }
    const int tid = threadIdx.x;
    const bool shared = MODE != MODE_DENSE && td.e == g.E;
    // first output row of the tile (shared-expert rows follow the T*k routed rows)
    const size_t obase = shared ? (size_t)g.T * g.k + td.p0 : (size_t)td.p0;

    ASlice<C> as;
    as.base = A;
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
        const int r = min((tid >> 3) + (C::NT / 8) * i, td.rows - 1);
        uint32_t arow;
        if constexpr (MODE == MODE_GATED) arow = shared ? (uint32_t)(td.p0 + r) : (uint32_t)(perm[td.p0 + r] / g.k);
        else arow = (uint32_t)(obase + r);
        as.off[i] = arow * (uint32_t)K + (tid & 7) * 8;
    }
    BSlice<C, BT> bs;
    const uint8_t* slot = MODE == MODE_DENSE ? nullptr : g.pool + (size_t)td.slot * g.slot_stride;
    const int i0 = nt * (C::BN / 2), n0 = nt * C::BN;
    const uint32_t rowb = BT == 0 ? (uint32_t)K * 2 : (uint32_t)K / 2;  // bytes per B row
    if constexpr (MODE == MODE_GATED) {
        bs.init(slot, tid,
                [&](int r) {
                    const uint32_t row = i0 + (r % (C::BN / 2));
                    return (uint32_t)(r < C::BN / 2 ? g.off[0] : g.off[1]) + row * rowb;
                },
                [&](int r) {
                    const uint32_t row = i0 + (r % (C::BN / 2));
                    return (uint32_t)(r < C::BN / 2 ? g.off[3] : g.off[4]) + row * (uint32_t)(K / 32);
                });
    } else if constexpr (MODE == MODE_LIST) {
        // rows past N (N not a multiple of BN) re-read row N-1; their columns are not stored
        bs.init(slot, tid,
                [&](int r) { return (uint32_t)g.off[2] + (uint32_t)min(n0 + r, N - 1) * rowb; },
                [&](int r) {
                    return (uint32_t)g.off[5] + (uint32_t)min(n0 + r, N - 1) * (uint32_t)(K / 32);
                });
    } else {
        bs.init(reinterpret_cast<const uint8_t*>(Bdense), tid,
                [&](int r) { return (uint32_t)min(n0 + r, N - 1) * rowb; },
                [&](int) { return 0u; });
    }

    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    f32x4_t acc[C::MT][C::NTL];
#pragma unroll
    for (int a = 0; a < C::MT; ++a)
#pragma unroll
        for (int b = 0; b < C::NTL; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = K / BK;
    as.load(0);
    bs.load(0);
    as.store(A0, tid);
    bs.store(B0, tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            as.load(kt + 1);
            bs.load(kt + 1);
        }
        const __bf16* Ac = A0 + cur * (C::BM * BK);
        const __bf16* Bc = B0 + cur * (C::BN * BK);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int ch = ks * 4 + (lane >> 4);
            bf16x8_t a[C::MT], b[C::NTL];
#pragma unroll
            for (int m = 0; m < C::MT; ++m) a[m] = frag(Ac, wm * C::WM + m * 16 + (lane & 15), ch);
#pragma unroll
            for (int n = 0; n < C::NTL; ++n) {
                int brow;
                if constexpr (MODE == MODE_GATED)  // first half of the wave's tiles: gate, second: up
                    brow = (n < C::NTL / 2 ? 0 : C::BN / 2) + wn * (C::WN / 2) + (n % (C::NTL / 2)) * 16;
                else
                    brow = wn * C::WN + n * 16;
                b[n] = frag(Bc, brow + (lane & 15), ch);
            }
#pragma unroll
            for (int m = 0; m < C::MT; ++m)
#pragma unroll
                for (int n = 0; n < C::NTL; ++n) acc[m][n] = mfma16(a[m], b[n], acc[m][n]);
        }
        if (kt + 1 < nk) {
            as.store(A0 + (cur ^ 1) * (C::BM * BK), tid);
            bs.store(B0 + (cur ^ 1) * (C::BN * BK), tid);
        }
        __syncthreads();
    }

    // epilogue: lane holds column (lane & 15), rows 4*(lane >> 4) + j of each 16 x 16 tile
#pragma unroll
    for (int m = 0; m < C::MT; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = wm * C::WM + m * 16 + 4 * (lane >> 4) + j;
            if (row >= td.rows) continue;
            if constexpr (MODE == MODE_GATED) {
#pragma unroll
                for (int n = 0; n < C::NTL / 2; ++n) {
                    const int col = i0 + wn * (C::WN / 2) + n * 16 + (lane & 15);
                    const float hv = silu_mul(acc[m][n][j], acc[m][n + C::NTL / 2][j]);
                    reinterpret_cast<uint16_t*>(out)[(obase + row) * g.I + col] =
                        (uint16_t)f32_to_bf16_bits(hv);
                }
            } else {
#pragma unroll
                for (int n = 0; n < C::NTL; ++n) {
                    const int col = n0 + wn * C::WN + n * 16 + (lane & 15);
                    if (col < N) {
                        const float v = acc[m][n][j];
                        if constexpr (sizeof(OutT) == 4)
                            reinterpret_cast<float*>(out)[(obase + row) * N + col] = v;
                        else
                            reinterpret_cast<uint16_t*>(out)[(obase + row) * N + col] =
                                (uint16_t)f32_to_bf16_bits(v);
                    }
                }
            }
        }
}

// ---------------------------------------------------------------------------
// Pipelined tile kernel for the expert GEMMs.  256 x 256 output tile, 4
// wavefronts (one per SIMD), each owning all 256 rows and a 64-column strip:
// 8 x 2 tiles of v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane),
// K in slices of 32 through five LDS stages.
// Slices are copied global -> LDS by the load units directly
// (global_load_lds_dwordx4: each wave instruction fills 1 KB of LDS, lane l
// its 16 bytes), so four slices are in flight while the fifth feeds the
// MFMAs and no registers hold staged data.  A wave waits for its own copies
// of a slice with s_waitcnt vmcnt and the block barrier then publishes it.
// The tile is as large as the 160 KB LDS allows so that every byte brought
// into the CU feeds as many MFMAs as possible: per slice 32 KB carry 4.2
// MFLOP.  MXFP4 weights stay packed in LDS (16 code bytes + 1 scale byte per
// row and slice) and are decoded to bf16 when a fragment is read.
// An expert's last M-tile is usually partly filled (routing gives each
// expert an arbitrary row count): since every wave spans all rows, all waves
// skip the MFMAs and fragment reads of 32-row sub-tiles past the tile's rows
// alike, and the block's time shrinks with its row count.
//
// LDS layout of a slice of rows: row r is 64 bytes = 4 chunks of 16 bytes,
// chunk c stored at position c ^ ((r >> 2) & 3): the 16 rows a fragment read
// touches then cover all 64 banks exactly once.
// ---------------------------------------------------------------------------
namespace pipe {
constexpr int BM = 256, BN = 256, KS = 32, NT = 256, NW = NT / 64, WN = BN / NW;
constexpr int STAGES = 5;   // 5 x 32 KB = all 160 KB of LDS (bf16)
constexpr int MT = BM / 32, NTL = WN / 32;   // 32 x 32 MFMA tiles per wavefront
constexpr int ROWB = KS * 2;                          // bytes of a bf16 row slice
constexpr int A_BYTES = BM * ROWB;                    // 16 KB
constexpr int AL = A_BYTES / 1024 / NW;               // A copies per wave per slice
// BT: 0 bf16 weights, 1 MXFP4, 2 FP8 (e4m3, one fp32 scale per matrix).
// MXFP4: codes [BN][16 B], then one 4-byte slot per row holding its scale byte
// (a 1-byte LDS-DMA load writes each lane's byte to a 4-byte slot).
// FP8: codes [BN][32 B]; the two 16-byte halves of rows 8..15 of every 16 are
// swapped (h ^ ((r >> 3) & 1)) so that fragment reads spread over the banks.
template <int BT> constexpr int b_bytes() { return BT == 0 ? BN * ROWB : BT == 1 ? BN * 16 + BN * 4 : BN * KS; }
template <int BT> constexpr int stage_bytes() { return A_BYTES + b_bytes<BT>(); }
constexpr size_t EPI_BYTES = (size_t)BM * (BN + 8) * 2;   // bf16 output tile (plain GEMM)
template <int BT> constexpr size_t lds_bytes() {
    return (size_t)STAGES * stage_bytes<BT>() > EPI_BYTES ? (size_t)STAGES * stage_bytes<BT>() : EPI_BYTES;
}
// global_load_lds instructions per wave per slice: A, then B (bf16 and FP8:
// 1 KB pieces; MXFP4: one codes piece of 64 rows and one scale byte per lane)
template <int BT> constexpr int b_copies() { return BT == 0 ? BN * ROWB / 1024 / NW : BT == 1 ? 1 : BN * KS / 1024 / NW; }
template <int BT> constexpr int loads_per_slice() { return AL + (BT == 1 ? 2 : b_copies<BT>()); }
__device__ __forceinline__ int fp8_half(int r, int h) { return h ^ ((r >> 3) & 1); }
__device__ __forceinline__ int sw(int r, int c) { return r * ROWB + ((c ^ ((r >> 2) & 3)) << 4); }
}  // namespace pipe

#define FT_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt vmcnt(n) lgkmcnt(0) (gfx9 encoding: vmcnt bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// 8 e4m3 codes (bytes of w0, then w1) -> 8 bf16, exact
__device__ __forceinline__ bf16x8_t fp8_frag(uint32_t w0, uint32_t w1) {
    u32x4_t d;
    d[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
    d[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
    d[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
    d[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
    return __builtin_bit_cast(bf16x8_t, d);
}

__device__ __forceinline__ bf16x8_t fp4_frag(uint32_t codes, uint32_t X) {
    const float sc = __uint_as_float(X << 23);
    u32x4_t d;
    d[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0));
    d[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1));
    d[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2));
    d[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3));
    return __builtin_bit_cast(bf16x8_t, d);
}

// f(std::integral_constant<int, M>) for the runtime M in [1, N].
template <int N, typename F>
__device__ __forceinline__ void with_count(int M, F&& f) {
    if constexpr (N >= 1) {
        if (M >= N) f(std::integral_constant<int, N>{});
        else with_count<N - 1>(M, f);
    }
}

template <int MODE, int BT, typename OutT>
__global__ __launch_bounds__(pipe::NT, 1) void gemm_pipe_kernel(
    ft::FfnGeom g, const __bf16* __restrict__ A, const int32_t* __restrict__ perm,
    const TileDesc* __restrict__ tiles, const int* __restrict__ n_tiles, int n_ntiles,
    OutT* __restrict__ out) {
    using namespace pipe;
    static_assert(STAGES == 5, "wait schedule below assumes five stages");
    extern __shared__ __attribute__((aligned(16))) unsigned char pipe_smem[];
    unsigned char* const smem = pipe_smem;
    // XCD-aware order: the dispatcher deals blocks to the 8 XCDs round-robin;
    // give XCD x a contiguous run of the real work so that the N-tiles of one
    // M-tile (same activation rows) share that XCD's L2.
    const int work = *n_tiles * n_ntiles;
    const int per_xcd = (work + 7) / 8;
    const int local = blockIdx.x / 8;
    const int lb = (blockIdx.x % 8) * per_xcd + local;
    if (local >= per_xcd || lb >= work) return;
    const int ti = lb / n_ntiles, nt = lb % n_ntiles;
    const TileDesc td = tiles[ti];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int K = MODE == MODE_GATED ? g.H : g.I;
    const int NOUT = MODE == MODE_GATED ? g.I : g.H;   // output columns (h or y)
    const bool shared = td.e == g.E;
    const size_t obase = shared ? (size_t)g.T * g.k + td.p0 : (size_t)td.p0;
    const uint8_t* slot = g.pool + (size_t)td.slot * g.slot_stride;
    // gated: B rows [0, 128) = gate rows c0.., [128, 256) = up rows c0..; plain: rows c0..
    const int c0 = nt * (MODE == MODE_GATED ? BN / 2 : BN);

    // A: copy i of this wave fills LDS rows 16 * (AL * wave + i) + lane / 4,
    // physical chunk lane % 4 (rows past the tile re-read its last row)
    uint32_t aoff[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int r = 16 * (AL * wave + i) + (lane >> 2);
        const int rc = min(r, td.rows - 1);
        uint32_t arow;
        if constexpr (MODE == MODE_GATED) arow = shared ? (uint32_t)(td.p0 + rc) : (uint32_t)(perm[td.p0 + rc] / g.k);
        else arow = (uint32_t)(obase + rc);
        aoff[i] = arow * (uint32_t)K + (uint32_t)(((lane & 3) ^ ((r >> 2) & 3)) * 8);
    }
    // B row r of the tile -> weight row (clamped: columns past NOUT are not stored)
    auto wrow = [&](int r) __attribute__((always_inline)) -> uint32_t {
        if constexpr (MODE == MODE_GATED) return (uint32_t)min(c0 + (r % (BN / 2)), NOUT - 1);
        else return (uint32_t)min(c0 + r, NOUT - 1);
    };
    auto wbase = [&](int r, int which) __attribute__((always_inline)) -> uint32_t {  // which: 0 codes/values, 1 scales
        if constexpr (MODE == MODE_GATED)
            return (uint32_t)(r < BN / 2 ? g.off[which ? 3 : 0] : g.off[which ? 4 : 1]);
        else
            return (uint32_t)g.off[which ? 5 : 2];
    };
    const uint32_t rowb = BT == 0 ? (uint32_t)K * 2 : BT == 1 ? (uint32_t)K / 2 : (uint32_t)K;
    // B value/code copies per wave: b_copies<BT>() <= 4 (a literal bound: a
    // call in an array bound reads as a variable-length array to the host pass)
    uint32_t boff[4], soff = 0;
    static_assert(b_copies<BT>() <= 4, "B copies per wave");
    if constexpr (BT == 0) {
#pragma unroll
        for (int i = 0; i < b_copies<BT>(); ++i) {
            const int r = 16 * (b_copies<BT>() * wave + i) + (lane >> 2);
            boff[i] = wbase(r, 0) + wrow(r) * rowb + (uint32_t)(((lane & 3) ^ ((r >> 2) & 3)) * 16);
        }
    } else if constexpr (BT == 1) {  // codes: row 64 * wave + lane, 16 bytes per slice; its scale byte likewise
        const int r = 64 * wave + lane;
        boff[0] = wbase(r, 0) + wrow(r) * rowb;
        soff = wbase(r, 1) + wrow(r) * (uint32_t)(K / 32);
    } else {  // FP8: copy i fills LDS 16-byte unit `lane` of rows 32 (2 wave + i) .. + 31
#pragma unroll
        for (int i = 0; i < b_copies<BT>(); ++i) {
            const int r = 32 * (b_copies<BT>() * wave + i) + (lane >> 1);
            boff[i] = wbase(r, 0) + wrow(r) * rowb + (uint32_t)(fp8_half(r, lane & 1) * 16);
        }
    }
    // FP8: the matrices' fp32 scales (gate / up, or down), applied in the epilogue
    float bsc0 = 1.0f, bsc1 = 1.0f;
    if constexpr (BT == 2) {
        bsc0 = *reinterpret_cast<const float*>(slot + (MODE == MODE_GATED ? g.off[3] : g.off[5]));
        bsc1 = *reinterpret_cast<const float*>(slot + (MODE == MODE_GATED ? g.off[4] : g.off[5]));
    }

    auto issue = [&](int stage, int kt) __attribute__((always_inline)) {
        unsigned char* st = smem + stage * stage_bytes<BT>();
#pragma unroll
        for (int i = 0; i < AL; ++i)
            __builtin_amdgcn_global_load_lds(A + aoff[i] + kt * KS, FT_LDS(st + (AL * wave + i) * 1024), 16, 0, 0);
        unsigned char* bst = st + A_BYTES;
        if constexpr (BT == 0 || BT == 2) {
            constexpr int bstep = BT == 0 ? ROWB : KS;  // bytes of a row slice
#pragma unroll
            for (int i = 0; i < b_copies<BT>(); ++i)
                __builtin_amdgcn_global_load_lds(slot + boff[i] + kt * bstep, FT_LDS(bst + (b_copies<BT>() * wave + i) * 1024), 16, 0, 0);
        } else {
            __builtin_amdgcn_global_load_lds(slot + boff[0] + kt * (KS / 2), FT_LDS(bst + wave * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(slot + soff + kt, FT_LDS(bst + BN * 16 + wave * 256), 1, 0, 0);
        }
    };

    const int wn = wave;
    f32x16_t acc[MT][NTL];
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int b = 0; b < NTL; ++b)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[a][b][q] = 0.f;

    constexpr int LPS = loads_per_slice<BT>();
    const int nk = K / KS;
    const int l32 = lane & 31, hi = lane >> 5;
    const int mact = min(MT, (td.rows + 31) / 32);  // 32-row sub-tiles holding rows

    // Fragments of one slice (both 16-deep k-steps): the wave reads slice k+1's
    // fragments from LDS while its MFMAs consume slice k's from registers.
    struct Frags {
        bf16x8_t a[2][MT], b[2][NTL];
    };
    auto load_frags = [&](int stage, Frags& F, auto mc) __attribute__((always_inline)) {
        constexpr int MA = decltype(mc)::value;
        const unsigned char* st = smem + stage * stage_bytes<BT>();
        const unsigned char* Bc = st + A_BYTES;
        if constexpr (BT == 2) {
            // FP8: a lane reads its B row's 16 codes k = 16 hi .. + 15 once and
            // fragment kk takes k = 16 hi + 8 kk .. + 7; A is read at the same
            // positions (chunk 2 hi + kk).  Both operands use this permutation of
            // the slice's 32 k, so the MFMA sums are those of the plain order.
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int m = 0; m < MA; ++m)
                    F.a[kk][m] = *reinterpret_cast<const bf16x8_t*>(st + sw(m * 32 + l32, 2 * hi + kk));
            if constexpr (MA > 0) {
#pragma unroll
                for (int n = 0; n < NTL; ++n) {
                    int brow;
                    if constexpr (MODE == MODE_GATED)
                        brow = (n < NTL / 2 ? 0 : BN / 2) + wn * (WN / 2) + (n % (NTL / 2)) * 32;
                    else
                        brow = wn * WN + n * 32;
                    const int row = brow + l32;
                    const u32x4_t c = *reinterpret_cast<const u32x4_t*>(Bc + row * KS + fp8_half(row, hi) * 16);
                    F.b[0][n] = fp8_frag(c[0], c[1]);
                    F.b[1][n] = fp8_frag(c[2], c[3]);
                }
            }
            return;
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            // 32x32x16 operands: lane holds row (lane % 32), k = 16 kk + 8 (lane / 32) .. + 7
            const int ch = 2 * kk + hi;
#pragma unroll
            for (int m = 0; m < MA; ++m)
                F.a[kk][m] = *reinterpret_cast<const bf16x8_t*>(st + sw(m * 32 + l32, ch));
#pragma unroll
            for (int n = 0; n < NTL; ++n) {
                int brow;
                if constexpr (MODE == MODE_GATED)  // the wave's gate tile, then its up tile
                    brow = (n < NTL / 2 ? 0 : BN / 2) + wn * (WN / 2) + (n % (NTL / 2)) * 32;
                else
                    brow = wn * WN + n * 32;
                const int row = brow + l32;
                if constexpr (BT == 0) {
                    F.b[kk][n] = *reinterpret_cast<const bf16x8_t*>(Bc + sw(row, ch));
                } else {
                    const uint32_t codes = *reinterpret_cast<const uint32_t*>(Bc + row * 16 + ch * 4);
                    F.b[kk][n] = fp4_frag(codes, Bc[BN * 16 + row * 4]);
                }
            }
        }
    };
    auto mfmas = [&](const Frags& F, auto mc) __attribute__((always_inline)) {
        constexpr int MA = decltype(mc)::value;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int m = 0; m < MA; ++m)
#pragma unroll
                for (int n = 0; n < NTL; ++n) acc[m][n] = mfma32(F.a[kk][m], F.b[kk][n], acc[m][n]);
    };
    // wait until a slice has landed (`later` slices issued after it may stay in
    // flight) and this wave's LDS reads are done, then meet the other waves
    auto wait_slice = [&](int later) __attribute__((always_inline)) {
        if (later >= 4) wait_vm_lgkm<4 * LPS>();
        else if (later == 3) wait_vm_lgkm<3 * LPS>();
        else if (later == 2) wait_vm_lgkm<2 * LPS>();
        else if (later == 1) wait_vm_lgkm<LPS>();
        else wait_vm_lgkm<0>();
        __builtin_amdgcn_s_barrier();
    };
    // One iteration: make slice kt+1 visible, refill the stage slice kt came from
    // (all waves read it one iteration ago) with slice kt+STAGES, read slice kt+1's
    // fragments into `nxt`, and run slice kt's MFMAs from `cur`.
    // The fragment reads are unconditional so that the compiler's LDS wait lands
    // before the next iteration's MFMAs, not before these: on the last slice they
    // read a stage no copy targets any more (every copy has been waited for) and the
    // values are not used.
    auto step = [&](int kt, const Frags& cur, Frags& nxt, auto mc) __attribute__((always_inline)) {
        constexpr int MA = decltype(mc)::value;
        if (kt + 1 < nk) {
            wait_slice(min(STAGES - 2, nk - 2 - kt));
            if (kt + STAGES < nk) issue(kt % STAGES, kt + STAGES);
        }
        load_frags((kt + 1) % STAGES, nxt, mc);
        mfmas(cur, mc);
        // interleave: one MFMA, one LDS read, ... so the reads hide under the MFMAs
        constexpr int NMF = 2 * MA * NTL, NDS = 2 * MA + (BT == 0 ? 2 : BT == 1 ? 4 : 1) * NTL;
        constexpr int NP = NMF < NDS ? NMF : NDS;
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        }
        if constexpr (NMF > NP) __builtin_amdgcn_sched_group_barrier(0x008, NMF - NP, 0);
        if constexpr (NDS > NP) __builtin_amdgcn_sched_group_barrier(0x100, NDS - NP, 0);
    };

    // prologue: all stages in flight
#pragma unroll
    for (int q = 0; q < STAGES; ++q)
        if (q < nk) issue(q, q);
    // the K loop, specialised on the number of 32-row sub-tiles holding rows
    Frags F0, F1;
    with_count<MT>(mact, [&](auto mc) __attribute__((always_inline)) {
        wait_slice(min(STAGES - 1, nk - 1));
        load_frags(0, F0, mc);
        for (int kt = 0; kt < nk; kt += 2) {
            step(kt, F0, F1, mc);
            if (kt + 1 < nk) step(kt + 1, F1, F0, mc);
        }
    });

    // Epilogue.  Register q of a 32 x 32 tile is row 8 (q / 4) + 4 (lane / 32) +
    // q % 4, column lane % 32.  bf16 results go through LDS (free once every
    // wave has passed the K loop) so that global stores write whole rows in
    // 16-byte pieces; fp32 results are stored directly (each store covers two
    // 128-byte row pieces).
    if constexpr (MODE == MODE_GATED || sizeof(OutT) == 2) {
        constexpr int TC = MODE == MODE_GATED ? BN / 2 : BN;  // tile columns
        constexpr int PITCH = TC + 8;                          // bf16 per LDS row (bank skew)
        __bf16* ts = reinterpret_cast<__bf16*>(smem);
        __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's LDS reads are done
        __builtin_amdgcn_s_barrier();        // ... and every other wave's
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m >= mact) break;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = m * 32 + 8 * (q >> 2) + 4 * hi + (q & 3);
                if constexpr (MODE == MODE_GATED) {
#pragma unroll
                    for (int n = 0; n < NTL / 2; ++n)
                        ts[row * PITCH + wn * (WN / 2) + n * 32 + l32] =
                            __builtin_bit_cast(__bf16, (uint16_t)f32_to_bf16_bits(
                                silu_mul_fast(acc[m][n][q] * bsc0, acc[m][n + NTL / 2][q] * bsc1)));
                } else {
#pragma unroll
                    for (int n = 0; n < NTL; ++n)
                        ts[row * PITCH + wn * WN + n * 32 + l32] =
                            __builtin_bit_cast(__bf16, (uint16_t)f32_to_bf16_bits(acc[m][n][q] * bsc0));
                }
            }
        }
        __syncthreads();
        constexpr int CPR = TC / 8;  // 16-byte pieces per tile row
        const int rows = td.rows;
        for (int c = threadIdx.x; c < rows * CPR; c += NT) {
            const int row = c / CPR, cc = c % CPR;
            const int col = c0 + cc * 8;
            if (col < NOUT)
                *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(out) + (obase + row) * NOUT + col) =
                    *reinterpret_cast<const u32x4_t*>(ts + row * PITCH + cc * 8);
        }
    } else {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m >= mact) break;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = m * 32 + 8 * (q >> 2) + 4 * hi + (q & 3);
                if (row >= td.rows) continue;
#pragma unroll
                for (int n = 0; n < NTL; ++n) {
                    const int col = c0 + wn * WN + n * 32 + l32;
                    if (col < NOUT) reinterpret_cast<float*>(out)[(obase + row) * NOUT + col] = acc[m][n][q] * bsc0;
                }
            }
        }
    }
}
#undef FT_LDS

template <int MODE, int BT, typename OutT>
hipError_t launch_pipe(unsigned grid, hipStream_t s, const ft::FfnGeom& g, const __bf16* A,
                       const int32_t* perm, const TileDesc* tiles, const int* n_tiles,
                       int n_ntiles, OutT* out) {
    static bool attr_set = false;
    auto kern = gemm_pipe_kernel<MODE, BT, OutT>;
    const size_t lds = pipe::lds_bytes<BT>();
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    kern<<<grid, pipe::NT, lds, s>>>(g, A, perm, tiles, n_tiles, n_ntiles, out);
    return hipGetLastError();
}

// Launch one instantiation (raising its dynamic LDS limit once).
template <class C, int MODE, int BT, typename OutT>
hipError_t launch_tile(unsigned grid, hipStream_t s, const ft::FfnGeom& g, const __bf16* A,
                       const int32_t* perm, const __bf16* Bd, int M, int N, int K,
                       const TileDesc* tiles, const int* n_tiles, int n_ntiles, OutT* out) {
    static bool attr_set = false;
    auto kern = gemm_tile_kernel<C, MODE, BT, OutT>;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    kern<<<grid, C::NT, C::LDS, s>>>(g, A, perm, Bd, M, N, K, tiles, n_tiles, n_ntiles, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// tile list
// ---------------------------------------------------------------------------
// Rows [start, start + rows) of tile m of a segment of c rows cut into
// n = ceil(c / BM) tiles (BM a multiple of 32): the segment's s = ceil(c / 32)
// sub-tiles of 32 rows are dealt evenly, the first s % n tiles taking one
// more, so no tile exceeds BM rows and none is empty.  An expert just past a
// multiple of BM rows thus gets two balanced tiles rather than a full one and
// a nearly empty one that streams the same weight panel, for the same number
// of MFMA sub-tiles.
__device__ __forceinline__ void tile_span(int c, int n, int m, int& start, int& rows) {
    const int s = (c + 31) / 32, q = s / n, r = s % n;
    start = 32 * (m * q + min(m, r));
    rows = min(32 * (q + (m < r ? 1 : 0)), c - start);
}

__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ slot_of,
                                                           int E, int T, int n_shared,
                                                           int shared_slot, int BMr,
                                                           TileDesc* tiles, int* n_tiles,
                                                           int max_tiles) {
    __shared__ int scan[1024];
    const int e = threadIdx.x;
    int cnt = 0, c = 0, off = 0, slot = -1;
    if (e < E) {
        off = offsets[e];
        c = offsets[e + 1] - off;
        slot = slot_of ? slot_of[e] : e;
        if (slot >= 0 && c > 0) cnt = (c + BMr - 1) / BMr;
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
        int idx = base + m, start, rows;
        tile_span(c, cnt, m, start, rows);
        if (idx < max_tiles) tiles[idx] = TileDesc{e, off + start, rows, slot};
    }
    int ns = n_shared ? (T + BMr - 1) / BMr : 0;
    for (int m = e; m < ns; m += 1024) {
        int idx = total + m, start, rows;
        tile_span(T, ns, m, start, rows);
        if (idx < max_tiles) tiles[idx] = TileDesc{E, start, rows, shared_slot};
    }
    if (e == 0) *n_tiles = min(total + ns, max_tiles);
}

}  // namespace

namespace ft {

int max_tiles_for(const FfnGeom& g, int bm) {
    const long tk = (long)g.T * g.k;
    const long act = tk < g.E ? tk : g.E;
    return (int)((tk + bm - 1) / bm + act + (g.n_shared ? (g.T + bm - 1) / bm : 0));
}

int tile_rows(const FfnGeom&) { return pipe::BM; }


ft_status launch_build_tiles(const FfnGeom& g, const int32_t* offsets,
                             const int32_t* slot_of_expert, int shared_slot, TileDesc* tiles,
                             int* n_tiles, int max_tiles, hipStream_t s) {
    build_tiles_kernel<<<1, 1024, 0, s>>>(offsets, slot_of_expert, g.E, g.T, g.n_shared,
                                          shared_slot, tile_rows(g), tiles, n_tiles, max_tiles);
    FT_LAUNCHED("build_tiles");
    return FT_OK;
}

ft_status launch_gemm1_mfma(const FfnGeom& g, const __bf16* x, const int32_t* perm,
                            const TileDesc* tiles, const int* n_tiles, int max_tiles,
                            __bf16* h, hipStream_t s) {
    const int mt = min(max_tiles, max_tiles_for(g, pipe::BM));
    const int nn = cdiv(g.I, pipe::BN / 2);
    const unsigned grid = (unsigned)(mt * nn + 7) / 8 * 8;  // whole rounds over the 8 XCDs
    hipError_t e = g.w_dt == FT_MXFP4 ? launch_pipe<MODE_GATED, 1, __bf16>(grid, s, g, x, perm, tiles, n_tiles, nn, h)
                 : g.w_dt == FT_FP8   ? launch_pipe<MODE_GATED, 2, __bf16>(grid, s, g, x, perm, tiles, n_tiles, nn, h)
                                      : launch_pipe<MODE_GATED, 0, __bf16>(grid, s, g, x, perm, tiles, n_tiles, nn, h);
    if (e != hipSuccess) return set_error(FT_ERR_HIP, "gemm1: %s", hipGetErrorString(e));
    return FT_OK;
}

ft_status launch_gemm2_mfma(const FfnGeom& g, const __bf16* h, const TileDesc* tiles,
                            const int* n_tiles, int max_tiles, void* y, ft_dtype y_dt,
                            hipStream_t s) {
    const int mt = min(max_tiles, max_tiles_for(g, pipe::BM));
    const int nn = cdiv(g.H, pipe::BN);
    const unsigned grid = (unsigned)(mt * nn + 7) / 8 * 8;
    hipError_t e;
    if (g.w_dt == FT_MXFP4)
        e = y_dt == FT_F32 ? launch_pipe<MODE_LIST, 1, float>(grid, s, g, h, nullptr, tiles, n_tiles, nn, (float*)y)
                           : launch_pipe<MODE_LIST, 1, __bf16>(grid, s, g, h, nullptr, tiles, n_tiles, nn, (__bf16*)y);
    else if (g.w_dt == FT_FP8)
        e = y_dt == FT_F32 ? launch_pipe<MODE_LIST, 2, float>(grid, s, g, h, nullptr, tiles, n_tiles, nn, (float*)y)
                           : launch_pipe<MODE_LIST, 2, __bf16>(grid, s, g, h, nullptr, tiles, n_tiles, nn, (__bf16*)y);
    else
        e = y_dt == FT_F32 ? launch_pipe<MODE_LIST, 0, float>(grid, s, g, h, nullptr, tiles, n_tiles, nn, (float*)y)
                           : launch_pipe<MODE_LIST, 0, __bf16>(grid, s, g, h, nullptr, tiles, n_tiles, nn, (__bf16*)y);
    if (e != hipSuccess) return set_error(FT_ERR_HIP, "gemm2: %s", hipGetErrorString(e));
    return FT_OK;
}

ft_status launch_dense_gemm_f32out(const void* A, const void* B, int M, int N, int K,
                                   float* out, hipStream_t s) {
    FfnGeom g{};
    const int n_ntiles = cdiv(N, RouterTile::BN);
    hipError_t e = launch_tile<RouterTile, MODE_DENSE, 0, float>(
        (unsigned)cdiv(M, RouterTile::BM) * n_ntiles, s, g, (const __bf16*)A, nullptr,
        (const __bf16*)B, M, N, K, nullptr, nullptr, n_ntiles, out);
    if (e != hipSuccess) return set_error(FT_ERR_HIP, "router gemm: %s", hipGetErrorString(e));
    return FT_OK;
}

}  // namespace ft
