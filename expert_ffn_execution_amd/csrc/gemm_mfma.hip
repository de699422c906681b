// gemm_mfma.hip -- MFMA kernels for many tokens (gfx950): the grouped expert
// GEMMs.
//
// The expert FFN over many tokens is a set of dense contractions, one per
// expert, over the rows routed to it (claypier.com article,
// "从 MoE「用不到的权重」入手的推理引擎": only the experts a token needs are
// computed).  build_tiles_kernel lists each expert's segment of the
// permutation as M-tiles of at most 256 rows; gemm_pipe_kernel computes a
// 256 x 256 output tile of one M-tile with v_mfma_f32_32x32x16_bf16, its K
// stages copied global -> LDS by the load units into two rings (activations,
// weights), several stages ahead.
//
// GEMM1 fuses SwiGLU: the B tile holds 128 gate rows and the same 128 up
// rows, each wavefront owns matching gate/up accumulators, and the epilogue
// writes h = silu(g) * u in bf16.  GEMM2 multiplies h by the down projection.
// Narrow weights (MXFP4, FP8, NVFP4) stay packed in LDS and are decoded
// exactly to bf16 when a fragment is read.
#include "gemm_mfma.h"
#include "lds_ring.h"

#include <type_traits>

namespace {

using ft::TileDesc;

// v_mfma_f32_32x32x16_bf16 sustains about twice the rate of the 16x16x32 form
// on gfx950 (measured), so the expert GEMMs use it
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// MODE_GATED: gate/up + SwiGLU -> h; MODE_LIST: down projection -> y
enum { MODE_GATED = 0, MODE_LIST = 1 };

// ---------------------------------------------------------------------------
// Pipelined tile kernel for the expert GEMMs.  256 x 256 output tile, 4
// wavefronts (one per SIMD), each owning all 256 rows and a 64-column strip:
// 8 x 2 tiles of v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane).
// K goes in stages of 64 through two LDS rings, one for A (the gathered
// activation rows) and one for B (the expert's weight rows), copied global ->
// LDS by the load units directly (global_load_lds_dwordx4: each wave
// instruction fills 1 KB of LDS, lane l its 16 bytes), so no registers hold
// staged data.  A bf16 row's stage is one whole 128-byte line, and a copy
// instruction reads 8 such lines.  With stages of 32 each instruction read
// 16 half lines, and a probe of this copy pattern alone moved L2-resident
// data at 15 TB/s with half lines against 32 TB/s with whole lines; the
// copies, not the MFMAs, set the K loop's pace.  Ring depths (stages of A,
// B): bf16 2, 3 and FP8 3, 4 -- the weights stream from HBM and need the
// longer lead, the activations (re-read by every N-tile of an M-tile) mostly
// hit in L2; bf16 with 3, 2 was 12% slower.  MXFP4, whose B stages are small,
// 4, 3 (2% faster than 3, 6).
// The MFMAs take a stage in two halves of 32 (two 16-deep k-steps each), one
// half per step: odd steps wait for the next stage (s_waitcnt vmcnt on the
// wave's own copies, counted from the fixed issue order), meet at the block
// barrier and copy the next A stage into the slot just freed; even steps copy
// the next B stage.  The tile is as large as the 160 KB LDS allows so that
// every byte brought into the CU feeds as many MFMAs as possible.  MXFP4
// weights stay packed in LDS (32 code bytes + 2 scale bytes per row and
// stage), FP8 likewise (64 code bytes), decoded to bf16 when a fragment is
// read.
// An expert's last M-tile is usually partly filled (routing gives each
// expert an arbitrary row count): since every wave spans all rows, all waves
// skip the MFMAs and fragment reads of 32-row sub-tiles past the tile's rows
// alike, and the block's time shrinks with its row count.
//
// LDS layout of a stage: bf16 rows are 8 chunks of 16 bytes, chunk c at
// position c ^ ((r >> 1) & 7); FP8 rows 4 chunks at c ^ ((r >> 2) & 3); MXFP4
// rows 2 halves at h ^ ((r >> 3) & 1).  The 16 rows one fragment read pass
// touches then spread over the 64 banks (MXFP4: two rows per bank group).
// ---------------------------------------------------------------------------
namespace pipe {
constexpr int BM = 256, BN = 256, NT = 256, NW = NT / 64, WN = BN / NW;
constexpr int KST = 64;                        // K per stage
constexpr int MT = BM / 32, NTL = WN / 32;     // 32 x 32 MFMA tiles per wavefront
constexpr int A_UNIT = BM * KST * 2;           // one A stage: 32 KB of bf16
constexpr int LA = A_UNIT / 1024 / NW;         // A copies per wave and stage, full tile
// BT: 0 bf16 weights, 1 MXFP4, 2 FP8 (e4m3, one fp32 scale per matrix), 3 NVFP4
// (e2m1 with an e4m3 scale per 16 and an fp32 scale per matrix).
template <int BT> constexpr int b_row() { return BT == 0 ? KST * 2 : BT == 2 ? KST : KST / 2; }
// MXFP4: codes [BN][32 B], then for each half of the stage a 4-byte slot per
// row holding its scale byte (a 1-byte LDS-DMA load writes each lane's byte
// to a 4-byte slot).  NVFP4: codes [BN][32 B], then the row's 4 block-scale
// bytes of the stage [BN][4 B].
template <int BT> constexpr int b_unit() {
    return BN * b_row<BT>() + (BT == 1 ? 2 * BN * 4 : BT == 3 ? BN * 4 : 0);
}
template <int BT> constexpr int n_a() { return BT == 0 ? 2 : BT == 2 ? 3 : 4; }  // A ring stages
template <int BT> constexpr int n_b() { return BT == 0 ? 3 : BT == 2 ? 4 : 3; }  // B ring stages
template <int BT> constexpr int b_code_copies() { return BN * b_row<BT>() / 1024 / NW; }
template <int BT> constexpr int b_copies() {  // per wave, stage
    return b_code_copies<BT>() + (BT == 1 ? 2 : BT == 3 ? 1 : 0);
}
constexpr size_t EPI_BYTES = (size_t)BM * (BN + 8) * 2;   // bf16 output tile (plain GEMM)
template <int BT> constexpr size_t ring_bytes() {
    return (size_t)n_a<BT>() * A_UNIT + (size_t)n_b<BT>() * b_unit<BT>();
}
template <int BT> constexpr size_t lds_bytes() { return ring_bytes<BT>() > EPI_BYTES ? ring_bytes<BT>() : EPI_BYTES; }
static_assert(lds_bytes<0>() <= 160 * 1024 && lds_bytes<1>() <= 160 * 1024 && lds_bytes<2>() <= 160 * 1024 &&
                  lds_bytes<3>() <= 160 * 1024,
              "rings fit the LDS");
__device__ __forceinline__ int swz_bf16(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }
__device__ __forceinline__ int swz_fp8(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }
__device__ __forceinline__ int swz_fp4(int r, int h) { return r * 32 + ((h ^ ((r >> 3) & 1)) << 4); }

// Copy issue order.  Step t (t < 0: before the K loop) issues, when the stage
// exists, A stage (t - 1) / 2 + n_a if t is odd, B stage (t - 2) / 2 + n_b if
// even; stage x of A thus goes out at step 2 (x - n_a) + 1, of B at 2 (x - n_b) + 2.
template <int BT> constexpr int step_of_a(int x) { return 2 * (x - n_a<BT>()) + 1; }
template <int BT> constexpr int step_of_b(int x) { return 2 * (x - n_b<BT>()) + 2; }
template <int BT> constexpr int first_step() {
    return step_of_a<BT>(0) < step_of_b<BT>(0) ? step_of_a<BT>(0) : step_of_b<BT>(0);
}
// Copies a wave may leave in flight when it waits for stage y having issued
// every step up to P (stages past the last, nst - 1, are never issued), with
// la A copies per stage (a tile of la 32-row sub-tiles copies la per wave).
template <int BT>
__host__ __device__ constexpr int copies_after(int y, int P, int nst, int la) {
    const int sa = step_of_a<BT>(y), sb = step_of_b<BT>(y);
    int n = 0;
    for (int t = (sa > sb ? sa : sb) + 1; t <= P; ++t) {
        const int x = (t & 1) ? (t - 1) / 2 + n_a<BT>() : (t - 2) / 2 + n_b<BT>();
        if (x >= 0 && x < nst) n += (t & 1) ? la : b_copies<BT>();
    }
    return n;
}
// in steady state (stage y = s + 1 at odd step 2 s + 1, every stage present)
template <int BT, int la> constexpr int steady_in_flight() { return copies_after<BT>(1, 0, 1 << 20, la); }
// the K loop's pairs of steps are straight-line once every copy of the pair exists
template <int BT> constexpr int steady_margin() {
    return n_b<BT>() - 1 > n_a<BT>() ? n_b<BT>() - 1 : n_a<BT>();
}
static_assert(steady_in_flight<0, LA>() == 8 && steady_in_flight<1, LA>() == 12 && steady_in_flight<2, LA>() == 16,
              "issue order");
}  // namespace pipe

using ft::wait_vm_lgkm;
using ft::wait_vm_lgkm_upto;

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

// NVFP4: 8 e2m1 codes times their block's e4m3 scale byte -> 8 bf16.  The
// product of an e2m1 and an e4m3 value has at most 6 significant bits, so the
// fp32 product converts to bf16 exactly.
__device__ __forceinline__ bf16x8_t nvfp4_frag(uint32_t codes, uint32_t scale_byte) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const float bs = __uint_as_float(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(scale_byte, 1.0f, false)) << 16);
    f32x2 v[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0),
                  __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1),
                  __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2),
                  __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3)};
    u32x4_t d;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        v[b].x *= bs;
        v[b].y *= bs;
        d[b] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v[b], bf16x2));
    }
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

// Scheduling groups of a steady K iteration in two phases: over the first P
// MFMAs the NX instructions of group MX, over the remaining ones the NY of
// group MY, each spread evenly (after MFMA i of a phase of n MFMAs, the ones
// that bring its count to (i + 1) * N / n).
template <int I, int NMF, int P, int MX, int NX, int MY, int NY>
__device__ __forceinline__ void sched_two() {
    if constexpr (I < NMF) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if constexpr (I < P) {
            constexpr int n = ((I + 1) * NX) / P - (I * NX) / P;
            if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(MX, n, 0);
        } else {
            constexpr int J = I - P, n = ((J + 1) * NY) / (NMF - P) - (J * NY) / (NMF - P);
            if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(MY, n, 0);
        }
        sched_two<I + 1, NMF, P, MX, NX, MY, NY>();
    }
}
template <int NX, int NY, int NMF>
constexpr int phase_split() {
    const int p = (NMF * NX + (NX + NY) / 2) / (NX + NY);
    return p < 1 ? 1 : p > NMF - 1 ? NMF - 1 : p;
}

template <int MODE, int BT, typename OutT>
__global__ __launch_bounds__(pipe::NT, 1) void gemm_pipe_kernel(
    ft::FfnGeom g, const __bf16* __restrict__ A, const int32_t* __restrict__ perm,
    const TileDesc* __restrict__ tiles, const int* __restrict__ n_tiles, int n_ntiles,
    OutT* __restrict__ out) {
    using namespace pipe;
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
    const uint8_t* slot = ft::slot_weights(g.pool, g.slot_stride, g.host_pool, g.host_stride, td.slot);
    // gated: B rows [0, 128) = gate rows c0.., [128, 256) = up rows c0..; plain: rows c0..
    const int c0 = nt * (MODE == MODE_GATED ? BN / 2 : BN);

    // A: copy i of this wave fills LDS rows 8 (NW i + wave) .. + 7, lane l row
    // + l / 8 at chunk position l % 8 (rows past the tile re-read its last
    // row).  Copy i lies in 32-row sub-tile i, so a tile of MA occupied
    // sub-tiles needs copies 0 .. MA - 1 of every wave and no others.
    uint32_t aoff[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int r = 8 * (NW * i + wave) + (lane >> 3);
        const int rc = min(r, td.rows - 1);
        uint32_t arow;
        if constexpr (MODE == MODE_GATED) arow = shared ? (uint32_t)(td.p0 + rc) : (uint32_t)(perm[td.p0 + rc] / g.k);
        else arow = (uint32_t)(obase + rc);
        aoff[i] = arow * (uint32_t)K + (uint32_t)(((lane & 7) ^ ((r >> 1) & 7)) * 8);
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
    const uint32_t rowb = BT == 0 ? (uint32_t)K * 2 : BT == 2 ? (uint32_t)K : (uint32_t)K / 2;
    // B code copies per wave: b_code_copies<BT>() <= 8 (a literal bound: a
    // call in an array bound reads as a variable-length array to the host pass)
    constexpr int NBC = b_code_copies<BT>();
    static_assert(NBC <= 8, "B copies per wave");
    uint32_t boff[8], soff = 0;
    if constexpr (BT == 0) {  // copy i: rows 8 (NBC wave + i) .. + 7, like A
#pragma unroll
        for (int i = 0; i < NBC; ++i) {
            const int r = 8 * (NBC * wave + i) + (lane >> 3);
            boff[i] = wbase(r, 0) + wrow(r) * rowb + (uint32_t)(((lane & 7) ^ ((r >> 1) & 7)) * 16);
        }
    } else if constexpr (BT == 1 || BT == 3) {  // copy i: rows 32 (NBC wave + i) .. + 31, two lanes a row; scales of row 64 wave + lane
#pragma unroll
        for (int i = 0; i < NBC; ++i) {
            const int r = 32 * (NBC * wave + i) + (lane >> 1);
            boff[i] = wbase(r, 0) + wrow(r) * rowb + (uint32_t)(((lane & 1) ^ ((r >> 3) & 1)) * 16);
        }
        const int r = 64 * wave + lane;
        soff = wbase(r, 1) + wrow(r) * (uint32_t)(K / (BT == 1 ? 32 : 16));
    } else {  // FP8 copy i: rows 16 (NBC wave + i) .. + 15, four lanes a row
#pragma unroll
        for (int i = 0; i < NBC; ++i) {
            const int r = 16 * (NBC * wave + i) + (lane >> 2);
            boff[i] = wbase(r, 0) + wrow(r) * rowb + (uint32_t)(((lane & 3) ^ ((r >> 2) & 3)) * 16);
        }
    }
    // FP8 matrix / NVFP4 tensor scales (gate / up, or down), applied in the epilogue
    float bsc0 = 1.0f, bsc1 = 1.0f;
    if constexpr (BT == 2) {
        bsc0 = *reinterpret_cast<const float*>(slot + (MODE == MODE_GATED ? g.off[3] : g.off[5]));
        bsc1 = *reinterpret_cast<const float*>(slot + (MODE == MODE_GATED ? g.off[4] : g.off[5]));
    } else if constexpr (BT == 3) {
        bsc0 = *reinterpret_cast<const float*>(slot + (MODE == MODE_GATED ? g.toff[0] : g.toff[2]));
        bsc1 = *reinterpret_cast<const float*>(slot + (MODE == MODE_GATED ? g.toff[1] : g.toff[2]));
    }

    // (constants, not calls: a constexpr template call evaluated at run time in
    // these lambdas keeps the host pass from emitting the kernel's launch stub)
    constexpr int NA = n_a<BT>(), NB = n_b<BT>(), LB = b_copies<BT>();
    constexpr int BUNIT = b_unit<BT>(), BROW = b_row<BT>();
    unsigned char* const aring = smem;
    unsigned char* const bring = smem + NA * A_UNIT;
    const int nst = K / KST;
    auto issue_a = [&](int x, auto mc) __attribute__((always_inline)) {  // A stage x into its ring slot
        constexpr int MA = decltype(mc)::value;
        unsigned char* dst = aring + (x % NA) * A_UNIT;
#pragma unroll
        for (int i = 0; i < MA; ++i)
            __builtin_amdgcn_global_load_lds(A + aoff[i] + x * KST, FT_LDS(dst + (NW * i + wave) * 1024), 16, 0, 0);
    };
    auto issue_b = [&](int x) __attribute__((always_inline)) {  // B stage x into its ring slot
        unsigned char* dst = bring + (x % NB) * BUNIT;
#pragma unroll
        for (int i = 0; i < NBC; ++i)
            __builtin_amdgcn_global_load_lds(slot + boff[i] + x * BROW, FT_LDS(dst + (NBC * wave + i) * 1024), 16, 0, 0);
        if constexpr (BT == 1) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
                __builtin_amdgcn_global_load_lds(slot + soff + 2 * x + h, FT_LDS(dst + BN * 32 + h * BN * 4 + wave * 256), 1, 0, 0);
        } else if constexpr (BT == 3) {  // the row's 4 block scales of the stage
            __builtin_amdgcn_global_load_lds(slot + soff + 4 * x, FT_LDS(dst + BN * 32 + wave * 256), 4, 0, 0);
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

    const int l32 = lane & 31, hi = lane >> 5;
    const int mact = min(MT, (td.rows + 31) / 32);  // 32-row sub-tiles holding rows

    // Fragments of one half stage (both 16-deep k-steps): the wave reads step
    // j+1's fragments from LDS while its MFMAs consume step j's from registers.
    struct Frags {
        bf16x8_t a[2][MT], b[2][NTL];
    };
    auto b_tile_row = [&](int n) __attribute__((always_inline)) {
        if constexpr (MODE == MODE_GATED)  // the wave's gate tile, then its up tile
            return (n < NTL / 2 ? 0 : BN / 2) + wn * (WN / 2) + (n % (NTL / 2)) * 32;
        else
            return wn * WN + n * 32;
    };
    auto load_frags = [&](int j, Frags& F, auto mc) __attribute__((always_inline)) {
        constexpr int MA = decltype(mc)::value;
        const int x = j >> 1, h = j & 1;  // stage, half
        const unsigned char* Au = aring + (x % NA) * A_UNIT;
        const unsigned char* Bu = bring + (x % NB) * BUNIT;
        if constexpr (BT == 2) {
            // FP8: a lane reads its B row's 16 codes k = 32 h + 16 hi .. + 15 once
            // and fragment kk takes k = 32 h + 16 hi + 8 kk .. + 7; A is read at the
            // same positions (chunk 4 h + 2 hi + kk).  Both operands use this
            // permutation of the half's 32 k, so the MFMA sums are those of the
            // plain order.
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int m = 0; m < MA; ++m)
                    F.a[kk][m] = *reinterpret_cast<const bf16x8_t*>(Au + swz_bf16(m * 32 + l32, 4 * h + 2 * hi + kk));
            if constexpr (MA > 0) {
#pragma unroll
                for (int n = 0; n < NTL; ++n) {
                    const u32x4_t c = *reinterpret_cast<const u32x4_t*>(Bu + swz_fp8(b_tile_row(n) + l32, 2 * h + hi));
                    F.b[0][n] = fp8_frag(c[0], c[1]);
                    F.b[1][n] = fp8_frag(c[2], c[3]);
                }
            }
            return;
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            // 32x32x16 operands: lane holds row (lane % 32), k = 32 h + 16 kk + 8 (lane / 32) .. + 7
            const int ch = 2 * kk + hi;
#pragma unroll
            for (int m = 0; m < MA; ++m)
                F.a[kk][m] = *reinterpret_cast<const bf16x8_t*>(Au + swz_bf16(m * 32 + l32, 4 * h + ch));
#pragma unroll
            for (int n = 0; n < NTL; ++n) {
                const int row = b_tile_row(n) + l32;
                if constexpr (BT == 0) {
                    F.b[kk][n] = *reinterpret_cast<const bf16x8_t*>(Bu + swz_bf16(row, 4 * h + ch));
                } else if constexpr (BT == 1) {
                    const uint32_t codes = *reinterpret_cast<const uint32_t*>(Bu + swz_fp4(row, h) + ch * 4);
                    F.b[kk][n] = fp4_frag(codes, Bu[BN * 32 + h * BN * 4 + row * 4]);
                } else {  // NVFP4: these 8 codes (k = 32 h + 8 ch ..) lie in block 2 h + ch / 2
                    const uint32_t codes = *reinterpret_cast<const uint32_t*>(Bu + swz_fp4(row, h) + ch * 4);
                    F.b[kk][n] = nvfp4_frag(codes, Bu[BN * 32 + row * 4 + 2 * h + ch / 2]);
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
    // Step j of the K loop (stage j / 2, half j % 2): odd steps wait until stage
    // (j + 1) / 2 has landed and every wave is done with stage (j - 1) / 2, then
    // copy A stage (j - 1) / 2 + NA into that stage's slot; even steps copy B
    // stage j / 2 - 1 + NB (its slot freed at the barrier of step j - 1).  Then
    // the wave reads step j+1's fragments into `nxt` and runs step j's MFMAs
    // from `cur`.  The fragment reads are unconditional so that the compiler's
    // LDS wait lands before the next step's MFMAs, not before these: on the last
    // step they read a slot no copy targets any more and the values are unused.
    // STEADY: every copy of the step exists, so the step is straight-line code
    // and its copies and reads each get a phase of the MFMAs; copies then reads
    // (bf16) or reads then copies (MXFP4, FP8), the order measured faster.
    auto step = [&](int j, const Frags& cur, Frags& nxt, auto mc, auto odd, auto steady) __attribute__((always_inline)) {
        constexpr int MA = decltype(mc)::value;
        constexpr bool ODD = decltype(odd)::value, STEADY = decltype(steady)::value;
        constexpr int NMF = 2 * MA * NTL, NDS = 2 * MA + (BT == 0 ? 2 : BT == 2 ? 1 : 4) * NTL;
        constexpr int NP = NMF < NDS ? NMF : NDS;
        constexpr int NC = ODD ? MA : LB;
        constexpr bool COPIES_FIRST = BT == 0;
        const int sx = ODD ? (j - 1) / 2 : j / 2;
        auto copy = [&]() __attribute__((always_inline)) {
            if constexpr (ODD) issue_a(sx + NA, mc);
            else issue_b(sx - 1 + NB);
        };
        if constexpr (ODD) {
            if constexpr (STEADY) {
                wait_vm_lgkm<steady_in_flight<BT, MA>()>();
                __builtin_amdgcn_s_barrier();
            } else if (sx + 1 < nst) {
                wait_vm_lgkm_upto<32>(copies_after<BT>(sx + 1, 2 * sx, nst, MA));
                __builtin_amdgcn_s_barrier();
            }
        }
        if constexpr (STEADY) {
            if constexpr (COPIES_FIRST) {
                copy();
                load_frags(j + 1, nxt, mc);
            } else {
                load_frags(j + 1, nxt, mc);
                copy();
            }
        } else {
            if ((ODD ? sx + NA : sx - 1 + NB) < nst) copy();
            load_frags(j + 1, nxt, mc);
        }
        mfmas(cur, mc);
        if constexpr (STEADY && NMF >= 2) {
            // The copies write LDS and the fragment reads read it, so neither may
            // pass the other: one phase each, in program order.
            if constexpr (COPIES_FIRST)
                sched_two<0, NMF, phase_split<NC, NDS, NMF>(), 0x010, NC, 0x100, NDS>();
            else
                sched_two<0, NMF, phase_split<NDS, NC, NMF>(), 0x100, NDS, 0x010, NC>();
        } else {
            // interleave: one MFMA, one LDS read, ... so the reads hide under the MFMAs
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
            }
            if constexpr (NMF > NP) __builtin_amdgcn_sched_group_barrier(0x008, NMF - NP, 0);
            if constexpr (NDS > NP) __builtin_amdgcn_sched_group_barrier(0x100, NDS - NP, 0);
        }
    };

    // the K loop, specialised on the number of 32-row sub-tiles holding rows
    Frags F0, F1;
    with_count<MT>(mact, [&](auto mc) __attribute__((always_inline)) {
        // prologue: the copies of every step before the first, in issue order
#pragma unroll
        for (int t = first_step<BT>(); t < 0; ++t) {
            if (t & 1) {
                const int x = (t - 1) / 2 + NA;
                if (x >= 0 && x < nst) issue_a(x, mc);
            } else {
                const int x = (t - 2) / 2 + NB;
                if (x >= 0 && x < nst) issue_b(x);
            }
        }
        wait_vm_lgkm_upto<32>(copies_after<BT>(0, -1, nst, decltype(mc)::value));
        __builtin_amdgcn_s_barrier();
        load_frags(0, F0, mc);
        int sx = 0;
        for (; sx < nst - steady_margin<BT>(); ++sx) {
            step(2 * sx, F0, F1, mc, std::false_type{}, std::true_type{});
            step(2 * sx + 1, F1, F0, mc, std::true_type{}, std::true_type{});
        }
        for (; sx < nst; ++sx) {
            step(2 * sx, F0, F1, mc, std::false_type{}, std::false_type{});
            step(2 * sx + 1, F1, F0, mc, std::true_type{}, std::false_type{});
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
        // Rows r, r + 1 of a lane's column c come from registers q, q + 1 (q
        // even).  Lanes 2i and 2i + 1 swap one value (DPP quad_perm [1,0,3,2])
        // so that the even lane holds row r, columns c, c + 1 and the odd lane
        // row r + 1, columns c - 1, c: one packed conversion (round to nearest
        // even) and one 32-bit LDS write per pair, half the writes of one bf16
        // each.
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bool odd = lane & 1;
        auto put = [&](int row, int col, float v0, float v1) __attribute__((always_inline)) {
            const float send = odd ? v0 : v1;
            const float recv = __builtin_bit_cast(
                float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, send), 0xB1, 0xF, 0xF, true));
            const f32x2 pr = odd ? f32x2{recv, v1} : f32x2{v0, recv};
            *reinterpret_cast<bf16x2*>(ts + (row + (odd ? 1 : 0)) * PITCH + (col & ~1)) =
                __builtin_convertvector(pr, bf16x2);
        };
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m >= mact) break;
#pragma unroll
            for (int q = 0; q < 16; q += 2) {
                const int row = m * 32 + 8 * (q >> 2) + 4 * hi + (q & 3);
                if constexpr (MODE == MODE_GATED) {
#pragma unroll
                    for (int n = 0; n < NTL / 2; ++n)
                        put(row, wn * (WN / 2) + n * 32 + l32,
                            silu_mul_fast(acc[m][n][q] * bsc0, acc[m][n + NTL / 2][q] * bsc1),
                            silu_mul_fast(acc[m][n][q + 1] * bsc0, acc[m][n + NTL / 2][q + 1] * bsc1));
                } else {
#pragma unroll
                    for (int n = 0; n < NTL; ++n)
                        put(row, wn * WN + n * 32 + l32, acc[m][n][q] * bsc0, acc[m][n][q + 1] * bsc0);
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
    return ft::launch_timed(MODE == MODE_GATED ? ft::PROF_FFN_GEMM1 : ft::PROF_FFN_GEMM2, kern,
                            dim3(grid), dim3(pipe::NT), lds, s, g, A, perm, tiles, n_tiles,
                            n_ntiles, out);
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
                                                           const void* host_pool,
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
        if (ft::slot_has_weights(slot, host_pool) && c > 0) cnt = (c + BMr - 1) / BMr;
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
    build_tiles_kernel<<<1, 1024, 0, s>>>(offsets, slot_of_expert, g.host_pool, g.E, g.T,
                                          g.n_shared, shared_slot, tile_rows(g), tiles, n_tiles,
                                          max_tiles);
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
                 : g.w_dt == FT_NVFP4 ? launch_pipe<MODE_GATED, 3, __bf16>(grid, s, g, x, perm, tiles, n_tiles, nn, h)
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
    else if (g.w_dt == FT_NVFP4)
        e = y_dt == FT_F32 ? launch_pipe<MODE_LIST, 3, float>(grid, s, g, h, nullptr, tiles, n_tiles, nn, (float*)y)
                           : launch_pipe<MODE_LIST, 3, __bf16>(grid, s, g, h, nullptr, tiles, n_tiles, nn, (__bf16*)y);
    else
        e = y_dt == FT_F32 ? launch_pipe<MODE_LIST, 0, float>(grid, s, g, h, nullptr, tiles, n_tiles, nn, (float*)y)
                           : launch_pipe<MODE_LIST, 0, __bf16>(grid, s, g, h, nullptr, tiles, n_tiles, nn, (__bf16*)y);
    if (e != hipSuccess) return set_error(FT_ERR_HIP, "gemm2: %s", hipGetErrorString(e));
    return FT_OK;
}

}  // namespace ft
