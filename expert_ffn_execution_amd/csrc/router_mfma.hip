// router_mfma.hip -- router logits for many tokens (gfx950).
//
// The router scores each token against every expert before a few experts are
// picked per token (claypier.com article, "从 MoE「用不到的权重」入手的推理引擎");
// for batches of more than 64 tokens the scores are a dense contraction of the
// activations with the router weight, done here with MFMA tiles.  Fewer
// tokens take the streaming kernel in route.hip.
#include "gemm_mfma.h"
#include "lds_ring.h"

namespace {

using ft::wait_vm_lgkm_upto;

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Router logits for many tokens: out[m][e] = sum_k x[m][k] W_r[e][k], fp32
// accumulation of bf16 products.  The contraction has few columns (E), so
// there are few output tiles, and a tile loop that loads one K slice ahead
// waits one memory round trip per slice (the plain tile kernel took 26 us for
// 4096 tokens x 128 experts x 2048).  Here a block takes BM rows x BN experts
// (32 x 64, or 64 x 128 for large grids) and walks K in stages of 64 through
// an LDS ring of RD stages, filled by direct global->LDS copies issued RD - 1
// stages ahead, so that many round trips are in flight at once; two blocks
// share a CU.  Rows past M and experts past N re-read the last row and are
// not stored.
// LDS stage: A rows 0..BM-1 then B rows 0..BN-1, 128 bytes each, chunk c of
// row r at position c ^ ((r >> 1) & 7).
namespace rpipe {
constexpr int KS = 64, NT = 256;
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
}  // namespace rpipe

// Copies of K stage st (taken at stage (st + rot) mod nst) into its ring slot.
template <int BM, int BN, int RD>
__device__ __forceinline__ void router_issue(unsigned char* ring, const unsigned char* const* asrc,
                                             const unsigned char* const* bsrc, int st, int rot, int nst,
                                             int wave) {
    constexpr int A_BYTES = BM * rpipe::KS * 2, STAGE = (BM + BN) * rpipe::KS * 2;
    constexpr int NCA = BM / 32, NCB = BN / 32;
    unsigned char* dst = ring + (st % RD) * STAGE;
    const int kst = st + rot < nst ? st + rot : st + rot - nst;
#pragma unroll
    for (int i = 0; i < NCA; ++i)
        __builtin_amdgcn_global_load_lds(asrc[i] + (size_t)kst * rpipe::KS * 2, FT_LDS(dst + (4 * i + wave) * 1024),
                                         16, 0, 0);
#pragma unroll
    for (int i = 0; i < NCB; ++i)
        __builtin_amdgcn_global_load_lds(bsrc[i] + (size_t)kst * rpipe::KS * 2,
                                         FT_LDS(dst + A_BYTES + (NCB * wave + i) * 1024), 16, 0, 0);
}

// BM x BN block tile, RD ring stages, OCC blocks per CU (launch bound).  The
// four waves form a 2 x 2 grid of (BM / 2) x (BN / 2) tiles of
// v_mfma_f32_16x16x32_bf16.  A copy instruction moves 8 rows of 128 bytes:
// copy i of a wave takes A rows 8 (4 i + wave) .. + 7 and B rows
// 8 (BN / 32 * wave + i) .. + 7.
template <int BM, int BN, int RD, int OCC>
__global__ __launch_bounds__(rpipe::NT, OCC) void router_pipe_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ wr, int M, int N, int K,
    float* __restrict__ out, int n_ntiles) {
    using namespace rpipe;
    constexpr int A_BYTES = BM * KS * 2, STAGE = (BM + BN) * KS * 2;
    constexpr int NCA = BM / 32, NCB = BN / 32, CPW = NCA + NCB;  // copies per wave and stage
    constexpr int WM = BM / 2, WN = BN / 2, MTL = WM / 16, NTL = WN / 16;
    static_assert(BM % 32 == 0 && BN % 32 == 0 && CPW * (RD - 2) < 64, "tile and ring");
    __shared__ __attribute__((aligned(16))) unsigned char ring[RD * STAGE];
    // the blocks the hardware deals to one XCD (every eighth) take consecutive
    // tiles, so the column tiles of one row strip share that XCD's L2 (when the
    // grid is a multiple of 8; the map is then a permutation)
    unsigned b = blockIdx.x;
    if (gridDim.x % 8 == 0) b = (b % 8) * (gridDim.x / 8) + b / 8;
    const int mi = (int)(b / (unsigned)n_ntiles);
    const int m0 = mi * BM, n0 = (int)(b % (unsigned)n_ntiles) * BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const size_t rowb = (size_t)K * 2;
    // this lane's copy sources: LDS position lane % 8 of row lane / 8 of the
    // copy's 1 KB piece takes the global chunk (lane % 8) ^ swz(row)
    const unsigned char* asrc[NCA];
#pragma unroll
    for (int i = 0; i < NCA; ++i) {
        const int ra = 8 * (4 * i + wave) + (lane >> 3);
        asrc[i] = reinterpret_cast<const unsigned char*>(x) + (size_t)min(m0 + ra, M - 1) * rowb +
                  ((lane & 7) ^ swz(ra)) * 16;
    }
    const unsigned char* bsrc[NCB];
#pragma unroll
    for (int i = 0; i < NCB; ++i) {
        const int rb = 8 * (NCB * wave + i) + (lane >> 3);
        bsrc[i] = reinterpret_cast<const unsigned char*>(wr) + (size_t)min(n0 + rb, N - 1) * rowb +
                  ((lane & 7) ^ swz(rb)) * 16;
    }
    const int nst = K / KS;
    // row strips start at different K stages (and wrap around), so that the
    // rows read at one moment sit at different offsets; the column tiles of one
    // strip keep in step, each reading the x stage the other just brought in
    const int rot = mi % nst;
    for (int st = 0; st < RD - 1 && st < nst; ++st) router_issue<BM, BN, RD>(ring, asrc, bsrc, st, rot, nst, wave);
    const int wm = wave & 1, wn = wave >> 1;
    f32x4_t acc[MTL][NTL];
#pragma unroll
    for (int mt = 0; mt < MTL; ++mt)
#pragma unroll
        for (int n = 0; n < NTL; ++n) acc[mt][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int st = 0; st < nst; ++st) {
        // stages st+1 .. min(st + RD - 2, nst - 1) may still be in flight; st must
        // have landed (copies complete in issue order, and this wave's LDS
        // reads of st - 1 are done), then every wave's has.  A plain barrier:
        // __syncthreads() would also wait for the copies in flight (its fence
        // covers them), which emptied the ring at every stage (17 vs 11.7 us
        // for 4096 x 128 x 2048 in isolation)
        wait_vm_lgkm_upto<CPW * (RD - 2)>(CPW * (min(st + RD - 2, nst - 1) - st));
        __builtin_amdgcn_s_barrier();
        // the slot of stage st - 1, which every wave has finished reading
        if (st + RD - 1 < nst) router_issue<BM, BN, RD>(ring, asrc, bsrc, st + RD - 1, rot, nst, wave);
        const unsigned char* sb = ring + (st % RD) * STAGE;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int c = 4 * ks + (lane >> 4);
            bf16x8_t a[MTL];
#pragma unroll
            for (int mt = 0; mt < MTL; ++mt) {
                const int ar = WM * wm + 16 * mt + (lane & 15);
                a[mt] = *reinterpret_cast<const bf16x8_t*>(sb + ar * 128 + ((c ^ swz(ar)) * 16));
            }
#pragma unroll
            for (int n = 0; n < NTL; ++n) {
                const int br = WN * wn + 16 * n + (lane & 15);
                const bf16x8_t b =
                    *reinterpret_cast<const bf16x8_t*>(sb + A_BYTES + br * 128 + ((c ^ swz(br)) * 16));
#pragma unroll
                for (int mt = 0; mt < MTL; ++mt) acc[mt][n] = mfma16(a[mt], b, acc[mt][n]);
            }
        }
    }
    // lane holds column lane & 15 and rows 4 (lane >> 4) + j of each 16 x 16 tile
#pragma unroll
    for (int mt = 0; mt < MTL; ++mt)
#pragma unroll
        for (int n = 0; n < NTL; ++n) {
            const int col = n0 + WN * wn + 16 * n + (lane & 15);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = m0 + WM * wm + 16 * mt + 4 * (lane >> 4) + j;
                if (row < M && col < N) out[(size_t)row * N + col] = acc[mt][n][j];
            }
        }
}

template <int BM, int BN, int RD, int OCC>
void launch_router(const void* A, const void* B, int M, int N, int K, float* out, hipStream_t s) {
    const int n_ntiles = ft::cdiv(N, BN);
    auto kern = router_pipe_kernel<BM, BN, RD, OCC>;
    kern<<<(unsigned)(ft::cdiv(M, BM) * n_ntiles), rpipe::NT, 0, s>>>((const __bf16*)A, (const __bf16*)B, M, N,
                                                                      K, out, n_ntiles);
}

}  // namespace

namespace ft {

ft_status launch_dense_gemm_f32out(const void* A, const void* B, int M, int N, int K,
                                   float* out, hipStream_t s) {
    if (K % rpipe::KS != 0) return set_error(FT_ERR_INVALID_ARG, "router GEMM: K must be a multiple of 64");
    // 64 x 128 tiles once they still fill the chip: x is then read half as
    // often from L2 (or HBM) and the LDS carries 1.5 rather than 2 bytes per
    // product pair; smaller grids keep the 32 x 64 tiles (four times as many
    // blocks).  Measured with routing's top-k included: 753B-A40B layer
    // (16384 x 256 x 6144) 168 -> 95 us, 284B-A13B layer (8192 x 256 x 4096)
    // 59 -> 47 us; the 35B-A3B layer (4096 x 128 x 2048: 64 large tiles) 18 us
    // with small tiles against 24 us with large ones.
    if ((long)ft::cdiv(M, 64) * ft::cdiv(N, 128) >= 256)
        launch_router<64, 128, 3, 2>(A, B, M, N, K, out, s);
    else
        launch_router<32, 64, 6, 2>(A, B, M, N, K, out, s);
    FT_LAUNCHED("router logits");
    return FT_OK;
}

}  // namespace ft
