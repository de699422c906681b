// gemm_mfma.h -- host launchers of the MFMA tile kernels (gfx950).
#pragma once
#include "common.h"

namespace ft {

// One M-tile of the grouped GEMMs: rows [p0, p0 + rows) of expert e's
// segment of the permutation (e == E is the shared expert, whose rows are
// token indices).
struct TileDesc {
    int e;
    int p0;
    int rows;
    int slot;
};

// rows per M-tile assumed when the workspace's tile list is sized: no more
// than the kernels' tile height (256), so the list always fits
constexpr int GEMM_BM = 128;

// Everything the FFN GEMM kernels need about the weights and the permutation.
struct FfnGeom {
    int E, H, I, k, T, n_shared;
    ft_dtype w_dt;
    const uint8_t* pool;
    size_t slot_stride;
    const uint8_t* host_pool;  // device-visible host experts (slot -2 - j), or null
    size_t host_stride;
    size_t off[6];  // gate, up, down, gate_sc, up_sc, down_sc (bytes within a slot)
    size_t toff[3];  // NVFP4: the fp32 tensor scales of gate, up, down
};

// A slot-table entry names where an expert's weights are: slot s >= 0 of the
// device pool, or (entry -2 - j, with a host pool) expert j of the host pool,
// read over the host link; -1 (or -2 - j without a host pool) skips the expert.
__host__ __device__ __forceinline__ bool slot_has_weights(int slot, const void* host_pool) {
    return slot >= 0 || (slot <= -2 && host_pool != nullptr);
}
__device__ __forceinline__ const uint8_t* slot_weights(const uint8_t* pool, size_t stride,
                                                       const uint8_t* host_pool, size_t host_stride,
                                                       int slot) {
    return slot >= 0 ? pool + (size_t)slot * stride : host_pool + (size_t)(-2 - slot) * host_stride;
}

// Build the M-tile list from offsets (one block).  tiles[0..max_tiles),
// *n_tiles receives the count.
ft_status launch_build_tiles(const FfnGeom& g, const int32_t* offsets,
                             const int32_t* slot_of_expert, int shared_slot, TileDesc* tiles,
                             int* n_tiles, int max_tiles, hipStream_t s);

// GEMM1 + SwiGLU: h[p][i] = bf16(silu(x_t . Wg_i) * (x_t . Wu_i)) over all tiles.
ft_status launch_gemm1_mfma(const FfnGeom& g, const __bf16* x, const int32_t* perm,
                            const TileDesc* tiles, const int* n_tiles, int max_tiles,
                            __bf16* h, hipStream_t s);
// GEMM2: y[p][d] = h[p] . Wd_d over all tiles; y is bf16 or f32.
ft_status launch_gemm2_mfma(const FfnGeom& g, const __bf16* h, const TileDesc* tiles,
                            const int* n_tiles, int max_tiles, void* y, ft_dtype y_dt,
                            hipStream_t s);
// Dense out[M][N] (fp32) = A[M][K] . B[N][K]^T, bf16 operands (router logits).
ft_status launch_dense_gemm_f32out(const void* A, const void* B, int M, int N, int K,
                                   float* out, hipStream_t s);

}  // namespace ft
