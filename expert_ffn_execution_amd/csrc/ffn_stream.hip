// ffn_stream.hip -- expert FFN for few tokens: weight streaming (gfx950).
//
// With a handful of tokens the layer reads every byte of each routed expert's
// weights once and does a few multiply-adds per byte, so the time is the HBM
// read of the active experts (the pages make the same point one level up:
// time goes to moving expert weights, not to arithmetic -- chenxutan.com
// article, "瓶颈为什么是带宽而不是容量").  These kernels therefore stream
// weights with 16-byte loads and keep the routed tokens' activations in LDS.
// bf16 (and fp32) weights use vector-ALU dot products (v_dot2_f32_bf16): the
// work per byte is too small for a matrix tile to pay off.  MXFP4 and FP8
// weights are decoded exactly to bf16 first, which costs as much ALU again
// per weight byte; with more than one token they go to matrix cores instead
// (the second kernel below).
//
// Streaming.  HBM stays busy only if every CU keeps enough bytes in flight,
// and the cross-lane sums at the end of each row must stay cheap.  A weight
// row is therefore read by a segment of LPR = 8, 16, 32 or 64 lanes (the
// fewest that cover the row in at most QMAX 16-byte loads per lane), so each
// load instruction reads 64/LPR rows, LPR*16 contiguous bytes of each, and
// every lane accumulates only its own row's products (one float per token
// and matrix).  An "item" is the 64/LPR rows of one such instruction group
// (or, for rows longer than 64*QMAX chunks, one pass over part of a row).
// The next item's loads are issued before the current item is multiplied
// (two register buffers), so a wave always has one item in flight while it
// computes.  A finished item's per-token sums are reduced over the segment
// with a butterfly that halves the token slots at each DPP exchange inside
// a 16-lane row, so R tokens cost about R exchanges rather than R full
// reductions.
//
// Grid: (group, block of weight rows), where a group is one expert and a
// chunk of at most RCAP of its token rows (their activations fill LDS).  A
// block finds its group from `offsets` with a wavefront scan, so no host
// round trip is needed; the host sizes the grid for the most groups T*k
// routed rows can make, and blocks past the last group exit.  An expert with
// more rows than RCAP (the shared expert sees all T) is split over several
// groups that run side by side and re-read its weights from cache.
#include "common.h"
#include "gemm_mfma.h"

#include <cstdlib>
#include <type_traits>

namespace {

constexpr int NWAVE = 4;  // wavefronts per block

// WT: 0 = fp32 weights (fp32 activations), 1 = bf16, 2 = MXFP4, 3 = FP8 e4m3,
// 4 = NVFP4 (bf16 activations)
template <int WT> struct W;
template <> struct W<0> { static constexpr int EPC = 4; };   // elements per 16 B chunk
template <> struct W<1> { static constexpr int EPC = 8; };
template <> struct W<2> { static constexpr int EPC = 32; };
template <> struct W<3> { static constexpr int EPC = 16; };
template <> struct W<4> { static constexpr int EPC = 32; };

// How a wavefront walks one weight matrix [N][K] of 16-byte chunks.
struct Walk {
    int nch;  // chunks per row
    int LPR;  // lanes per row segment: 8, 16, 32 or 64
    int Q;    // loads per lane and matrix in one item (<= QMAX)
    int P;    // passes per row (P > 1 only with LPR == 64 and Q == QMAX)
    int CPP;  // chunks per pass (== nch when P == 1)
};

// Everything a streaming launch needs (passed by value).
struct StreamArgs {
    const uint8_t* pool;
    size_t slot_stride;
    const uint8_t* host_pool;  // slot-table entries -2 - j: expert j of this pool
    size_t host_stride;
    size_t moff[2], soff[2];  // matrix / scale byte offsets inside a slot
    size_t toff[2];           // NVFP4: the matrices' fp32 tensor scales
    const int32_t* offsets;
    const int32_t* perm;  // gate/up: source token = perm[p] / k; null for down
    const int32_t* slot_of;
    int E, T, k, shared_slot, n_routed_groups;
    int N, K;  // weight rows, row length in elements
    Walk wk;
    int RPB, NB, RCAP;
    int target;  // grid target in blocks (0: the default for the token rows)
    const void* src;  // x (gate/up) or h (down)
    void* dst;        // h (gate/up) or y (down)
};

// Inclusive prefix sum over the 64 lanes: DPP shifts inside each row of 16
// lanes, then row broadcasts carry the row totals forward.
__device__ __forceinline__ int wave_scan_incl(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false); // row_bcast:15 -> rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false); // row_bcast:31 -> rows 2, 3
    return v;
}

// Group j of the routed experts -> (expert e, token chunk c).  Experts with
// rows and a slot contribute ceil(rows / RCAP) groups each, in id order; the
// loads for 256 experts are issued together, then a wavefront scan places j.
// Returns false when j is past the last group.
// The expert's row range [lo, hi) and slot come back from the scan's own
// registers, so the block's first weight address needs no further load.
struct Group { int e, c, lo, hi, slot; };
__device__ bool find_group(const int32_t* __restrict__ offsets, const int32_t* __restrict__ slot_of,
                           const void* host_pool, int E, int RCAP, int j, int lane, Group& g) {
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += 256) {
        int nc[4], lo[4], hi[4], sl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = e0 + 64 * i + lane;
            lo[i] = hi[i] = 0;
            sl[i] = e;
            if (e < E) {
                lo[i] = offsets[e];
                hi[i] = offsets[e + 1];
                if (slot_of) sl[i] = slot_of[e];
            }
            nc[i] = hi[i] > lo[i] && ft::slot_has_weights(sl[i], host_pool) ? (hi[i] - lo[i] + RCAP - 1) / RCAP : 0;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int incl = wave_scan_incl(nc[i]);
            const int total = __shfl(incl, 63, 64);
            if (j < base + total) {
                const uint64_t m = __ballot(j < base + incl);
                const int l = __builtin_ctzll(m);
                g.e = e0 + 64 * i + l;
                g.c = j - base - __shfl(incl - nc[i], l, 64);
                g.lo = __shfl(lo[i], l, 64);
                g.hi = __shfl(hi[i], l, 64);
                g.slot = __shfl(sl[i], l, 64);
                return g.e < E;
            }
            base += total;
        }
    }
    return false;
}

// The token rows of block group j: an expert (or the shared expert) and a
// chunk of at most RCAP of its rows.  All block-uniform; readfirstlane makes
// them scalar so that row loops branch on SGPRs instead of masking lanes.
struct GroupRows {
    int slot, r0, R;     // weight slot, first row of the chunk in the group, rows
    size_t p_lo, orow0;  // first permutation position of the expert; output row base
    bool shared;
};
__device__ __forceinline__ bool resolve_group(const StreamArgs& a, int j, int lane, GroupRows& gr) {
    if (j < a.n_routed_groups) {
        Group g;
        if (!find_group(a.offsets, a.slot_of, a.host_pool, a.E, a.RCAP, j, lane, g)) return false;
        const int c = __builtin_amdgcn_readfirstlane(g.c);
        gr.slot = __builtin_amdgcn_readfirstlane(g.slot);
        const int lo = __builtin_amdgcn_readfirstlane(g.lo);
        const int hi = __builtin_amdgcn_readfirstlane(g.hi);
        gr.p_lo = lo;
        gr.r0 = c * a.RCAP;
        gr.R = min(a.RCAP, hi - lo - gr.r0);
        gr.orow0 = gr.p_lo;
        gr.shared = false;
    } else {
        gr.slot = a.shared_slot;
        gr.p_lo = 0;
        gr.r0 = (j - a.n_routed_groups) * a.RCAP;
        gr.R = min(a.RCAP, a.T - gr.r0);
        gr.orow0 = (size_t)a.T * a.k;
        gr.shared = true;
    }
    return gr.R > 0;
}
// Source row of token row r of the group: x row (gate/up) or h row (down).
__device__ __forceinline__ size_t source_row(const StreamArgs& a, const GroupRows& gr, int r) {
    if (!a.perm) return gr.orow0 + gr.r0 + r;
    if (gr.shared) return (size_t)(gr.r0 + r);
    return (size_t)(a.perm[gr.p_lo + gr.r0 + r] / a.k);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// One butterfly exchange with the lane that DPP control CTRL pairs with this
// one (the pair differs in lane bit BIT).  With N >= 2 slots the upper half
// of the slots goes to the lane whose bit is 0 and the lower half to the
// other; each lane keeps N/2 slots, summed over the pair.  With N == 1 the
// pair's values are simply added.
template <int CTRL, int BIT, int N, int NM, int RP>
__device__ __forceinline__ void bstep(float (&v)[NM][RP], int lane) {
    if constexpr (N >= 2) {
        const bool up = (lane >> BIT) & 1;
#pragma unroll
        for (int i = 0; i < N / 2; ++i)
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const float lo = v[m][i], hi = v[m][i + N / 2];
                v[m][i] = (up ? hi : lo) + dpp_f<CTRL>(up ? lo : hi);
            }
    } else {
#pragma unroll
        for (int m = 0; m < NM; ++m) v[m][0] += dpp_f<CTRL>(v[m][0]);
    }
}

// Sum v[m][r] over each LPR-lane segment.  Afterwards v[m][0] of lane l holds
// the segment's sum for token slot seg_slot<RP, LPR>(l); RP is a power of two
// <= 16 (<= 8 when LPR == 8).  Exchanges: row_mirror (bit 3), row_half_mirror
// (bit 2), quad_perm [2,3,0,1] (bit 1), quad_perm [1,0,3,2] (bit 0); each
// pairs lanes that hold the same slots so far.  Segments of 32 and 64 lanes
// finish with cross-row swaps.
template <int LPR, int NM, int RP>
__device__ __forceinline__ void seg_reduce(float (&v)[NM][RP], int lane) {
    constexpr int R1 = RP / 2 > 0 ? RP / 2 : 1, R2 = RP / 4 > 0 ? RP / 4 : 1;
    constexpr int R3 = RP / 8 > 0 ? RP / 8 : 1;
    if constexpr (LPR >= 16) {
        bstep<0x140, 3, RP, NM, RP>(v, lane);
        bstep<0x141, 2, R1, NM, RP>(v, lane);
        bstep<0x4E, 1, R2, NM, RP>(v, lane);
        bstep<0xB1, 0, R3, NM, RP>(v, lane);
    } else {
        bstep<0x141, 2, RP, NM, RP>(v, lane);
        bstep<0x4E, 1, R1, NM, RP>(v, lane);
        bstep<0xB1, 0, R2, NM, RP>(v, lane);
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        if constexpr (LPR >= 32) v[m][0] += __shfl_xor(v[m][0], 16, 64);
        if constexpr (LPR == 64) v[m][0] += __shfl_xor(v[m][0], 32, 64);
    }
}
// token slot held by lane l after seg_reduce, and whether l writes it
template <int RP, int LPR>
__device__ __forceinline__ int seg_slot(int lane) {
    constexpr int LB = LPR >= 16 ? 4 : 3;  // lane bits used by the DPP steps
    constexpr int SB = RP == 1 ? 0 : RP == 2 ? 1 : RP == 4 ? 2 : RP == 8 ? 3 : 4;
    return (lane & ((1 << LB) - 1)) >> (LB - SB);
}
template <int RP, int LPR>
__device__ __forceinline__ bool seg_writer(int lane) {
    constexpr int LB = LPR >= 16 ? 4 : 3;
    constexpr int SB = RP == 1 ? 0 : RP == 2 ? 1 : RP == 4 ? 2 : RP == 8 ? 3 : 4;
    return (lane % LPR) < (1 << LB) && (lane & ((1 << (LB - SB)) - 1)) == 0;
}

// acc += (16-byte weight chunk) . (matching activations of one token row).
// xr points at the token row in LDS; col is the chunk column.  MXFP4 rows are
// held in LDS sub-chunk-major (8-element unit w of chunk c at (w*nch + c)*8)
// so that lanes reading consecutive chunks touch consecutive 16-byte words.
// FP8 chunks (16 codes, decoded into dec[0..7]) meet 16 plain-layout values.
// NVFP4 chunks (two blocks of 16 codes, laid out like MXFP4) sum each block
// in fp32 and add it times the block's scale (bs0, bs1).
template <int WT, typename AT>
__device__ __forceinline__ float chunk_dot(const u32x4_t& wv, const uint32_t* dec, const AT* xr,
                                           int col, int nch, float acc, float bs0 = 0.f,
                                           float bs1 = 0.f) {
    if constexpr (WT == 0) {
        const f32x4_t xv = *reinterpret_cast<const f32x4_t*>(xr + col * 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = fmaf(__uint_as_float(wv[q]), xv[q], acc);
    } else if constexpr (WT == 1) {
        const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xr + col * 8);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = dot2_bf16(wv[q], xv[q], acc);
    } else if constexpr (WT == 3) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xr + col * 16 + 8 * h);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc = dot2_bf16(dec[4 * h + q], xv[q], acc);
        }
    } else if constexpr (WT == 4) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            float p = 0.f;
#pragma unroll
            for (int w = 2 * blk; w < 2 * blk + 2; ++w) {
                const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xr + ((size_t)w * nch + col) * 8);
#pragma unroll
                for (int b = 0; b < 4; ++b) p = dot2_bf16(dec[4 * w + b], xv[b], p);
            }
            acc = fmaf(p, blk ? bs1 : bs0, acc);
        }
    } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xr + ((size_t)w * nch + col) * 8);
#pragma unroll
            for (int b = 0; b < 4; ++b) acc = dot2_bf16(dec[4 * w + b], xv[b], acc);
        }
    }
    return acc;
}

// two e4m3 bytes (the low half of w) -> floats, exact
__device__ __forceinline__ void e4m3x2_f32(uint32_t w, float& lo, float& hi) {
    const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    lo = __uint_as_float(b << 16);
    hi = __uint_as_float(b & 0xFFFF0000u);
}

// f(std::integral_constant<int, R>) for the runtime R in [1, N].
template <int N, typename F>
__device__ __forceinline__ void with_rows(int R, F&& f) {
    if constexpr (N >= 1) {
        if (R == N) f(std::integral_constant<int, N>{});
        else with_rows<N - 1>(R, f);
    }
}

// NM = 2: gate and up rows -> h = silu(gate) * up (row length H, N = I).
// NM = 1: down rows -> y (row length I, N = H).
template <int WT, int NM, int QMAX, int RMAX, typename OT>
__device__ __forceinline__ void stream_body(const StreamArgs& a) {
    using AT = typename std::conditional<WT == 0, float, __bf16>::type;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    AT* xs = reinterpret_cast<AT*>(smem);
    const int j = blockIdx.x / a.NB, nb = blockIdx.x % a.NB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

    // this block's group: an expert (or the shared expert) and its token chunk
    // (all block-uniform; readfirstlane makes them scalar so the token-row
    // loops below branch on SGPRs instead of masking lanes).  Written out here
    // rather than through resolve_group(): this kernel sits at the register
    // limit of two wavefronts per SIMD, and the helper's struct costs 15 VGPRs.
    int slot, r0, R;
    size_t p_lo, orow0;
    bool shared;
    if (j < a.n_routed_groups) {
        Group g;
        if (!find_group(a.offsets, a.slot_of, a.host_pool, a.E, a.RCAP, j, lane, g)) return;
        const int c = __builtin_amdgcn_readfirstlane(g.c);
        slot = __builtin_amdgcn_readfirstlane(g.slot);
        const int lo = __builtin_amdgcn_readfirstlane(g.lo);
        const int hi = __builtin_amdgcn_readfirstlane(g.hi);
        p_lo = lo;
        r0 = c * a.RCAP;
        R = min(a.RCAP, hi - lo - r0);
        orow0 = p_lo;
        shared = false;
    } else {
        slot = a.shared_slot;
        p_lo = 0;
        r0 = (j - a.n_routed_groups) * a.RCAP;
        R = min(a.RCAP, a.T - r0);
        orow0 = (size_t)a.T * a.k;
        shared = true;
    }
    if (R <= 0) return;
    const uint8_t* sl = ft::slot_weights(a.pool, a.slot_stride, a.host_pool, a.host_stride, slot);
    const u32x4_t* mat[NM];
    const uint8_t* scl[NM];
    float msc[NM];  // FP8: the matrix scales (applied to the reduced sums); else 1
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        mat[m] = reinterpret_cast<const u32x4_t*>(sl + a.moff[m]);
        scl[m] = sl + a.soff[m];
        if constexpr (WT == 3) msc[m] = *reinterpret_cast<const float*>(scl[m]);
        else if constexpr (WT == 4) msc[m] = *reinterpret_cast<const float*>(sl + a.toff[m]);
        else msc[m] = 1.0f;
    }
    const Walk wk = a.wk;
    const int K = a.K;
    const int RS = 64 / wk.LPR;                           // rows per item
    const int seg = lane / wk.LPR, sg = lane % wk.LPR;    // this lane's row in the item, place in it
    const int n0 = nb * a.RPB, n1 = min(n0 + a.RPB, a.N);
    const int ng = (n1 - n0 + RS - 1) / RS;                          // items per pass, block
    const int gw = ng > wave ? (ng - wave + NWAVE - 1) / NWAVE : 0;  // ... of this wave
    const int U = gw * wk.P;                                         // items of this wave

    struct Item { int row, p, cend; };
    auto item = [&](int u) __attribute__((always_inline)) {
        const int gi = u / wk.P;
        Item it;
        it.p = u - gi * wk.P;
        it.row = n0 + (wave + NWAVE * gi) * RS + seg;
        it.cend = min(wk.nch, (it.p + 1) * wk.CPP);
        return it;
    };
    auto col_of = [&](const Item& it, int q) __attribute__((always_inline)) {
        return it.p * wk.CPP + sg + wk.LPR * q;
    };
    auto valid = [&](const Item& it, int q) __attribute__((always_inline)) {
        return q < wk.Q && it.row < n1 && col_of(it, q) < it.cend;
    };
    struct Buf {
        u32x4_t v[NM][QMAX];
        uint32_t s[NM][QMAX];
    };
    // Every issue() runs all NM*QMAX loads on every lane, without branches, so
    // that the number of loads in flight is the same on every path and the
    // compiler's wait before consume() only covers the buffer it reads (a
    // load under a branch makes it wait for everything).  Loads that are not
    // part of the item (and issues past the wave's last item) point every
    // lane at the matrix's first 16 bytes: one cache line.
    auto issue = [&](Buf& b, int u) __attribute__((always_inline)) {
        const bool live = u < U;  // wave-uniform
        const Item it = item(u);
#pragma unroll
        for (int q = 0; q < QMAX; ++q) {
            const size_t ci = live && valid(it, q) ? (size_t)it.row * wk.nch + col_of(it, q) : 0;
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                b.v[m][q] = __builtin_nontemporal_load(mat[m] + ci);
                if constexpr (WT == 2) b.s[m][q] = scl[m][ci];
                if constexpr (WT == 4) b.s[m][q] = reinterpret_cast<const uint16_t*>(scl[m])[ci];
            }
        }
    };

    float acc[NM][RMAX];
    auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int r = 0; r < RMAX; ++r) acc[m][r] = 0.f;
    };

    // consume(b, u, rows): rows is a std::integral_constant, the number of
    // token rows of this group, so that the row loops have fixed trip counts
    // (a runtime count makes the compiler keep every chunk's values live).
    auto consume = [&](const Buf& b, int u, auto rows) __attribute__((always_inline)) {
        constexpr int RR = decltype(rows)::value;
        const Item it = item(u);
#pragma unroll
        for (int q = 0; q < QMAX; ++q) {
            if (q >= wk.Q) break;  // uniform
            const bool ok = valid(it, q);
            const int col = ok ? col_of(it, q) : 0;
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                uint32_t dec[WT == 2 || WT == 4 ? 16 : WT == 3 ? 8 : 1];
                float bs0 = 0.f, bs1 = 0.f;  // NVFP4 block scales of the chunk
                u32x4_t wv = b.v[m][q];
#pragma unroll
                for (int w = 0; w < 4; ++w) wv[w] = ok ? wv[w] : 0u;  // +0 codes / +0.0 weights
                if constexpr (WT == 2) {
                    const float sc = __uint_as_float(b.s[m][q] << 23);
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const uint32_t cw = wv[w];
                        dec[4 * w + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 0));
                        dec[4 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 1));
                        dec[4 * w + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 2));
                        dec[4 * w + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 3));
                    }
                } else if constexpr (WT == 4) {
                    // e2m1 codes to bf16 (exact); each block's sum is scaled later
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const uint32_t cw = wv[w];
                        dec[4 * w + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 0));
                        dec[4 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 1));
                        dec[4 * w + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 2));
                        dec[4 * w + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 3));
                    }
                    e4m3x2_f32(ok ? b.s[m][q] : 0u, bs0, bs1);
                } else if constexpr (WT == 3) {
                    // e4m3 codes to bf16 (exact; the conversion's scale operand only
                    // takes a power of two, so the matrix scale comes later)
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        dec[2 * w + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wv[w], 1.0f, false));
                        dec[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wv[w], 1.0f, true));
                    }
                }
#pragma unroll
                for (int r = 0; r < RR; ++r)
                    acc[m][r] = chunk_dot<WT, AT>(wv, dec, xs + (size_t)r * K, col, wk.nch, acc[m][r], bs0, bs1);
            }
        }
        if (it.p != wk.P - 1) return;
        // item finished: reduce each token's sums over the row's segment
        constexpr int RP = RR <= 1 ? 1 : RR <= 2 ? 2 : RR <= 4 ? 4 : RR <= 8 ? 8 : 16;
        float v[NM][RP];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int r = 0; r < RP; ++r) v[m][r] = r < RR ? acc[m][r] : 0.f;
        int rs;
        bool wr;
        switch (wk.LPR) {
            case 8:
                seg_reduce<8>(v, lane);
                rs = seg_slot<RP, 8>(lane);
                wr = seg_writer<RP, 8>(lane);
                break;
            case 16:
                seg_reduce<16>(v, lane);
                rs = seg_slot<RP, 16>(lane);
                wr = seg_writer<RP, 16>(lane);
                break;
            case 32:
                seg_reduce<32>(v, lane);
                rs = seg_slot<RP, 32>(lane);
                wr = seg_writer<RP, 32>(lane);
                break;
            default:
                seg_reduce<64>(v, lane);
                rs = seg_slot<RP, 64>(lane);
                wr = seg_writer<RP, 64>(lane);
                break;
        }
        if (wr && rs < RR && it.row < n1) {
            const size_t idx = (orow0 + r0 + rs) * (size_t)a.N + it.row;
            float val;
            if constexpr (NM == 2) val = silu_mul(v[0][0] * msc[0], v[1][0] * msc[1]);
            else val = v[0][0] * msc[0];
            using DT = typename std::conditional<NM == 2, AT, OT>::type;
            if constexpr (sizeof(DT) == 4) reinterpret_cast<float*>(a.dst)[idx] = val;
            else reinterpret_cast<uint16_t*>(a.dst)[idx] = (uint16_t)f32_to_bf16_bits(val);
        }
        zero_acc();
    };

    const AT* src = reinterpret_cast<const AT*>(a.src);
    const int units = K * (int)sizeof(AT) / 16;  // 16-byte units per activation row
    Buf A, B;
    // the first two items are in flight while the activations are staged
    issue(A, 0);
    issue(B, 1);
    for (int i = threadIdx.x; i < R * units; i += blockDim.x) {
        const int r = i / units, uu = i - r * units;
        const size_t srow = a.perm ? (shared ? (size_t)(r0 + r) : (size_t)(a.perm[p_lo + r0 + r] / a.k))
                                   : orow0 + r0 + r;
        const int du = (WT == 2 || WT == 4) ? (uu & 3) * (units >> 2) + (uu >> 2) : uu;
        reinterpret_cast<u32x4_t*>(xs + (size_t)r * K)[du] =
            reinterpret_cast<const u32x4_t*>(src + srow * K)[uu];
    }
    __syncthreads();
    zero_acc();
    // Two items always in flight; issues past the end are single-line reads.
    auto stream = [&](auto rows) __attribute__((always_inline)) {
        for (int u = 0; u < U; u += 2) {
            consume(A, u, rows);
            issue(A, u + 2);
            if (u + 1 < U) consume(B, u + 1, rows);
            issue(B, u + 3);
        }
    };
    with_rows<RMAX>(R, stream);
}

template <int WT, int NM, int QMAX, int RMAX, typename OT>
__global__ __launch_bounds__(256) void stream_kernel(const StreamArgs a) {
    stream_body<WT, NM, QMAX, RMAX, OT>(a);
}
// The same held to 168 VGPRs, so that three wavefronts fit a SIMD
template <int WT, int NM, int QMAX, int RMAX, typename OT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void stream_kernel_w3(const StreamArgs a) {
    stream_body<WT, NM, QMAX, RMAX, OT>(a);
}

// ---------------------------------------------------------------------------
// Narrow weights on matrix cores.  Decoding an e2m1 or e4m3 code to bf16
// costs one instruction per two weights, and a dot product per token row one
// more, with the activations read from LDS again for every token row.  Here
// the decoded weights feed v_mfma_f32_16x16x32_bf16 instead: the group's
// token rows are the MFMA's M (padded to 16 with zeros), 16 weight rows its
// N, and every token row costs nothing beyond the decode.  Exact like the
// version above: codes decode exactly to bf16 (MXFP4 times the block's
// power-of-two scale; the FP8 matrix scale multiplies the finished sums),
// products and sums in fp32.
//
// Lane l takes LE weights of row 16 g + (l & 15) at K offset LE (l >> 4) of
// each 4 LE-wide step, with two 16-byte loads: the four lane groups together
// read a whole 128-byte line of each of the 16 rows (LE = 64 for MXFP4, 32
// for FP8).  The weights decode to 8-wide B fragments, fragment f covering
// k = LE (l >> 4) + 8 f.  Every lane's k positions form a permutation of the
// step's, the same for A (read from LDS at those positions) and B, so the
// MFMA's sum over its K is the sum over the step.  No cross-lane reduction
// is needed: the accumulator of lane l holds token rows 4 (l >> 4) .. + 3 of
// weight row 16 g + (l & 15).  NM = 2 runs the gate and up rows of the same
// 16 row numbers side by side and writes silu(gate) * up.
//
// A wavefront walks (row group of 16, K step) pairs in order with D steps of
// loads in flight (a rolling register buffer, branch-free like the kernel
// above); the block's four wavefronts take every fourth row group of its rows.
// MXFP4 scales: one 16-byte load per lane every two steps brings a row's
// scale bytes of those steps; one-byte loads per step, from 16 rows at once,
// cost more than the codes.
// Measured (MXFP4 284B-A13B layer, 2 to 64 tokens): half a line per row and
// step (one load per lane) was up to 20% slower than whole lines, and 8
// steps in flight (148 VGPRs) slower than 4 (108) where blocks are short.
// Against the kernel above: gate/up 33 vs 56 us at 2 tokens and 353 vs 418
// us at 64; down 195 vs 223 us at 64 tokens.
// ---------------------------------------------------------------------------
// Steps in flight per wavefront (a multiple of 2): 4 for bf16 down rows, 2 for
// bf16 gate/up rows and the narrow formats, whose registers then leave room
// for more wavefronts (bf16 gate/up at 4 tokens 43.1 vs 45.5 us).
// Narrow rows with 2 against 4 (us): 284B-A13B MXFP4 gate/up 89.0 vs 94.0 at 8
// tokens and 346 vs 352 at 64; 753B-A40B MXFP4 298 vs 305 at 32; 35B-A3B FP8
// 49.0 vs 52.3 at 16 and 79.0 vs 81.8 at 64.  bf16 down rows at 64 tokens
// were 2% slower with 2 (74.8 vs 73.5), 6 and 8 slower for every format.
template <int WT, int NM = 1> constexpr int mx_d() { return WT == 1 && NM == 1 ? 4 : 2; }

__device__ __forceinline__ bf16x8_t fp4x8_bf16(uint32_t codes, float sc) {
    u32x4_t d;
    d[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0));
    d[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1));
    d[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2));
    d[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3));
    return __builtin_bit_cast(bf16x8_t, d);
}

// 8 e4m3 codes (two words) -> 8 bf16, exact
__device__ __forceinline__ bf16x8_t fp8x8_bf16(uint32_t lo, uint32_t hi) {
    u32x4_t d;
    d[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
    d[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
    d[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
    d[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
    return __builtin_bit_cast(bf16x8_t, d);
}

// NVFP4: 8 codes times their block scale -> 8 bf16.  e2m1 times e4m3 has at
// most 6 significant bits, so the product (in fp32) converts to bf16 exactly.
__device__ __forceinline__ bf16x8_t nvfp4x8_bf16(uint32_t codes, float bs) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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

// Per-step shape of the matrix-core kernel (WT: 1 = bf16, 2 = MXFP4, 3 = FP8,
// 4 = NVFP4).  bf16 rows need no decode: each 16-byte load is one fragment.
template <int WT> struct MxShape {
    static constexpr int LPS = 2;                                // 16-byte code loads per lane, step, matrix
    static constexpr int EPL = WT == 1 ? 8 : WT == 3 ? 16 : 32;  // weights per 16-byte load
    static constexpr int LE = LPS * EPL;                         // weights per lane and step
    static constexpr int KS = 4 * LE;                            // K per step (128 code bytes of a row)
    static constexpr int NF = LE / 8;                            // 8-wide B fragments per lane, step
    static constexpr int SPW = WT == 2 ? 16 / (4 * LPS) : 1;     // MXFP4: steps per 16-byte scale word
    static constexpr int NSV = WT == 2 ? 2 * mx_d<WT>() / SPW : 1;  // MXFP4: scale-word slots (D = 2 for both NM)
};

template <int WT, int NM, typename OT>
__global__ __launch_bounds__(256) void stream_mx_kernel(const StreamArgs a) {
    static_assert(WT >= 1 && WT <= 4, "bf16 or narrow weights");
    using S = MxShape<WT>;
    constexpr int D = mx_d<WT, NM>(), LPS = S::LPS, KS = S::KS, NF = S::NF, SPW = S::SPW, NSV = S::NSV;
    static_assert(D % SPW == 0, "a scale word's steps share one register round");
    static_assert(WT != 2 || NSV == 2 * D / SPW, "scale-word slots for D steps in flight");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __bf16* xs = reinterpret_cast<__bf16*>(smem);
    const int j = blockIdx.x / a.NB, nb = blockIdx.x % a.NB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    GroupRows gr;
    if (!resolve_group(a, j, lane, gr)) return;
    const int R = gr.R;
    const int K = a.K, pitch = K + 8;  // bf16 per LDS row (the skew spreads rows over banks)
    const int nks = K / KS;
    const int n0 = nb * a.RPB, n1 = min(n0 + a.RPB, a.N);
    const int nrg = (n1 - n0) / 16;                                       // row groups of the block
    const int rgw = nrg > wave ? (nrg - wave + NWAVE - 1) / NWAVE : 0;    // ... of this wave
    const int U = rgw * nks;                                              // (group, step) pairs
    const int ln = lane & 15, q = lane >> 4;
    const uint8_t* sl = ft::slot_weights(a.pool, a.slot_stride, a.host_pool, a.host_stride, gr.slot);
    const size_t rowb = WT == 1 ? (size_t)K * 2 : WT == 3 ? (size_t)K : (size_t)K / 2;
    const size_t srowb = (size_t)K / (WT == 4 ? 16 : 32);
    float msc[NM];  // FP8 matrix / NVFP4 tensor scales (applied to the finished sums)
#pragma unroll
    for (int m = 0; m < NM; ++m)
        msc[m] = WT == 3 ? *reinterpret_cast<const float*>(sl + a.soff[m])
               : WT == 4 ? *reinterpret_cast<const float*>(sl + a.toff[m]) : 1.0f;

    // Loads of pair u into code buffer b; pairs past the end re-read the first
    // one.  MXFP4: a pair u == 0 mod SPW also loads the row's 16 scale bytes of
    // pairs u .. u + SPW - 1 (nks is a multiple of SPW: one row group) into
    // scale slot t; the loop below runs two rounds of D pairs per iteration so
    // that slot t's readers (SPW pairs, D pairs earlier) are done when it is
    // refilled.
    u32x4_t cb[D][NM][LPS];
    u32x4_t sv[NSV][NM];
    // NVFP4: the 4 block-scale bytes of this lane's 64 weights of each step
    uint32_t s4[WT == 4 ? D : 1][NM];
    auto row_of = [&](int uu) __attribute__((always_inline)) {
        const int rgi = uu / nks;
        // (clamped into the block: a wavefront without row groups still issues)
        return (size_t)min(n0 + 16 * (wave + NWAVE * rgi) + ln, n1 - 1);
    };
    auto issue = [&](int b, int t, int u) __attribute__((always_inline)) {
        const int uu = u < U ? u : 0;
        const int ks = uu % nks;
        const size_t row = row_of(uu);
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int h = 0; h < LPS; ++h)
                cb[b][m][h] = *(reinterpret_cast<const u32x4_t*>(sl + a.moff[m] + row * rowb) +
                                4 * LPS * ks + LPS * q + h);
        if (WT == 2 && b % SPW == 0) {
#pragma unroll
            for (int m = 0; m < NM; ++m)
                sv[t][m] = *reinterpret_cast<const u32x4_t*>(sl + a.soff[m] + row * srowb + 4 * LPS * ks);
        }
        if constexpr (WT == 4) {
#pragma unroll
            for (int m = 0; m < NM; ++m)
                s4[b][m] = *reinterpret_cast<const uint32_t*>(sl + a.soff[m] + row * srowb + 16 * ks + 4 * q);
        }
    };
#pragma unroll
    for (int b = 0; b < D; ++b) issue(b, (b / SPW) % NSV, b);

    // the group's activation rows, plain layout
    const __bf16* src = reinterpret_cast<const __bf16*>(a.src);
    const int units = K / 8;
    for (int i = threadIdx.x; i < R * units; i += blockDim.x) {
        const int r = i / units, uu = i - r * units;
        *reinterpret_cast<u32x4_t*>(xs + (size_t)r * pitch + 8 * uu) =
            reinterpret_cast<const u32x4_t*>(src + source_row(a, gr, r) * K)[uu];
    }
    __syncthreads();

    // A: this lane's token row (rows past R read row R - 1 and are zeroed),
    // at the lane group's K offset
    const bool mrow = ln < R;
    const __bf16* xa = xs + (size_t)min(ln, R - 1) * pitch + S::LE * q;
    f32x4_t acc[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int u0 = 0; u0 < U; u0 += 2 * D) {
#pragma unroll
        for (int v = 0; v < 2 * D; ++v) {
            const int u = u0 + v, b = v % D, t = (v / SPW) % NSV;
            if (u < U) {  // wave-uniform
                const int rgi = u / nks, ks = u - rgi * nks;
                bf16x8_t av[NF];
#pragma unroll
                for (int f = 0; f < NF; ++f) {
                    av[f] = *reinterpret_cast<const bf16x8_t*>(xa + ks * KS + 8 * f);
                    if (!mrow) av[f] = bf16x8_t{};
                }
#pragma unroll
                for (int m = 0; m < NM; ++m) {
#pragma unroll
                    for (int f = 0; f < NF; ++f) {
                        bf16x8_t bw;
                        if constexpr (WT == 1) {
                            bw = __builtin_bit_cast(bf16x8_t, cb[b][m][f]);
                        } else if constexpr (WT == 2) {
                            // scale byte of this lane's 32-block: byte SPW-step s, group q, load h
                            const int h = f / 4, by = (v % SPW) * 4 * LPS + LPS * q + h;
                            const uint32_t word = sv[t][m][by >> 2];
                            const float sc = __uint_as_float(((word >> (8 * (by & 3))) & 0xFFu) << 23);
                            bw = fp4x8_bf16(cb[b][m][h][f % 4], sc);
                        } else if constexpr (WT == 4) {
                            // fragment f lies in this lane's block f / 2 (16 weights)
                            float bs0, bs1;
                            e4m3x2_f32(s4[b][m] >> (16 * (f / 4)), bs0, bs1);
                            bw = nvfp4x8_bf16(cb[b][m][f / 4][f % 4], (f / 2) % 2 ? bs1 : bs0);
                        } else {
                            const int h = f / 2, w0 = 2 * (f % 2);
                            bw = fp8x8_bf16(cb[b][m][h][w0], cb[b][m][h][w0 + 1]);
                        }
                        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[f], bw, acc[m], 0, 0, 0);
                    }
                }
                if (ks == nks - 1) {  // row group done: token rows 4 q + i of weight row
                    const int row = n0 + 16 * (wave + NWAVE * rgi) + ln;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int mo = 4 * q + i;
                        if (mo < R) {
                            const size_t idx = (gr.orow0 + gr.r0 + mo) * (size_t)a.N + row;
                            if constexpr (NM == 2) {  // h = silu(gate) * up, bf16
                                const float hv = silu_mul(acc[0][i] * msc[0], acc[1][i] * msc[1]);
                                reinterpret_cast<uint16_t*>(a.dst)[idx] = (uint16_t)f32_to_bf16_bits(hv);
                            } else if constexpr (sizeof(OT) == 4) {
                                reinterpret_cast<float*>(a.dst)[idx] = acc[0][i] * msc[0];
                            } else {
                                reinterpret_cast<uint16_t*>(a.dst)[idx] =
                                    (uint16_t)f32_to_bf16_bits(acc[0][i] * msc[0]);
                            }
                        }
                    }
#pragma unroll
                    for (int m = 0; m < NM; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
            }
            issue(b, ((v + D) / SPW) % NSV, u + D);
        }
    }
}

// Segment width: the fewest lanes per row (8..64) that cover a row in at most
// QMAX loads per lane; rows longer than 64*QMAX chunks take several passes.
Walk make_walk(int K, int epc, int QMAX) {
    Walk w;
    w.nch = K / epc;
    for (int lpr = 8; lpr <= 64; lpr *= 2) {
        const int q = (w.nch + lpr - 1) / lpr;
        if (q <= QMAX) {
            w.LPR = lpr;
            w.Q = q;
            w.P = 1;
            w.CPP = w.nch;
            return w;
        }
    }
    w.LPR = 64;
    w.Q = QMAX;
    w.CPP = 64 * QMAX;
    w.P = (w.nch + w.CPP - 1) / w.CPP;
    return w;
}

// Rows per block grow (by doubling) until the grid holds at most `target`
// blocks.  With one token per group the whole layer is a few items per wave
// and a grid that stays resident at once is fastest; with more tokens per
// group a finer grid balances groups of unequal size.
// `hint` (StreamArgs::target) overrides the default for one launch.
int target_blocks(int rmax, int hint = 0) {
    static const int forced = [] {
        const char* s = getenv("FTMOE_STREAM_BLOCKS");
        return s ? atoi(s) : 0;
    }();
    if (forced > 0) return forced;
    if (hint > 0) return hint;
    return rmax == 1 ? 1024 : 4096;
}
int pick_rpb(long groups, int N, int rows_per_item, int target) {
    int rpb = rows_per_item * NWAVE;
    while (rpb < N && groups * ((N + rpb - 1) / rpb) > target) rpb *= 2;
    return rpb;
}

template <int WT, int NM, int QMAX, int RMAX, typename OT>
ft_status launch_one(StreamArgs a, int n_shared, size_t max_lds, hipStream_t s) {
    using AT = typename std::conditional<WT == 0, float, __bf16>::type;
    const size_t row_bytes = (size_t)a.K * sizeof(AT);
    int rcap = a.T < RMAX ? a.T : RMAX;
    while (rcap > 1 && rcap * row_bytes > max_lds) --rcap;
    const size_t lds = rcap * row_bytes;
    if (lds > max_lds)
        return ft::set_error(FT_ERR_UNSUPPORTED, "ffn stream: an activation row of %zu bytes exceeds LDS",
                             row_bytes);
    a.RCAP = rcap;
    // groups: sum over experts of ceil(rows / RCAP) <= (T*k + active*(RCAP-1)) / RCAP
    const long tk = (long)a.T * a.k;
    const long act = tk < a.E ? tk : a.E;
    a.n_routed_groups = (int)((tk + act * (rcap - 1)) / rcap);
    const long groups = a.n_routed_groups + (n_shared ? (a.T + rcap - 1) / rcap : 0);
    a.wk = make_walk(a.K, W<WT>::EPC, QMAX);
    a.RPB = pick_rpb(groups, a.N, 64 / a.wk.LPR, target_blocks(RMAX, a.target));
    a.NB = (a.N + a.RPB - 1) / a.RPB;
    // bf16 gate/up rows at up to 4 token rows fit 168 VGPRs: three wavefronts
    // per SIMD instead of two (35B-A3B at 8 / 16 tokens 64.3 / 87.9 -> 57.5 /
    // 84.5 us; 753B-A40B at 2 tokens 127.5 -> 122.2 us)
    auto kern = stream_kernel<WT, NM, QMAX, RMAX, OT>;
    if constexpr (WT == 1 && NM == 2 && RMAX == 4) kern = stream_kernel_w3<WT, NM, QMAX, RMAX, OT>;
    if (lds > 65536)
        FT_HIP(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)lds));
    FT_HIP(ft::launch_timed(NM == 2 ? ft::PROF_FFN_GEMM1 : ft::PROF_FFN_GEMM2, kern,
                        dim3((unsigned)(groups * a.NB)), dim3(64 * NWAVE), lds, s, a));
    FT_LAUNCHED("ffn_stream");
    return FT_OK;
}

// Token rows held per group: 1 for single-token decode (a lean kernel), else
// up to `cap` (4 when rows are long: LDS and registers).
template <int WT, int NM, int QMAX, typename OT>
ft_status launch_rows(const StreamArgs& a, int n_shared, int cap, size_t max_lds, hipStream_t s) {
    if (a.T <= 1) return launch_one<WT, NM, QMAX, 1, OT>(a, n_shared, max_lds, s);
    if (a.T <= 4 || cap <= 4) return launch_one<WT, NM, QMAX, 4, OT>(a, n_shared, max_lds, s);
    return launch_one<WT, NM, QMAX, 8, OT>(a, n_shared, max_lds, s);
}

// Rows on matrix cores: MXFP4 rows whose length is a multiple of 512 (each
// 16-byte scale word then lies within its row), FP8 rows whose length is a
// multiple of 128.  Only with more than one token: at one token the lean
// one-row dot-product kernel is as fast for MXFP4 and faster for FP8
// (35B-A3B gate/up 12.8 vs 17.5 us).
int mx_min_t() {
    static const int min_t = [] {
        const char* e = getenv("FTMOE_MX_MIN_T");
        return e ? atoi(e) : 2;
    }();
    return min_t;
}
// At one token (FTMOE_MX_MIN_T unset) only where measured faster: MXFP4 down
// rows (284B-A13B 12.2 -> 10.9 us, 753B-A40B 16.5 -> 14.5), MXFP4 gate/up rows
// of at most 4096 (284B-A13B 21.0 -> 19.1; 753B-A40B's 6144-long rows 27.5 vs
// 28.1) and NVFP4 down rows (35B-A3B 7.8 -> 7.0); FP8 and NVFP4 gate/up rows
// stay on the dot-product kernel (11.5 vs 15.8 us).
bool mx_eligible(int WT, int NM, int K, int T) {
    static const bool off = getenv("FTMOE_MX_DOT") != nullptr;  // keep the dot-product kernel
    static const bool forced = getenv("FTMOE_MX_MIN_T") != nullptr;
    if (off || T < 1 || T < mx_min_t()) {
        const bool one = !off && !forced && T == 1 &&
                         ((WT == 2 && (NM == 1 || K <= 4096)) || (WT == 4 && NM == 1));
        if (!one) return false;
    }
    if (WT == 2) return K % 512 == 0;
    if (WT == 4) return K % 256 == 0;
    return WT == 3 && K % 128 == 0;
}
// bf16 rows on matrix cores (more than one token, K a multiple of 64).  The
// down rows always: 35B-A3B layer at 2 / 4 / 16 / 64 tokens 18.8 / 31.9 /
// 69.4 / 98.0 us on the dot-product kernel, 14.8 / 21.1 / 52.5 / 76.8 us here;
// 753B-A40B at 32 tokens 570 -> 515 us.  The gate/up rows only at up to 4
// tokens with rows of at most 2048 (35B-A3B: 38.2 -> 25.9 us at 2 tokens,
// 50.7 -> 46.9 at 4; but 88 -> 112 at 16, and the 753B-A40B layer's 6144-long
// rows 128 -> 140 at 2 tokens).  FTMOE_BF16_MX forces 0 neither, 1 the down
// rows only, 2 both.
bool bf16_mx_eligible(int NM, int K, int T) {
    static const int mode = [] {
        const char* e = getenv("FTMOE_BF16_MX");
        return e ? atoi(e) : -1;
    }();
    if (T < mx_min_t() || K % 64 != 0) return false;
    if (mode >= 0) return mode >= 2 || (mode == 1 && NM == 1);
    return NM == 1 || (T <= 4 && K <= 2048);
}
template <int WT, int NM, typename OT>
ft_status launch_mx(StreamArgs a, int n_shared, size_t max_lds, hipStream_t s) {
    // Token rows per group: up to 8, within 64 KB of LDS (two blocks or more
    // per CU).  Fewer rows per group split busy experts into more groups that
    // re-read the same weights (FP8 35B-A3B layer at 64 tokens: 73 -> 60 us
    // for the down rows going from 4 to 8).
    static const int rcap_max = [] {
        const char* e = getenv("FTMOE_MX_RCAP");
        const int v = e ? atoi(e) : 8;
        return v < 1 ? 1 : v > 16 ? 16 : v;
    }();
    const size_t row_bytes = ((size_t)a.K + 8) * 2;
    const size_t lds_cap = max_lds < 65536 ? max_lds : 65536;
    int rcap = a.T < rcap_max ? a.T : rcap_max;
    while (rcap > 1 && rcap * row_bytes > lds_cap) --rcap;
    const size_t lds = rcap * row_bytes;
    if (lds > max_lds)
        return ft::set_error(FT_ERR_UNSUPPORTED, "ffn stream: an activation row of %zu bytes exceeds LDS",
                             row_bytes);
    a.RCAP = rcap;
    const long tk = (long)a.T * a.k;
    const long act = tk < a.E ? tk : a.E;
    a.n_routed_groups = (int)((tk + act * (rcap - 1)) / rcap);
    const long groups = a.n_routed_groups + (n_shared ? (a.T + rcap - 1) / rcap : 0);
    // Rows per block.  A wavefront's start-up (group lookup, activation
    // staging, the first loads' latency) is fixed, so each wavefront streams
    // at least wave_bytes of weights (32 KB: measured best; bf16 35B-A3B down
    // rows at 16 / 64 tokens 49.4 / 73.7 us with 32 KB, 52.7 / 76.8 with 64 KB,
    // 61.1 / 79.8 with 128 KB; FP8 down rows, two steps in flight, 28.8 / 43.7
    // with 32 KB, 35.1 / 45.7 with 64 KB);
    // then the grid is held to at most target_blocks() and, while the rows can
    // still halve, to at least 512 blocks.  FP8 35B-A3B down rows (768 B) at
    // 4 / 16 / 64 tokens: 29 / 66 / 60 us with one row group per wavefront,
    // 18 / 36 / 49 us with this rule.
    static const int wave_kb = [] {
        const char* e = getenv("FTMOE_MX_WAVE_KB");
        return e ? atoi(e) : 0;
    }();
    const size_t wave_bytes = (size_t)(wave_kb > 0 ? wave_kb : 32) * 1024;
    const size_t row_w = (WT == 1 ? (size_t)a.K * 2 : WT == 3 ? (size_t)a.K
                                                  : (size_t)a.K / 2 + a.K / (WT == 4 ? 16 : 32)) * NM;  // weight bytes per row
    auto nblk = [&](int rpb) { return groups * ((a.N + rpb - 1) / rpb); };
    int rpb = 16 * NWAVE;
    while (rpb < a.N && (size_t)(rpb / NWAVE) * row_w < wave_bytes) rpb *= 2;
    while (rpb < a.N && nblk(rpb) > target_blocks(rcap, a.target)) rpb *= 2;
    while (rpb > 16 * NWAVE && nblk(rpb) < 512) rpb /= 2;
    a.RPB = rpb;
    a.NB = (a.N + a.RPB - 1) / a.RPB;
    auto kern = stream_mx_kernel<WT, NM, OT>;
    if (lds > 65536)
        FT_HIP(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)lds));
    FT_HIP(ft::launch_timed(NM == 2 ? ft::PROF_FFN_GEMM1 : ft::PROF_FFN_GEMM2, kern,
                        dim3((unsigned)(groups * a.NB)), dim3(64 * NWAVE), lds, s, a));
    FT_LAUNCHED("ffn_stream_mx");
    return FT_OK;
}

}  // namespace

namespace ft {

ft_status launch_ffn_stream(const FfnGeom& g, const void* x, const int32_t* perm,
                            const int32_t* offsets, const int32_t* slot_of, int shared_slot,
                            void* h, void* y, ft_dtype y_dt, hipStream_t s) {
    const size_t max_lds = 160 * 1024;
    const bool big = g.H > 2048 || g.I > 2048;

    StreamArgs a{};
    a.pool = g.pool;
    a.slot_stride = g.slot_stride;
    a.host_pool = g.host_pool;
    a.host_stride = g.host_stride;
    a.offsets = offsets;
    a.slot_of = slot_of;
    a.E = g.E;
    a.T = g.T;
    a.k = g.k;
    a.shared_slot = shared_slot;
    // bf16 weights of a layer with rows longer than 2048, from 8 tokens on: a
    // finer grid (753B-A40B gate/up + down at 8 / 16 / 32 / 64 tokens: 586 /
    // 934 / 1466 / 2152 us with 4096 blocks, 558 / 923 / 1430 / 2055 with
    // 8192; at 2 tokens 8192 was slower, and on the 35B-A3B layer at every
    // token count)
    a.target = (g.w_dt == FT_BF16 && big && g.T >= 8) ? 8192 : 0;

    // gate/up + SwiGLU: rows I of length H
    StreamArgs a1 = a;
    a1.moff[0] = g.off[0];
    a1.moff[1] = g.off[1];
    a1.soff[0] = g.off[3];
    a1.soff[1] = g.off[4];
    a1.toff[0] = g.toff[0];
    a1.toff[1] = g.toff[1];
    a1.perm = perm;
    a1.N = g.I;
    a1.K = g.H;
    a1.src = x;
    a1.dst = h;
    const int cap = (g.w_dt != FT_F32 && big) ? 4 : 8;
    // bf16 gate/up groups of at most 4 token rows (the three-wavefront kernel)
    // while routed rows average at most 2 per expert; beyond that more experts
    // would be split into groups that re-read their weights (35B-A3B at 64
    // tokens: 138 us with 8 rows a group, 172 with 4)
    const int cap1 = g.w_dt == FT_BF16 && (long)g.T * g.k <= 2L * g.E ? 4 : cap;
    ft_status r;
    if (g.w_dt == FT_F32) r = launch_rows<0, 2, 4, float>(a1, g.n_shared, cap, max_lds, s);
    else if (g.w_dt == FT_BF16) {
        if (bf16_mx_eligible(2, a1.K, a1.T)) r = launch_mx<1, 2, float>(a1, g.n_shared, max_lds, s);
        else r = launch_rows<1, 2, 4, float>(a1, g.n_shared, cap1, max_lds, s);
    }
    else if (g.w_dt == FT_FP8) {
        if (mx_eligible(3, 2, a1.K, a1.T)) r = launch_mx<3, 2, float>(a1, g.n_shared, max_lds, s);
        else r = launch_rows<3, 2, 4, float>(a1, g.n_shared, cap, max_lds, s);
    } else if (g.w_dt == FT_NVFP4) {
        if (mx_eligible(4, 2, a1.K, a1.T)) r = launch_mx<4, 2, float>(a1, g.n_shared, max_lds, s);
        else r = launch_rows<4, 2, 4, float>(a1, g.n_shared, cap, max_lds, s);
    } else if (mx_eligible(2, 2, a1.K, a1.T)) {
        r = launch_mx<2, 2, float>(a1, g.n_shared, max_lds, s);
    } else {
        r = launch_rows<2, 2, 4, float>(a1, g.n_shared, cap, max_lds, s);
    }
    if (r != FT_OK) return r;

    // down: rows H of length I
    StreamArgs a2 = a;
    // MXFP4 down rows of a layer with rows longer than 2048 from 16 tokens on:
    // the finer grid too (753B-A40B at 32 tokens 149 -> 138 us, 284B-A13B at
    // 64 187 -> 178; their gate/up rows were as fast or slower with it)
    if (g.w_dt == FT_MXFP4 && big && g.T >= 16) a2.target = 8192;
    a2.moff[0] = g.off[2];
    a2.soff[0] = g.off[5];
    a2.toff[0] = g.toff[2];
    a2.perm = nullptr;
    a2.N = g.H;
    a2.K = g.I;
    a2.src = h;
    a2.dst = y;
    if (g.w_dt == FT_F32) r = launch_rows<0, 1, 8, float>(a2, g.n_shared, cap, max_lds, s);
    else if (g.w_dt == FT_BF16) {
        if (bf16_mx_eligible(1, a2.K, a2.T)) {
            if (y_dt == FT_F32) r = launch_mx<1, 1, float>(a2, g.n_shared, max_lds, s);
            else r = launch_mx<1, 1, __bf16>(a2, g.n_shared, max_lds, s);
        } else {
            if (y_dt == FT_F32) r = launch_rows<1, 1, 8, float>(a2, g.n_shared, cap, max_lds, s);
            else r = launch_rows<1, 1, 8, __bf16>(a2, g.n_shared, cap, max_lds, s);
        }
    } else if (g.w_dt == FT_FP8) {
        if (mx_eligible(3, 1, a2.K, a2.T)) {
            if (y_dt == FT_F32) r = launch_mx<3, 1, float>(a2, g.n_shared, max_lds, s);
            else r = launch_mx<3, 1, __bf16>(a2, g.n_shared, max_lds, s);
        } else {
            if (y_dt == FT_F32) r = launch_rows<3, 1, 8, float>(a2, g.n_shared, cap, max_lds, s);
            else r = launch_rows<3, 1, 8, __bf16>(a2, g.n_shared, cap, max_lds, s);
        }
    } else if (g.w_dt == FT_NVFP4) {
        if (mx_eligible(4, 1, a2.K, a2.T)) {
            if (y_dt == FT_F32) r = launch_mx<4, 1, float>(a2, g.n_shared, max_lds, s);
            else r = launch_mx<4, 1, __bf16>(a2, g.n_shared, max_lds, s);
        } else {
            if (y_dt == FT_F32) r = launch_rows<4, 1, 8, float>(a2, g.n_shared, cap, max_lds, s);
            else r = launch_rows<4, 1, 8, __bf16>(a2, g.n_shared, cap, max_lds, s);
        }
    } else if (mx_eligible(2, 1, a2.K, a2.T)) {
        if (y_dt == FT_F32) r = launch_mx<2, 1, float>(a2, g.n_shared, max_lds, s);
        else r = launch_mx<2, 1, __bf16>(a2, g.n_shared, max_lds, s);
    } else {
        if (y_dt == FT_F32) r = launch_rows<2, 1, 8, float>(a2, g.n_shared, cap, max_lds, s);
        else r = launch_rows<2, 1, 8, __bf16>(a2, g.n_shared, cap, max_lds, s);
    }
    return r;
}

}  // namespace ft
