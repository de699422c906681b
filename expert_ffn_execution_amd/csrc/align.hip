// align.hip -- token-to-expert alignment: histogram, offsets, stable permutation.
//
// The expert GEMMs read the tokens routed to one expert as one contiguous
// segment (claypier.com article, "从 MoE「用不到的权重」入手的推理引擎": each
// step touches only the experts it routes to).  perm lists the flat slots
// f = t*k + j grouped by expert, increasing f inside a group: a stable
// counting sort, so the result is unique and bitwise reproducible.
//
// Stable ranks come from wavefront ballots: a wave takes 64 consecutive
// slots, one per lane; for each distinct expert among them, a ballot finds the
// lanes holding it, the rank of a lane is the popcount of the matching lanes
// below it, and a running per-expert base (kept in LDS, touched only by this
// wave) advances by the match count.  Waves own contiguous chunks, and a
// per-(chunk, expert) prefix scan gives each chunk its starting positions.
#include "common.h"
#include "route_core.h"

namespace {

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
    return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// Scatter 64 consecutive slots [f0, f0 + 64) ∩ [0, n) held one per lane.
// run[e] is this wave's next free position for expert e (LDS, wave-private).
__device__ __forceinline__ void wave_scatter(const int32_t* __restrict__ ids, int f0, int n,
                                             int* run, int32_t* __restrict__ perm,
                                             int32_t* __restrict__ inv, int lane) {
    const int f = f0 + lane;
    const bool valid = f < n;
    const int v = valid ? ids[f] : -1;
    uint64_t remaining = __ballot(valid);
    while (remaining) {
        const int leader = __builtin_ctzll(remaining);
        const int vl = __shfl(v, leader, 64);
        const uint64_t peers = __ballot(v == vl);
        const int base = run[vl];  // same address for every lane: broadcast read
        if (v == vl) {
            const int pos = base + __popcll(peers & lanemask_lt(lane));
            perm[pos] = f;
            inv[f] = pos;
        }
        if (lane == leader) run[vl] = base + __popcll(peers);
        remaining &= ~peers;
    }
}

// ---------------------------------------------------------------------------
// Small problems: one block of 8 waves does everything.
// LDS: hist[8][E] (then running bases), tot[E].  `ids` may point into LDS.
// ---------------------------------------------------------------------------
constexpr int SW = 8;
__device__ __forceinline__ void align_block(const int32_t* ids, int n, int E,
                                            int32_t* __restrict__ counts,
                                            int32_t* __restrict__ offsets,
                                            int32_t* __restrict__ perm,
                                            int32_t* __restrict__ inv, int* lds) {
    int* hist = lds;            // [SW][E]
    int* tot = lds + SW * E;    // [E] inclusive scan scratch
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < SW * E; i += SW * 64) hist[i] = 0;
    __syncthreads();
    const int chunk = ((n + SW - 1) / SW + 63) & ~63;
    const int f_lo = w * chunk, f_hi = min(n, f_lo + chunk);
    for (int f = f_lo + lane; f < f_hi; f += 64) atomicAdd(&hist[w * E + ids[f]], 1);
    __syncthreads();
    // totals and exclusive offsets (Hillis-Steele over E, E <= 1024)
    for (int e = tid; e < E; e += SW * 64) {
        int s = 0;
        for (int q = 0; q < SW; ++q) s += hist[q * E + e];
        tot[e] = s;
        counts[e] = s;
    }
    __syncthreads();
    for (int o = 1; o < E; o <<= 1) {
        int v[2] = {0, 0};
        for (int i = 0, e = tid; e < E; e += SW * 64, ++i) v[i] = e >= o ? tot[e - o] : 0;
        __syncthreads();
        for (int i = 0, e = tid; e < E; e += SW * 64, ++i) tot[e] += v[i];
        __syncthreads();
    }
    for (int e = tid; e < E; e += SW * 64) {
        int base = (e ? tot[e - 1] : 0);
        offsets[e] = base;
        if (e == E - 1) offsets[E] = tot[e];
        for (int q = 0; q < SW; ++q) {
            int c = hist[q * E + e];
            hist[q * E + e] = base;
            base += c;
        }
    }
    __syncthreads();
    for (int f0 = f_lo; f0 < f_hi; f0 += 64)
        wave_scatter(ids, f0, f_hi, hist + w * E, perm, inv, lane);
}

// At most 64 slots (decode: T*k <= 64): one wavefront, no barriers.  Lane f
// holds slot f; its position is the number of slots with a smaller expert
// plus the number of earlier slots with the same expert (the stable counting
// sort), and the counts and offsets of every expert are counted the same way,
// with each slot's expert read as a scalar.  The same results as align_block.
// EPL: experts per lane (E <= 64 EPL).
template <int EPL>
__device__ __forceinline__ void align_wave(const int32_t* ids, int n, int E,
                                           int32_t* __restrict__ counts,
                                           int32_t* __restrict__ offsets,
                                           int32_t* __restrict__ perm,
                                           int32_t* __restrict__ inv, int lane) {
    const int v = lane < n ? ids[lane] : 0x7fffffff;
    int cnt[EPL], off[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) cnt[i] = off[i] = 0;
    int pos = 0;
    for (int f = 0; f < n; ++f) {
        const int vf = __builtin_amdgcn_readlane(v, f);
        pos += (vf < v) || (vf == v && f < lane);
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            cnt[i] += vf == e;
            off[i] += vf < e;
        }
    }
    if (lane < n) {
        perm[pos] = lane;
        inv[lane] = pos;
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E) {
            counts[e] = cnt[i];
            offsets[e] = off[i];
        }
    }
    if (lane == 0) offsets[E] = n;
}

__global__ __launch_bounds__(SW * 64) void align_small_kernel(const int32_t* __restrict__ ids,
                                                              int n, int E,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ perm,
                                                              int32_t* __restrict__ inv) {
    extern __shared__ int lds[];
    if (n <= 64) {  // block-uniform
        if (threadIdx.x >= 64) return;
        const int l = threadIdx.x;
        if (E <= 64) align_wave<1>(ids, n, E, counts, offsets, perm, inv, l);
        else if (E <= 128) align_wave<2>(ids, n, E, counts, offsets, perm, inv, l);
        else if (E <= 256) align_wave<4>(ids, n, E, counts, offsets, perm, inv, l);
        else if (E <= 512) align_wave<8>(ids, n, E, counts, offsets, perm, inv, l);
        else align_wave<16>(ids, n, E, counts, offsets, perm, inv, l);
        return;
    }
    align_block(ids, n, E, counts, offsets, perm, inv, lds);
}

// Top-k of every token, then the alignment of the picks, in one block: for a
// decode-sized batch the two steps are each a few microseconds of launch and
// memory round trip around very little work.  Wave w picks tokens w, w + SW,
// ... (the top-k kernel's per-token code, so the same picks and gates); the
// picks also go to LDS, where the alignment reads them after a barrier.
// LDS: ids[T*k], then the alignment's hist[SW][E] and tot[E].
template <int NPL>
__global__ __launch_bounds__(SW * 64) void topk_align_small_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    extern __shared__ int lds[];
    const int n = T * k;
    int* ids_s = lds;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int t = wave; t < T; t += SW)
        topk_token<NPL>(logits + (size_t)t * E, bias, E, k, ids + (size_t)t * k, w + (size_t)t * k,
                        ids_s + t * k, lane);
    __syncthreads();
    if (n <= 64) {  // block-uniform
        if (wave == 0) align_wave<NPL>(ids_s, n, E, counts, offsets, perm, inv, lane);
        return;
    }
    align_block(ids_s, n, E, counts, offsets, perm, inv, lds + ((n + 3) & ~3));
}

// ---------------------------------------------------------------------------
// Large problems: units of UB = 256 consecutive slots, one block of 4 waves each.
//   1) per-unit histograms hist[u][e]
//   2) per-expert exclusive scan over units (in place), counts[e]
//   3) per-unit scatter: wave w of unit u starts expert e at
//      offsets[e] + hist[u][e] + (slots of e in the unit's earlier waves)
// hist is read along units by consecutive experts (coalesced) in step 2.
// ---------------------------------------------------------------------------
constexpr int UB = 256;

__global__ __launch_bounds__(256) void unit_hist_kernel(const int32_t* __restrict__ ids, int n,
                                                        int E, int* __restrict__ hist) {
    extern __shared__ int h[];  // [E]
    const int u = blockIdx.x, tid = threadIdx.x;
    for (int e = tid; e < E; e += 256) h[e] = 0;
    __syncthreads();
    const int f = u * UB + tid;
    if (f < n) atomicAdd(&h[ids[f]], 1);
    __syncthreads();
    for (int e = tid; e < E; e += 256) hist[(size_t)u * E + e] = h[e];
}

// 64 experts per block, one per lane; wave w sums units [U w / 16, U (w + 1) / 16)
constexpr int SCAN_W = 16;
__global__ __launch_bounds__(SCAN_W * 64) void unit_scan_kernel(int* __restrict__ hist, int E, int U,
                                                                int32_t* __restrict__ counts) {
    __shared__ int part[SCAN_W][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + lane;
    const int u0 = (int)((long)U * w / SCAN_W), u1 = (int)((long)U * (w + 1) / SCAN_W);
    int s = 0;
    if (e < E) {
#pragma unroll 8
        for (int u = u0; u < u1; ++u) s += hist[(size_t)u * E + e];
    }
    part[w][lane] = s;
    __syncthreads();
    int carry = 0;
    for (int q = 0; q < w; ++q) carry += part[q][lane];
    if (e < E) {
        for (int u = u0; u < u1; ++u) {
            const int v = hist[(size_t)u * E + e];
            hist[(size_t)u * E + e] = carry;
            carry += v;
        }
        if (w == SCAN_W - 1) counts[e] = carry;
    }
}

__global__ __launch_bounds__(256) void unit_scatter_kernel(const int32_t* __restrict__ ids,
                                                           int n, int E,
                                                           const int* __restrict__ hist,
                                                           const int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ inv) {
    extern __shared__ int lds[];  // off[E], sub[4][E], tot[4]
    int* off = lds;
    int* sub = lds + E;
    int* tot = lds + 5 * E;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int u = blockIdx.x;
    for (int i = tid; i < 4 * E; i += 256) sub[i] = 0;
    // exclusive scan of counts: each wave scans a quarter, then the quarters combine
    const int per = (E + 3) / 4;
    {
        int carry = 0;
        const int e_lo = w * per, e_hi = min(E, e_lo + per);
        for (int e0 = e_lo; e0 < e_hi; e0 += 64) {
            const int e = e0 + lane;
            const int v = e < e_hi ? counts[e] : 0;
            int incl = v;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int t = __shfl_up(incl, o, 64);
                if (lane >= o) incl += t;
            }
            if (e < e_hi) off[e] = carry + incl - v;
            carry += __shfl(incl, 63, 64);
        }
        if (lane == 0) tot[w] = carry;
    }
    __syncthreads();
    const int f = u * UB + tid;
    if (f < n) atomicAdd(&sub[w * E + ids[f]], 1);  // the four waves' sub-histograms
    int add = 0;
    for (int q = 0; q < w; ++q) add += tot[q];
    {
        const int e_lo = w * per, e_hi = min(E, e_lo + per);
        for (int e = e_lo + lane; e < e_hi; e += 64) off[e] += add;
    }
    __syncthreads();
    if (u == 0) {
        for (int e = tid; e < E; e += 256) offsets[e] = off[e];
        if (tid == 0) offsets[E] = tot[0] + tot[1] + tot[2] + tot[3];
    }
    // running bases of the four waves
    for (int e = tid; e < E; e += 256) {
        int b = off[e] + hist[(size_t)u * E + e];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = sub[q * E + e];
            sub[q * E + e] = b;
            b += c;
        }
    }
    __syncthreads();
    wave_scatter(ids, u * UB + 64 * w, n, sub + w * E, perm, inv, lane);
}

__global__ void fill_i32_kernel(int32_t* p, long n, int32_t v) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

}  // namespace

namespace ft {

ft_status launch_fill_i32(int32_t* p, long n, int32_t v, hipStream_t s) {
    if (n <= 0) return FT_OK;
    fill_i32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p, n, v);
    FT_LAUNCHED("fill_i32");
    return FT_OK;
}

constexpr long ALIGN_SMALL_MAX = 4096;

size_t align_workspace(int T, int k, int E) {
    long n = (long)T * k;
    if (n <= ALIGN_SMALL_MAX) return 0;
    long U = (n + UB - 1) / UB;
    return (size_t)(U * E) * sizeof(int);
}

ft_status launch_align(const int32_t* ids, int T, int k, int E, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* inv, void* ws,
                       hipStream_t s) {
    const long n = (long)T * k;
    if (n <= ALIGN_SMALL_MAX) {
        size_t lds = (size_t)(SW + 1) * E * sizeof(int);
        align_small_kernel<<<1, SW * 64, lds, s>>>(ids, (int)n, E, counts, offsets, perm, inv);
        FT_LAUNCHED("align_small");
        return FT_OK;
    }
    const int U = (int)((n + UB - 1) / UB);
    int* hist = (int*)ws;
    unit_hist_kernel<<<U, 256, E * sizeof(int), s>>>(ids, (int)n, E, hist);
    FT_LAUNCHED("align_hist");
    unit_scan_kernel<<<cdiv(E, 64), SCAN_W * 64, 0, s>>>(hist, E, U, counts);
    FT_LAUNCHED("align_scan");
    unit_scatter_kernel<<<U, 256, (5 * E + 4) * sizeof(int), s>>>(ids, (int)n, E, hist, counts,
                                                                   offsets, perm, inv);
    FT_LAUNCHED("align_scatter");
    return FT_OK;
}

bool topk_align_small_ok(int T, int k) {
    // at most one token per wavefront of the one block: with more, the tokens
    // of a wavefront are picked in turn and the separate top-k launch (one
    // wavefront per token) wins (35B-A3B layer, graph replays: T = 1 44.3 vs
    // 48.5 us per step; T = 64 307 vs 277 us)
    return T >= 1 && T <= SW && (long)T * k <= ALIGN_SMALL_MAX;
}

ft_status launch_topk_align_small(const float* logits, const float* bias, int T, int E, int k,
                                  int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                                  int32_t* perm, int32_t* inv, hipStream_t s) {
    const int n = T * k;
    const size_t lds = (size_t)(((n + 3) & ~3) + (SW + 1) * E) * sizeof(int);
    if (E <= 64)
        topk_align_small_kernel<1><<<1, SW * 64, lds, s>>>(logits, bias, T, E, k, ids, w, counts, offsets, perm, inv);
    else if (E <= 128)
        topk_align_small_kernel<2><<<1, SW * 64, lds, s>>>(logits, bias, T, E, k, ids, w, counts, offsets, perm, inv);
    else if (E <= 256)
        topk_align_small_kernel<4><<<1, SW * 64, lds, s>>>(logits, bias, T, E, k, ids, w, counts, offsets, perm, inv);
    else if (E <= 512)
        topk_align_small_kernel<8><<<1, SW * 64, lds, s>>>(logits, bias, T, E, k, ids, w, counts, offsets, perm, inv);
    else
        topk_align_small_kernel<16><<<1, SW * 64, lds, s>>>(logits, bias, T, E, k, ids, w, counts, offsets, perm, inv);
    FT_LAUNCHED("topk_align_small");
    return FT_OK;
}

}  // namespace ft
