/*
 * ftmoe.h -- C ABI of the MI355X (gfx950) MoE-layer FFN library (libftmoe.so).
 *
 * One MoE layer, T tokens of hidden size H, E routed experts, k experts per
 * token, expert intermediate size I, optionally one always-on shared expert:
 *
 *   ft_moe_route    router logits (optional) -> top-k expert ids + gates
 *   ft_moe_align    expert histogram, offsets, token->expert permutation
 *   ft_moe_ffn      grouped gate/up GEMM + SwiGLU + down GEMM over the routed
 *                   experts only, weights read through a slot table
 *   ft_moe_combine  gate-weighted sum back to token order
 *   ft_moe_step_run / ft_moe_graph_*  the four as one step, eager or as a
 *                   captured HIP graph
 *   ft_moe_step_fused  a decode step (up to 4 tokens) as one kernel launch
 *   ft_slot_cache_* LRU expert-slot cache over a pinned host expert pool, with
 *                   the next layer's missing experts copied while this layer
 *                   computes
 *
 * Sources.  The pages describe the engine around this path: a few experts per
 * token out of hundreds, only those brought to the GPU, a global LRU expert
 * cache sized in slots, and the next layer's weights streamed double-buffered
 * while the current layer computes (claypier.com article,
 * "从 MoE「用不到的权重」入手的推理引擎" and "按带宽决定分工的思路";
 * FreeToken hub article, paragraphs on prefill overlap and on the WSL pinned
 * memory limit; refft.com guide, "深度解析"; freelamp.com article, section 2.3).
 * They do not spell out the routing rule or the expert FFN; the readings used
 * (top-k on fp32 logits with ties to the lower expert id, softmax over the k
 * picks, SwiGLU experts) are stated at each entry point.
 *
 * Conventions (all entry points):
 *   - Device pointers are HIP device memory (or host-pinned memory mapped for
 *     the device) on the current device; host pointers are ordinary memory.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Work is enqueued asynchronously; no entry point synchronises the stream
 *     unless stated.  The caller owns every buffer; the library never
 *     allocates device memory in these calls (workspace is passed in), except
 *     the fused step's exchange buffer, made once per device on its first call.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     failed check returns FT_ERR_INVALID_ARG / FT_ERR_UNSUPPORTED and
 *     enqueues nothing.  A HIP launch error returns FT_ERR_HIP.  The message
 *     of the last failure on the calling thread is ft_last_error().
 *   - T == 0 is a valid no-op.  T*k must be < 2^31; E <= 1024; k in [1, E].
 *   - Results are deterministic: identical inputs give bitwise identical
 *     outputs (no floating-point atomics anywhere).
 */
#ifndef FTMOE_H
#define FTMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FT_OK = 0,
    FT_ERR_INVALID_ARG = 1,
    FT_ERR_UNSUPPORTED = 2,
    FT_ERR_CAPACITY = 3,
    FT_ERR_NOT_PINNED = 4,
    FT_ERR_BUSY = 5,
    FT_ERR_HIP = 6,
    FT_WARN_OVERLAP_DISABLED = 100
} ft_status;

typedef enum { FT_F32 = 0, FT_BF16 = 1, FT_MXFP4 = 2, FT_FP8 = 3, FT_NVFP4 = 4 } ft_dtype;

/* Message of the last non-OK status returned on this thread ("" if none). */
const char* ft_last_error(void);
/* Library version string. */
const char* ft_version(void);
/* Device-visible address of page-locked host memory (hipHostGetDevicePointer),
 * e.g. for ft_moe_weights.host_pool.  FT_ERR_INVALID_ARG for a null argument,
 * FT_ERR_UNSUPPORTED when `host` is not mapped for the current device. */
ft_status ft_host_device_pointer(const void* host, void** dev);

/* --------------------------------------------------------------------------
 * ft_moe_route -- router top-k gating.
 *
 * Logits: either supplied (`logits_in` [T][E] fp32, device; then x and
 * w_router must be NULL) or computed here as l = x W_r^T with fp32
 * accumulation (x [T][H], w_router [E][H], both in x_dt = FT_BF16 or FT_F32,
 * device; then logits_out [T][E] fp32 must be given and receives l).
 * `bias` [E] fp32 (device, may be NULL) is added to every row:
 * l' = fl32(l + b).  The pages only imply routing (chenxutan.com article,
 * "瓶颈为什么是带宽而不是容量": prefill tokens reach almost every expert;
 * freelamp.com article, section 2.1: the router's choice changes with the
 * content); the rule implemented is:
 *   topk_ids[t][0..k-1] (int32, device) = the k largest l'[t][.] in
 *     decreasing order, equal values ordered by increasing expert id
 *     (-0.0 equals +0.0);
 *   topk_w[t][j] (fp32, device) = exp(l'_j - l'_0) / sum_{i<k} exp(l'_i - l'_0),
 *     i.e. the softmax over all experts restricted to the picks and
 *     renormalised.
 * Logits must be finite (not checked on the device; the result is unspecified
 * otherwise).
 * Computed logits are deterministic for a given batch, but their fp32
 * summation order depends on the batch: up to 64 tokens take a dot-product
 * kernel, more take matrix-core tiles whose blocks start their K loop at
 * different stages.  A token's logits can thus differ in the last bits
 * between batch sizes or positions (each within 1e-5 relative of the exact
 * sum), and with them the picks at near-ties.  Routing from supplied logits
 * is exact and position-independent.
 * ------------------------------------------------------------------------ */
ft_status ft_moe_route(const void* x, ft_dtype x_dt, const void* w_router,
                       const float* logits_in, const float* bias, int T, int H, int E,
                       int k, float* logits_out, int32_t* topk_ids, float* topk_w,
                       void* stream);

/* --------------------------------------------------------------------------
 * ft_moe_align -- token-to-expert alignment (stable counting sort).
 *
 * In: topk_ids [T*k] int32 device, every id in [0, E).
 * Out (device, int32): counts[E]; offsets[E+1] exclusive prefix sums;
 *   perm[T*k] = flat slots f = t*k + j grouped by expert, increasing f within
 *   an expert; inv_perm[T*k] with inv_perm[perm[p]] = p.
 * ws: device workspace of at least ft_moe_align_workspace(T, k, E) bytes
 *   (may be NULL when that is 0); contents need not be initialised.
 * Ids outside [0, E) give unspecified results (not checked on the device).
 * ------------------------------------------------------------------------ */
size_t ft_moe_align_workspace(int T, int k, int E);
ft_status ft_moe_align(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* ws,
                       size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------
 * Expert weight storage ("slot" layout).  One contiguous block per expert so
 * that one copy moves one expert (the pages' pre-merged runtime weight
 * layout: FreeToken hub article, paragraph on the FTW format).  Within a slot:
 *   FT_F32 / FT_BF16: gate [I][H] | up [I][H] | down [H][I], row-major,
 *     element size 4 / 2.
 *   FT_MXFP4: gate codes [I][H/2] | up codes [I][H/2] | down codes [H][I/2] |
 *     gate scales [I][H/32] | up scales [I][H/32] | down scales [H][I/32].
 *     Codes are e2m1 (bit 3 sign, bits 2..1 exponent, bit 0 mantissa), element
 *     2j of a row in the low nibble of byte j, 2j+1 in the high nibble; scales
 *     are e8m0 bytes 2^(X-127) for 32 consecutive elements along the
 *     contraction dimension (OCP Microscaling Formats v1.0).
 *   FT_FP8: gate codes [I][H] | up codes [I][H] | down codes [H][I], one e4m3
 *     byte each (OCP 8-bit floating point v1.0, E4M3: bias 7, no infinities,
 *     S.1111.111 is NaN) | three fp32 scales (gate, up, down), one per matrix:
 *     weight = value(code) * scale.  The pages list FP8 weights (refft.com
 *     guide, the format list) without their scaling; one scale per matrix is
 *     the plainest reading.
 *   FT_NVFP4: gate codes [I][H/2] | up codes [I][H/2] | down codes [H][I/2]
 *     (e2m1 nibbles as for MXFP4) | gate scales [I][H/16] | up scales [I][H/16]
 *     | down scales [H][I/16] (one e4m3 byte per 16 consecutive elements along
 *     the contraction dimension) | three fp32 tensor scales (gate, up, down) at
 *     byte offsets offs[5] + H*I/16 + 0, 4, 8: weight = e2m1(code) *
 *     e4m3(block scale) * tensor scale.  The pages list NVFP4 (refft.com
 *     guide, the format list) without its layout; this is NVIDIA's published
 *     NVFP4 definition.
 * All formats: H % 64 == 0 and I % 64 == 0.
 * ft_expert_layout fills offs[6] = byte offsets of {gate, up, down,
 * gate_sc, up_sc, down_sc} (scale arrays for MXFP4 and NVFP4, the fp32 scales
 * for FP8, 0 otherwise) and returns the
 * slot size in bytes (0 for an unsupported combination).
 * ------------------------------------------------------------------------ */
size_t ft_expert_layout(ft_dtype w_dt, int H, int I, size_t offs[6]);

typedef struct {
    ft_dtype w_dt;        /* FT_F32, FT_BF16, FT_MXFP4, FT_FP8 or FT_NVFP4 */
    int E;                /* routed experts */
    int H;                /* hidden size */
    int I;                /* expert intermediate size */
    int n_shared;         /* 0 or 1 always-on shared expert */
    const void* pool;     /* device base of the slot array */
    size_t slot_stride;   /* bytes between slots (>= ft_expert_layout(), multiple of 256) */
    int shared_slot;      /* slot index of the shared expert (n_shared == 1) */
    /* Optional host tier: the device-visible address of a page-locked host
     * array of experts in the same slot layout (NULL: none).  A slot table
     * entry -2 - j then reads expert j's weights from host_pool + j *
     * host_stride over the host link (zero-copy) instead of a device slot.
     * 256-byte aligned; host_stride >= ft_expert_layout(), a multiple of 256. */
    const void* host_pool;
    size_t host_stride;
} ft_moe_weights;

/* --------------------------------------------------------------------------
 * ft_moe_ffn -- grouped expert FFN over the routed experts only.
 *
 * For every position p of the permutation (expert e = the segment of
 * `offsets` holding p, token t = perm[p] / k):
 *   g = W_gate,e x_t,  u = W_up,e x_t,  h = silu(g) * u,  y_perm[p] = W_down,e h
 * with fp32 accumulation; h is rounded to bf16 for bf16 / MXFP4 weights.
 * With n_shared == 1, rows T*k + t of y_perm receive the shared expert's FFN
 * of x_t (weight 1 in the combine).  MXFP4 weights are decoded exactly to bf16
 * on chip and multiplied with bf16 activations; FP8 codes likewise, the matrix
 * scale applied to each fp32 sum; NVFP4 codes times their block scales
 * likewise (exactly representable in bf16), the tensor scale applied to each
 * fp32 sum.
 *   x [T][H] device, act_dt = FT_BF16 (FT_F32 only with FT_F32 weights);
 *   perm, offsets: ft_moe_align's outputs for the same ids;
 *   slot_of_expert [E] int32 device, or NULL for slot e = expert e: the slot
 *     in `pool` holding expert e; -1 skips expert e (its rows of y_perm are
 *     not written); -2 - j reads expert e's weights from expert j of
 *     w->host_pool (skips it when there is no host pool);
 *   y_perm [T*k + n_shared*T][H] device, y_dt = FT_BF16 (bf16 weights/MXFP4)
 *     or FT_F32 (any weights);
 *   ws: device workspace of >= ft_moe_ffn_workspace(w, T, k) bytes.
 * The kernels address activation rows with 32-bit element offsets and weight
 * rows inside a slot with 32-bit byte offsets: T*H, (T*k + n_shared*T)*I and
 * the expert's slot bytes (ft_expert_layout) must each be below 2^32, else
 * FT_ERR_UNSUPPORTED and nothing is enqueued.
 * ------------------------------------------------------------------------ */
size_t ft_moe_ffn_workspace(const ft_moe_weights* w, int T, int k);
ft_status ft_moe_ffn(const ft_moe_weights* w, const void* x, ft_dtype act_dt, int T, int k,
                     const int32_t* perm, const int32_t* offsets,
                     const int32_t* slot_of_expert, void* y_perm, ft_dtype y_dt, void* ws,
                     size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------
 * ft_moe_ffn_noalloc -- ft_moe_ffn without a caller workspace, for callers
 * that cannot allocate device memory: code under HIP graph capture, serving
 * loops and harnesses that forbid hipMalloc.
 *
 * The workspace is a static device array of FT_NOALLOC_SCRATCH_BYTES
 * (64 MiB) inside the library, which the HIP runtime places on every GPU the
 * library runs on and keeps until the process ends; its device address is
 * looked up once per device, on the first call with that device current.
 * The call itself allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).
 *   Arguments, results (bit for bit) and errors: those of ft_moe_ffn on the
 *   same inputs, without ws / ws_bytes.  FT_ERR_CAPACITY (nothing enqueued)
 *   when ft_moe_ffn_workspace(w, T, k) exceeds FT_NOALLOC_SCRATCH_BYTES;
 *   FT_ERR_HIP when the array's address cannot be obtained.
 *   Every call on one GPU uses that GPU's one array and leaves its last
 *   contents there; nothing in it needs clearing (every byte a call reads was
 *   written earlier in the same call).  Calls that can overlap on one GPU
 *   (other streams, other threads, without ordering between them) race on the
 *   array and give undefined results: order them on one stream.
 * ------------------------------------------------------------------------ */
#define FT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ft_status ft_moe_ffn_noalloc(const ft_moe_weights* w, const void* x, ft_dtype act_dt, int T,
                             int k, const int32_t* perm, const int32_t* offsets,
                             const int32_t* slot_of_expert, void* y_perm, ft_dtype y_dt,
                             void* stream);

/* Kernel family used by ft_moe_ffn: 0 = choose by size (default),
 * 1 = weight-streaming (small token counts), 2 = MFMA tiles (large token
 * counts).  Process-wide; a tuning and test knob.  Returns the previous value. */
int ft_moe_ffn_set_path(int path);

/* Profiling hook: HIP events (hipEvent_t as void*) that time one stage, so
 * that a caller can read them with hipEventElapsedTime.  which: 0 = the FFN's
 * gate/up kernel (+SwiGLU), 1 = its down kernel, 2 = the whole ft_moe_ffn,
 * 3 = ft_moe_route, 4 = ft_moe_align, 5 = ft_moe_combine.  Stages 0 and 1 are
 * one kernel each and their events are attached to that kernel's dispatch
 * (hipExtLaunchKernel): they time the kernel itself and add no packet to the
 * stream.  The others are recorded on the launch stream right before / after
 * the stage's kernels (each such record can leave the GPU idle for a few
 * microseconds).  NULL events switch a stage off.  Process-wide setting, not
 * synchronised between threads; not applied while a graph is captured. */
ft_status ft_set_profile_events(int which, void* start, void* stop);

/* --------------------------------------------------------------------------
 * ft_moe_combine -- weighted combine back to token order.
 *   out[t] = sum_{j<k} topk_w[t][j] * y_perm[inv_perm[t*k + j]]
 *            (+ y_perm[T*k + t] when n_shared == 1)
 * summed in fp32 in increasing j, then the shared row, rounded once to
 * out_dt (FT_BF16 or FT_F32).  y_perm in y_dt (FT_BF16 or FT_F32).
 * All pointers device; out [T][H].
 * ------------------------------------------------------------------------ */
ft_status ft_moe_combine(const void* y_perm, ft_dtype y_dt, const int32_t* inv_perm,
                         const float* topk_w, int T, int k, int H, int n_shared, void* out,
                         ft_dtype out_dt, void* stream);

/* --------------------------------------------------------------------------
 * Whole-layer step and its graph.
 *
 * ft_moe_step_run enqueues one MoE-layer step on `stream`: ft_moe_route (from
 * x and w_router), ft_moe_align, ft_moe_ffn, ft_moe_combine, with the buffers
 * named in the descriptor; it returns the first failing call's status (the
 * calls before it stay enqueued).
 *
 * ft_moe_graph_create runs the step once eagerly on `stream` (checking every
 * argument), waits for it, then captures the same step on a private stream
 * into a HIP graph.  ft_moe_graph_launch replays it on any stream: the kernels
 * read and write the descriptor's buffers as they were at capture time, so a
 * caller refills x (and, with a slot cache, the slot table) in place between
 * replays.  The pages list graph-compatible execution among the runtime's
 * features (refft.com guide, "深度解析", the runtime feature list).  The
 * descriptor is copied; the buffers it names must outlive the graph.  Profile
 * events (ft_set_profile_events) are not captured.  Replays of one graph must
 * not overlap (they share every buffer).  Errors: FT_ERR_INVALID_ARG for a
 * NULL descriptor / graph, the step's own errors, FT_ERR_HIP when capture or
 * instantiation fails.
 * ------------------------------------------------------------------------ */
typedef struct {
    ft_moe_weights weights;
    const void* x;            /* [T][H] device, act_dt */
    ft_dtype act_dt;          /* FT_BF16 (FT_F32 with FT_F32 weights) */
    const void* w_router;     /* [E][H] device, act_dt */
    const float* bias;        /* [E] device or NULL */
    int T, k;
    const int32_t* slot_of_expert; /* [E] device or NULL (identity) */
    float* logits;            /* [T][E] device */
    int32_t* topk_ids;        /* [T][k] device */
    float* topk_w;            /* [T][k] device */
    int32_t* counts;          /* [E] device */
    int32_t* offsets;         /* [E+1] device */
    int32_t* perm;            /* [T*k] device */
    int32_t* inv_perm;        /* [T*k] device */
    void* align_ws;           /* >= ft_moe_align_workspace(T, k, E) bytes */
    size_t align_ws_bytes;
    void* y_perm;             /* [T*k + n_shared*T][H] device, y_dt */
    ft_dtype y_dt;
    void* ffn_ws;             /* >= ft_moe_ffn_workspace(&weights, T, k) bytes */
    size_t ffn_ws_bytes;
    void* out;                /* [T][H] device, out_dt */
    ft_dtype out_dt;
} ft_moe_step;

typedef struct ft_moe_graph ft_moe_graph;

ft_status ft_moe_step_run(const ft_moe_step* step, void* stream);
ft_status ft_moe_graph_create(const ft_moe_step* step, void* stream, ft_moe_graph** out);
ft_status ft_moe_graph_launch(ft_moe_graph* graph, void* stream);
ft_status ft_moe_graph_destroy(ft_moe_graph* graph);

/* --------------------------------------------------------------------------
 * Fused decode step: the whole layer in one kernel launch.
 *
 * ft_moe_step_fused enqueues the step of `step` as one kernel: router logits,
 * top-k gating (the rule of ft_moe_route), gate/up + SwiGLU, down projection
 * and the gated combine, with one grid-wide exchange after the logits and one
 * after h; the down weights are loaded while the exchange of h is pending.
 * The pages list graph-compatible execution among the runtime's features
 * (refft.com guide, "深度解析", the runtime feature list); the launch gaps
 * between the separate kernels are what this removes.
 *   Writes logits [T][E], topk_ids, topk_w (each token's picks and gates by
 *   the same rule as ft_moe_route, from these logits) and out [T][H]
 *   (out_dt FT_BF16 or FT_F32).  counts, offsets, perm, inv_perm, y_perm and
 *   the workspaces are neither read nor written (they may be NULL).
 *   out[t] = sum over the picks j (and the shared expert, gate 1) of
 *   topk_w[t][j] * (W_down h), each expert's down-projection row sum taken in
 *   fp32 and never rounded to y_dt; h is rounded to bf16 as in ft_moe_ffn.
 *   The sums run in another fixed order than the separate kernels', so the
 *   logits and out agree with ft_moe_step_run to rounding, not bit for bit;
 *   each is deterministic from run to run.
 *   slot_of_expert as in ft_moe_ffn; an expert whose entry is -1 (or -2 - j
 *   without a host pool) adds nothing to out.
 * Supported: bf16 weights and activations, 1 <= T <= 4, E <= 512,
 * T*k + n_shared*T <= 64, T*H and (T*k + n_shared*T)*I bf16 values of at
 * most 128 KiB each; other steps return FT_ERR_UNSUPPORTED before anything
 * is enqueued (T == 0 returns FT_OK and enqueues nothing).
 * The grid is one block per CU and every block waits for the others twice:
 * the device must have all its CUs free for the launch (another kernel that
 * never ends on the same device would hold blocks back; each wait gives up
 * after 0.1 s and is counted, see ft_moe_fused_timeouts).  The blocks
 * exchange data through a buffer of about 150 KiB per device, allocated
 * uncached on the first call on that device and held until the process ends;
 * that first call synchronises the device and must not be captured.  Fused
 * steps on one device must not overlap (they share that buffer); use one
 * stream, or order them.
 *
 * ft_moe_graph_create_fused is ft_moe_graph_create for the fused step: one
 * eager fused step, then the step captured as a graph of one kernel node,
 * replayed with ft_moe_graph_launch and freed with ft_moe_graph_destroy.
 *
 * ft_moe_fused_timeouts waits for the current device, returns in *count the
 * number of fused-step waits that gave up since the last call, and resets it.
 * ------------------------------------------------------------------------ */
ft_status ft_moe_step_fused(const ft_moe_step* step, void* stream);
ft_status ft_moe_graph_create_fused(const ft_moe_step* step, void* stream, ft_moe_graph** out);
ft_status ft_moe_fused_timeouts(int* count);

/* --------------------------------------------------------------------------
 * Expert slot cache.
 *
 * The full expert pool sits in pinned host memory; a fixed number of device
 * slots hold the working set under LRU replacement, counted in slots (refft.com
 * guide, "深度解析": global LRU expert caching; freelamp.com article, section
 * 2.3: the expert cache is sized in slots).  Missing experts are copied
 * host->device asynchronously on a copy stream; the next layer's misses are
 * copied while the current layer computes, which needs room for two whole
 * layers, else the overlap is reported as disabled (FreeToken hub article,
 * paragraph on prefill overlap and its WARNING).  Asynchronous copies need
 * pinned host memory (FreeToken hub article, install caveat on WSL).
 *
 * The library owns host metadata and HIP events only; the caller owns the
 * host pool and the device slot array.
 * ------------------------------------------------------------------------ */
typedef struct ft_slot_cache ft_slot_cache;

typedef enum { FT_SCOPE_GLOBAL = 0, FT_SCOPE_PER_LAYER = 1 } ft_slot_scope;

typedef struct {
    int n_layers;
    int n_experts;            /* experts per layer (routed + shared) */
    size_t expert_bytes;      /* bytes copied per expert */
    const void* host_pool;    /* pinned host memory, expert (l, e) at
                                 host_pool + (l * n_experts + e) * host_stride */
    size_t host_stride;       /* >= expert_bytes */
    void* dev_slots;          /* device memory, slot s at dev_slots + s * slot_stride */
    size_t slot_stride;       /* >= expert_bytes */
    int n_slots;              /* total device slots */
    int scope;                /* FT_SCOPE_GLOBAL: one LRU over all slots;
                                 FT_SCOPE_PER_LAYER: n_slots / n_layers per layer */
} ft_slot_cache_desc;

typedef struct {
    int n_demand;      /* distinct experts requested */
    int n_hit;         /* resident before the call (demand hits) */
    int n_prefetch_hit;/* resident or in flight because of a prefetch */
    int n_miss;        /* copied by this call */
    size_t bytes_h2d;  /* bytes enqueued by this call */
} ft_map_stats;

typedef struct {
    long long maps, demand, hits, prefetch_hits, misses, prefetch_issued, evictions;
    long long bytes_h2d;
    int resident, held, in_flight, n_slots;
} ft_cache_stats;

/* Create / destroy.  Fails with FT_ERR_NOT_PINNED when host_pool is not
 * pinned (page-locked) host memory, FT_ERR_INVALID_ARG on bad sizes. */
ft_status ft_slot_cache_create(const ft_slot_cache_desc* desc, ft_slot_cache** out);
ft_status ft_slot_cache_destroy(ft_slot_cache* c);

/* ft_slot_cache_map -- make layer `layer`'s experts `experts_host[0..n-1]`
 * (host int32, distinct, ascending) resident and write the device slot table
 * slot_table_dev[0..n_experts-1] (int32; -1 for experts not requested).
 * Hits are touched (most recent) and held until ft_slot_cache_release;
 * misses take free slots, else evict least-recently-used entries that are
 * neither held nor in flight, and are copied on `copy_stream`.  `compute`
 * waits (on the device) for every copy the table depends on, and the table is
 * written on `compute`.  FT_ERR_CAPACITY when the held set plus the request
 * exceeds the slots (nothing changes).  st may be NULL. */
ft_status ft_slot_cache_map(ft_slot_cache* c, int layer, const int32_t* experts_host, int n,
                            int32_t* slot_table_dev, void* compute, void* copy_stream,
                            ft_map_stats* st);

/* ft_slot_cache_release -- the work enqueued on `compute` so far is the last
 * reader of layer `layer`'s held slots: an event is recorded there and later
 * copies into those slots wait for it.  The entries become evictable. */
ft_status ft_slot_cache_release(ft_slot_cache* c, int layer, void* compute);

/* ft_slot_cache_prefetch -- start copying layer `layer`'s experts that are not
 * resident (host int32, distinct, ascending) on `copy_stream`, into free or
 * evictable slots, without holding them.  Entries of the layer being computed
 * are held and so are never victims.  When fewer than n slots can be
 * obtained, issues what fits and returns FT_WARN_OVERLAP_DISABLED.
 * n_issued (may be NULL) receives the number of copies started. */
ft_status ft_slot_cache_prefetch(ft_slot_cache* c, int layer, const int32_t* experts_host,
                                 int n, void* copy_stream, int* n_issued);

/* ft_slot_cache_evict -- drop (layer, expert) from the cache, or the whole
 * layer when expert == -1.  FT_ERR_BUSY (nothing dropped) if an entry is held
 * or its copy is in flight. */
ft_status ft_slot_cache_evict(ft_slot_cache* c, int layer, int expert);

/* ft_slot_cache_resize -- change the number of device slots at run time,
 * keeping what fits resident (no copy from the host pool): the pages describe
 * the expert cache being resized in slots while the engine runs, without a
 * restart or a reload of the weights (freelamp.com article, section 2.3;
 * refft.com guide, "深度解析").  Global scope only (FT_ERR_UNSUPPORTED for
 * per-layer caches); nothing may be held (FT_ERR_BUSY, nothing changes; also
 * when more than n_slots copies are in flight).
 *   Least-recently-used entries that no copy is filling are evicted until the
 *   residents fit.  Survivors keep their slot index when it is below n_slots;
 *   the others move to the lowest free slots below n_slots, by device-to-device
 *   copies on `copy_stream`.
 *   dev_slots: NULL or the current array to keep it (it must hold n_slots
 *   slots of slot_stride bytes), or a new device array of n_slots slots, into
 *   which every survivor is copied; free the old array only after
 *   `copy_stream` has passed this call's copies.
 * Slot tables written by earlier maps are stale afterwards: map again.  The
 * copies are ordered after each source slot's fill and each destination
 * slot's last reader; later maps make `compute` wait for them.  A failed copy
 * returns FT_ERR_HIP and leaves the cache empty at the new size. */
ft_status ft_slot_cache_resize(ft_slot_cache* c, int n_slots, void* dev_slots, void* copy_stream);

/* Counters since creation. */
ft_status ft_slot_cache_stats(const ft_slot_cache* c, ft_cache_stats* out);

/* --------------------------------------------------------------------------
 * ft_slot_stack_forward -- one pass through a stack of MoE layers whose
 * experts come through the cache, as one call (the per-layer host work runs
 * here rather than in the caller).  For each layer l in order: the routing
 * and alignment of layer l + 2 are enqueued first (a layer's input must not
 * depend on the outputs of the layers before it), then layer l's FFN, combine and
 * ft_slot_cache_release; then, once layer l + 1's expert counts have reached
 * the host, its missing experts are prefetched on `copy_stream` (every expert
 * of the layer when `prefill`) while layer l computes, and mapped into its
 * slot table.  The pages describe this double-buffered streaming of the next
 * layer's experts (claypier.com article, "按带宽决定分工的思路"; FreeToken hub
 * article, paragraph on prefill overlap).
 *   layers [n_layers]: one ft_moe_step per layer with its buffers; its
 *     weights.pool is the cache's device slot array, slot_of_expert that
 *     layer's device slot table (E + n_shared entries, written by the map),
 *     counts its device expert histogram; T >= 1; E and n_shared equal for all
 *     layers, E + n_shared == the cache's experts per layer; weights.shared_slot
 *     is ignored (looked up per layer).
 *   logits_in: NULL, or [n_layers] device fp32 logits per layer (NULL entries
 *     compute the router GEMM from x and w_router).
 *   counts_host: pinned host [n_layers][E] int32, written (the expert lists).
 * The host waits for each layer's counts: it polls a flag that the kernel
 * copying them sets (when counts_host has a device mapping), else
 * hipEventSynchronize; everything else is asynchronous on `compute` /
 * `copy_stream`.  Stops at the first failing call and returns its status
 * (earlier layers stay enqueued).  FT_WARN_OVERLAP_DISABLED from a prefetch
 * is counted, not returned.
 * stats (may be NULL): demand, hits, prefetch hits and misses of the maps,
 * H2D bytes enqueued, prefetch warnings.
 *
 * flags & FT_STACK_DEVICE_TABLE (decode; ignored with `prefill`, which runs
 * as above): the pass does not wait for the host.  The cache keeps a device
 * slot table [layers][E] that the FFN reads directly: an expert resident in a
 * slot (its copy landed) is read there, any other one straight from the
 * pinned host pool over the host link (ft_moe_weights.host_pool, table entry
 * -2 - (l * E + e)), so the pass's kernels are enqueued back to back and give
 * the same bits either way.  The LRU learns the pass's routing afterwards: a
 * small kernel copies every layer's counts into a ring of pinned buffers in
 * the cache and sets a flag, and a later call (or a flush) takes each
 * finished pass's experts through map and release in order, which copies
 * missed experts into slots on `copy_stream` (after the slot's last reader);
 * the table maps them once their copies have landed.  Stats of a call count
 * the passes it took through the LRU (the host runs at most one pass ahead of
 * that, FTMOE_DT_LAG = 0..3 in the environment changes it); a call with
 * n_layers == 0 only flushes (waits for and counts every pending pass).
 * Needs n_shared == 0, E <= 512, n_layers <= 64 and a device mapping of the
 * host pool; otherwise FT_ERR_UNSUPPORTED.  counts_host is not used. */
#define FT_STACK_DEVICE_TABLE 1
typedef struct {
    int n_layers;
    const ft_moe_step* layers;
    const float* const* logits_in;
    int32_t* counts_host;
    int prefill;
    int flags;  /* FT_STACK_DEVICE_TABLE or 0 */
} ft_stack_pass;

typedef struct {
    long long demand, hits, prefetch_hits, misses, bytes_h2d;
    int prefetch_warnings;
} ft_stack_stats;

ft_status ft_slot_stack_forward(ft_slot_cache* c, const ft_stack_pass* p, void* compute,
                                void* copy_stream, ft_stack_stats* stats);

/* Slot of (layer, expert), or -1 when not cached.  Host query, no device work. */
int ft_slot_cache_lookup(const ft_slot_cache* c, int layer, int expert);

/* --------------------------------------------------------------------------
 * Host expert FFN: the CPU side of the bandwidth-adaptive split of cache
 * misses.  The pages' hybrid backend sends part of a step's missed experts
 * over PCIe to the GPU and computes the rest on the CPU straight from host
 * memory, at the same time, in the ratio of the measured PCIe and host
 * bandwidths so that both finish together (chenxutan.com article, "瓶颈为什么是
 * 带宽而不是容量", the q* strategy and the MoE backend list; freelamp.com
 * article, section 2.1).  This call is that CPU share for one expert; the
 * split is the caller's (expert_ffn_execution_amd/stack.py).
 *   y[r] = W_down (bf16(silu(W_gate x[r]) * (W_up x[r]))) for r < T, fp32 sums,
 *   h rounded to bf16 as on the GPU.
 *   slot: host pointer to one expert slot (ft_expert_layout; FT_BF16 only);
 *   x [T][H] host, x_dt = FT_BF16; y [T][H] fp32 host; n_threads in [1, 256]
 *   host threads (a persistent pool; the caller's thread is one of them).
 * Synchronous; no device work.  Other weight or activation formats return
 * FT_ERR_INVALID_ARG. */
ft_status ft_host_expert_ffn(ft_dtype w_dt, int H, int I, const void* slot, const void* x,
                             ft_dtype x_dt, int T, float* y, int n_threads);

/* --------------------------------------------------------------------------
 * Host MoE FFN over a list of experts, asynchronous: the whole CPU share of
 * one layer's missed experts in one job, run on the library's host threads
 * while the caller goes on enqueueing GPU work (the same passages as
 * ft_host_expert_ffn: the CPU and the PCIe copies work at the same time).
 * For the listed experts in list order, and for each row j in
 * [offsets[e], offsets[e+1]) of expert e in the aligned order (token
 * t = perm[j] / k), with b counting the output rows up from 0:
 *   rows[b] = W_down_e bf16(silu(W_gate_e x[t]) * (W_up_e x[t])),  pos[b] = j,
 * the same arithmetic, and the same bits, as ft_host_expert_ffn.  The caller
 * moves rows[b] to row pos[b] of the layer's y_perm.
 * Descriptor (all pointers are host memory):
 *   w_dt = FT_BF16, x_dt = FT_BF16; E experts, H, I multiples of 64, top-k k;
 *   pool: expert e's slot at pool + e * slot_stride (ft_expert_layout);
 *   experts [n_experts] distinct, in [0, E);
 *   offsets [E+1] and perm [T*k] as ft_moe_align writes them;
 *   x [T][H]; rows [max_rows][H] fp32 and pos [max_rows] int64, written;
 *   n_threads in [1, 256].
 * ft_host_moe_ffn_submit checks the descriptor (FT_ERR_INVALID_ARG; offsets
 * and perm are read here, so they must be final; FT_ERR_CAPACITY when the
 * experts hold more than max_rows rows), copies it and the expert list,
 * queues the job and returns with *job set and *n_rows = the number of output
 * rows.  Jobs run one at a time, in submission order.  Every buffer the
 * descriptor names must stay as it is (rows, pos: unread) until
 * ft_host_job_wait(job) returns: it waits for the job, returns its status and
 * frees the handle; wait for every job exactly once.  No device work. */
typedef struct {
    ft_dtype w_dt;
    int E, H, I, k;
    const void* pool;
    size_t slot_stride;
    const int32_t* experts;
    int n_experts;
    const int32_t* offsets;
    const int32_t* perm;
    const void* x;
    ft_dtype x_dt;
    int T;
    float* rows;
    int64_t* pos;
    int max_rows;
    int n_threads;
} ft_host_moe_job_desc;

typedef struct ft_host_job_s ft_host_job;

ft_status ft_host_moe_ffn_submit(const ft_host_moe_job_desc* d, ft_host_job** job, int* n_rows);
ft_status ft_host_job_wait(ft_host_job* job);

/* --------------------------------------------------------------------------
 * ft_split_misses -- how many of a decode step's m missed experts to copy to
 * the GPU; the other m - n are computed on host cores (ft_host_moe_ffn_submit)
 * at the same time (chenxutan.com article, "瓶颈为什么是带宽而不是容量", the
 * q* strategy; freelamp.com article, section 2.1).  Copying n experts takes
 * n W / Bp and the host FFN of m - n takes (m - n) W / Bh; they overlap, so the
 * step waits for the slower.  The printed formula is garbled; balancing the
 * two sides gives n* = m Bp / (Bp + Bh), and of the integers on either side
 * the one that finishes sooner is returned (the lower one on a tie).
 *   bp: measured pinned host-to-device GB/s; bh: measured host FFN GB/s of
 *   expert weights.  bh <= 0 returns m, bp <= 0 returns 0, m <= 0 returns 0.
 * Host arithmetic only; never fails. */
int ft_split_misses(int m, double bp, double bh);

/* --------------------------------------------------------------------------
 * ft_moe_scatter_rows -- place expert output rows computed elsewhere (the
 * host's share of a hybrid decode step, ft_host_moe_ffn_submit) into y_perm:
 *   y_perm[pos[i]] = rows[i] for i < n, rounded to y_dt (FT_BF16: to nearest
 *   even; FT_F32: copied).
 * rows [n][H] fp32, pos [n] int64 (distinct rows of y_perm), y_perm
 * [..][H] in y_dt: all device memory; H % 8 == 0, rows and y_perm 16-byte
 * aligned.  Asynchronous on `stream`; n == 0 is a no-op. */
ft_status ft_moe_scatter_rows(const float* rows, const int64_t* pos, int n, int H, void* y_perm,
                              ft_dtype y_dt, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FTMOE_H */
