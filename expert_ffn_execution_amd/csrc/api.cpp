// api.cpp -- C entry points of libftmoe: argument checks and dispatch.
//
// Every check runs on the host before anything is enqueued; the kernels
// assume the shapes validated here (H and I multiples of 64, 16-byte aligned
// operands, 256-byte aligned slots).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>

#include "common.h"
#include "gemm_mfma.h"

namespace ft {

ft_status launch_topk(const float*, const float*, int, int, int, int32_t*, float*, hipStream_t);
ft_status launch_router_logits(const void*, ft_dtype, const void*, int, int, int, float*,
                               hipStream_t);
size_t align_workspace(int T, int k, int E);
ft_status launch_align(const int32_t*, int, int, int, int32_t*, int32_t*, int32_t*, int32_t*,
                       void*, hipStream_t);
ft_status launch_fill_i32(int32_t*, long, int32_t, hipStream_t);
ft_status launch_ffn_stream(const FfnGeom&, const void*, const int32_t*, const int32_t*,
                            const int32_t*, int, void*, void*, ft_dtype, hipStream_t);
ft_status launch_combine(const void*, ft_dtype, const int32_t*, const float*, int, int, int, int,
                         void*, ft_dtype, hipStream_t);
ft_status launch_scatter_rows(const float*, const int64_t*, int, int, void*, ft_dtype, hipStream_t);
bool topk_align_small_ok(int T, int k);
ft_status launch_topk_align_small(const float*, const float*, int, int, int, int32_t*, float*,
                                  int32_t*, int32_t*, int32_t*, int32_t*, hipStream_t);
bool fused_shape_ok(int T, int k, int E, int H, int I, int n_shared);
ft_status launch_fused_decode(const ft_moe_step* st, const size_t offs[3], hipStream_t s);

static thread_local char g_err[512] = "";

ft_status set_error(ft_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}
void clear_error() { g_err[0] = 0; }

static hipEvent_t g_prof[PROF_N][2];
// Set while this thread captures a step into a graph: the profiling events
// are then not recorded (they would become graph nodes).
static thread_local bool g_capturing = false;
void set_capturing(bool on) { g_capturing = on; }
void prof_begin(int which, hipStream_t s) {
    if (g_prof[which][0] && !g_capturing) (void)hipEventRecord(g_prof[which][0], s);
}
void prof_end(int which, hipStream_t s) {
    if (g_prof[which][1] && !g_capturing) (void)hipEventRecord(g_prof[which][1], s);
}
StageEvents prof_stage(int which) {
    if (g_capturing || !g_prof[which][0] || !g_prof[which][1]) return StageEvents{nullptr, nullptr};
    return StageEvents{g_prof[which][0], g_prof[which][1]};
}

static std::atomic<int> g_ffn_path{0};

}  // namespace ft

using namespace ft;

namespace {

constexpr int MAX_E = 1024;
constexpr int MFMA_MIN_ROWS = 32;  // average routed rows per active expert for MFMA tiles

bool valid_act(ft_dtype d) { return d == FT_F32 || d == FT_BF16; }

size_t layout(ft_dtype w, int H, int I, size_t offs[6]) {
    for (int i = 0; i < 6; ++i) offs[i] = 0;
    if (H <= 0 || I <= 0 || H % 64 || I % 64) return 0;
    const size_t HI = (size_t)H * I;
    if (w == FT_F32 || w == FT_BF16) {
        const size_t es = w == FT_F32 ? 4 : 2;
        offs[1] = HI * es;
        offs[2] = 2 * HI * es;
        return 3 * HI * es;
    }
    if (w == FT_FP8) {  // codes, then the three fp32 matrix scales
        offs[1] = HI;
        offs[2] = 2 * HI;
        offs[3] = 3 * HI;
        offs[4] = offs[3] + 4;
        offs[5] = offs[3] + 8;
        return offs[3] + 16;
    }
    if (w == FT_NVFP4) {  // codes, e4m3 block scales, then the three fp32 tensor scales
        offs[1] = HI / 2;
        offs[2] = HI;
        offs[3] = 3 * HI / 2;
        offs[4] = offs[3] + HI / 16;
        offs[5] = offs[4] + HI / 16;
        return offs[5] + HI / 16 + 16;
    }
    if (w == FT_MXFP4) {
        offs[1] = HI / 2;
        offs[2] = HI;
        offs[3] = HI * 3 / 2;
        offs[4] = offs[3] + HI / 32;
        offs[5] = offs[4] + HI / 32;
        return offs[5] + HI / 32;
    }
    return 0;
}

struct FfnPlan {
    size_t h_bytes, tiles_off, count_off, total;
    int max_tiles;
};

FfnPlan plan_ffn(const ft_moe_weights& w, int T, int k) {
    FfnPlan p{};
    const long tk = (long)T * k;
    const long hrows = tk + (long)w.n_shared * T;
    const size_t es = w.w_dt == FT_F32 ? 4 : 2;
    p.h_bytes = ((size_t)hrows * w.I * es + 255) & ~(size_t)255;
    const long act = tk < w.E ? tk : w.E;
    p.max_tiles = (int)((tk + GEMM_BM - 1) / GEMM_BM + act +
                        (w.n_shared ? (T + GEMM_BM - 1) / GEMM_BM : 0));
    if (p.max_tiles < 1) p.max_tiles = 1;
    p.tiles_off = p.h_bytes;
    p.count_off = p.tiles_off + (((size_t)p.max_tiles * sizeof(TileDesc) + 255) & ~(size_t)255);
    p.total = p.count_off + 256;
    return p;
}

ft_status check_weights(const ft_moe_weights* w) {
    FT_CHECK_ARG(w, "null weights");
    FT_CHECK_ARG(w->w_dt == FT_F32 || w->w_dt == FT_BF16 || w->w_dt == FT_MXFP4 || w->w_dt == FT_FP8 ||
                     w->w_dt == FT_NVFP4,
                 "bad w_dt");
    FT_CHECK_ARG(w->E >= 1 && w->E <= MAX_E, "E must be in [1, %d]", MAX_E);
    FT_CHECK_ARG(w->H > 0 && w->I > 0 && w->H % 64 == 0 && w->I % 64 == 0,
                 "H and I must be positive multiples of 64 (H=%d I=%d)", w->H, w->I);
    FT_CHECK_ARG(w->n_shared == 0 || w->n_shared == 1, "n_shared must be 0 or 1");
    size_t offs[6];
    const size_t need = layout(w->w_dt, w->H, w->I, offs);
    FT_CHECK_ARG(need > 0 && w->slot_stride >= need && w->slot_stride % 256 == 0,
                 "slot_stride %zu must be a multiple of 256 and >= %zu", w->slot_stride, need);
    FT_CHECK_ARG(w->pool && ((uintptr_t)w->pool & 255) == 0, "pool must be 256-byte aligned");
    FT_CHECK_ARG(!w->host_pool || (((uintptr_t)w->host_pool & 255) == 0 && w->host_stride >= need &&
                                   w->host_stride % 256 == 0),
                 "host_pool must be 256-byte aligned with host_stride a multiple of 256 and >= %zu",
                 need);
    FT_CHECK_ARG(!w->n_shared || w->shared_slot >= 0, "bad shared_slot");
    return FT_OK;
}

}  // namespace

extern "C" {

const char* ft_last_error(void) { return g_err; }
const char* ft_version(void) { return "ftmoe 0.1 gfx950"; }

ft_status ft_host_device_pointer(const void* host, void** dev) {
    clear_error();
    FT_CHECK_ARG(host && dev, "null host / dev");
    *dev = nullptr;
    // (the runtime only reads the host address; its signature is not const)
    if (hipHostGetDevicePointer(dev, const_cast<void*>(host), 0) != hipSuccess || !*dev) {
        (void)hipGetLastError();
        *dev = nullptr;
        return set_error(FT_ERR_UNSUPPORTED, "host address %p is not mapped for the current device", host);
    }
    return FT_OK;
}

int ft_moe_ffn_set_path(int path) { return g_ffn_path.exchange(path); }

// Profiling hook: hipEvent_t handles recorded on the launch stream right
// before / after the kernels named by `which` (0 GEMM1, 1 GEMM2, 2 whole FFN,
// 3 route, 4 align, 5 combine).  NULL clears.  Process-wide; not thread-safe.
ft_status ft_set_profile_events(int which, void* start, void* stop) {
    clear_error();
    FT_CHECK_ARG(which >= 0 && which < PROF_N, "bad profile slot");
    g_prof[which][0] = (hipEvent_t)start;
    g_prof[which][1] = (hipEvent_t)stop;
    return FT_OK;
}

size_t ft_expert_layout(ft_dtype w_dt, int H, int I, size_t offs[6]) {
    size_t tmp[6];
    return layout(w_dt, H, I, offs ? offs : tmp);
}

ft_status ft_moe_route(const void* x, ft_dtype x_dt, const void* w_router, const float* logits_in,
                       const float* bias, int T, int H, int E, int k, float* logits_out,
                       int32_t* topk_ids, float* topk_w, void* stream) {
    clear_error();
    FT_CHECK_ARG(T >= 0, "T must be >= 0");
    FT_CHECK_ARG(E >= 1 && E <= MAX_E, "E must be in [1, %d]", MAX_E);
    FT_CHECK_ARG(k >= 1 && k <= E, "k must be in [1, E]");
    FT_CHECK_ARG((long long)T * k < (1ll << 31), "T*k must be < 2^31");
    if (T == 0) return FT_OK;
    FT_CHECK_ARG(topk_ids && topk_w, "null outputs");
    hipStream_t s = (hipStream_t)stream;
    if (logits_in) {
        FT_CHECK_ARG(!x && !w_router, "give either logits_in or x and w_router, not both");
    } else {
        FT_CHECK_ARG(x && w_router && logits_out, "x, w_router and logits_out are required");
        FT_CHECK_ARG(valid_act(x_dt), "x_dt must be FT_F32 or FT_BF16");
        FT_CHECK_ARG(H > 0 && H % 64 == 0, "H must be a positive multiple of 64");
        FT_CHECK_ARG(aligned16(x) && aligned16(w_router), "x / w_router must be 16-byte aligned");
    }
    prof_begin(PROF_ROUTE, s);
    ft_status r = FT_OK;
    if (!logits_in) r = launch_router_logits(x, x_dt, w_router, T, H, E, logits_out, s);
    if (r == FT_OK)
        r = launch_topk(logits_in ? logits_in : logits_out, bias, T, E, k, topk_ids, topk_w, s);
    prof_end(PROF_ROUTE, s);
    return r;
}

size_t ft_moe_align_workspace(int T, int k, int E) {
    if (T <= 0 || k <= 0 || E <= 0) return 0;
    return align_workspace(T, k, E);
}

ft_status ft_moe_align(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* ws,
                       size_t ws_bytes, void* stream) {
    clear_error();
    FT_CHECK_ARG(T >= 0, "T must be >= 0");
    FT_CHECK_ARG(E >= 1 && E <= MAX_E, "E must be in [1, %d]", MAX_E);
    FT_CHECK_ARG(k >= 1 && k <= E, "k must be in [1, E]");
    FT_CHECK_ARG((long long)T * k < (1ll << 31), "T*k must be < 2^31");
    FT_CHECK_ARG(counts && offsets, "null counts/offsets");
    hipStream_t s = (hipStream_t)stream;
    if (T == 0) {
        // empty batch: all counts and offsets are zero (a fill kernel, not a
        // memset node, so that the call can sit inside a captured graph)
        ft_status r = launch_fill_i32(counts, E, 0, s);
        if (r == FT_OK) r = launch_fill_i32(offsets, E + 1, 0, s);
        return r;
    }
    FT_CHECK_ARG(topk_ids && perm && inv_perm, "null ids/perm/inv_perm");
    const size_t need = align_workspace(T, k, E);
    FT_CHECK_ARG(ws_bytes >= need && (need == 0 || ws), "workspace too small (%zu < %zu)",
                 ws_bytes, need);
    prof_begin(PROF_ALIGN, s);
    ft_status r = launch_align(topk_ids, T, k, E, counts, offsets, perm, inv_perm, ws, s);
    prof_end(PROF_ALIGN, s);
    return r;
}

size_t ft_moe_ffn_workspace(const ft_moe_weights* w, int T, int k) {
    if (!w || T < 0 || k < 1 || w->E < 1 || w->I < 1) return 0;
    return plan_ffn(*w, T, k).total;
}

ft_status ft_moe_ffn(const ft_moe_weights* w, const void* x, ft_dtype act_dt, int T, int k,
                     const int32_t* perm, const int32_t* offsets, const int32_t* slot_of_expert,
                     void* y_perm, ft_dtype y_dt, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    ft_status v = check_weights(w);
    if (v != FT_OK) return v;
    FT_CHECK_ARG(T >= 0, "T must be >= 0");
    FT_CHECK_ARG(k >= 1 && k <= w->E, "k must be in [1, E]");
    FT_CHECK_ARG((long long)T * k < (1ll << 31), "T*k must be < 2^31");
    if (T == 0) return FT_OK;
    FT_CHECK_ARG(x && perm && offsets && y_perm, "null x/perm/offsets/y_perm");
    FT_CHECK_ARG(aligned16(x) && aligned16(y_perm), "x and y_perm must be 16-byte aligned");
    if (w->w_dt == FT_F32) {
        FT_CHECK_ARG(act_dt == FT_F32 && y_dt == FT_F32, "fp32 weights take fp32 x and y");
    } else {
        FT_CHECK_ARG(act_dt == FT_BF16, "bf16/MXFP4/FP8/NVFP4 weights take bf16 activations");
        FT_CHECK_ARG(y_dt == FT_BF16 || y_dt == FT_F32, "y_dt must be FT_BF16 or FT_F32");
    }
    {
        // The kernels address an activation row (x for gate/up, h for down)
        // with a 32-bit element offset and a weight row inside a slot with a
        // 32-bit byte offset: refuse shapes past either range.
        const uint64_t hrows = (uint64_t)T * k + (uint64_t)w->n_shared * T;
        size_t offs[6];
        const uint64_t slot_bytes = layout(w->w_dt, w->H, w->I, offs);
        if ((uint64_t)T * w->H >= (1ull << 32) || hrows * w->I >= (1ull << 32) ||
            slot_bytes >= (1ull << 32))
            return set_error(FT_ERR_UNSUPPORTED,
                             "shape beyond 32-bit offsets: T*H = %llu, (T*k + n_shared*T)*I = %llu, "
                             "expert bytes = %llu (each must be < 2^32)",
                             (unsigned long long)T * w->H, (unsigned long long)(hrows * w->I),
                             (unsigned long long)slot_bytes);
    }
    const FfnPlan p = plan_ffn(*w, T, k);
    FT_CHECK_ARG(ws && ws_bytes >= p.total && ((uintptr_t)ws & 255) == 0,
                 "workspace must be 256-byte aligned and >= %zu bytes", p.total);
    hipStream_t s = (hipStream_t)stream;

    FfnGeom g;
    g.E = w->E;
    g.H = w->H;
    g.I = w->I;
    g.k = k;
    g.T = T;
    g.n_shared = w->n_shared;
    g.w_dt = w->w_dt;
    g.pool = (const uint8_t*)w->pool;
    g.slot_stride = w->slot_stride;
    g.host_pool = (const uint8_t*)w->host_pool;
    g.host_stride = w->host_stride;
    layout(w->w_dt, w->H, w->I, g.off);
    for (int m = 0; m < 3; ++m)  // NVFP4 tensor scales follow the down block scales
        g.toff[m] = g.off[5] + (size_t)w->H * w->I / 16 + 4 * (size_t)m;

    const long tk = (long)T * k;
    const long act = tk < w->E ? tk : w->E;
    int path = g_ffn_path.load();
    if (path == 0) path = (w->w_dt != FT_F32 && tk >= (long)MFMA_MIN_ROWS * act) ? 2 : 1;
    if (path == 2 && w->w_dt == FT_F32) path = 1;  // no fp32 MFMA tiles: fp32 is the tiny case

    char* wsb = (char*)ws;
    void* h = wsb;
    prof_begin(PROF_FFN, s);
    ft_status r;
    if (path == 1) {
        r = launch_ffn_stream(g, x, perm, offsets, slot_of_expert, w->shared_slot, h, y_perm, y_dt, s);
    } else {
        TileDesc* tiles = (TileDesc*)(wsb + p.tiles_off);
        int* n_tiles = (int*)(wsb + p.count_off);
        r = launch_build_tiles(g, offsets, slot_of_expert, w->shared_slot, tiles, n_tiles,
                               p.max_tiles, s);
        if (r == FT_OK)
            r = launch_gemm1_mfma(g, (const __bf16*)x, perm, tiles, n_tiles, p.max_tiles,
                                  (__bf16*)h, s);
        if (r == FT_OK)
            r = launch_gemm2_mfma(g, (const __bf16*)h, tiles, n_tiles, p.max_tiles, y_perm, y_dt, s);
    }
    prof_end(PROF_FFN, s);
    return r;
}

ft_status ft_moe_combine(const void* y_perm, ft_dtype y_dt, const int32_t* inv_perm,
                         const float* topk_w, int T, int k, int H, int n_shared, void* out,
                         ft_dtype out_dt, void* stream) {
    clear_error();
    FT_CHECK_ARG(T >= 0 && k >= 1 && H > 0 && H % 8 == 0, "bad T/k/H (H must be a multiple of 8)");
    FT_CHECK_ARG(n_shared == 0 || n_shared == 1, "n_shared must be 0 or 1");
    FT_CHECK_ARG(valid_act(y_dt) && valid_act(out_dt), "y_dt/out_dt must be FT_F32 or FT_BF16");
    FT_CHECK_ARG((long long)T * k < (1ll << 31), "T*k must be < 2^31");
    if (T == 0) return FT_OK;
    FT_CHECK_ARG(y_perm && inv_perm && topk_w && out, "null pointer");
    FT_CHECK_ARG(aligned16(y_perm) && aligned16(out), "y_perm/out must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    prof_begin(PROF_COMBINE, s);
    ft_status r = launch_combine(y_perm, y_dt, inv_perm, topk_w, T, k, H, n_shared, out, out_dt, s);
    prof_end(PROF_COMBINE, s);
    return r;
}

ft_status ft_moe_scatter_rows(const float* rows, const int64_t* pos, int n, int H, void* y_perm,
                              ft_dtype y_dt, void* stream) {
    clear_error();
    FT_CHECK_ARG(n >= 0 && H > 0 && H % 8 == 0, "bad n/H (H must be a multiple of 8)");
    FT_CHECK_ARG(y_dt == FT_BF16 || y_dt == FT_F32, "y_dt must be FT_BF16 or FT_F32");
    if (n == 0) return FT_OK;
    FT_CHECK_ARG(rows && pos && y_perm, "null pointer");
    FT_CHECK_ARG(aligned16(rows) && aligned16(y_perm), "rows / y_perm must be 16-byte aligned");
    return launch_scatter_rows(rows, pos, n, H, y_perm, y_dt, (hipStream_t)stream);
}

}  // extern "C"

namespace ft {

// Route and align of a whole-layer step.  A decode-sized batch runs the
// router logits, then top-k and alignment fused in one launch (same picks,
// gates, counts, offsets and permutation as ft_moe_route + ft_moe_align, whose
// argument checks are repeated here); larger batches call the two entry points.
ft_status route_align(const ft_moe_step* st, hipStream_t s) {
    const int T = st->T, E = st->weights.E, k = st->k, H = st->weights.H;
    if (!topk_align_small_ok(T, k) || E < 1 || E > MAX_E || k < 1 || k > E) {  // (their checks reject bad E, k)
        ft_status r = ft_moe_route(st->x, st->act_dt, st->w_router, nullptr, st->bias, T, H, E, k,
                                   st->logits, st->topk_ids, st->topk_w, s);
        if (r != FT_OK) return r;
        return ft_moe_align(st->topk_ids, T, k, E, st->counts, st->offsets, st->perm, st->inv_perm,
                            st->align_ws, st->align_ws_bytes, s);
    }
    clear_error();
    FT_CHECK_ARG(st->topk_ids && st->topk_w, "null outputs");
    FT_CHECK_ARG(st->x && st->w_router && st->logits, "x, w_router and logits_out are required");
    FT_CHECK_ARG(valid_act(st->act_dt), "x_dt must be FT_F32 or FT_BF16");
    FT_CHECK_ARG(H > 0 && H % 64 == 0, "H must be a positive multiple of 64");
    FT_CHECK_ARG(aligned16(st->x) && aligned16(st->w_router), "x / w_router must be 16-byte aligned");
    FT_CHECK_ARG(st->counts && st->offsets, "null counts/offsets");
    FT_CHECK_ARG(st->perm && st->inv_perm, "null ids/perm/inv_perm");
    prof_begin(PROF_ROUTE, s);
    ft_status r = launch_router_logits(st->x, st->act_dt, st->w_router, T, H, E, st->logits, s);
    if (r == FT_OK)
        r = launch_topk_align_small(st->logits, st->bias, T, E, k, st->topk_ids, st->topk_w,
                                    st->counts, st->offsets, st->perm, st->inv_perm, s);
    prof_end(PROF_ROUTE, s);
    return r;
}

// Checks of the fused decode step (ft_moe_step_fused), then its launch.
ft_status fused_step(const ft_moe_step* st, hipStream_t s) {
    clear_error();
    FT_CHECK_ARG(st, "null step");
    const ft_moe_weights& w = st->weights;
    ft_status v = check_weights(&w);
    if (v != FT_OK) return v;
    FT_CHECK_ARG(st->T >= 0, "T must be >= 0");
    FT_CHECK_ARG(st->k >= 1 && st->k <= w.E, "k must be in [1, E]");
    if (w.w_dt != FT_BF16 || st->act_dt != FT_BF16)
        return set_error(FT_ERR_UNSUPPORTED, "the fused step takes bf16 weights and activations");
    if (!fused_shape_ok(st->T > 0 ? st->T : 1, st->k, w.E, w.H, w.I, w.n_shared))
        return set_error(FT_ERR_UNSUPPORTED,
                         "the fused step takes T <= 4, E <= 512, T*k + n_shared*T <= 64, T*H and "
                         "(T*k + n_shared*T)*I bf16 values within 128 KiB (T=%d k=%d E=%d H=%d I=%d)",
                         st->T, st->k, w.E, w.H, w.I);
    if (st->T == 0) return FT_OK;
    FT_CHECK_ARG(st->x && st->w_router && st->logits && st->topk_ids && st->topk_w && st->out,
                 "x, w_router, logits, topk_ids, topk_w and out are required");
    FT_CHECK_ARG(aligned16(st->x) && aligned16(st->w_router), "x / w_router must be 16-byte aligned");
    FT_CHECK_ARG(st->out_dt == FT_BF16 || st->out_dt == FT_F32, "out_dt must be FT_BF16 or FT_F32");
    size_t offs[6];
    layout(w.w_dt, w.H, w.I, offs);
    return launch_fused_decode(st, offs, s);
}

}  // namespace ft
