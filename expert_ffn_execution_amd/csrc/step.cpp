// step.cpp -- one whole MoE-layer step (route -> align -> ffn -> combine) as a
// single call, and the same step captured once into a HIP graph.
//
// At decode the step is a handful of small kernels, and the host time to
// enqueue them (argument checks, launch calls) and the gaps between them
// exceed the FFN's own few microseconds.  The pages list graph-compatible
// execution among the runtime's features (refft.com guide, "深度解析", the
// runtime feature list); here a step is captured on a private stream into a
// hipGraph whose replay enqueues every kernel with one call.  Nothing in the
// step allocates, synchronises or writes memset nodes (empty inputs are
// cleared by a fill kernel), so the captured graph holds kernel nodes only.
#include <hip/hip_runtime.h>

#include "common.h"

namespace ft {
void set_capturing(bool on);
ft_status route_align(const ft_moe_step* st, hipStream_t s);
ft_status fused_step(const ft_moe_step* st, hipStream_t s);
ft_status fused_timeouts(int* count);
}

using namespace ft;

struct ft_moe_graph {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

namespace {

ft_status run_step(const ft_moe_step* st, void* stream) {
    // route + align (top-k and alignment in one launch for decode-sized batches)
    ft_status r = route_align(st, (hipStream_t)stream);
    if (r != FT_OK) return r;
    r = ft_moe_ffn(&st->weights, st->x, st->act_dt, st->T, st->k, st->perm, st->offsets,
                   st->slot_of_expert, st->y_perm, st->y_dt, st->ffn_ws, st->ffn_ws_bytes, stream);
    if (r != FT_OK) return r;
    return ft_moe_combine(st->y_perm, st->y_dt, st->inv_perm, st->topk_w, st->T, st->k,
                          st->weights.H, st->weights.n_shared, st->out, st->out_dt, stream);
}

ft_status run_fused(const ft_moe_step* st, void* stream) { return fused_step(st, (hipStream_t)stream); }

// Runs `run` once eagerly on `stream` (every argument check, first-use set-up
// outside the capture), waits, then captures it on a private stream.
ft_status create_graph(const ft_moe_step* st, void* stream, ft_moe_graph** out,
                       ft_status (*run)(const ft_moe_step*, void*)) {
    *out = nullptr;
    ft_status r = run(st, stream);
    if (r != FT_OK) return r;
    FT_HIP(hipStreamSynchronize((hipStream_t)stream));

    hipStream_t cap = nullptr;
    FT_HIP(hipStreamCreateWithFlags(&cap, hipStreamNonBlocking));
    ft_moe_graph* g = new ft_moe_graph;
    hipError_t e = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
        set_capturing(true);  // profile events stay out of the graph
        r = run(st, cap);
        set_capturing(false);
        e = hipStreamEndCapture(cap, &g->graph);
    }
    if (e == hipSuccess && r == FT_OK) e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0);
    (void)hipStreamDestroy(cap);
    if (r != FT_OK || e != hipSuccess) {
        if (g->exec) (void)hipGraphExecDestroy(g->exec);
        if (g->graph) (void)hipGraphDestroy(g->graph);
        delete g;
        if (r != FT_OK) return r;
        return set_error(FT_ERR_HIP, "graph capture failed: %s", hipGetErrorString(e));
    }
    *out = g;
    return FT_OK;
}

}  // namespace

extern "C" {

ft_status ft_moe_step_run(const ft_moe_step* st, void* stream) {
    clear_error();
    FT_CHECK_ARG(st, "null step");
    return run_step(st, stream);
}

ft_status ft_moe_graph_create(const ft_moe_step* st, void* stream, ft_moe_graph** out) {
    clear_error();
    FT_CHECK_ARG(st && out, "null step / out");
    return create_graph(st, stream, out, run_step);
}

ft_status ft_moe_step_fused(const ft_moe_step* st, void* stream) {
    return fused_step(st, (hipStream_t)stream);
}

ft_status ft_moe_graph_create_fused(const ft_moe_step* st, void* stream, ft_moe_graph** out) {
    clear_error();
    FT_CHECK_ARG(st && out, "null step / out");
    return create_graph(st, stream, out, run_fused);
}

ft_status ft_moe_fused_timeouts(int* count) {
    clear_error();
    FT_CHECK_ARG(count, "null count");
    *count = 0;
    return fused_timeouts(count);
}

ft_status ft_moe_graph_launch(ft_moe_graph* g, void* stream) {
    clear_error();
    FT_CHECK_ARG(g && g->exec, "null graph");
    FT_HIP(hipGraphLaunch(g->exec, (hipStream_t)stream));
    return FT_OK;
}

ft_status ft_moe_graph_destroy(ft_moe_graph* g) {
    clear_error();
    if (!g) return FT_OK;
    ft_status r = FT_OK;
    if (g->exec && hipGraphExecDestroy(g->exec) != hipSuccess) r = FT_ERR_HIP;
    if (g->graph && hipGraphDestroy(g->graph) != hipSuccess) r = FT_ERR_HIP;
    delete g;
    if (r != FT_OK) return set_error(r, "graph destroy failed");
    return FT_OK;
}

}  // extern "C"
