// slot_cache.cpp -- HIP copy engine and C entry points of the expert-slot cache.
//
// Copies run as hipMemcpyAsync from the pinned host pool on the caller's copy
// stream; each slot has a "filled" event (recorded after its copy) and a
// "read" event (recorded on the compute stream when the layer that used it is
// released).  A copy into a slot first waits for the slot's read event, and
// the compute stream waits for the filled events of the slots a layer maps:
// the next layer's weights travel while the current layer computes, with no
// host synchronisation (FreeToken hub article, paragraph on prefill overlap;
// claypier.com article, "按带宽决定分工的思路": whole-layer double-buffered
// streaming).  Asynchronous copies need page-locked host memory, so a pageable
// pool is refused (FreeToken hub article, install caveat on WSL).
#include <hip/hip_runtime.h>

#include <cstring>
#include <new>
#include <vector>

#include "common.h"
#include "slot_policy.h"

struct ft_slot_cache {
    ft_slot_cache_desc d;
    ftp::Policy policy;
    std::vector<hipEvent_t> filled, read;
    std::vector<char> read_valid;
    // pinned staging ring for slot-table uploads
    int32_t* stage = nullptr;
    std::vector<hipEvent_t> stage_ev;
    std::vector<char> stage_used;
    int ring = 0, ring_pos = 0;

    explicit ft_slot_cache(const ft_slot_cache_desc& dd)
        : d(dd), policy(dd.n_layers, dd.n_experts, dd.n_slots, dd.scope, dd.expert_bytes) {}
};

namespace {

struct HipEngine final : ftp::Engine {
    ft_slot_cache* c;
    hipStream_t compute, copy_s;
    hipError_t err = hipSuccess;
    HipEngine(ft_slot_cache* cc, hipStream_t comp, hipStream_t cp) : c(cc), compute(comp), copy_s(cp) {}

    bool ok(hipError_t e) {
        if (e != hipSuccess && err == hipSuccess) err = e;
        return e == hipSuccess;
    }
    bool copy(int slot, int layer, int expert) override {
        if (c->read_valid[slot] && !ok(hipStreamWaitEvent(copy_s, c->read[slot], 0))) return false;
        const char* src = (const char*)c->d.host_pool +
                          ((size_t)layer * c->d.n_experts + expert) * c->d.host_stride;
        char* dst = (char*)c->d.dev_slots + (size_t)slot * c->d.slot_stride;
        if (!ok(hipMemcpyAsync(dst, src, c->d.expert_bytes, hipMemcpyHostToDevice, copy_s)))
            return false;
        return ok(hipEventRecord(c->filled[slot], copy_s));
    }
    bool copy_done(int slot) override {
        hipError_t e = hipEventQuery(c->filled[slot]);
        if (e == hipErrorNotReady) return false;
        return ok(e);
    }
    bool compute_wait(int slot) override {
        return ok(hipStreamWaitEvent(compute, c->filled[slot], 0));
    }
    bool record_read(int slot) override {
        if (!ok(hipEventRecord(c->read[slot], compute))) return false;
        c->read_valid[slot] = 1;
        return true;
    }
    bool move(int, int) override { return false; }  // only ResizeEngine moves slots
};

// Engine of a resize: moves copy slot src of the current array into slot dst
// of the (possibly new) array on the copy stream, ordered after src's fill and
// dst's last reader; dst's fill event (of the new event set) marks completion.
struct ResizeEngine final : ftp::Engine {
    ft_slot_cache* c;
    hipStream_t copy_s;
    char* dst_base;
    std::vector<hipEvent_t>& filled_new;
    std::vector<hipEvent_t>& read_new;
    std::vector<char>& read_valid_new;
    hipError_t err = hipSuccess;
    ResizeEngine(ft_slot_cache* cc, hipStream_t cp, char* base, std::vector<hipEvent_t>& f,
                 std::vector<hipEvent_t>& r, std::vector<char>& rv)
        : c(cc), copy_s(cp), dst_base(base), filled_new(f), read_new(r), read_valid_new(rv) {}
    bool ok(hipError_t e) {
        if (e != hipSuccess && err == hipSuccess) err = e;
        return e == hipSuccess;
    }
    bool copy(int, int, int) override { return false; }
    bool copy_done(int slot) override {
        hipError_t e = hipEventQuery(c->filled[slot]);
        if (e == hipErrorNotReady) return false;
        return ok(e);
    }
    bool compute_wait(int) override { return false; }
    bool record_read(int) override { return false; }
    bool move(int src, int dst) override {
        if (!ok(hipStreamWaitEvent(copy_s, c->filled[src], 0))) return false;
        if (read_valid_new[dst] && !ok(hipStreamWaitEvent(copy_s, read_new[dst], 0))) return false;
        const char* from = (const char*)c->d.dev_slots + (size_t)src * c->d.slot_stride;
        char* to = dst_base + (size_t)dst * c->d.slot_stride;
        if (!ok(hipMemcpyAsync(to, from, c->d.expert_bytes, hipMemcpyDeviceToDevice, copy_s)))
            return false;
        return ok(hipEventRecord(filled_new[dst], copy_s));
    }
};

ft_status hip_status(hipError_t err, ft_status st) {
    if (err != hipSuccess)
        return ft::set_error(FT_ERR_HIP, "slot cache: %s", hipGetErrorString(err));
    if (st == FT_ERR_CAPACITY)
        return ft::set_error(st, "slot cache: held slots plus this request exceed capacity");
    if (st == FT_ERR_INVALID_ARG)
        return ft::set_error(st, "slot cache: bad layer/expert list (ids must be distinct, ascending, in range)");
    if (st == FT_ERR_BUSY)
        return ft::set_error(st, "slot cache: entry is held or its copy is in flight");
    if (st == FT_WARN_OVERLAP_DISABLED)
        return ft::set_error(st,
                             "Disabling MoE prefetch overlap: the slot cache cannot hold the "
                             "next layer's experts beside the held ones");
    if (st == FT_ERR_UNSUPPORTED)
        return ft::set_error(st, "slot cache: resizing needs the global scope");
    return st;
}
ft_status hip_status(const HipEngine& eng, ft_status st) { return hip_status(eng.err, st); }

hipError_t make_event(hipEvent_t* e) { return hipEventCreateWithFlags(e, hipEventDisableTiming); }

}  // namespace

extern "C" {

ft_status ft_slot_cache_create(const ft_slot_cache_desc* desc, ft_slot_cache** out) {
    ft::clear_error();
    FT_CHECK_ARG(desc && out, "null desc/out");
    const ft_slot_cache_desc& d = *desc;
    FT_CHECK_ARG(d.n_layers > 0 && d.n_experts > 0 && d.n_slots > 0, "sizes must be positive");
    FT_CHECK_ARG(d.expert_bytes > 0 && d.host_stride >= d.expert_bytes &&
                     d.slot_stride >= d.expert_bytes,
                 "strides must cover expert_bytes");
    FT_CHECK_ARG(d.host_pool && d.dev_slots, "null pool");
    FT_CHECK_ARG(d.scope == FT_SCOPE_GLOBAL || d.scope == FT_SCOPE_PER_LAYER, "bad scope");
    FT_CHECK_ARG(d.scope == FT_SCOPE_GLOBAL || d.n_slots % d.n_layers == 0,
                 "per-layer scope needs n_slots divisible by n_layers");
    hipPointerAttribute_t attr;
    hipError_t pe = hipPointerGetAttributes(&attr, d.host_pool);
    if (pe != hipSuccess || attr.type != hipMemoryTypeHost) {
        (void)hipGetLastError();
        return ft::set_error(FT_ERR_NOT_PINNED,
                             "host_pool is not page-locked host memory; asynchronous copies "
                             "(and the overlap) need pinned memory");
    }
    ft_slot_cache* c = new (std::nothrow) ft_slot_cache(d);
    if (!c) return ft::set_error(FT_ERR_CAPACITY, "out of host memory");
    c->filled.resize(d.n_slots);
    c->read.resize(d.n_slots);
    c->read_valid.assign(d.n_slots, 0);
    for (int s = 0; s < d.n_slots; ++s) {
        if (hipEventCreateWithFlags(&c->filled[s], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&c->read[s], hipEventDisableTiming) != hipSuccess) {
            ft_slot_cache_destroy(c);
            return ft::set_error(FT_ERR_HIP, "hipEventCreate failed");
        }
    }
    c->ring = 8;
    if (hipHostMalloc((void**)&c->stage, sizeof(int32_t) * (size_t)d.n_experts * c->ring,
                      hipHostMallocDefault) != hipSuccess) {
        c->stage = nullptr;
        ft_slot_cache_destroy(c);
        return ft::set_error(FT_ERR_HIP, "hipHostMalloc of the slot-table staging ring failed");
    }
    c->stage_ev.resize(c->ring);
    c->stage_used.assign(c->ring, 0);
    for (int i = 0; i < c->ring; ++i)
        if (hipEventCreateWithFlags(&c->stage_ev[i], hipEventDisableTiming) != hipSuccess) {
            ft_slot_cache_destroy(c);
            return ft::set_error(FT_ERR_HIP, "hipEventCreate failed");
        }
    *out = c;
    return FT_OK;
}

ft_status ft_slot_cache_destroy(ft_slot_cache* c) {
    if (!c) return FT_OK;
    for (hipEvent_t e : c->filled)
        if (e) (void)hipEventSynchronize(e), (void)hipEventDestroy(e);
    for (hipEvent_t e : c->read)
        if (e) (void)hipEventSynchronize(e), (void)hipEventDestroy(e);
    for (hipEvent_t e : c->stage_ev)
        if (e) (void)hipEventSynchronize(e), (void)hipEventDestroy(e);
    if (c->stage) (void)hipHostFree(c->stage);
    delete c;
    return FT_OK;
}

ft_status ft_slot_cache_map(ft_slot_cache* c, int layer, const int32_t* experts_host, int n,
                            int32_t* slot_table_dev, void* compute, void* copy_stream,
                            ft_map_stats* st) {
    ft::clear_error();
    FT_CHECK_ARG(c && slot_table_dev, "null cache/slot table");
    HipEngine eng(c, (hipStream_t)compute, (hipStream_t)copy_stream);
    std::vector<int32_t> slot_of((size_t)(n > 0 ? n : 1));
    ft_status r = c->policy.map(eng, layer, experts_host, n, slot_of.data(), st);
    if (r != FT_OK) return hip_status(eng, r);
    // slot table through the pinned staging ring
    const int i = c->ring_pos;
    c->ring_pos = (c->ring_pos + 1) % c->ring;
    if (c->stage_used[i]) FT_HIP(hipEventSynchronize(c->stage_ev[i]));
    int32_t* tab = c->stage + (size_t)i * c->d.n_experts;
    for (int e = 0; e < c->d.n_experts; ++e) tab[e] = -1;
    for (int q = 0; q < n; ++q) tab[experts_host[q]] = slot_of[q];
    FT_HIP(hipMemcpyAsync(slot_table_dev, tab, sizeof(int32_t) * c->d.n_experts,
                          hipMemcpyHostToDevice, (hipStream_t)compute));
    FT_HIP(hipEventRecord(c->stage_ev[i], (hipStream_t)compute));
    c->stage_used[i] = 1;
    return FT_OK;
}

ft_status ft_slot_cache_release(ft_slot_cache* c, int layer, void* compute) {
    ft::clear_error();
    FT_CHECK_ARG(c, "null cache");
    HipEngine eng(c, (hipStream_t)compute, nullptr);
    return hip_status(eng, c->policy.release(eng, layer));
}

ft_status ft_slot_cache_prefetch(ft_slot_cache* c, int layer, const int32_t* experts_host, int n,
                                 void* copy_stream, int* n_issued) {
    ft::clear_error();
    FT_CHECK_ARG(c, "null cache");
    HipEngine eng(c, nullptr, (hipStream_t)copy_stream);
    return hip_status(eng, c->policy.prefetch(eng, layer, experts_host, n, n_issued));
}

ft_status ft_slot_cache_evict(ft_slot_cache* c, int layer, int expert) {
    ft::clear_error();
    FT_CHECK_ARG(c, "null cache");
    HipEngine eng(c, nullptr, nullptr);
    return hip_status(eng, c->policy.evict(eng, layer, expert));
}

ft_status ft_slot_cache_stats(const ft_slot_cache* c, ft_cache_stats* out) {
    ft::clear_error();
    FT_CHECK_ARG(c && out, "null cache/out");
    *out = c->policy.stats();
    return FT_OK;
}

ft_status ft_slot_cache_resize(ft_slot_cache* c, int n_slots, void* dev_slots, void* copy_stream) {
    ft::clear_error();
    FT_CHECK_ARG(c && n_slots > 0, "null cache or n_slots <= 0");
    const int old_n = c->d.n_slots;
    const bool moved = dev_slots && dev_slots != c->d.dev_slots;
    // the event set of the new size: slots below min(old, new) keep theirs
    std::vector<hipEvent_t> filled(n_slots, nullptr), read(n_slots, nullptr);
    std::vector<char> read_valid(n_slots, 0);
    for (int s = 0; s < n_slots; ++s) {
        if (s < old_n) {
            filled[s] = c->filled[s];
            read[s] = c->read[s];
            read_valid[s] = c->read_valid[s];
        } else if (make_event(&filled[s]) != hipSuccess || make_event(&read[s]) != hipSuccess) {
            for (int q = old_n; q <= s; ++q) {
                if (filled[q]) (void)hipEventDestroy(filled[q]);
                if (read[q]) (void)hipEventDestroy(read[q]);
            }
            return ft::set_error(FT_ERR_HIP, "hipEventCreate failed");
        }
    }
    char* base = (char*)(moved ? dev_slots : c->d.dev_slots);
    ResizeEngine eng(c, (hipStream_t)copy_stream, base, filled, read, read_valid);
    const ft_status r = c->policy.resize(eng, n_slots, moved);
    if (r != FT_OK && r != FT_ERR_HIP) {  // nothing changed
        for (int s = old_n; s < n_slots; ++s) (void)hipEventDestroy(filled[s]), (void)hipEventDestroy(read[s]);
        return hip_status(eng.err, r);
    }
    // the policy now has n_slots slots: retire the events of dropped slots
    // (after the work they mark) and switch to the new set and array
    for (int s = n_slots; s < old_n; ++s) {
        (void)hipEventSynchronize(c->filled[s]), (void)hipEventDestroy(c->filled[s]);
        (void)hipEventSynchronize(c->read[s]), (void)hipEventDestroy(c->read[s]);
    }
    c->filled.swap(filled);
    c->read.swap(read);
    c->read_valid.swap(read_valid);
    c->d.n_slots = n_slots;
    c->d.dev_slots = base;
    return hip_status(eng.err, r);
}

int ft_slot_cache_lookup(const ft_slot_cache* c, int layer, int expert) {
    return c ? c->policy.lookup(layer, expert) : -1;
}

}  // extern "C"
