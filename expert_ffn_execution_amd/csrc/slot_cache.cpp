// slot_cache.cpp -- HIP copy engine and C entry points of the expert-slot cache.
//
// Copies run as hipMemcpyAsync from the pinned host pool on the caller's copy
// stream; each slot has a "filled" event (recorded after its copy) and refers
// to a "read" event recorded on the compute stream when the layer that used it
// is released (one event per release, shared by that layer's slots, from a
// small pool; a slot keeps the generation it saw, and once the pool has
// recorded that event again the copy waits for the newer point, which comes
// later on the same stream).  A copy into a slot first waits for that event, and
// the compute stream waits for the filled events of the slots a layer maps:
// the next layer's weights travel while the current layer computes, with no
// host synchronisation (FreeToken hub article, paragraph on prefill overlap;
// claypier.com article, "按带宽决定分工的思路": whole-layer double-buffered
// streaming).  Asynchronous copies need page-locked host memory, so a pageable
// pool is refused (FreeToken hub article, install caveat on WSL).
//
// Device-table passes (FT_STACK_DEVICE_TABLE) turn the order around for
// decode: the FFN reads a device slot table that maps each expert either to
// its slot (once the copy into it has landed) or to the pinned host pool, so a
// whole pass is enqueued without the host waiting for any layer's routing.  A
// kernel then brings every layer's counts to a pinned ring and sets a flag;
// later calls take each finished pass through the same LRU map and release,
// whose copies fill slots for the passes after.  A pass records one read
// event for all the slots its table maps, which is what a copy into one of
// them waits for.
#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "common.h"
#include "slot_policy.h"

namespace ft {
ft_status route_align(const ft_moe_step* st, hipStream_t s);
ft_status launch_copy_i32(const int32_t* src, int32_t* dst, int n, hipStream_t s);
ft_status launch_copy_i32_flag(const int32_t* src, int32_t* dst, int n, int32_t* flag, int32_t epoch,
                               hipStream_t s);
ft_status launch_set_table(const int32_t* table, int n, int32_t* dst, hipStream_t s);
ft_status launch_copy_counts_flag(const int32_t* const* src, int n_layers, int n, int32_t* dst,
                                  int32_t* flag, int32_t epoch, hipStream_t s);
}

struct ft_slot_cache {
    ft_slot_cache_desc d;
    ftp::Policy policy;
    std::vector<hipEvent_t> filled;
    std::vector<int> read_ev;          // slot -> pool event of its last release (-1: none)
    std::vector<long long> read_gen;   // slot -> that event's generation at the release
    std::vector<hipEvent_t> rpool;     // release events
    std::vector<long long> rgen;       // times each was recorded
    int rpos = 0;
    // pinned staging ring for slot-table uploads, and its device mapping (a
    // one-block kernel uploads a table; null: hipMemcpyAsync)
    int32_t* stage = nullptr;
    const int32_t* stage_dev = nullptr;
    std::vector<hipEvent_t> stage_ev;
    std::vector<char> stage_used;
    int ring = 0, ring_pos = 0;
    // ft_slot_stack_forward: one event per layer marks its expert counts on the
    // host, or (mapped buffers) a flag per layer that the copying kernel sets
    // to the pass's epoch after the counts
    std::vector<hipEvent_t> counts_ev;
    int32_t* flags = nullptr;        // pinned [n_layers]
    int32_t* flags_dev = nullptr;    // its device mapping, or null
    int32_t epoch = 0;
    // device-table passes (FT_STACK_DEVICE_TABLE), set up on first use
    static constexpr int DT_RING = 4;      // passes routed but not yet taken through the LRU, at most
    int32_t* dtab = nullptr;               // device [n_layers][n_experts]: slot, or -2 - host index
    std::vector<int32_t> htab;             // what dtab holds
    const uint8_t* host_dev = nullptr;     // device address of the host pool
    int32_t* dt_counts = nullptr;          // pinned [DT_RING][n_layers][n_experts]
    int32_t* dt_counts_dev = nullptr;
    int32_t* dt_flags = nullptr;           // pinned [DT_RING]: the pass number whose counts are there
    int32_t* dt_flags_dev = nullptr;
    long long dt_enq = 0, dt_done = 0;     // passes enqueued / taken through the LRU
    int dt_layers[DT_RING] = {};

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
    int shared_ev = -1;  // this call's release event, once recorded
    bool wait_read(int slot) {  // the copy stream waits for the slot's last reader
        const int ev = c->read_ev[slot];
        if (ev < 0) return true;
        if (c->rgen[ev] != c->read_gen[slot]) {
            // recorded again since: the slot's release is earlier on the compute
            // stream than that newer point, so it is done once the newer one is
            hipError_t q = hipEventQuery(c->rpool[ev]);
            if (q == hipSuccess) return true;
            if (q != hipErrorNotReady) return ok(q);
        }
        return ok(hipStreamWaitEvent(copy_s, c->rpool[ev], 0));
    }
    bool copy(int slot, int layer, int expert) override {
        if (!wait_read(slot)) return false;
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
    bool copy_wait(int slot) override { return ok(hipEventSynchronize(c->filled[slot])); }
    // device-table bookkeeping: kernels find slots through the device table,
    // which maps a slot only once its copy has landed, and each pass records
    // one read event for every slot the table maps; so the compute stream
    // neither waits for copies nor records reads here
    bool dt = false;
    bool compute_wait(int slot) override {
        if (dt) return true;
        return ok(hipStreamWaitEvent(compute, c->filled[slot], 0));
    }
    bool record_read(int slot) override {
        if (dt) return true;
        if (shared_ev < 0) {
            shared_ev = c->rpos;
            c->rpos = (c->rpos + 1) % (int)c->rpool.size();
            if (!ok(hipEventRecord(c->rpool[shared_ev], compute))) return false;
            ++c->rgen[shared_ev];
        }
        c->read_ev[slot] = shared_ev;
        c->read_gen[slot] = c->rgen[shared_ev];
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
    std::vector<int>& read_ev_new;
    hipError_t err = hipSuccess;
    ResizeEngine(ft_slot_cache* cc, hipStream_t cp, char* base, std::vector<hipEvent_t>& f,
                 std::vector<int>& r)
        : c(cc), copy_s(cp), dst_base(base), filled_new(f), read_ev_new(r) {}
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
    bool copy_wait(int) override { return false; }
    bool compute_wait(int) override { return false; }
    bool record_read(int) override { return false; }
    bool move(int src, int dst) override {
        if (!ok(hipStreamWaitEvent(copy_s, c->filled[src], 0))) return false;
        // (a reused pool event is a later point of the compute stream: waiting
        // for it is conservative)
        if (read_ev_new[dst] >= 0 && !ok(hipStreamWaitEvent(copy_s, c->rpool[read_ev_new[dst]], 0)))
            return false;
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

// ---- device-table passes ---------------------------------------------------

ft_status dt_setup(ft_slot_cache* c) {
    if (c->dtab) return FT_OK;
    const ft_slot_cache_desc& d = c->d;
    if (d.n_experts > ft::TABLE_MAX)
        return ft::set_error(FT_ERR_UNSUPPORTED, "device-table passes: %d experts per layer > %d",
                             d.n_experts, ft::TABLE_MAX);
    void* hp = nullptr;
    // (the runtime only reads the host address; its signature is not const)
    if (hipHostGetDevicePointer(&hp, const_cast<void*>(d.host_pool), 0) != hipSuccess || !hp) {
        (void)hipGetLastError();
        return ft::set_error(FT_ERR_UNSUPPORTED, "device-table passes: the host pool has no device mapping");
    }
    if (((uintptr_t)hp & 255) || d.host_stride % 256)
        return ft::set_error(FT_ERR_UNSUPPORTED,
                             "device-table passes: the host pool must be 256-byte aligned with a "
                             "stride that is a multiple of 256");
    // all or nothing: the cache keeps these only when every one was obtained
    const size_t n = (size_t)d.n_layers * d.n_experts;
    int32_t *tab = nullptr, *cnt = nullptr, *flg = nullptr;
    void *cnt_dev = nullptr, *flg_dev = nullptr;
    hipError_t e = hipMalloc((void**)&tab, sizeof(int32_t) * n);
    if (e == hipSuccess)
        e = hipHostMalloc((void**)&cnt, sizeof(int32_t) * n * ft_slot_cache::DT_RING, hipHostMallocDefault);
    if (e == hipSuccess)
        e = hipHostMalloc((void**)&flg, sizeof(int32_t) * ft_slot_cache::DT_RING, hipHostMallocDefault);
    if (e == hipSuccess) e = hipHostGetDevicePointer(&cnt_dev, cnt, 0);
    if (e == hipSuccess) e = hipHostGetDevicePointer(&flg_dev, flg, 0);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        if (tab) (void)hipFree(tab);
        if (cnt) (void)hipHostFree(cnt);
        if (flg) (void)hipHostFree(flg);
        return ft::set_error(FT_ERR_HIP, "device-table passes: allocating the table and count ring: %s",
                             hipGetErrorString(e));
    }
    for (int i = 0; i < ft_slot_cache::DT_RING; ++i) flg[i] = 0;
    c->dtab = tab;
    c->dt_counts = cnt;
    c->dt_counts_dev = (int32_t*)cnt_dev;
    c->dt_flags = flg;
    c->dt_flags_dev = (int32_t*)flg_dev;
    c->htab.assign(n, INT32_MIN);  // nothing uploaded yet: every row differs
    c->host_dev = (const uint8_t*)hp;
    return FT_OK;
}

// Take the oldest pass not yet counted through the LRU: map and release each
// of its layers' experts (ascending layer), as the per-layer path would have.
// Returns FT_OK with *done = false when its counts are not there and !block.
ft_status dt_account_one(ft_slot_cache* c, HipEngine& eng, bool block, bool* done, ft_stack_stats* acc) {
    *done = false;
    if (c->dt_done >= c->dt_enq) return FT_OK;
    const int ring = (int)(c->dt_done % ft_slot_cache::DT_RING);
    const int32_t want = (int32_t)(c->dt_done + 1);
    if (__atomic_load_n(c->dt_flags + ring, __ATOMIC_ACQUIRE) != want) {
        if (!block) return FT_OK;
        // bounded: a stream that stopped (an earlier failure) gives an error
        // rather than a hung host
        const auto t0 = std::chrono::steady_clock::now();
        while (__atomic_load_n(c->dt_flags + ring, __ATOMIC_ACQUIRE) != want) {
            if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(20))
                return ft::set_error(FT_ERR_HIP, "the expert counts of pass %lld did not arrive",
                                     c->dt_done + 1);
#if defined(__x86_64__)
            __builtin_ia32_pause();
#endif
        }
    }
    const int E = c->d.n_experts, L = c->dt_layers[ring];
    const int32_t* cnt = c->dt_counts + (size_t)ring * c->d.n_layers * E;
    std::vector<int32_t> need, slots((size_t)E);
    for (int l = 0; l < L; ++l) {
        need.clear();
        for (int e = 0; e < E; ++e)
            if (cnt[(size_t)l * E + e] > 0) need.push_back(e);
        ft_map_stats ms{};
        ft_status r = c->policy.map(eng, l, need.data(), (int)need.size(), slots.data(), &ms);
        if (r == FT_ERR_CAPACITY) {
            // more distinct experts than the layer's slots can take (the map
            // checks this before changing anything): the pass already read
            // them from the host pool; count the non-resident ones as misses
            ms = ft_map_stats{};
            ms.n_demand = (int)need.size();
            for (int32_t e : need)
                if (c->policy.lookup(l, e) >= 0) ++ms.n_hit; else ++ms.n_miss;
            r = FT_OK;
        } else if (r == FT_OK) {
            r = c->policy.release(eng, l);
        }
        if (r != FT_OK) return hip_status(eng, r);
        acc->demand += ms.n_demand;
        acc->hits += ms.n_hit;
        acc->prefetch_hits += ms.n_prefetch_hit;
        acc->misses += ms.n_miss;
    }
    ++c->dt_done;
    *done = true;
    return FT_OK;
}

// Bring the device table to the cache's state: an expert maps to its slot
// once the copy into it has landed, else to the host pool.  Rows that change
// are written on the compute stream, ahead of the pass that reads them.
ft_status dt_sync(ft_slot_cache* c, hipStream_t cs) {
    const int E = c->d.n_experts;
    std::vector<int32_t> row((size_t)E);
    for (int l = 0; l < c->d.n_layers; ++l) {
        for (int e = 0; e < E; ++e) {
            const int sl = c->policy.lookup(l, e);
            bool landed = sl >= 0;
            if (landed && c->policy.entry(sl).copying) {
                const hipError_t q = hipEventQuery(c->filled[sl]);
                if (q != hipSuccess && q != hipErrorNotReady) FT_HIP(q);
                landed = q == hipSuccess;
            }
            row[e] = landed ? sl : -2 - (l * E + e);
        }
        int32_t* have = c->htab.data() + (size_t)l * E;
        if (std::memcmp(row.data(), have, sizeof(int32_t) * E) != 0) {
            const ft_status r = ft::launch_set_table(row.data(), E, c->dtab + (size_t)l * E, cs);
            if (r != FT_OK) return r;
            std::memcpy(have, row.data(), sizeof(int32_t) * E);
        }
    }
    return FT_OK;
}

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
    c->filled.assign(d.n_slots, nullptr);
    c->read_ev.assign(d.n_slots, -1);
    c->read_gen.assign(d.n_slots, 0);
    for (int s = 0; s < d.n_slots; ++s) {
        if (make_event(&c->filled[s]) != hipSuccess) {
            ft_slot_cache_destroy(c);
            return ft::set_error(FT_ERR_HIP, "hipEventCreate failed");
        }
    }
    // release events: enough that one is recorded again only long after its
    // slots' copies were issued (4 per layer)
    c->rpool.assign((size_t)4 * d.n_layers + 4, nullptr);
    c->rgen.assign(c->rpool.size(), 0);
    for (auto& e : c->rpool)
        if (make_event(&e) != hipSuccess) {
            ft_slot_cache_destroy(c);
            return ft::set_error(FT_ERR_HIP, "hipEventCreate failed");
        }
    c->ring = 8;
    if (hipHostMalloc((void**)&c->stage, sizeof(int32_t) * (size_t)d.n_experts * c->ring,
                      hipHostMallocDefault) != hipSuccess) {
        c->stage = nullptr;
        ft_slot_cache_destroy(c);
        return ft::set_error(FT_ERR_HIP, "hipHostMalloc of the slot-table staging ring failed");
    }
    {
        void* dp = nullptr;
        if (hipHostGetDevicePointer(&dp, c->stage, 0) == hipSuccess) c->stage_dev = (const int32_t*)dp;
        else (void)hipGetLastError();
        if (hipHostMalloc((void**)&c->flags, sizeof(int32_t) * (size_t)d.n_layers, hipHostMallocDefault) ==
            hipSuccess) {
            for (int l = 0; l < d.n_layers; ++l) c->flags[l] = 0;
            dp = nullptr;
            if (hipHostGetDevicePointer(&dp, c->flags, 0) == hipSuccess) c->flags_dev = (int32_t*)dp;
            else (void)hipGetLastError();
        } else {
            c->flags = nullptr;
            (void)hipGetLastError();
        }
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
    for (hipEvent_t e : c->rpool)
        if (e) (void)hipEventSynchronize(e), (void)hipEventDestroy(e);
    for (hipEvent_t e : c->stage_ev)
        if (e) (void)hipEventSynchronize(e), (void)hipEventDestroy(e);
    for (hipEvent_t e : c->counts_ev)
        if (e) (void)hipEventSynchronize(e), (void)hipEventDestroy(e);
    if (c->stage) (void)hipHostFree(c->stage);
    if (c->flags) (void)hipHostFree(c->flags);
    if (c->dtab) (void)hipFree(c->dtab);  // after the read events above: no pass still reads it
    if (c->dt_counts) (void)hipHostFree(c->dt_counts);
    if (c->dt_flags) (void)hipHostFree(c->dt_flags);
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
    if (c->d.n_experts <= ft::TABLE_MAX) {  // the table rides in a kernel's arguments
        int32_t tab[ft::TABLE_MAX];
        for (int e = 0; e < c->d.n_experts; ++e) tab[e] = -1;
        for (int q = 0; q < n; ++q) tab[experts_host[q]] = slot_of[q];
        return ft::launch_set_table(tab, c->d.n_experts, slot_table_dev, (hipStream_t)compute);
    }
    // larger tables through the pinned staging ring
    const int i = c->ring_pos;
    c->ring_pos = (c->ring_pos + 1) % c->ring;
    if (c->stage_used[i]) FT_HIP(hipEventSynchronize(c->stage_ev[i]));
    int32_t* tab = c->stage + (size_t)i * c->d.n_experts;
    for (int e = 0; e < c->d.n_experts; ++e) tab[e] = -1;
    for (int q = 0; q < n; ++q) tab[experts_host[q]] = slot_of[q];
    if (c->stage_dev) {
        ft_status r2 = ft::launch_copy_i32(c->stage_dev + (size_t)i * c->d.n_experts, slot_table_dev,
                                           c->d.n_experts, (hipStream_t)compute);
        if (r2 != FT_OK) return r2;
    } else {
        FT_HIP(hipMemcpyAsync(slot_table_dev, tab, sizeof(int32_t) * c->d.n_experts,
                              hipMemcpyHostToDevice, (hipStream_t)compute));
    }
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
    std::vector<hipEvent_t> filled(n_slots, nullptr);
    std::vector<int> read_ev(n_slots, -1);
    std::vector<long long> read_gen(n_slots, 0);
    for (int s = 0; s < n_slots; ++s) {
        if (s < old_n) {
            filled[s] = c->filled[s];
            read_ev[s] = c->read_ev[s];
            read_gen[s] = c->read_gen[s];
        } else if (make_event(&filled[s]) != hipSuccess) {
            for (int q = old_n; q < s; ++q) (void)hipEventDestroy(filled[q]);
            return ft::set_error(FT_ERR_HIP, "hipEventCreate failed");
        }
    }
    char* base = (char*)(moved ? dev_slots : c->d.dev_slots);
    ResizeEngine eng(c, (hipStream_t)copy_stream, base, filled, read_ev);
    const ft_status r = c->policy.resize(eng, n_slots, moved);
    if (r != FT_OK && r != FT_ERR_HIP) {  // nothing changed
        for (int s = old_n; s < n_slots; ++s) (void)hipEventDestroy(filled[s]);
        return hip_status(eng.err, r);
    }
    // the policy now has n_slots slots: retire the fill events of dropped
    // slots (after the copies they mark) and switch to the new set and array
    for (int s = n_slots; s < old_n; ++s)
        (void)hipEventSynchronize(c->filled[s]), (void)hipEventDestroy(c->filled[s]);
    c->filled.swap(filled);
    c->read_ev.swap(read_ev);
    c->read_gen.swap(read_gen);
    c->d.n_slots = n_slots;
    c->d.dev_slots = base;
    return hip_status(eng.err, r);
}

int ft_slot_cache_lookup(const ft_slot_cache* c, int layer, int expert) {
    return c ? c->policy.lookup(layer, expert) : -1;
}

// One pass through a stack of layers whose experts come through the cache:
// per layer l, the routing of layer l + 2 is enqueued first (its inputs do
// not depend on the layers before it here), then layer l's FFN and combine and its
// release; once layer l + 1's expert counts are on the host its missing
// experts are prefetched on the copy stream (the next layer's weights travel
// while this layer computes: claypier.com article, "按带宽决定分工的思路";
// FreeToken hub article, paragraph on prefill overlap) and mapped.
namespace {

// One FT_STACK_DEVICE_TABLE pass (or, with n_layers == 0, a flush).
ft_status dt_forward(ft_slot_cache* c, const ft_stack_pass* p, hipStream_t cs, hipStream_t copy_s,
                     ft_stack_stats* out) {
    const int L = p->n_layers, E = c->d.n_experts;
    FT_CHECK_ARG(L >= 0 && L <= c->d.n_layers, "n_layers must be in [0, %d]", c->d.n_layers);
    if (L > ft::STACK_MAX_LAYERS)
        return ft::set_error(FT_ERR_UNSUPPORTED, "device-table passes: %d layers > %d", L,
                             ft::STACK_MAX_LAYERS);
    const ft_moe_step* S = p->layers;
    FT_CHECK_ARG(L == 0 || S, "null layers");
    for (int l = 0; l < L; ++l) {
        if (S[l].weights.n_shared)
            return ft::set_error(FT_ERR_UNSUPPORTED, "device-table passes: no shared expert");
        FT_CHECK_ARG(S[l].T >= 1 && S[l].weights.E == E && S[l].counts,
                     "layer %d: T >= 1, E == the cache's experts per layer, counts", l);
        FT_CHECK_ARG(S[l].weights.pool == c->d.dev_slots && S[l].weights.slot_stride == c->d.slot_stride,
                     "layer %d: weights.pool / slot_stride must be the cache's slot array", l);
    }
    if (L == 0 && !c->dtab) {  // a flush before any device-table pass
        if (out) *out = ft_stack_stats{};
        return FT_OK;
    }
    ft_status r = dt_setup(c);
    if (r != FT_OK) return r;
    HipEngine eng(c, cs, copy_s);
    eng.dt = true;
    ft_stack_stats acc{};
    const long long h2d0 = c->policy.stats().bytes_h2d;
    // passes whose counts are back, then (blocking) room in the ring for this
    // one; a flush takes every pending pass
    bool done = true;
    while (done) {
        r = dt_account_one(c, eng, false, &done, &acc);
        if (r != FT_OK) return r;
    }
    // passes left pending while this one is enqueued: the host may run that
    // far ahead of the GPU, and a missed expert is read from the host pool
    // until its pass is counted and its copy lands.  One: on the 8-layer
    // 35B-A3B stack, 0.44-0.49 ms per pass against 0.46-0.54 with three
    static const int lag = [] {
        const char* e = getenv("FTMOE_DT_LAG");
        const int v = e ? atoi(e) : 1;
        return v < 0 ? 0 : v > ft_slot_cache::DT_RING - 1 ? ft_slot_cache::DT_RING - 1 : v;
    }();
    const long long keep = L > 0 ? lag : 0;
    while (c->dt_enq - c->dt_done > keep) {
        r = dt_account_one(c, eng, true, &done, &acc);
        if (r != FT_OK) return r;
    }
    // one read point after the pass's kernels (also after a partly enqueued
    // pass that failed) for every slot the table maps: a copy into such a
    // slot waits for it
    auto mark_reads = [&]() -> ft_status {
        const int ev = c->rpos;
        c->rpos = (c->rpos + 1) % (int)c->rpool.size();
        FT_HIP(hipEventRecord(c->rpool[ev], cs));
        ++c->rgen[ev];
        for (int32_t v : c->htab)
            if (v >= 0) {
                c->read_ev[v] = ev;
                c->read_gen[v] = c->rgen[ev];
            }
        return FT_OK;
    };
    if (L > 0) {
        r = dt_sync(c, cs);
        if (r != FT_OK) return r;
        const int32_t* cnts[ft::STACK_MAX_LAYERS];
        for (int l = 0; l < L; ++l) {
            const ft_moe_step& st = S[l];
            const float* lin = p->logits_in ? p->logits_in[l] : nullptr;
            if (lin) {
                r = ft_moe_route(nullptr, st.act_dt, nullptr, lin, st.bias, st.T, st.weights.H, E, st.k,
                                 nullptr, st.topk_ids, st.topk_w, cs);
                if (r == FT_OK)
                    r = ft_moe_align(st.topk_ids, st.T, st.k, E, st.counts, st.offsets, st.perm,
                                     st.inv_perm, st.align_ws, st.align_ws_bytes, cs);
            } else {
                r = ft::route_align(&st, cs);
            }
            ft_moe_weights w = st.weights;
            w.host_pool = c->host_dev;
            w.host_stride = c->d.host_stride;
            if (r == FT_OK)
                r = ft_moe_ffn(&w, st.x, st.act_dt, st.T, st.k, st.perm, st.offsets, c->dtab + (size_t)l * E,
                               st.y_perm, st.y_dt, st.ffn_ws, st.ffn_ws_bytes, cs);
            if (r == FT_OK)
                r = ft_moe_combine(st.y_perm, st.y_dt, st.inv_perm, st.topk_w, st.T, st.k, w.H, 0,
                                   st.out, st.out_dt, cs);
            if (r != FT_OK) {
                (void)mark_reads();
                return r;
            }
            cnts[l] = st.counts;
        }
        const int ring = (int)(c->dt_enq % ft_slot_cache::DT_RING);
        r = ft::launch_copy_counts_flag(cnts, L, E, c->dt_counts_dev + (size_t)ring * c->d.n_layers * E,
                                        c->dt_flags_dev + ring, (int32_t)(c->dt_enq + 1), cs);
        const ft_status rm = mark_reads();
        if (r != FT_OK) return r;
        if (rm != FT_OK) return rm;
        c->dt_layers[ring] = L;
        ++c->dt_enq;
    }
    acc.bytes_h2d = c->policy.stats().bytes_h2d - h2d0;
    if (out) *out = acc;
    return hip_status(eng, FT_OK);
}

}  // namespace

ft_status ft_slot_stack_forward(ft_slot_cache* c, const ft_stack_pass* p, void* compute,
                                void* copy_stream, ft_stack_stats* out) {
    ft::clear_error();
    FT_CHECK_ARG(c && p, "null cache / pass");
    FT_CHECK_ARG((p->flags & ~FT_STACK_DEVICE_TABLE) == 0, "unknown flags 0x%x", p->flags);
    ft_stack_stats flushed{};
    if (p->flags & FT_STACK_DEVICE_TABLE) {
        if (!p->prefill) return dt_forward(c, p, (hipStream_t)compute, (hipStream_t)copy_stream, out);
        if (c->dt_enq > c->dt_done) {  // a prefill: count the pending passes first
            ft_stack_pass flush{};
            flush.flags = FT_STACK_DEVICE_TABLE;
            const ft_status r = dt_forward(c, &flush, (hipStream_t)compute, (hipStream_t)copy_stream, &flushed);
            if (r != FT_OK) return r;
        }
    }
    FT_CHECK_ARG(p->layers && p->counts_host, "null layers / counts_host");
    const int L = p->n_layers;
    FT_CHECK_ARG(L >= 1 && L <= c->d.n_layers, "n_layers must be in [1, %d]", c->d.n_layers);
    const ft_moe_step* S = p->layers;
    const int E = S[0].weights.E, ns = S[0].weights.n_shared;
    FT_CHECK_ARG(E + ns == c->d.n_experts, "E + n_shared must equal the cache's experts per layer");
    for (int l = 0; l < L; ++l)
        FT_CHECK_ARG(S[l].T >= 1 && S[l].weights.E == E && S[l].weights.n_shared == ns &&
                         S[l].slot_of_expert && S[l].counts,
                     "layer %d: T >= 1, the same E and n_shared, a slot table and counts", l);
    hipStream_t cs = (hipStream_t)compute;
    while ((int)c->counts_ev.size() < L) {
        hipEvent_t e = nullptr;
        FT_HIP(make_event(&e));
        c->counts_ev.push_back(e);
    }
    // the counts go to the host through the buffer's device mapping when it
    // has one (a one-block kernel), else by hipMemcpyAsync
    int32_t* counts_dev_map = nullptr;
    {
        void* dp = nullptr;
        if (hipHostGetDevicePointer(&dp, p->counts_host, 0) == hipSuccess) counts_dev_map = (int32_t*)dp;
        else (void)hipGetLastError();
    }
    const bool use_flags = counts_dev_map && c->flags_dev;
    const int32_t epoch = ++c->epoch;  // this pass's flag value
    ft_stack_stats acc = flushed;
    const ft_cache_stats before = c->policy.stats();
    std::vector<int32_t> need, all(E + ns);
    for (int e = 0; e < E + ns; ++e) all[e] = e;

    auto route = [&](int l) -> ft_status {
        const ft_moe_step& st = S[l];
        ft_status r;
        const float* lin = p->logits_in ? p->logits_in[l] : nullptr;
        if (lin) {
            r = ft_moe_route(nullptr, st.act_dt, nullptr, lin, st.bias, st.T, st.weights.H, E, st.k,
                             nullptr, st.topk_ids, st.topk_w, compute);
            if (r == FT_OK)
                r = ft_moe_align(st.topk_ids, st.T, st.k, E, st.counts, st.offsets, st.perm,
                                 st.inv_perm, st.align_ws, st.align_ws_bytes, compute);
        } else {
            r = ft::route_align(&st, cs);
        }
        if (r != FT_OK) return r;
        if (use_flags) {
            return ft::launch_copy_i32_flag(st.counts, counts_dev_map + (size_t)l * E, E,
                                            c->flags_dev + l, epoch, cs);
        }
        FT_HIP(hipMemcpyAsync(p->counts_host + (size_t)l * E, st.counts, sizeof(int32_t) * E,
                              hipMemcpyDeviceToHost, cs));
        FT_HIP(hipEventRecord(c->counts_ev[l], cs));
        return FT_OK;
    };
    auto experts_of = [&](int l) -> ft_status {  // distinct experts with rows, ascending (+ shared)
        if (use_flags) {
            // the kernel sets the flag after the counts (system-scope release);
            // the counts are usually there already (routing runs ahead).  A
            // bounded wait: a stream that stopped (an earlier failure) gives
            // an error rather than a hung host
            const auto t0 = std::chrono::steady_clock::now();
            while (__atomic_load_n(c->flags + l, __ATOMIC_ACQUIRE) != epoch) {
                if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(20))
                    return ft::set_error(FT_ERR_HIP, "layer %d's expert counts did not arrive", l);
#if defined(__x86_64__)
                __builtin_ia32_pause();
#endif
            }
        } else {
            // poll briefly before a blocking wait
            hipError_t q = hipErrorNotReady;
            for (int i = 0; i < 2000 && q == hipErrorNotReady; ++i) q = hipEventQuery(c->counts_ev[l]);
            if (q == hipErrorNotReady) q = hipEventSynchronize(c->counts_ev[l]);
            FT_HIP(q);
        }
        need.clear();
        const int32_t* cnt = p->counts_host + (size_t)l * E;
        for (int e = 0; e < E; ++e)
            if (cnt[e] > 0) need.push_back(e);
        if (ns) need.push_back(E);
        return FT_OK;
    };
    auto map = [&](int l) -> ft_status {
        ft_map_stats ms{};
        // (the step's slot table is the map's output here; the descriptor holds
        // it as the FFN's read-only input)
        ft_status r = ft_slot_cache_map(c, l, need.data(), (int)need.size(),
                                        const_cast<int32_t*>(S[l].slot_of_expert), compute,
                                        copy_stream, &ms);
        acc.demand += ms.n_demand;
        acc.hits += ms.n_hit;
        acc.prefetch_hits += ms.n_prefetch_hit;
        acc.misses += ms.n_miss;
        return r;
    };
    auto prefetch = [&](int l, const std::vector<int32_t>& ex) -> ft_status {
        ft_status r = ft_slot_cache_prefetch(c, l, ex.data(), (int)ex.size(), copy_stream, nullptr);
        if (r == FT_WARN_OVERLAP_DISABLED) {
            ++acc.prefetch_warnings;
            return FT_OK;
        }
        return r;
    };
#define FT_STACK_TRY(call)              \
    do {                                \
        const ft_status r_ = (call);    \
        if (r_ != FT_OK) return r_;     \
    } while (0)
    // Routing runs two layers ahead of the FFN, so that while the host waits
    // for layer l + 1's counts and maps its experts the GPU still has layer
    // l + 2's routing and layer l's FFN queued.
    FT_STACK_TRY(route(0));
    if (L > 1) FT_STACK_TRY(route(1));
    FT_STACK_TRY(experts_of(0));
    FT_STACK_TRY(map(0));
    for (int l = 0; l < L; ++l) {
        if (l + 2 < L) FT_STACK_TRY(route(l + 2));
        ft_moe_step st = S[l];
        if (ns) st.weights.shared_slot = c->policy.lookup(l, E);
        FT_STACK_TRY(ft_moe_ffn(&st.weights, st.x, st.act_dt, st.T, st.k, st.perm, st.offsets,
                                st.slot_of_expert, st.y_perm, st.y_dt, st.ffn_ws, st.ffn_ws_bytes,
                                compute));
        FT_STACK_TRY(ft_moe_combine(st.y_perm, st.y_dt, st.inv_perm, st.topk_w, st.T, st.k,
                                    st.weights.H, ns, st.out, st.out_dt, compute));
        FT_STACK_TRY(ft_slot_cache_release(c, l, compute));
        if (l + 1 < L) {
            // layer l + 1's counts come after layer l - 1's map on the compute
            // stream, so once they are here its copies have landed and its
            // slots can take layer l + 1's experts
            FT_STACK_TRY(experts_of(l + 1));
            FT_STACK_TRY(prefetch(l + 1, p->prefill ? all : need));
            FT_STACK_TRY(map(l + 1));
        }
    }
#undef FT_STACK_TRY
    acc.bytes_h2d = flushed.bytes_h2d + c->policy.stats().bytes_h2d - before.bytes_h2d;
    if (out) *out = acc;
    return FT_OK;
}

}  // extern "C"
