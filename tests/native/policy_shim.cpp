// policy_shim.cpp -- C entry points over the slot-cache policy with a mock copy
// engine, for CPU tests of the LRU bookkeeping (no HIP involved).
//
// The mock records every engine call; copies either complete at once or stay
// "in flight" until pol_complete_all(), and the next copy can be made to fail.
#include <vector>

#include "../../expert_ffn_execution_amd/csrc/slot_policy.h"

namespace {

struct Mock final : ftp::Engine {
    explicit Mock(int n_slots) : pending(n_slots, 0) {}
    std::vector<int> log;  // (kind, slot, layer, expert): kind 0 copy, 1 wait, 2 read, 3 move, 4 host wait
    std::vector<char> pending;
    bool auto_complete = true, fail_next = false;

    void rec(int kind, int slot, int layer, int expert) {
        log.push_back(kind);
        log.push_back(slot);
        log.push_back(layer);
        log.push_back(expert);
    }
    bool copy(int slot, int layer, int expert) override {
        if (fail_next) {
            fail_next = false;
            return false;
        }
        rec(0, slot, layer, expert);
        pending[slot] = auto_complete ? 0 : 1;
        return true;
    }
    bool copy_done(int slot) override { return !pending[slot]; }
    bool copy_wait(int slot) override {  // the copy completes while the host waits
        rec(4, slot, -1, -1);
        pending[slot] = 0;
        return true;
    }
    bool compute_wait(int slot) override {
        rec(1, slot, -1, -1);
        return true;
    }
    bool record_read(int slot) override {
        rec(2, slot, -1, -1);
        return true;
    }
    bool move(int src, int dst) override {
        if (fail_next) {
            fail_next = false;
            return false;
        }
        rec(3, src, dst, -1);
        if ((int)pending.size() <= dst) pending.resize(dst + 1, 0);
        pending[dst] = auto_complete ? 0 : 1;
        return true;
    }
};

struct Shim {
    Shim(int L, int E, int S, int scope) : pol(L, E, S, scope, 1000), eng(S) {}
    ftp::Policy pol;
    Mock eng;
};

}  // namespace

extern "C" {

void* pol_create(int L, int E, int S, int scope) { return new Shim(L, E, S, scope); }
void pol_destroy(void* h) { delete static_cast<Shim*>(h); }

int pol_map(void* h, int layer, const int* experts, int n, int* slots, int* st4) {
    Shim* s = static_cast<Shim*>(h);
    ft_map_stats ms{};
    int r = s->pol.map(s->eng, layer, experts, n, slots, &ms);
    if (st4) {
        st4[0] = ms.n_demand;
        st4[1] = ms.n_hit;
        st4[2] = ms.n_prefetch_hit;
        st4[3] = ms.n_miss;
    }
    return r;
}
int pol_release(void* h, int layer) {
    Shim* s = static_cast<Shim*>(h);
    return s->pol.release(s->eng, layer);
}
int pol_prefetch(void* h, int layer, const int* experts, int n, int* issued) {
    Shim* s = static_cast<Shim*>(h);
    return s->pol.prefetch(s->eng, layer, experts, n, issued);
}
int pol_evict(void* h, int layer, int expert) {
    Shim* s = static_cast<Shim*>(h);
    return s->pol.evict(s->eng, layer, expert);
}
int pol_resize(void* h, int n_slots, int moved_array) {
    Shim* s = static_cast<Shim*>(h);
    int r = s->pol.resize(s->eng, n_slots, moved_array != 0);
    if (r == FT_OK || r == FT_ERR_HIP) s->eng.pending.resize(n_slots, 0);
    return r;
}
int pol_lookup(void* h, int layer, int expert) {
    return static_cast<Shim*>(h)->pol.lookup(layer, expert);
}
void pol_set_auto_complete(void* h, int on) { static_cast<Shim*>(h)->eng.auto_complete = on != 0; }
void pol_complete_all(void* h) {
    Shim* s = static_cast<Shim*>(h);
    for (auto& p : s->eng.pending) p = 0;
}
void pol_fail_next_copy(void* h) { static_cast<Shim*>(h)->eng.fail_next = true; }
int pol_log(void* h, int* out, int max) {
    Shim* s = static_cast<Shim*>(h);
    int n = (int)s->eng.log.size();
    for (int i = 0; i < n && i < max; ++i) out[i] = s->eng.log[i];
    s->eng.log.clear();
    return n;
}
void pol_stats(void* h, long long* out) {
    ft_cache_stats c = static_cast<Shim*>(h)->pol.stats();
    long long v[12] = {c.maps, c.demand, c.hits, c.prefetch_hits, c.misses, c.prefetch_issued,
                       c.evictions, c.bytes_h2d, c.resident, c.held, c.in_flight, c.n_slots};
    for (int i = 0; i < 12; ++i) out[i] = v[i];
}

}  // extern "C"
