// slot_policy.h -- LRU expert-slot policy (host C++, no HIP).
//
// The device holds a fixed number of expert slots; the full pool of
// (layer, expert) weights lives in host memory.  A request for a layer's
// routed experts takes the resident ones (touching them as most recent) and
// brings the others into free slots, else into the least-recently-used slots
// that no one is reading and no copy is filling (refft.com guide, "深度解析":
// global LRU expert caching; freelamp.com article, section 2.3: the expert
// cache is counted in slots; claypier.com article,
// "从 MoE「用不到的权重」入手的推理引擎": weights not used for a while are
// evicted).  The next layer's experts can be prefetched into slots while the
// current layer computes (FreeToken hub article, paragraph on prefill overlap).
//
// The policy is pure bookkeeping; an Engine performs copies and orders them
// against the compute stream (a HIP engine in the library, a recording mock
// in the CPU tests).  Every call visits its experts in ascending id order, so
// timestamps and victims are deterministic.
#pragma once

#include <cstddef>
#include <cstdint>
#include <algorithm>
#include <vector>

#include "../../include/ftmoe.h"

namespace ftp {

struct Engine {
    virtual ~Engine() {}
    // enqueue host (layer, expert) -> device slot; must first wait for the
    // slot's last reader (if one was recorded) and leave a completion marker.
    virtual bool copy(int slot, int layer, int expert) = 0;
    // has the last copy into `slot` completed?
    virtual bool copy_done(int slot) = 0;
    // block the host until the last copy into `slot` has completed
    virtual bool copy_wait(int slot) = 0;
    // make the compute stream wait for the last copy into `slot`
    virtual bool compute_wait(int slot) = 0;
    // record: work enqueued on the compute stream so far is the last reader of `slot`
    virtual bool record_read(int slot) = 0;
    // resize: copy the device contents of slot `src` into slot `dst` of the
    // (possibly new) slot array, after the last copy into `src` and the last
    // reader of `dst`, leaving a completion marker for `dst`
    virtual bool move(int src, int dst) = 0;
};

struct Entry {
    int layer = -1, expert = -1;   // -1: free
    uint64_t last = 0;             // LRU timestamp
    bool held = false;             // demanded by a map, not yet released
    bool prefetched = false;       // brought by prefetch and not yet demanded
    bool copying = false;          // a copy was issued and not yet seen complete
};

class Policy {
  public:
    Policy(int n_layers, int n_experts, int n_slots, int scope, size_t expert_bytes)
        : L_(n_layers), E_(n_experts), S_(n_slots), scope_(scope), bytes_(expert_bytes),
          slots_(n_slots), where_((size_t)n_layers * n_experts, -1) {
        st_ = ft_cache_stats{};
        st_.n_slots = n_slots;
    }

    int lookup(int layer, int expert) const {
        if (layer < 0 || layer >= L_ || expert < 0 || expert >= E_) return -1;
        return where_[(size_t)layer * E_ + expert];
    }

    // slot_of[i] receives the slot of experts[i].  Resident experts are touched
    // and held first (ascending ids), then the missing ones are brought in
    // (ascending ids), so a request never evicts one of its own experts.
    ft_status map(Engine& eng, int layer, const int32_t* experts, int n, int32_t* slot_of,
                  ft_map_stats* ms) {
        ft_status v = check_list(layer, experts, n);
        if (v != FT_OK) return v;
        refresh(eng);
        // capacity: the misses must fit in free slots plus slots that are neither
        // held nor hold a requested expert.  Those whose copy is still in flight
        // become evictable when it lands: if the request needs them, the host
        // waits for the least recently used ones (a request that fits is never
        // refused for timing).
        int need = 0;
        for (int i = 0; i < n; ++i)
            if (lookup(layer, experts[i]) < 0) ++need;
        const int have = obtainable(layer, experts, n);
        if (need > have) {
            std::vector<int> landing;
            for (int s = lo(layer); s < hi(layer); ++s) {
                const Entry& en = slots_[s];
                if (en.layer >= 0 && !en.held && en.copying && !requested(en, layer, experts, n))
                    landing.push_back(s);
            }
            if (need > have + (int)landing.size()) return FT_ERR_CAPACITY;
            std::sort(landing.begin(), landing.end(),
                      [&](int a, int b) { return slots_[a].last < slots_[b].last; });
            for (int i = 0; i < need - have; ++i) {
                if (!eng.copy_wait(landing[i])) return FT_ERR_HIP;
                slots_[landing[i]].copying = false;
            }
        }
        ft_map_stats m{};
        m.n_demand = n;
        for (int i = 0; i < n; ++i) {
            const int s = lookup(layer, experts[i]);
            if (s < 0) continue;
            Entry& en = slots_[s];
            if (en.prefetched) ++m.n_prefetch_hit; else ++m.n_hit;
            en.prefetched = false;
            en.last = ++clock_;
            en.held = true;
            if (en.copying && !eng.compute_wait(s)) return FT_ERR_HIP;
            slot_of[i] = s;
        }
        for (int i = 0; i < n; ++i) {
            if (lookup(layer, experts[i]) >= 0) continue;
            const int s = take_slot(eng, layer);
            if (s < 0) return FT_ERR_CAPACITY;  // cannot happen after the check above
            if (!start_copy(eng, s, layer, experts[i])) return FT_ERR_HIP;
            ++m.n_miss;
            m.bytes_h2d += bytes_;
            Entry& en = slots_[s];
            en.last = ++clock_;
            en.held = true;
            if (!eng.compute_wait(s)) return FT_ERR_HIP;
            slot_of[i] = s;
        }
        st_.maps++;
        st_.demand += m.n_demand;
        st_.hits += m.n_hit;
        st_.prefetch_hits += m.n_prefetch_hit;
        st_.misses += m.n_miss;
        st_.bytes_h2d += (long long)m.bytes_h2d;
        if (ms) *ms = m;
        return FT_OK;
    }

    ft_status release(Engine& eng, int layer) {
        if (layer < 0 || layer >= L_) return FT_ERR_INVALID_ARG;
        for (int s = 0; s < S_; ++s) {
            Entry& en = slots_[s];
            if (en.held && en.layer == layer) {
                if (!eng.record_read(s)) return FT_ERR_HIP;
                en.held = false;
            }
        }
        return FT_OK;
    }

    // Resident experts are touched first, then the missing ones are copied into
    // free or evictable slots while any remain; held entries are never victims.
    ft_status prefetch(Engine& eng, int layer, const int32_t* experts, int n, int* n_issued) {
        ft_status v = check_list(layer, experts, n);
        if (v != FT_OK) return v;
        refresh(eng);
        for (int i = 0; i < n; ++i) {
            const int s = lookup(layer, experts[i]);
            if (s >= 0) slots_[s].last = ++clock_;
        }
        int issued = 0;
        bool short_of_room = false;
        for (int i = 0; i < n; ++i) {
            if (lookup(layer, experts[i]) >= 0) continue;
            const int s = take_slot(eng, layer, experts, n);
            if (s < 0) {
                short_of_room = true;
                break;
            }
            if (!start_copy(eng, s, layer, experts[i])) return FT_ERR_HIP;
            Entry& en = slots_[s];
            en.prefetched = true;
            en.last = ++clock_;
            ++issued;
            st_.bytes_h2d += (long long)bytes_;
        }
        st_.prefetch_issued += issued;
        if (n_issued) *n_issued = issued;
        return short_of_room ? FT_WARN_OVERLAP_DISABLED : FT_OK;
    }

    ft_status evict(Engine& eng, int layer, int expert) {
        if (layer < 0 || layer >= L_ || expert < -1 || expert >= E_) return FT_ERR_INVALID_ARG;
        refresh(eng);
        const int lo = expert < 0 ? 0 : expert, hi = expert < 0 ? E_ : expert + 1;
        for (int e = lo; e < hi; ++e) {
            int s = lookup(layer, e);
            if (s >= 0 && (slots_[s].held || slots_[s].copying)) return FT_ERR_BUSY;
        }
        for (int e = lo; e < hi; ++e) {
            int s = lookup(layer, e);
            if (s >= 0) drop(s);
        }
        return FT_OK;
    }

    // Change the number of slots to n_new (global scope; the pages describe the
    // expert cache being resized in slots at run time, without a restart or a
    // reload of the weights: freelamp.com article, section 2.3; refft.com
    // guide, "深度解析").  Nothing may be held.  Least-recently-used entries
    // that no copy is filling are dropped until the residents fit; survivors
    // keep their slot when it is below n_new, else move (ascending old slot) to
    // the lowest free slot below n_new.  With `moved_array` (the caller gives a
    // new slot array) every survivor is copied, else only the relocated ones;
    // copied entries count as in flight until their move completes.
    // FT_ERR_BUSY / FT_ERR_INVALID_ARG / FT_ERR_UNSUPPORTED change nothing.  A
    // failed move leaves the cache empty at the new size (FT_ERR_HIP).
    ft_status resize(Engine& eng, int n_new, bool moved_array) {
        if (n_new <= 0) return FT_ERR_INVALID_ARG;
        if (scope_ != FT_SCOPE_GLOBAL) return FT_ERR_UNSUPPORTED;
        refresh(eng);
        int inflight = 0, resident = 0;
        for (const Entry& en : slots_) {
            if (en.held) return FT_ERR_BUSY;
            if (en.copying) ++inflight;
            if (en.layer >= 0) ++resident;
        }
        if (inflight > n_new) return FT_ERR_BUSY;
        while (resident > n_new) {  // an evictable entry exists: inflight <= n_new
            int best = -1;
            for (int s = 0; s < S_; ++s) {
                const Entry& en = slots_[s];
                if (en.layer < 0 || !evictable(en)) continue;
                if (best < 0 || en.last < slots_[best].last) best = s;
            }
            drop(best);
            st_.evictions++;
            --resident;
        }
        std::vector<int> dst_of(S_, -1);
        std::vector<char> taken(n_new, 0);
        for (int s = 0; s < S_ && s < n_new; ++s)
            if (slots_[s].layer >= 0) dst_of[s] = s, taken[s] = 1;
        int d = 0;
        for (int s = n_new; s < S_; ++s) {
            if (slots_[s].layer < 0) continue;
            while (taken[d]) ++d;  // d < n_new: resident <= n_new
            taken[d] = 1;
            dst_of[s] = d;
        }
        bool failed = false;
        for (int s = 0; s < S_ && !failed; ++s)
            if (dst_of[s] >= 0 && (dst_of[s] != s || moved_array)) failed = !eng.move(s, dst_of[s]);
        std::vector<Entry> next(n_new);
        for (int s = 0; s < S_; ++s) {
            if (dst_of[s] < 0) continue;
            Entry& en = slots_[s];
            if (failed) {
                where_[(size_t)en.layer * E_ + en.expert] = -1;
                continue;
            }
            next[dst_of[s]] = en;
            if (dst_of[s] != s || moved_array) next[dst_of[s]].copying = true;
            where_[(size_t)en.layer * E_ + en.expert] = dst_of[s];
        }
        slots_.swap(next);
        S_ = n_new;
        st_.n_slots = n_new;
        return failed ? FT_ERR_HIP : FT_OK;
    }

    ft_cache_stats stats() const {
        ft_cache_stats o = st_;
        o.resident = o.held = o.in_flight = 0;
        for (const Entry& en : slots_) {
            if (en.layer >= 0) o.resident++;
            if (en.held) o.held++;
            if (en.copying) o.in_flight++;
        }
        return o;
    }

    const Entry& entry(int s) const { return slots_[s]; }
    int n_slots() const { return S_; }

  private:
    int L_, E_, S_, scope_;
    size_t bytes_;
    std::vector<Entry> slots_;
    std::vector<int> where_;
    uint64_t clock_ = 0;
    ft_cache_stats st_;

    int lo(int layer) const { return scope_ == FT_SCOPE_PER_LAYER ? layer * (S_ / L_) : 0; }
    int hi(int layer) const { return scope_ == FT_SCOPE_PER_LAYER ? (layer + 1) * (S_ / L_) : S_; }

    ft_status check_list(int layer, const int32_t* experts, int n) const {
        if (layer < 0 || layer >= L_ || n < 0 || (n > 0 && !experts)) return FT_ERR_INVALID_ARG;
        for (int i = 0; i < n; ++i) {
            if (experts[i] < 0 || experts[i] >= E_) return FT_ERR_INVALID_ARG;
            if (i && experts[i] <= experts[i - 1]) return FT_ERR_INVALID_ARG;
        }
        return FT_OK;
    }

    // mark copies seen complete
    void refresh(Engine& eng) {
        for (int s = 0; s < S_; ++s)
            if (slots_[s].copying && eng.copy_done(s)) slots_[s].copying = false;
    }

    bool evictable(const Entry& en) const { return !en.held && !en.copying; }

    bool requested(const Entry& en, int layer, const int32_t* experts, int n) const {
        if (en.layer != layer) return false;
        for (int i = 0; i < n; ++i)
            if (experts[i] == en.expert) return true;
        return false;
    }

    // free slots plus evictable slots (not holding a requested expert) in the range
    int obtainable(int layer, const int32_t* experts, int n) const {
        int c = 0;
        for (int s = lo(layer); s < hi(layer); ++s) {
            const Entry& en = slots_[s];
            if (en.layer < 0 || (evictable(en) && !requested(en, layer, experts, n))) ++c;
        }
        return c;
    }

    // lowest free slot, else the least recently used evictable slot that holds
    // none of the experts of the current request
    int take_slot(Engine&, int layer, const int32_t* experts = nullptr, int n = 0) {
        for (int s = lo(layer); s < hi(layer); ++s)
            if (slots_[s].layer < 0) return s;
        int best = -1;
        for (int s = lo(layer); s < hi(layer); ++s) {
            const Entry& en = slots_[s];
            if (!evictable(en) || requested(en, layer, experts, n)) continue;
            if (best < 0 || en.last < slots_[best].last) best = s;
        }
        if (best >= 0) {
            drop(best);
            st_.evictions++;
        }
        return best;
    }

    void drop(int s) {
        Entry& en = slots_[s];
        if (en.layer >= 0) where_[(size_t)en.layer * E_ + en.expert] = -1;
        en = Entry{};
    }

    bool start_copy(Engine& eng, int s, int layer, int e) {
        if (!eng.copy(s, layer, e)) return false;
        Entry& en = slots_[s];
        en.layer = layer;
        en.expert = e;
        en.copying = true;
        en.prefetched = false;
        where_[(size_t)layer * E_ + e] = s;
        return true;
    }
};

}  // namespace ftp
