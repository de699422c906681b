// san_policy.cpp -- a seeded random walk over the slot-cache policy (through
// the test shim and its mock copy engine), built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_sanitizers.py.  Exits non-zero on
// a broken invariant; the sanitizers abort on a memory or UB error.
#include <cstdio>
#include <random>
#include <vector>

#include "policy_shim.cpp"

#define REQUIRE(c)                                                        \
    do {                                                                  \
        if (!(c)) {                                                       \
            std::fprintf(stderr, "invariant failed: %s (line %d)\n", #c, __LINE__); \
            return 1;                                                     \
        }                                                                 \
    } while (0)

static int walk(int L, int E, int S, int scope, unsigned seed) {
    void* h = pol_create(L, E, S, scope);
    std::mt19937 rng(seed);
    std::vector<int> slots(E), ex;
    int st4[4];
    long long stats[12];
    for (int step = 0; step < 4000; ++step) {
        const int layer = (int)(rng() % L);
        const int op = (int)(rng() % 10);
        ex.clear();
        const int want = 1 + (int)(rng() % (unsigned)(E < 6 ? E : 6));
        for (int e = 0; e < E && (int)ex.size() < want; ++e)
            if (rng() % 3 == 0) ex.push_back(e);
        if (op < 5) {
            const int r = pol_map(h, layer, ex.data(), (int)ex.size(), slots.data(), st4);
            REQUIRE(r == FT_OK || r == FT_ERR_CAPACITY);
            if (r == FT_OK) {
                for (size_t i = 0; i < ex.size(); ++i)  // slot of experts[i] in slots[i]
                    REQUIRE(slots[i] >= 0 && pol_lookup(h, layer, ex[i]) == slots[i]);
                REQUIRE(st4[1] + st4[2] + st4[3] == st4[0]);
            }
            REQUIRE(pol_release(h, layer) == FT_OK);
        } else if (op < 7) {
            int issued = 0;
            const int r = pol_prefetch(h, layer, ex.data(), (int)ex.size(), &issued);
            REQUIRE(r == FT_OK || r == FT_WARN_OVERLAP_DISABLED);
            REQUIRE(issued >= 0 && issued <= (int)ex.size());
        } else if (op == 7) {
            const int r = pol_evict(h, layer, (int)(rng() % (unsigned)(E + 1)) - 1);
            REQUIRE(r == FT_OK || r == FT_ERR_BUSY);
        } else if (op == 8) {
            pol_set_auto_complete(h, (int)(rng() & 1));
            pol_complete_all(h);
        } else if (scope == FT_SCOPE_GLOBAL) {
            pol_complete_all(h);
            const int ns = 1 + (int)(rng() % (unsigned)(2 * S));
            const int r = pol_resize(h, ns, (int)(rng() & 1));
            REQUIRE(r == FT_OK || r == FT_ERR_BUSY);
        }
        pol_stats(h, stats);
        REQUIRE(stats[8] <= stats[11]);              // resident <= slots
        REQUIRE(stats[2] + stats[3] + stats[4] == stats[1]);  // hits + prefetch hits + misses = demand
        std::vector<int> log(4 * 4096);
        REQUIRE(pol_log(h, log.data(), (int)log.size()) >= 0);
    }
    pol_destroy(h);
    return 0;
}

int main() {
    int rc = 0;
    rc |= walk(4, 16, 24, FT_SCOPE_GLOBAL, 1);
    rc |= walk(3, 8, 12, FT_SCOPE_PER_LAYER, 2);
    rc |= walk(8, 128, 512, FT_SCOPE_GLOBAL, 3);
    if (rc == 0) std::printf("policy walk ok\n");
    return rc;
}
