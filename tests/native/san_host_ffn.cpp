// san_host_ffn.cpp -- the host expert FFN and its job queue (csrc/host_ffn.cpp)
// under AddressSanitizer + UndefinedBehaviorSanitizer or ThreadSanitizer,
// built by tests/test_sanitizers.py.  One expert's FFN must give the same
// bits for any thread count, and jobs submitted from several threads at once
// must each give the bits of the same job run alone.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <thread>
#include <vector>

#include "ftmoe.h"

// the library's error helpers (defined in api.cpp, which needs HIP)
namespace ft {
static thread_local char g_msg[256];
ft_status set_error(ft_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_msg, sizeof g_msg, fmt, ap);
    va_end(ap);
    return st;
}
void clear_error() { g_msg[0] = 0; }
}  // namespace ft

#define REQUIRE(c)                                                        \
    do {                                                                  \
        if (!(c)) {                                                       \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            std::exit(1);                                                 \
        }                                                                 \
    } while (0)

static uint16_t bf16_of(float f) {  // truncation is enough for test data
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

int main() {
    const int E = 6, H = 256, I = 128, k = 2, T = 10;
    const size_t bytes = 3 * (size_t)H * I * 2;  // bf16 slot: gate | up | down
    std::mt19937 rng(7);
    std::normal_distribution<float> nd(0.f, 0.1f);
    std::vector<uint16_t> pool(E * bytes / 2), x(T * H);
    for (auto& v : pool) v = bf16_of(nd(rng));
    for (auto& v : x) v = bf16_of(nd(rng) * 10.f);
    // one expert, 1 and 4 threads: same bits
    std::vector<float> y1(T * H), y4(T * H);
    REQUIRE(ft_host_expert_ffn(FT_BF16, H, I, pool.data(), x.data(), FT_BF16, T, y1.data(), 1) == FT_OK);
    REQUIRE(ft_host_expert_ffn(FT_BF16, H, I, pool.data(), x.data(), FT_BF16, T, y4.data(), 4) == FT_OK);
    REQUIRE(std::memcmp(y1.data(), y4.data(), y1.size() * 4) == 0);
    REQUIRE(ft_host_expert_ffn(FT_MXFP4, H, I, pool.data(), x.data(), FT_BF16, T, y4.data(), 4) ==
            FT_ERR_INVALID_ARG);
    // an alignment: token t picks experts t % E and (t + 1) % E
    std::vector<int32_t> ids(T * k), offsets(E + 1, 0), perm(T * k);
    for (int t = 0; t < T; ++t) ids[t * k] = t % E, ids[t * k + 1] = (t + 1) % E;
    for (int f = 0; f < T * k; ++f) offsets[ids[f] + 1]++;
    for (int e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
    {
        std::vector<int32_t> fill(offsets.begin(), offsets.end() - 1);
        for (int f = 0; f < T * k; ++f) perm[fill[ids[f]]++] = f;
    }
    auto run_job = [&](const std::vector<int32_t>& experts, std::vector<float>& rows,
                       std::vector<int64_t>& pos) {
        ft_host_moe_job_desc d{};
        d.w_dt = FT_BF16;
        d.E = E, d.H = H, d.I = I, d.k = k;
        d.pool = pool.data();
        d.slot_stride = bytes;
        d.experts = experts.data();
        d.n_experts = (int)experts.size();
        d.offsets = offsets.data();
        d.perm = perm.data();
        d.x = x.data();
        d.x_dt = FT_BF16;
        d.T = T;
        rows.assign((size_t)T * k * H, 0.f);
        pos.assign(T * k, -1);
        d.rows = rows.data();
        d.pos = pos.data();
        d.max_rows = T * k;
        d.n_threads = 3;
        ft_host_job* job = nullptr;
        int n = 0;
        REQUIRE(ft_host_moe_ffn_submit(&d, &job, &n) == FT_OK);
        REQUIRE(ft_host_job_wait(job) == FT_OK);
        return n;
    };
    const std::vector<std::vector<int32_t>> lists = {{0, 3}, {5, 1}, {2}, {4, 0, 1}};
    std::vector<std::vector<float>> want_rows(lists.size());
    std::vector<std::vector<int64_t>> want_pos(lists.size());
    std::vector<int> want_n(lists.size());
    for (size_t i = 0; i < lists.size(); ++i) want_n[i] = run_job(lists[i], want_rows[i], want_pos[i]);
    std::vector<std::thread> ths;
    std::vector<int> bad(lists.size(), 0);
    for (size_t i = 0; i < lists.size(); ++i)
        ths.emplace_back([&, i] {
            std::vector<float> rows;
            std::vector<int64_t> pos;
            for (int rep = 0; rep < 4; ++rep) {
                const int n = run_job(lists[i], rows, pos);
                if (n != want_n[i] || std::memcmp(rows.data(), want_rows[i].data(), (size_t)n * H * 4) ||
                    std::memcmp(pos.data(), want_pos[i].data(), (size_t)n * 8))
                    bad[i] = 1;
            }
        });
    for (auto& t : ths) t.join();
    for (int b : bad) REQUIRE(b == 0);
    std::printf("host ffn ok\n");
    return 0;
}
