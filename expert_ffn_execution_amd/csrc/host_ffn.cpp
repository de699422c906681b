// host_ffn.cpp -- one expert's SwiGLU FFN on host cores, straight from an
// expert slot in (pinned) host memory: the CPU side of the bandwidth-adaptive
// split of cache misses.
//
// The pages describe a hybrid MoE backend that, at each decode step, sends part
// of the experts that missed the GPU's slot cache over PCIe to the GPU and
// computes the rest on the CPU from host memory, both at once, in the ratio of
// the two measured bandwidths so that both sides finish together
// (chenxutan.com article, "瓶颈为什么是带宽而不是容量", the q* strategy and the
// MoE backend list; freelamp.com article section 2.1, the q* strategy).  The
// split itself is host scheduling (the slot stack); this file is the CPU's
// share of the arithmetic.
//
// Arithmetic as on the GPU: bf16 weights and activations, fp32 sums, h =
// silu(g) * u rounded to bf16 before the down projection, fp32 output rows.
// Rows are split over a small persistent thread pool (gate/up rows, then down
// rows); each dot product keeps 16 separate fp32 partial sums so that the
// compiler can vectorise it without reassociating, and the partial sums are
// added in a fixed order (deterministic whatever the thread count: every row
// is summed by one thread).
//
// Plain host C++ (built with the host compiler, no device pass): only the C
// header and the library's error helpers.
#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "ftmoe.h"

namespace ft {
ft_status set_error(ft_status st, const char* fmt, ...);
void clear_error();
}  // namespace ft

#define HOST_CHECK_ARG(cond, ...) \
    do {                         \
        if (!(cond)) return ::ft::set_error(FT_ERR_INVALID_ARG, __VA_ARGS__); \
    } while (0)

namespace {

// ---- a persistent pool: run(n, f) calls f(0..n-1) on n threads (the caller is 0)
class Pool {
public:
    ~Pool() {
        {
            std::lock_guard<std::mutex> g(mu_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto& t : th_) t.join();
    }
    void run(int n, const std::function<void(int)>& f) {
        std::lock_guard<std::mutex> one(call_mu_);  // one job at a time
        grow(n - 1);
        {
            std::lock_guard<std::mutex> g(mu_);
            job_ = &f;
            active_ = n - 1;
            pending_ = n - 1;
            ++gen_;
        }
        cv_.notify_all();
        f(0);
        std::unique_lock<std::mutex> g(mu_);
        done_.wait(g, [&] { return pending_ == 0; });
        job_ = nullptr;
    }

private:
    void grow(int want) {
        while ((int)th_.size() < want) {
            const int id = (int)th_.size() + 1;
            th_.emplace_back([this, id] { loop(id); });
        }
    }
    void loop(int id) {
        unsigned seen = 0;
        for (;;) {
            const std::function<void(int)>* f;
            {
                std::unique_lock<std::mutex> g(mu_);
                cv_.wait(g, [&] { return stop_ || gen_ != seen; });
                if (stop_) return;
                seen = gen_;
                if (id > active_) continue;  // not part of this job
                f = job_;
            }
            (*f)(id);
            std::lock_guard<std::mutex> g(mu_);
            if (--pending_ == 0) done_.notify_all();
        }
    }
    std::vector<std::thread> th_;
    std::mutex mu_, call_mu_;
    std::condition_variable cv_, done_;
    const std::function<void(int)>* job_ = nullptr;
    unsigned gen_ = 0;
    int active_ = 0, pending_ = 0;
    bool stop_ = false;
};

Pool& pool() {
    static Pool p;
    return p;
}

inline float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}
inline float round_bf16(float f) {  // to the nearest bf16 (ties to even), as a float
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return f;  // NaN
    u = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
    std::memcpy(&f, &u, 4);
    return f;
}

// sum_k w[k] * a[k], w bf16, a fp32, n % 16 == 0
template <int V>
inline float dot_bf16(const uint16_t* __restrict__ w, const float* __restrict__ a, int n) {
    float acc[V];
    for (int j = 0; j < V; ++j) acc[j] = 0.f;
    for (int k = 0; k < n; k += V)
        for (int j = 0; j < V; ++j) acc[j] += bf16_to_f32(w[k + j]) * a[k + j];
    float s = 0.f;
    for (int j = 0; j < V; ++j) s += acc[j];
    return s;
}
__attribute__((target("avx2,fma"))) float dot_avx2(const uint16_t* w, const float* a, int n) {
    return dot_bf16<16>(w, a, n);
}
float dot_generic(const uint16_t* w, const float* a, int n) { return dot_bf16<16>(w, a, n); }

using DotFn = float (*)(const uint16_t*, const float*, int);
DotFn pick_dot() {
    __builtin_cpu_init();
    return (__builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma")) ? dot_avx2 : dot_generic;
}

}  // namespace

extern "C" ft_status ft_host_expert_ffn(ft_dtype w_dt, int H, int I, const void* slot, const void* x,
                                        ft_dtype x_dt, int T, float* y, int n_threads) {
    ft::clear_error();
    HOST_CHECK_ARG(w_dt == FT_BF16 && x_dt == FT_BF16, "host FFN: bf16 weights and activations only");
    HOST_CHECK_ARG(H > 0 && I > 0 && H % 64 == 0 && I % 64 == 0, "H and I must be positive multiples of 64");
    HOST_CHECK_ARG(T >= 0 && n_threads >= 1 && n_threads <= 256, "T >= 0 and n_threads in [1, 256]");
    HOST_CHECK_ARG(T == 0 || (slot && x && y), "null slot / x / y");
    if (T == 0) return FT_OK;
    static const DotFn dot = pick_dot();
    const uint16_t* wg = static_cast<const uint16_t*>(slot);
    const uint16_t* wu = wg + (size_t)I * H;
    const uint16_t* wd = wu + (size_t)I * H;
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    std::vector<float> xf((size_t)T * H), hf((size_t)T * I);
    for (size_t i = 0; i < xf.size(); ++i) xf[i] = bf16_to_f32(xb[i]);
    const int nt = n_threads;
    // gate/up rows, then down rows, each split over the threads in contiguous ranges
    pool().run(nt, [&](int t) {
        const int i0 = (int)((long)I * t / nt), i1 = (int)((long)I * (t + 1) / nt);
        for (int i = i0; i < i1; ++i)
            for (int r = 0; r < T; ++r) {
                const float g = dot(wg + (size_t)i * H, xf.data() + (size_t)r * H, H);
                const float u = dot(wu + (size_t)i * H, xf.data() + (size_t)r * H, H);
                hf[(size_t)r * I + i] = round_bf16(g / (1.0f + std::exp(-g)) * u);
            }
    });
    pool().run(nt, [&](int t) {
        const int d0 = (int)((long)H * t / nt), d1 = (int)((long)H * (t + 1) / nt);
        for (int d = d0; d < d1; ++d)
            for (int r = 0; r < T; ++r) y[(size_t)r * H + d] = dot(wd + (size_t)d * I, hf.data() + (size_t)r * I, I);
    });
    return FT_OK;
}
