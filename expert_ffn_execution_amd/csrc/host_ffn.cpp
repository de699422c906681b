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
// Weight rows are split over a small persistent thread pool (gate/up rows of
// every expert of the job, then down rows); each dot product keeps 16
// separate fp32 partial sums so that the compiler can vectorise it without
// reassociating, and the partial sums are added in a fixed order
// (deterministic whatever the thread count or the job's expert list: every
// output element is one thread's one dot product).
//
// ft_host_moe_ffn_submit queues a whole layer's CPU share as one job for a
// dispatcher thread, so the caller's thread only enqueues and later waits
// (a decode step's CPU experts then overlap the GPU's copies and kernels).
//
// Plain host C++ (built with the host compiler, no device pass): only the C
// header and the library's error helpers.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <deque>
#include <memory>
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

inline void cpu_relax() {
#if defined(__x86_64__) || defined(__i386__)
    __builtin_ia32_pause();
#endif
}

// Spin until pred() holds or about kSpinUs microseconds have passed; true if it held.
constexpr int kSpinUs = 250;
template <class P>
bool spin_until(P pred) {
    const auto t0 = std::chrono::steady_clock::now();
    for (;;) {
        for (int i = 0; i < 64; ++i) {
            if (pred()) return true;
            cpu_relax();
        }
        if (std::chrono::steady_clock::now() - t0 > std::chrono::microseconds(kSpinUs)) return pred();
    }
}

// ---- a persistent pool: run(n, f) calls f(0..n-1) on n threads (the caller is 0).
// Workers spin for up to kSpinUs after each job before sleeping (a decode
// step brings a layer's job about every 0.2 ms), so the
// back-to-back phases of one job (and a next job soon after) start without a
// wake-up from the kernel.
class Pool {
public:
    ~Pool() {
        {
            std::lock_guard<std::mutex> g(mu_);
            stop_ = true;
            agen_.store(~0u, std::memory_order_release);
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
            pending_.store(n - 1, std::memory_order_relaxed);
            ++gen_;
            agen_.store(gen_, std::memory_order_release);
        }
        cv_.notify_all();
        f(0);
        if (!spin_until([&] { return pending_.load(std::memory_order_acquire) == 0; })) {
            std::unique_lock<std::mutex> g(mu_);
            done_.wait(g, [&] { return pending_.load(std::memory_order_acquire) == 0; });
        }
        std::lock_guard<std::mutex> g(mu_);
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
            spin_until([&] { return agen_.load(std::memory_order_acquire) != seen; });
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
            if (pending_.fetch_sub(1, std::memory_order_acq_rel) == 1) {
                std::lock_guard<std::mutex> g(mu_);
                done_.notify_all();
            }
        }
    }
    std::vector<std::thread> th_;
    std::mutex mu_, call_mu_;
    std::condition_variable cv_, done_;
    const std::function<void(int)>* job_ = nullptr;
    unsigned gen_ = 0;
    std::atomic<unsigned> agen_{0};
    std::atomic<int> pending_{0};
    int active_ = 0;
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

// one expert's share of a job: its slot, its output rows [b, b + n) and the
// first of its rows in the aligned order
struct Span {
    const uint16_t* w;
    int b, n, lo;
};

// out[b + r] = FFN(xf[b + r]) for every span; xf [rows][H], hf [rows][I] scratch.
// Gate/up weight rows of all spans are split over the threads in contiguous
// ranges, then the down rows likewise.
void ffn_spans(const std::vector<Span>& sp, int H, int I, const float* xf, float* hf, float* out,
               int nt) {
    static const DotFn dot = pick_dot();
    const long n_sp = (long)sp.size();
    pool().run(nt, [&](int t) {
        const long u0 = n_sp * I * t / nt, u1 = n_sp * I * (t + 1) / nt;
        for (long u = u0; u < u1; ++u) {
            const Span& s = sp[u / I];
            const int i = (int)(u % I);
            const uint16_t* wg = s.w + (size_t)i * H;
            const uint16_t* wu = s.w + (size_t)I * H + (size_t)i * H;
            for (int r = 0; r < s.n; ++r) {
                const float* a = xf + (size_t)(s.b + r) * H;
                const float g = dot(wg, a, H);
                const float v = dot(wu, a, H);
                hf[(size_t)(s.b + r) * I + i] = round_bf16(g / (1.0f + std::exp(-g)) * v);
            }
        }
    });
    pool().run(nt, [&](int t) {
        const long u0 = n_sp * H * t / nt, u1 = n_sp * H * (t + 1) / nt;
        for (long u = u0; u < u1; ++u) {
            const Span& s = sp[u / H];
            const int d = (int)(u % H);
            const uint16_t* wd = s.w + 2 * (size_t)I * H + (size_t)d * I;
            for (int r = 0; r < s.n; ++r)
                out[(size_t)(s.b + r) * H + d] = dot(wd, hf + (size_t)(s.b + r) * I, I);
        }
    });
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
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    std::vector<float> xf((size_t)T * H), hf((size_t)T * I);
    for (size_t i = 0; i < xf.size(); ++i) xf[i] = bf16_to_f32(xb[i]);
    ffn_spans({Span{static_cast<const uint16_t*>(slot), 0, T, 0}}, H, I, xf.data(), hf.data(), y, n_threads);
    return FT_OK;
}

// ---------------------------------------------------------------------------
// asynchronous jobs: one dispatcher thread runs queued jobs in order
struct ft_host_job_s {
    ft_host_moe_job_desc d;
    std::vector<Span> spans;
    std::vector<int32_t> src;  // token of each output row
    int n_rows = 0;
    std::mutex mu;
    std::condition_variable cv;
    bool done = false;
    ft_status st = FT_OK;
};

namespace {

void run_job(ft_host_job* j) {
    const ft_host_moe_job_desc& d = j->d;
    const int H = d.H, I = d.I, n = j->n_rows;
    const uint16_t* xb = static_cast<const uint16_t*>(d.x);
    std::vector<float> xf((size_t)n * H), hf((size_t)n * I);
    const int nt = d.n_threads;
    pool().run(nt, [&](int t) {  // gather and widen the rows' inputs
        for (long r = (long)n * t / nt; r < (long)n * (t + 1) / nt; ++r) {
            const uint16_t* src = xb + (size_t)j->src[r] * H;
            float* dst = xf.data() + (size_t)r * H;
            for (int c = 0; c < H; ++c) dst[c] = bf16_to_f32(src[c]);
        }
    });
    ffn_spans(j->spans, H, I, xf.data(), hf.data(), d.rows, nt);
}

class Dispatcher {
public:
    Dispatcher() {
        pool();  // constructed first, so destroyed after this dispatcher
        th_ = std::thread([this] { loop(); });
    }
    ~Dispatcher() {
        {
            std::lock_guard<std::mutex> g(mu_);
            stop_ = true;
        }
        cv_.notify_all();
        th_.join();
    }
    void submit(ft_host_job* j) {
        {
            std::lock_guard<std::mutex> g(mu_);
            q_.push_back(j);
        }
        cv_.notify_one();
    }

private:
    void loop() {
        for (;;) {
            ft_host_job* j;
            {
                std::unique_lock<std::mutex> g(mu_);
                cv_.wait(g, [&] { return stop_ || !q_.empty(); });
                if (q_.empty()) return;  // stopping with nothing queued
                j = q_.front();
                q_.pop_front();
            }
            run_job(j);
            {
                // notify under the job's lock: once it is released the waiter
                // may return and free the job (its condition variable too)
                std::lock_guard<std::mutex> g(j->mu);
                j->done = true;
                j->cv.notify_all();
            }
        }
    }
    std::thread th_;
    std::mutex mu_;
    std::condition_variable cv_;
    std::deque<ft_host_job*> q_;
    bool stop_ = false;
};

Dispatcher& dispatcher() {
    static Dispatcher d;
    return d;
}

}  // namespace

extern "C" ft_status ft_host_moe_ffn_submit(const ft_host_moe_job_desc* d, ft_host_job** job, int* n_rows) {
    ft::clear_error();
    HOST_CHECK_ARG(d && job && n_rows, "null descriptor / job / n_rows");
    *job = nullptr;
    *n_rows = 0;
    HOST_CHECK_ARG(d->w_dt == FT_BF16 && d->x_dt == FT_BF16, "host MoE FFN: bf16 weights and activations only");
    HOST_CHECK_ARG(d->H > 0 && d->I > 0 && d->H % 64 == 0 && d->I % 64 == 0,
                   "H and I must be positive multiples of 64");
    HOST_CHECK_ARG(d->E > 0 && d->k > 0 && d->k <= d->E && d->T >= 0 && d->n_experts >= 0 &&
                       d->n_experts <= d->E && d->max_rows >= 0,
                   "need E > 0, 0 < k <= E, T >= 0, 0 <= n_experts <= E, max_rows >= 0");
    HOST_CHECK_ARG(d->n_threads >= 1 && d->n_threads <= 256, "n_threads in [1, 256]");
    HOST_CHECK_ARG(d->slot_stride >= (size_t)3 * d->H * d->I * 2, "slot_stride below one bf16 expert");
    HOST_CHECK_ARG(d->n_experts == 0 || (d->experts && d->offsets && d->pool),
                   "null experts / offsets / pool");
    const long TK = (long)d->T * d->k;
    auto j = std::make_unique<ft_host_job>();
    j->d = *d;
    std::vector<char> seen(d->E, 0);
    int b = 0;
    for (int q = 0; q < d->n_experts; ++q) {
        const int e = d->experts[q];
        HOST_CHECK_ARG(e >= 0 && e < d->E && !seen[e], "experts must be distinct and in [0, E)");
        seen[e] = 1;
        const int lo = d->offsets[e], hi = d->offsets[e + 1];
        HOST_CHECK_ARG(0 <= lo && lo <= hi && hi <= TK, "offsets of expert %d out of [0, T*k]", e);
        if (hi == lo) continue;
        HOST_CHECK_ARG(d->perm && d->x, "null perm / x");
        if ((long)b + (hi - lo) > d->max_rows)
            return ft::set_error(FT_ERR_CAPACITY, "the experts hold more than max_rows = %d rows", d->max_rows);
        for (int r = lo; r < hi; ++r) {
            HOST_CHECK_ARG(d->perm[r] >= 0 && d->perm[r] < TK, "perm[%d] out of [0, T*k)", r);
            j->src.push_back(d->perm[r] / d->k);
        }
        j->spans.push_back(Span{reinterpret_cast<const uint16_t*>(static_cast<const char*>(d->pool) +
                                                                  (size_t)e * d->slot_stride),
                                b, hi - lo, lo});
        b += hi - lo;
    }
    HOST_CHECK_ARG(b == 0 || (d->rows && d->pos), "null rows / pos");
    for (const Span& s : j->spans)
        for (int r = 0; r < s.n; ++r) d->pos[s.b + r] = s.lo + r;
    j->n_rows = b;
    j->d.experts = nullptr;  // the list is not read after this call
    *n_rows = b;
    ft_host_job* h = j.release();
    if (b == 0) {
        h->done = true;  // nothing to compute
    } else {
        dispatcher().submit(h);
    }
    *job = h;
    return FT_OK;
}

extern "C" ft_status ft_host_job_wait(ft_host_job* job) {
    ft::clear_error();
    HOST_CHECK_ARG(job, "null job");
    {
        std::unique_lock<std::mutex> g(job->mu);
        job->cv.wait(g, [&] { return job->done; });
    }
    const ft_status st = job->st;
    delete job;
    return st;
}

// The split of a decode step's m missed experts (chenxutan.com article,
// "瓶颈为什么是带宽而不是容量", the q* strategy; freelamp.com article, section
// 2.1): n go over PCIe to the GPU (n W / Bp) while m - n are computed here
// from host memory ((m - n) W / Bh), at the same time.  The printed formula is
// garbled; balancing the two sides gives n* = m Bp / (Bp + Bh), and of the two
// integers around it the one whose slower side finishes sooner is taken (the
// lower one on a tie).
extern "C" int ft_split_misses(int m, double bp, double bh) {
    if (m <= 0) return 0;
    if (!(bh > 0.0)) return m;   // no host side: everything to the GPU
    if (!(bp > 0.0)) return 0;   // no link: everything on the host
    const double q = (double)m * bp / (bp + bh);
    int lo = (int)q;
    lo = lo < 0 ? 0 : lo > m ? m : lo;
    const int hi = lo + 1 > m ? m : lo + 1;
    auto cost = [&](int n) { return std::max(n / bp, (m - n) / bh); };
    return cost(lo) <= cost(hi) ? lo : hi;
}
