// pi_host.cpp -- the cold partition computed on the host cores.
//
// The pages' hybrid execution keeps the frequently active (hot) neurons on the
// GPU and computes the rest (cold) on the CPU, next to their weights in host
// memory; the two partial outputs are then merged (CSDN article, section on
// the CPU/GPU hybrid design and its figure; hada.io README summary,
// hybrid-approach section).  This file is that CPU side: the sparse FFN over a
// list of rows held in host memory, accumulated in fp32, on a persistent pool
// of worker threads, with AVX2 / F16C / FMA code chosen at run time when the
// processor has them.
//
// Work split: worker t takes the t-th contiguous run of the list and
// accumulates its own partial of y; the partials are then added element by
// element in worker order (the element ranges spread over the workers), so a
// call's result is reproducible for a given thread count.
//
// Built by the host compiler alone (no device code here).
#include "pi_host.h"

#include <immintrin.h>
#include <sched.h>
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

namespace pi {
namespace host {
namespace {

// Worker pool: run(n, fn) calls fn(t) for t in [0, n) on n threads (the
// caller takes t = 0) and returns when all are done.  Created on first use and
// never destroyed; its workers end with the process.  A worker that finished a
// job polls for the next one for SPIN_US before it blocks on a condition
// variable: decode steps call every few hundred microseconds, and waking a
// blocked thread costs tens of microseconds or more (more again under a
// hypervisor), which is the size of the work itself.
class Pool {
  public:
    static constexpr double SPIN_US = 2000.0;

    explicit Pool(int n) {
        size_ = n;
        for (int i = 1; i < n; ++i) std::thread([this, i] { loop(i); }).detach();
    }
    int size() const { return size_; }
    void run(int n, const std::function<void(int)>& fn) {
        n = std::max(1, std::min(n, size()));
        if (n == 1) {
            fn(0);
            return;
        }
        // every worker acknowledges every job (those with t >= n without running it),
        // so none can still be reading job_ or njob_ when the next call rewrites them
        job_ = &fn;
        njob_ = n;
        pending_.store(size() - 1, std::memory_order_relaxed);
        {
            // under the lock, so a worker about to block either sees the new
            // generation or is counted in sleepers_ before it is read below
            std::lock_guard<std::mutex> lk(m_);
            gen_.fetch_add(1, std::memory_order_release);
        }
        if (sleepers_.load(std::memory_order_acquire) > 0) cv_.notify_all();
        fn(0);
        while (pending_.load(std::memory_order_acquire) != 0) _mm_pause();
    }

  private:
    void loop(int i) {
        uint64_t seen = 0;
        for (;;) {
            auto t0 = std::chrono::steady_clock::now();
            uint64_t g;
            unsigned spins = 0;
            while ((g = gen_.load(std::memory_order_acquire)) == seen) {
                _mm_pause();
                if ((++spins & 1023u) == 0 &&
                    std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count() >
                        SPIN_US) {
                    std::unique_lock<std::mutex> lk(m_);
                    sleepers_.fetch_add(1, std::memory_order_acq_rel);
                    cv_.wait(lk, [&] { return gen_.load(std::memory_order_acquire) != seen; });
                    sleepers_.fetch_sub(1, std::memory_order_acq_rel);
                    t0 = std::chrono::steady_clock::now();
                }
            }
            seen = g;
            if (i < njob_) (*job_)(i);
            pending_.fetch_sub(1, std::memory_order_acq_rel);
        }
    }
    int size_ = 1;
    std::mutex m_;
    std::condition_variable cv_;
    std::atomic<uint64_t> gen_{0};
    std::atomic<int> pending_{0}, sleepers_{0};
    const std::function<void(int)>* job_ = nullptr;
    int njob_ = 0;
};

constexpr int MAX_THREADS = 64;

int allowed_cpus() {
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof(set), &set) == 0) return std::max(1, (int)CPU_COUNT(&set));
    return std::max(1, (int)std::thread::hardware_concurrency());
}

// The pool of this process.  A child created by fork() has none of its
// parent's worker threads: it builds a pool of its own on first use (the
// parent's copy is left alone).
Pool& pool() {
    static std::mutex mu;
    static Pool* p = nullptr;
    static pid_t owner = 0;
    std::lock_guard<std::mutex> lk(mu);
    if (!p || owner != getpid()) {
        p = new Pool(std::min(allowed_cpus(), MAX_THREADS));
        owner = getpid();
    }
    return *p;
}

// AVX2 + FMA + F16C code when the processor has it; PI_HOST_PLAIN=1 in the
// environment (read once) selects the portable code instead.
bool has_avx2() {
    static const bool ok = [] {
        const char* plain = std::getenv("PI_HOST_PLAIN");
        if (plain && plain[0] == '1') return false;
        return __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma") &&
               __builtin_cpu_supports("f16c");
    }();
    return ok;
}

// IEEE binary16 -> binary32, exact for every input (subnormals, inf, NaN)
float half_to_float(uint16_t h) {
    const uint32_t s = (uint32_t)(h & 0x8000u) << 16, e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
    uint32_t bits;
    if (e == 0) {
        const float f = (float)m * 5.9604644775390625e-8f;    // m * 2^-24, exact
        std::memcpy(&bits, &f, 4);
        bits |= s;
    } else if (e == 31) {
        bits = s | 0x7f800000u | (m << 13);
    } else {
        bits = s | ((e + 112u) << 23) | (m << 13);
    }
    float f;
    std::memcpy(&f, &bits, 4);
    return f;
}

int64_t row_bytes(int wt, int d) {
    return wt == PI_F32 ? 4LL * d : wt == PI_F16 ? 2LL * d : (int64_t)d / 2 + (int64_t)d / 16;
}

// ---- one row's weights, eight at a time ------------------------------------------
// Elements k .. k+7 (k % 8 == 0) of a row as fp32.  A Q4_0 row holds d/2 code
// bytes then d/32 fp16 scales; element t of block j is the low nibble of code
// byte 16 j + t (t < 16) or the high nibble of byte 16 j + t - 16, and its value
// is (code - 8) * scale_j.
template <int WT> struct Row8;

template <> struct Row8<PI_F32> {
    __attribute__((target("avx2,fma,f16c"))) static __m256 avx(const uint8_t* row, int, int k) {
        return _mm256_loadu_ps(reinterpret_cast<const float*>(row) + k);
    }
    static void plain(const uint8_t* row, int, int k, float* w) {
        std::memcpy(w, row + 4 * (int64_t)k, 32);
    }
};

template <> struct Row8<PI_F16> {
    __attribute__((target("avx2,fma,f16c"))) static __m256 avx(const uint8_t* row, int, int k) {
        return _mm256_cvtph_ps(_mm_loadu_si128(reinterpret_cast<const __m128i*>(row + 2 * (int64_t)k)));
    }
    static void plain(const uint8_t* row, int, int k, float* w) {
        for (int e = 0; e < 8; ++e) {
            uint16_t h;
            std::memcpy(&h, row + 2 * ((int64_t)k + e), 2);
            w[e] = half_to_float(h);
        }
    }
};

template <> struct Row8<PI_Q4_0> {
    __attribute__((target("avx2,fma,f16c"))) static __m256 avx(const uint8_t* row, int d, int k) {
        const int j = k >> 5, t = k & 31;
        uint64_t c8;
        std::memcpy(&c8, row + 16 * (int64_t)j + (t & 15), 8);
        if (t >= 16) c8 >>= 4;
        const __m256i q = _mm256_and_si256(_mm256_cvtepu8_epi32(_mm_cvtsi64_si128((long long)c8)),
                                           _mm256_set1_epi32(15));
        uint16_t sh;
        std::memcpy(&sh, row + d / 2 + 2 * (int64_t)j, 2);
        const __m256 s = _mm256_set1_ps(_cvtsh_ss(sh));
        return _mm256_mul_ps(_mm256_cvtepi32_ps(_mm256_sub_epi32(q, _mm256_set1_epi32(8))), s);
    }
    static void plain(const uint8_t* row, int d, int k, float* w) {
        const int j = k >> 5, t = k & 31;
        uint16_t sh;
        std::memcpy(&sh, row + d / 2 + 2 * (int64_t)j, 2);
        const float s = half_to_float(sh);
        for (int e = 0; e < 8; ++e) {
            const int te = t + e;
            const uint8_t c = row[16 * (int64_t)j + (te & 15)];
            w[e] = (float)((te < 16 ? (c & 15) : (c >> 4)) - 8) * s;
        }
    }
};

// ---- per-row products --------------------------------------------------------------
// dot[b] = row . xs[b] for the B tokens of xs (fp32 [B][d]); four accumulators
// per token (d % 64 == 0, so the 32-element steps tile the row)
template <int WT>
__attribute__((target("avx2,fma,f16c"))) void dots_avx(const uint8_t* row, int d, const float* xs, int B,
                                                        float* dot) {
    for (int b = 0; b < B; ++b) {
        const float* x = xs + (int64_t)b * d;
        __m256 a0 = _mm256_setzero_ps(), a1 = a0, a2 = a0, a3 = a0;
        for (int k = 0; k < d; k += 32) {
            a0 = _mm256_fmadd_ps(Row8<WT>::avx(row, d, k), _mm256_loadu_ps(x + k), a0);
            a1 = _mm256_fmadd_ps(Row8<WT>::avx(row, d, k + 8), _mm256_loadu_ps(x + k + 8), a1);
            a2 = _mm256_fmadd_ps(Row8<WT>::avx(row, d, k + 16), _mm256_loadu_ps(x + k + 16), a2);
            a3 = _mm256_fmadd_ps(Row8<WT>::avx(row, d, k + 24), _mm256_loadu_ps(x + k + 24), a3);
        }
        const __m256 s = _mm256_add_ps(_mm256_add_ps(a0, a1), _mm256_add_ps(a2, a3));
        alignas(32) float t[8];
        _mm256_store_ps(t, s);
        dot[b] = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
    }
}

// y[b] += h[b] * row, for the tokens with h[b] != 0
template <int WT>
__attribute__((target("avx2,fma,f16c"))) void axpys_avx(const uint8_t* row, int d, const float* h, int B,
                                                         float* y) {
    for (int k = 0; k < d; k += 8) {
        const __m256 w = Row8<WT>::avx(row, d, k);
        for (int b = 0; b < B; ++b) {
            if (h[b] == 0.0f) continue;
            float* yb = y + (int64_t)b * d + k;
            _mm256_storeu_ps(yb, _mm256_fmadd_ps(_mm256_set1_ps(h[b]), w, _mm256_loadu_ps(yb)));
        }
    }
}

template <int WT>
void dots_plain(const uint8_t* row, int d, const float* xs, int B, float* dot) {
    float w[8];
    for (int b = 0; b < B; ++b) dot[b] = 0.0f;
    for (int k = 0; k < d; k += 8) {
        Row8<WT>::plain(row, d, k, w);
        for (int b = 0; b < B; ++b)
            for (int e = 0; e < 8; ++e) dot[b] += w[e] * xs[(int64_t)b * d + k + e];
    }
}

template <int WT>
void axpys_plain(const uint8_t* row, int d, const float* h, int B, float* y) {
    float w[8];
    for (int k = 0; k < d; k += 8) {
        Row8<WT>::plain(row, d, k, w);
        for (int b = 0; b < B; ++b)
            if (h[b] != 0.0f)
                for (int e = 0; e < 8; ++e) y[(int64_t)b * d + k + e] += h[b] * w[e];
    }
}

// Entries idx[lo .. hi) of the list into y (fp32 [B][d], accumulated).  Per
// row: the up (and gate) dot products for every token, the activation, then
// the down row scaled by h into y (CSDN article, section on sparse activation:
// a neuron that does not fire adds nothing, so its down row is skipped).
constexpr int64_t PREFETCH_BYTES = 2048;

template <int WT>
void rows_range(const pi_ffn_part& p, const float* xs, int B, const int32_t* idx, int lo, int hi, float* y,
                bool avx) {
    const int d = p.d;
    const int64_t rb = row_bytes(WT, d);
    float up[PI_MAX_BATCH], gate[PI_MAX_BATCH], h[PI_MAX_BATCH];
    const uint8_t* Wu = static_cast<const uint8_t*>(p.W_up);
    const uint8_t* Wg = static_cast<const uint8_t*>(p.W_gate);
    const uint8_t* Wd = static_cast<const uint8_t*>(p.W_downT);
    for (int e = lo; e < hi; ++e) {
        const int row = idx[e];
        if (row < 0 || row >= p.rows) continue;        // not a row of this partition: nothing
        if (e + 1 < hi) {
            // the start of the next listed rows, while this one streams: the hardware
            // prefetchers pick a row up only after its first misses
            const int nx = idx[e + 1];
            if (nx >= 0 && nx < p.rows) {
                for (int64_t o = 0; o < std::min<int64_t>(rb, PREFETCH_BYTES); o += 64) {
                    __builtin_prefetch(Wu + nx * rb + o);
                    __builtin_prefetch(Wd + nx * rb + o);
                    if (p.act == PI_REGLU) __builtin_prefetch(Wg + nx * rb + o);
                }
            }
        }
        if (avx) dots_avx<WT>(Wu + row * rb, d, xs, B, up);
        else dots_plain<WT>(Wu + row * rb, d, xs, B, up);
        if (p.act == PI_REGLU) {
            if (avx) dots_avx<WT>(Wg + row * rb, d, xs, B, gate);
            else dots_plain<WT>(Wg + row * rb, d, xs, B, gate);
        }
        bool any = false;
        for (int b = 0; b < B; ++b) {
            const float u = up[b] + (p.b_up ? p.b_up[row] : 0.0f);
            float v;
            if (p.act == PI_RELU) {
                v = u > 0.0f ? u : 0.0f;
            } else if (p.act == PI_SQRELU) {
                const float r = u > 0.0f ? u : 0.0f;
                v = r * r;
            } else {
                const float g = gate[b] + (p.b_gate ? p.b_gate[row] : 0.0f);
                v = (g > 0.0f ? g : 0.0f) * u;
            }
            h[b] = v;
            any |= v != 0.0f;
        }
        if (!any) continue;
        if (avx) axpys_avx<WT>(Wd + row * rb, d, h, B, y);
        else axpys_plain<WT>(Wd + row * rb, d, h, B, y);
    }
}

__attribute__((target("avx2,fma,f16c"))) void halves_to_floats_avx(const uint16_t* src, int64_t len, float* dst) {
    int64_t i = 0;
    for (; i + 8 <= len; i += 8)
        _mm256_storeu_ps(dst + i, _mm256_cvtph_ps(_mm_loadu_si128(reinterpret_cast<const __m128i*>(src + i))));
    for (; i < len; ++i) dst[i] = half_to_float(src[i]);
}

// Buffers reused across calls (grown on demand); calls are serialised.
std::mutex g_call;
std::vector<float> g_x, g_part;

}  // namespace

int threads_available() { return pool().size(); }

void sparse_ffn(const pi_ffn_part& p, const void* x, int B, int xdtype, const int32_t* idx, int count, float* y,
                int nthreads) {
    std::lock_guard<std::mutex> call(g_call);
    const int d = p.d;
    const int64_t len = (int64_t)B * d;
    const bool avx = has_avx2();
    const float* xs;
    if (xdtype == PI_F32) {
        xs = static_cast<const float*>(x);
    } else {
        if ((int64_t)g_x.size() < len) g_x.resize(len);
        if (avx) {
            halves_to_floats_avx(static_cast<const uint16_t*>(x), len, g_x.data());
        } else {
            const uint16_t* xh = static_cast<const uint16_t*>(x);
            for (int64_t i = 0; i < len; ++i) g_x[i] = half_to_float(xh[i]);
        }
        xs = g_x.data();
    }
    count = std::max(count, 0);
    Pool& P = pool();
    const int want = nthreads > 0 ? nthreads : P.size();
    const int n = std::max(1, std::min({want, P.size(), std::max(count, 1)}));
    float* part;
    if (n == 1) {
        part = y;                                   // a single worker accumulates into y itself
    } else {
        if ((int64_t)g_part.size() < n * len) g_part.resize((size_t)n * len);
        part = g_part.data();
    }
    P.run(n, [&](int t) {
        float* yt = part + (size_t)t * len;
        std::fill(yt, yt + len, 0.0f);
        const int lo = (int)((int64_t)count * t / n), hi = (int)((int64_t)count * (t + 1) / n);
        if (p.wdtype == PI_F32) rows_range<PI_F32>(p, xs, B, idx, lo, hi, yt, avx);
        else if (p.wdtype == PI_F16) rows_range<PI_F16>(p, xs, B, idx, lo, hi, yt, avx);
        else rows_range<PI_Q4_0>(p, xs, B, idx, lo, hi, yt, avx);
    });
    if (n == 1) return;
    // y = partial 0 + partial 1 + ... in that order, element ranges split over the workers
    P.run(n, [&](int t) {
        const int64_t a = len * t / n, b = len * (t + 1) / n;
        for (int64_t i = a; i < b; ++i) {
            float s = part[i];
            for (int u = 1; u < n; ++u) s += part[(size_t)u * len + i];
            y[i] = s;
        }
    });
}

int cold_list(const uint64_t* mask, int n_hot, int n, int32_t* out) {
    int c = 0;
    for (int i = n_hot; i < n;) {
        const int w = i >> 6, lo = i & 63;
        uint64_t v = mask[w] >> lo;
        const int span = std::min(64 - lo, n - i);
        if (span < 64) v &= (1ull << span) - 1ull;
        while (v) {
            out[c++] = i + __builtin_ctzll(v) - n_hot;
            v &= v - 1;
        }
        i += span;
    }
    return c;
}

}  // namespace host
}  // namespace pi
