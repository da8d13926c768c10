// Host kernels: bf16 working-copy cast, AdamW, gradient-slab accumulation,
// embedding gather / scatter-add, RoPE table.
//
// The optimizer runs on the CPU where the fp32 master, grad and Adam m/v live,
// so optimizer state is never moved to the GPU (zhichai.net
// "MegaTrain：单卡训百亿大模型的突破与实践", design point 1; m.lqnn.cn MegaTrain
// article, 二: SIMD CPU Adam over ParameterState).  A CPU worker adds each
// gradient slab into the fp32 host gradient (lqnn 三.3).
//
// Arithmetic order is fixed and written out (compiled without FP contraction)
// so results do not depend on the thread count.
#include "host_ops.h"

#include <immintrin.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <chrono>

namespace mt {

ThreadPool::ThreadPool(int n) {
  for (int i = 1; i < n; ++i) workers_.emplace_back([this] { loop(); });
}

ThreadPool::~ThreadPool() {
  {
    std::lock_guard<std::mutex> g(mu_);
    stop_ = true;
  }
  cv_.notify_all();
  for (auto& t : workers_) t.join();
}

void ThreadPool::loop() {
  uint64_t seen = 0;
  for (;;) {
    std::unique_lock<std::mutex> lk(mu_);
    cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
    if (stop_) return;
    seen = gen_;
    for (;;) {
      if (next_ >= n_) break;
      int64_t i = next_++;
      lk.unlock();
      (*fn_)(i);
      lk.lock();
      if (--pending_ == 0) done_cv_.notify_all();
    }
  }
}

void ThreadPool::run(int64_t n, const std::function<void(int64_t)>& fn) {
  if (n <= 0) return;
  std::lock_guard<std::mutex> rg(run_mu_);
  std::unique_lock<std::mutex> lk(mu_);
  fn_ = &fn;
  n_ = n;
  next_ = 0;
  pending_ = n;
  ++gen_;
  cv_.notify_all();
  for (;;) {
    if (next_ >= n_) break;
    int64_t i = next_++;
    lk.unlock();
    fn(i);
    lk.lock();
    --pending_;
  }
  done_cv_.wait(lk, [&] { return pending_ == 0; });
  fn_ = nullptr;
  n_ = 0;
}

int default_threads() {
  unsigned hc = std::thread::hardware_concurrency();
  int n = hc ? (int)hc : 4;
  return std::max(1, std::min(n, 16));
}

// Round to nearest even; NaN stays a (quiet) NaN.  Branch-free so that the
// loops calling it vectorise.
static inline uint16_t rne_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t q = (u >> 16) | 0x40u;
  return (uint16_t)(((u & 0x7fffffffu) > 0x7f800000u) ? q : r);
}

static constexpr int64_t kChunk = 1 << 18;  // elements per task
static constexpr int64_t kStage = 2048;     // elements staged in L1 before a streaming copy-out

// Copies an L1-resident staging block to dst with non-temporal stores for its
// 32-byte-aligned middle.  Lines that a loop only writes then go to memory
// without first being read into the cache (no read-for-ownership), which
// would otherwise add their size again to the host-memory traffic.  The
// caller issues an sfence before the data is handed on.
static inline void stream_out(void* dst, const void* src, size_t bytes) {
  char* d = static_cast<char*>(dst);
  const char* s = static_cast<const char*>(src);
  size_t head = (32 - ((uintptr_t)d & 31)) & 31;
  if (head > bytes) head = bytes;
  memcpy(d, s, head);
  d += head;
  s += head;
  bytes -= head;
  for (; bytes >= 32; bytes -= 32, d += 32, s += 32)
    _mm256_stream_si256(reinterpret_cast<__m256i*>(d),
                        _mm256_loadu_si256(reinterpret_cast<const __m256i*>(s)));
  memcpy(d, s, bytes);
}

template <class F>
static void chunked(ThreadPool& pool, int64_t n, F&& f) {
  const int64_t nt = (n + kChunk - 1) / kChunk;
  pool.run(nt, [&](int64_t t) {
    const int64_t b = t * kChunk, e = std::min(n, b + kChunk);
    f(b, e);
  });
}

void cast_bf16(ThreadPool& pool, const float* src, uint16_t* dst, int64_t n) {
  chunked(pool, n, [&](int64_t b, int64_t e) {
    const float* __restrict s = src;
    uint16_t* __restrict d = dst;
    for (int64_t i = b; i < e; ++i) d[i] = rne_bf16(s[i]);
  });
}

namespace {
// fp32 AdamW coefficients, formed in double from the exact hyper-parameters.
struct AdamCoef {
  float decay, b1, b2, c1, c2, bc1, bc2, lr, eps;
  AdamCoef(const mt_adamw_hparams& hp, int64_t step)
      : decay((float)(1.0 - hp.lr * hp.weight_decay)),
        b1((float)hp.beta1),
        b2((float)hp.beta2),
        c1((float)(1.0 - hp.beta1)),
        c2((float)(1.0 - hp.beta2)),
        bc1((float)(1.0 - pow(hp.beta1, (double)step))),
        bc2((float)(1.0 - pow(hp.beta2, (double)step))),
        lr((float)hp.lr),
        eps((float)hp.eps) {}
};

inline float bf16_bits_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// One element of the update, in the order of the per-element definition:
// decay, first and second moments, bias-corrected step.  Every operation is a
// separately rounded fp32 operation (built with contraction off).
template <bool BF>
inline void adam_range(const AdamCoef& k, float* __restrict p, const float* __restrict g,
                       float* __restrict m, float* __restrict v, uint16_t* __restrict bf,
                       int64_t b, int64_t e) {
  alignas(64) uint16_t bs[BF ? kStage : 1];  // the bf16 copy is written only: streamed out
  for (int64_t b0 = b; b0 < e; b0 += kStage) {
    const int64_t n = std::min(kStage, e - b0);
    for (int64_t j = 0; j < n; ++j) {
      const int64_t i = b0 + j;
      const float gi = g[i];
      float pi = p[i] * k.decay;
      float mi = m[i] * k.b1;
      mi = mi + k.c1 * gi;
      float vi = v[i] * k.b2;
      vi = vi + k.c2 * (gi * gi);
      const float mh = mi / k.bc1;
      const float vh = vi / k.bc2;
      pi = pi - (k.lr * mh) / (sqrtf(vh) + k.eps);
      p[i] = pi;
      m[i] = mi;
      v[i] = vi;
      if (BF) bs[j] = rne_bf16(pi);
    }
    if (BF) stream_out(bf + b0, bs, (size_t)n * sizeof(uint16_t));
  }
  if (BF) _mm_sfence();
}
}  // namespace

// Gradient element i of a slab job: (add ? grad[i] : 0) + slab[i], stored back
// into grad (one fp32 add, as accumulate does), then the update.
template <bool BF, bool SB, bool ADD>
inline void adam_slab_range(const AdamCoef& k, float* __restrict p, float* __restrict g,
                            float* __restrict m, float* __restrict v, uint16_t* __restrict bf,
                            const void* __restrict slab, int64_t b, int64_t e) {
  const uint16_t* __restrict s16 = static_cast<const uint16_t*>(slab);
  const float* __restrict s32 = static_cast<const float*>(slab);
  // Written-only outputs (the gradient when nothing is added to it, the bf16
  // copy) are staged and streamed out.
  alignas(64) float gs[ADD ? 1 : kStage];
  alignas(64) uint16_t bs[BF ? kStage : 1];
  for (int64_t b0 = b; b0 < e; b0 += kStage) {
    const int64_t n = std::min(kStage, e - b0);
    for (int64_t j = 0; j < n; ++j) {
      const int64_t i = b0 + j;
      const float si = SB ? bf16_bits_to_f32(s16[i]) : s32[i];
      float gi;
      if constexpr (ADD) {
        gi = g[i] + si;
        g[i] = gi;
      } else {
        gi = si;
        gs[j] = gi;
      }
      float pi = p[i] * k.decay;
      float mi = m[i] * k.b1;
      mi = mi + k.c1 * gi;
      float vi = v[i] * k.b2;
      vi = vi + k.c2 * (gi * gi);
      const float mh = mi / k.bc1;
      const float vh = vi / k.bc2;
      pi = pi - (k.lr * mh) / (sqrtf(vh) + k.eps);
      p[i] = pi;
      m[i] = mi;
      v[i] = vi;
      if (BF) bs[j] = rne_bf16(pi);
    }
    if (!ADD) stream_out(g + b0, gs, (size_t)n * sizeof(float));
    if (BF) stream_out(bf + b0, bs, (size_t)n * sizeof(uint16_t));
  }
  if (!ADD || BF) _mm_sfence();
}

void adamw(ThreadPool& pool, float* p, const float* g, float* m, float* v, uint16_t* bf, int64_t n,
           const mt_adamw_hparams& hp, int64_t step) {
  const AdamCoef k(hp, step);
  chunked(pool, n, [&](int64_t b, int64_t e) {
    if (bf)
      adam_range<true>(k, p, g, m, v, bf, b, e);
    else
      adam_range<false>(k, p, g, m, v, nullptr, b, e);
  });
}

void adamw_slab(ThreadPool& pool, float* p, float* g, float* m, float* v, uint16_t* bf,
                const void* slab, bool slab_bf16, bool add, int64_t n, const mt_adamw_hparams& hp,
                int64_t step) {
  const AdamCoef k(hp, step);
  chunked(pool, n, [&](int64_t b, int64_t e) {
#define MT_SLAB_CASE(BFV, SBV, ADDV)                                        \
  if ((bf != nullptr) == BFV && slab_bf16 == SBV && add == ADDV) {          \
    adam_slab_range<BFV, SBV, ADDV>(k, p, g, m, v, bf, slab, b, e);         \
    return;                                                                 \
  }
    MT_SLAB_CASE(true, true, true) MT_SLAB_CASE(true, true, false)
    MT_SLAB_CASE(true, false, true) MT_SLAB_CASE(true, false, false)
    MT_SLAB_CASE(false, true, true) MT_SLAB_CASE(false, true, false)
    MT_SLAB_CASE(false, false, true) MT_SLAB_CASE(false, false, false)
#undef MT_SLAB_CASE
  });
}

void accumulate(ThreadPool& pool, float* grad, const float* src, int64_t n, bool add) {
  chunked(pool, n, [&](int64_t b, int64_t e) {
    float* __restrict d = grad;
    const float* __restrict s = src;
    if (add) {
      for (int64_t i = b; i < e; ++i) d[i] += s[i];
    } else {
      stream_out(d + b, s + b, (size_t)(e - b) * sizeof(float));
      _mm_sfence();
    }
  });
}

static inline float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

void accumulate_bf16(ThreadPool& pool, float* grad, const uint16_t* src, int64_t n, bool add) {
  chunked(pool, n, [&](int64_t b, int64_t e) {
    float* __restrict d = grad;
    const uint16_t* __restrict s = src;
    if (add) {
      for (int64_t i = b; i < e; ++i) d[i] += bf16_to_f32(s[i]);
    } else {
      alignas(64) float st[kStage];
      for (int64_t b0 = b; b0 < e; b0 += kStage) {
        const int64_t n = std::min(kStage, e - b0);
        for (int64_t j = 0; j < n; ++j) st[j] = bf16_to_f32(s[b0 + j]);
        stream_out(d + b0, st, (size_t)n * sizeof(float));
      }
      _mm_sfence();
    }
  });
}

void embed_gather(ThreadPool& pool, const float* emb, const int32_t* tok, int64_t T, int64_t h,
                  float* x0) {
  const int64_t per = 64;
  pool.run((T + per - 1) / per, [&](int64_t k) {
    for (int64_t t = k * per; t < std::min(T, (k + 1) * per); ++t)
      memcpy(x0 + t * h, emb + (int64_t)tok[t] * h, (size_t)h * sizeof(float));
  });
}

// The tokens are ordered by id with a stable counting sort, so that a task
// owns a run of embedding rows and adds into each of them its tokens' rows
// of dx0 in token order: per element the same additions in the same order as
// one pass over t, with whole rows read and written (a split by columns read
// dx0 in 256-byte pieces at a 16 KB stride).
void embed_scatter(ThreadPool& pool, float* demb, int64_t rows, const int32_t* tok, int64_t T,
                   int64_t h, const float* dx0, bool add) {
  std::vector<int64_t> start((size_t)rows + 1, 0);
  for (int64_t t = 0; t < T; ++t) ++start[(size_t)tok[t] + 1];
  for (int64_t r = 0; r < rows; ++r) start[(size_t)r + 1] += start[(size_t)r];
  std::vector<int32_t> order((size_t)T);
  {
    std::vector<int64_t> next(start.begin(), start.end() - 1);
    for (int64_t t = 0; t < T; ++t) order[(size_t)next[(size_t)tok[t]]++] = (int32_t)t;
  }
  const int64_t nb = std::min<int64_t>(rows, 4 * (int64_t)pool.size());
  pool.run(nb, [&](int64_t k) {
    const int64_t r0 = rows * k / nb, r1 = rows * (k + 1) / nb;
    if (!add) memset(demb + r0 * h, 0, (size_t)((r1 - r0) * h) * sizeof(float));
    for (int64_t r = r0; r < r1; ++r) {
      float* __restrict dst = demb + r * h;
      for (int64_t i = start[(size_t)r]; i < start[(size_t)r + 1]; ++i) {
        const float* __restrict s = dx0 + (int64_t)order[(size_t)i] * h;
        for (int64_t c = 0; c < h; ++c) dst[c] += s[c];
      }
    }
  });
}

void rope_table(int seq, int d, float base, float* cos_out, float* sin_out) {
  const int half = d / 2;
  for (int i = 0; i < half; ++i) {
    const double theta = pow((double)base, -2.0 * (double)i / (double)d);
    for (int pos = 0; pos < seq; ++pos) {
      const double a = (double)pos * theta;
      cos_out[(int64_t)pos * half + i] = (float)cos(a);
      sin_out[(int64_t)pos * half + i] = (float)sin(a);
    }
  }
}

}  // namespace mt

// ---------------------------------------------------------------- C ABI
using namespace mt;

static int nthreads(int32_t t) { return t > 0 ? std::min<int>(t, 256) : default_threads(); }

extern "C" mt_status mt_host_cast_bf16(const float* src, uint16_t* dst, int64_t n,
                                       int32_t threads) {
  if (n < 0 || (n > 0 && (!src || !dst))) return MT_E_ARG;
  ThreadPool pool(nthreads(threads));
  cast_bf16(pool, src, dst, n);
  return MT_OK;
}

extern "C" mt_status mt_host_adamw(float* master, const float* grad, float* m, float* v,
                                   uint16_t* bf16_out, int64_t n, const mt_adamw_hparams* hp,
                                   int64_t step, int32_t threads) {
  if (n < 0 || !hp || step < 1) return MT_E_ARG;
  if (n > 0 && (!master || !grad || !m || !v)) return MT_E_ARG;
  ThreadPool pool(nthreads(threads));
  adamw(pool, master, grad, m, v, bf16_out, n, *hp, step);
  return MT_OK;
}

extern "C" mt_status mt_host_adamw_slab(float* master, float* grad, float* m, float* v,
                                        uint16_t* bf16_out, const void* slab, int32_t slab_bf16,
                                        int32_t accumulate_flag, int64_t n,
                                        const mt_adamw_hparams* hp, int64_t step,
                                        int32_t threads) {
  if (n < 0 || !hp || step < 1) return MT_E_ARG;
  if ((slab_bf16 != 0 && slab_bf16 != 1) || (accumulate_flag != 0 && accumulate_flag != 1))
    return MT_E_ARG;
  if (n > 0 && (!master || !grad || !m || !v || !slab)) return MT_E_ARG;
  ThreadPool pool(nthreads(threads));
  adamw_slab(pool, master, grad, m, v, bf16_out, slab, slab_bf16 != 0, accumulate_flag != 0, n,
             *hp, step);
  return MT_OK;
}

extern "C" mt_status mt_host_accumulate(float* grad, const float* src, int64_t n,
                                        int32_t accumulate_flag, int32_t threads) {
  if (n < 0 || (n > 0 && (!grad || !src))) return MT_E_ARG;
  ThreadPool pool(nthreads(threads));
  accumulate(pool, grad, src, n, accumulate_flag != 0);
  return MT_OK;
}

extern "C" mt_status mt_host_triad(float* a, const float* b, const float* c, float s, int64_t n,
                                   int32_t reps, int32_t threads, double* best_s) {
  if (n < 1 || reps < 1 || !a || !b || !c || !best_s) return MT_E_ARG;
  ThreadPool pool(nthreads(threads));
  double best = 1e30;
  for (int32_t r = 0; r < reps; ++r) {
    const auto t0 = std::chrono::steady_clock::now();
    chunked(pool, n, [&](int64_t lo, int64_t hi) {
      float* __restrict x = a;
      const float* __restrict y = b;
      const float* __restrict z = c;
      for (int64_t i = lo; i < hi; ++i) x[i] = y[i] + s * z[i];
    });
    best = std::min(best, std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count());
  }
  *best_s = best;
  return MT_OK;
}

extern "C" mt_status mt_host_rope_table(int32_t seq_len, int32_t head_dim, float base,
                                        float* cos_out, float* sin_out) {
  if (seq_len < 1 || head_dim < 2 || head_dim % 2 || !(base > 0.0f) || !cos_out || !sin_out)
    return MT_E_ARG;
  rope_table(seq_len, head_dim, base, cos_out, sin_out);
  return MT_OK;
}
