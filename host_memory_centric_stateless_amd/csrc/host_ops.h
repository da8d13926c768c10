// Host-side kernels and the CPU thread pool they run on.
#pragma once

#include <stdint.h>

#include <condition_variable>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "../../include/mt.h"

namespace mt {

// Fixed pool: run(n, fn) calls fn(i) for i in [0, n) spread over the workers
// and the caller, and returns when all are done.  One run at a time (callers
// from different threads queue on a mutex).
class ThreadPool {
 public:
  explicit ThreadPool(int n);
  ~ThreadPool();
  int size() const { return (int)workers_.size() + 1; }
  void run(int64_t n, const std::function<void(int64_t)>& fn);

 private:
  void loop();
  std::vector<std::thread> workers_;
  std::mutex run_mu_, mu_;
  std::condition_variable cv_, done_cv_;
  const std::function<void(int64_t)>* fn_ = nullptr;
  int64_t n_ = 0, next_ = 0, pending_ = 0;
  uint64_t gen_ = 0;
  bool stop_ = false;
};

int default_threads();

// Chunked element-wise ops over n elements, split across the pool.
void cast_bf16(ThreadPool& pool, const float* src, uint16_t* dst, int64_t n);
void adamw(ThreadPool& pool, float* p, const float* g, float* m, float* v, uint16_t* bf, int64_t n,
           const mt_adamw_hparams& hp, int64_t step);
// grad = (add ? grad : 0) + slab, then adamw on that gradient, in one pass:
// the same values as accumulate/accumulate_bf16 followed by adamw.
void adamw_slab(ThreadPool& pool, float* p, float* g, float* m, float* v, uint16_t* bf,
                const void* slab, bool slab_bf16, bool add, int64_t n, const mt_adamw_hparams& hp,
                int64_t step);
void accumulate(ThreadPool& pool, float* grad, const float* src, int64_t n, bool add);
// grad = float(src) or grad += float(src) for bf16 src.
void accumulate_bf16(ThreadPool& pool, float* grad, const uint16_t* src, int64_t n, bool add);
// x0[t, :] = emb[tok[t], :]
void embed_gather(ThreadPool& pool, const float* emb, const int32_t* tok, int64_t T, int64_t h,
                  float* x0);
// demb[tok[t], :] += dx0[t, :] in token order, for demb of `rows` rows
// (zeroed first unless add).  Token ids must lie in [0, rows).
void embed_scatter(ThreadPool& pool, float* demb, int64_t rows, const int32_t* tok, int64_t T,
                   int64_t h, const float* dx0, bool add);
void rope_table(int seq, int d, float base, float* cos_out, float* sin_out);

}  // namespace mt
