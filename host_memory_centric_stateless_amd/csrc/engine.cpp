// The streaming engine behind mt_forward / mt_backward / mt_flush_grads /
// mt_adamw_step.
//
// Method (citations by page and section):
//   * fp32 master, grad and Adam m/v stay in host memory; the GPU only holds a
//     ping-pong pair of flat bf16 layer buffers, one K-layer activation window
//     and a pool of flat gradient slabs (zhichai.net
//     "MegaTrain：单卡训百亿大模型的突破与实践", design points 1-2; m.lqnn.cn
//     MegaTrain article, 二 and 三.1).
//   * three streams -- prefetch (host->device weights), compute, offload
//     (device->host gradients) -- ordered by events: a compute step waits for
//     its buffer's weight_ready event, a copy into a buffer waits for the
//     buffer_free event recorded after the last step that read it (lqnn 三.2;
//     zhichai design point 4; blog.travelaiplan.net
//     "單卡也能練 100B+：MegaTrain 實戰", 核心功能 2).
//   * each streamed unit's gradient is written into a free slab, copied to a
//     pinned host slab and added into the fp32 host gradient by a CPU worker;
//     the slab returns to the pool afterwards (lqnn 三.3, 12 slabs by
//     default).  Gradients are never accumulated across units on the GPU.
//   * a checkpoint (the layer input, fp32) every K layers; backward walks the
//     segments last to first, recomputes a segment's forwards into the window
//     from its checkpoint, then runs its blocks backwards (zhichai design
//     point 3; lqnn 三.4).
//
// MI355X choices (not from the pages):
//   * which buffer a load goes into is decided ahead of time by simulating the
//     two buffers over the whole pass (a unit still resident is reused
//     instead of re-copied, e.g. the last layers of a segment when its
//     backward starts); the forward of the last segment writes the window
//     directly, so that segment is not recomputed; the LM head is streamed
//     through the same buffers in vocabulary chunks;
//   * slabs drain through a small copy kernel writing pinned host memory;
//   * with mt_backward_step, each unit's last slab of the step is added and
//     stepped by AdamW in one host pass on the optimizer thread, units served
//     in the order the next forward reads them;
//   * optionally several micro-batches share one pass (layer-major gradient
//     accumulation, mt_config.micro_batches_per_pass).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <deque>
#include <functional>
#include <map>
#include <memory>
#include <string>
#include <vector>

#include "common.h"
#include "host_ops.h"
#include "moe.h"
#include "plan.h"

using namespace mt;

namespace {

enum Kind { K_FWD, K_HEAD_LOGITS, K_CE, K_HEAD_GRAD, K_RECOMP, K_BWD, K_EMBED_GRAD };

struct Step {
  Kind kind;
  int layer = -1, chunk = -1, slot = -1;
  bool write_y = true;
  int unit = -1;  // streamed unit needed (layer l -> l, head chunk c -> L + c)
  int buf = -1;   // buffer holding it
  int load = -1;  // load that brings it in (first user only), else -1
};

struct Load {
  int unit, buf, after;  // issue once step `after` is enqueued (-1: at once)
};

struct Job {
  enum { SLAB, EMBED } kind;
  int slab = -1, group = 0, parity = 0;
  int64_t e0 = 0, n = 0;
  bool add = false;
  bool adamw = false;  // run the optimizer on this range once it is accumulated
  int unit = -1;       // streamed unit whose working copy the update refreshes
  std::vector<int32_t> tok;
};

enum State { ST_UNBOUND, ST_IDLE, ST_FWD, ST_BWD, ST_FLUSHED };

// Slabs leave the device either by the DMA engine or by a copy kernel that
// writes the pinned host slab (mt_config.drain_workgroups).  Measured on the
// MI355X host link with 405 MB slabs: beside the weight loads, the runtime
// ran many DMA device->host copies as blit kernels on the CUs, and the rest
// fell to 7-16 GB/s on the copy engine.  A 4-workgroup copy kernel keeps
// ~38 GB/s device->host with host->device unchanged at ~57 GB/s; with 8 or
// more workgroups the two directions saturate the link and kernels sharing
// CUs with the copy stall on its host stores for milliseconds.  When a step
// has several micro-batches, three workgroups do better: the drain (~24 GB/s)
// then trails into the next micro-batch's forward, whose device->host
// direction is otherwise idle, and the weight loads keep ~51 GB/s instead of
// ~46 beside four.

double now_s() {
  return std::chrono::duration<double>(std::chrono::steady_clock::now().time_since_epoch())
      .count();
}

}  // namespace

struct mt_ctx {
  Plan p;
  int device = 0;
  hipStream_t sp = nullptr, sc = nullptr, so = nullptr;
  uint16_t* wbuf[2] = {nullptr, nullptr};
  float* dslab[64] = {};
  uint8_t* window = nullptr;
  uint8_t* ckpt = nullptr;
  uint8_t* ws = nullptr;
  int nslab = 0;

  struct Bind {
    float *master = nullptr, *grad = nullptr, *m = nullptr, *v = nullptr;
    int64_t n = 0;
    uint16_t* pinned = nullptr;  // bf16 working copy (blocks, head)
  };
  std::vector<Bind> layers;
  Bind head, embed;

  float* hslab[64] = {};
  float* x0_stage[2] = {};
  float* dx0_stage[2] = {};
  int32_t* lab_stage[2] = {};
  float* loss_pin = nullptr;
  static constexpr int kLossRing = 4096;

  hipEvent_t ev_ready[2] = {}, ev_free[2] = {}, ev_x0[2] = {}, ev_bwd_done[2] = {};
  hipEvent_t ev_written[64] = {}, ev_copied[64] = {}, ev_dx0[2] = {}, ev_dx0_copied[2] = {};
  hipEvent_t ev_loss = nullptr;  // after the last forward's loss copy to the pinned ring
  hipEvent_t ev_origin = nullptr;  // timing origin, recorded when kernel timing is enabled
  bool x0_used[2] = {false, false}, bwd_used[2] = {false, false};

  int buf_unit[2] = {-1, -1};
  std::vector<Step> steps;
  std::vector<Load> loads;
  size_t next_load = 0, next_step = 0, split = 0;
  int64_t mb = 0;
  int parity = 0;
  int dy_idx = 0;
  bool head_grad_first = true;
  // labelled tokens of each micro-batch of the current pass and its loss
  // scale (the cross-entropy coefficients of the head's backward)
  int64_t n_valid[32] = {};
  float grad_scale = 1.0f;
  std::vector<int32_t> tok_cur;
  State state = ST_UNBOUND;
  int accumulate = 0;

  std::unique_ptr<ThreadPool> pool;
  std::unique_ptr<ThreadPool> opt_pool;  // optimizer work, separate from slab draining
  // Caller-thread work (embedding gather): its own few threads, so that the
  // next micro-batch's input is never queued behind gradient accumulation.
  std::unique_ptr<ThreadPool> io_pool;
  std::thread opt_worker;
  std::deque<Job> opt_jobs;
  std::condition_variable opt_cv;
  std::thread worker;
  std::mutex mu;
  std::condition_variable cv, slab_cv, idle_cv;
  std::deque<Job> jobs;
  int outstanding = 0;
  bool stop = false;
  std::vector<int> free_slabs;
  int embed_busy[2] = {0, 0};
  int delay_us = 0;
  // overlapped optimizer (mt_backward_step)
  bool fused = false;
  mt_adamw_hparams hp{};
  int64_t opt_step = 0;
  std::vector<char> upd_pending;  // per streamed unit: update not applied yet
  bool embed_upd_pending = false;

  // live per-kernel timing (mt_kernel_timing)
  struct KRec {
    hipEvent_t a, b;
    const char* name;
    double flop, bytes;
  };
  struct KTot {
    int64_t n = 0;
    double ms = 0, flop = 0, bytes = 0;
  };
  bool ktiming = false;
  std::vector<hipEvent_t> ev_pool;
  std::vector<KRec> krec;
  std::map<std::string, KTot> ktot;
  hipEvent_t take_event() {
    if (!ev_pool.empty()) {
      hipEvent_t e = ev_pool.back();
      ev_pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  // Timed intervals of one flush: host-link copies and compute kernels, as
  // [start, end) in ms from ev_origin; their union measures and the measure
  // of their intersection go into the stats.
  static bool is_copy(const char* n) {
    return !strcmp(n, "h2d_load") || !strcmp(n, "h2d_input") || !strcmp(n, "drain_d2h");
  }
  static std::vector<std::pair<double, double>> union_of(std::vector<std::pair<double, double>> v) {
    std::sort(v.begin(), v.end());
    std::vector<std::pair<double, double>> u;
    for (auto& x : v) {
      if (!u.empty() && x.first <= u.back().second)
        u.back().second = std::max(u.back().second, x.second);
      else
        u.push_back(x);
    }
    return u;
  }
  static double measure(const std::vector<std::pair<double, double>>& u) {
    double m = 0;
    for (auto& x : u) m += x.second - x.first;
    return m;
  }
  hipError_t collect_overlap() {
    std::vector<std::pair<double, double>> cp, kn;
    for (auto& r : krec) {
      float a = 0.0f, b = 0.0f;
      hipError_t e = hipEventElapsedTime(&a, ev_origin, r.a);
      if (e == hipSuccess) e = hipEventElapsedTime(&b, ev_origin, r.b);
      if (e != hipSuccess) return e;
      (is_copy(r.name) ? cp : kn).emplace_back(a, b);
    }
    const auto uc = union_of(cp), uk = union_of(kn);
    double both = 0;
    for (size_t i = 0, j = 0; i < uc.size() && j < uk.size();) {
      const double lo = std::max(uc[i].first, uk[j].first), hi = std::min(uc[i].second, uk[j].second);
      if (lo < hi) both += hi - lo;
      if (uc[i].second < uk[j].second) ++i; else ++j;
    }
    st.timed_copy_ms += measure(uc);
    st.timed_kernel_ms += measure(uk);
    st.timed_overlap_ms += both;
    return hipSuccess;
  }
  hipError_t collect_kernel_times() {
    if (!krec.empty()) {
      hipError_t e = collect_overlap();
      if (e != hipSuccess) return e;
    }
    for (auto& r : krec) {
      float ms = 0.0f;
      hipError_t e = hipEventElapsedTime(&ms, r.a, r.b);
      if (e != hipSuccess) return e;
      KTot& t = ktot[r.name];
      t.n += 1;
      t.ms += ms;
      t.flop += r.flop;
      t.bytes += r.bytes;
      ev_pool.push_back(r.a);
      ev_pool.push_back(r.b);
    }
    krec.clear();
    return hipSuccess;
  }

  std::mutex err_mu;
  std::string err;
  std::atomic<bool> poisoned{false};
  std::vector<std::pair<float*, int>> pending_loss;
  int loss_next = 0;
  // loss ring slots of the passes of the open optimizer step, and of the last
  // completed one (mt_step_loss)
  std::vector<int> step_slots, last_step_slots;
  mt_stats st{};

  void set_err(const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    std::lock_guard<std::mutex> g(err_mu);
    err = buf;
  }
  mt_status fail_hip(hipError_t e, const char* what) {
    set_err("%s: %s", what, hipGetErrorString(e));
    poisoned = true;
    return MT_E_HIP;
  }

  uint8_t* slot_base(int w) const { return window + (size_t)w * p.slot.bytes; }
  float* ckpt_ptr(int j) {
    if (j == 0) return reinterpret_cast<float*>(ws + p.ws.x0[parity]);
    return reinterpret_cast<float*>(ckpt + (size_t)(j - 1) * round_bytes((size_t)p.T * p.c.hidden * 4));
  }
  float* slot_x(int w) { return reinterpret_cast<float*>(slot_base(w) + p.slot.x); }
  template <class T>
  T* wsp(size_t off) { return reinterpret_cast<T*>(ws + off); }

  const Bind& bind_of(int group) const {
    if (group == MT_GROUP_HEAD) return head;
    if (group == MT_GROUP_EMBED) return embed;
    return layers[group];
  }
  // Pinned source and element count of a streamed unit.
  void unit_src(int u, const uint16_t** src, int64_t* n) const {
    const int L = p.c.n_layers;
    if (u < L) {
      *src = layers[u].pinned;
      *n = p.block_elems(u);
    } else {
      const int c = u - L;
      *src = head.pinned + p.chunk_e0[c];
      *n = p.chunk_e0[c + 1] - p.chunk_e0[c];
    }
  }
};

#define MT_HIP(ctx, expr)                                          \
  do {                                                             \
    hipError_t e_ = (expr);                                        \
    if (e_ != hipSuccess) return (ctx)->fail_hip(e_, #expr);       \
  } while (0)

namespace {

// ------------------------------------------------------------ activations
struct Acts {
  float* x;
  float* rstd1;
  uint16_t* n1;
  uint16_t* qkv;
  uint16_t* o;
  float* lse;
  float* h1;
  float* rstd2;
  uint16_t* n2;
  uint16_t* gu;
  uint16_t* m;
  // mixture-of-experts blocks
  float* mlog;
  int32_t *msel, *mpos, *moff, *mrowtok;
  float* mgate;
  uint16_t *mx, *mgu, *mm;
  float* myo;
};

Acts acts_of(mt_ctx* c, int w, float* x) {
  uint8_t* b = c->slot_base(w);
  const SlotLayout& s = c->p.slot;
  return Acts{x,
              reinterpret_cast<float*>(b + s.rstd1),
              reinterpret_cast<uint16_t*>(b + s.n1),
              reinterpret_cast<uint16_t*>(b + s.qkv),
              reinterpret_cast<uint16_t*>(b + s.o),
              reinterpret_cast<float*>(b + s.lse),
              reinterpret_cast<float*>(b + s.h1),
              reinterpret_cast<float*>(b + s.rstd2),
              reinterpret_cast<uint16_t*>(b + s.n2),
              reinterpret_cast<uint16_t*>(b + s.gu),
              reinterpret_cast<uint16_t*>(b + s.m),
              reinterpret_cast<float*>(b + s.mlog),
              reinterpret_cast<int32_t*>(b + s.msel),
              reinterpret_cast<int32_t*>(b + s.mpos),
              reinterpret_cast<int32_t*>(b + s.moff),
              reinterpret_cast<int32_t*>(b + s.mrowtok),
              reinterpret_cast<float*>(b + s.mgate),
              reinterpret_cast<uint16_t*>(b + s.mx),
              reinterpret_cast<uint16_t*>(b + s.mgu),
              reinterpret_cast<uint16_t*>(b + s.mm),
              reinterpret_cast<float*>(b + s.myo)};
}

// Records timing events around one launch when mt_kernel_timing is on.
struct KScope {
  mt_ctx* c;
  hipStream_t s;
  hipEvent_t a = nullptr;
  const char* name;
  double flop, bytes;
  KScope(mt_ctx* c_, hipStream_t s_, const char* n, double f, double b)
      : c(c_), s(s_), name(n), flop(f), bytes(b) {
    if (c->ktiming && (a = c->take_event()) && hipEventRecord(a, s) != hipSuccess) a = nullptr;
  }
  ~KScope() {
    if (!a) return;
    hipEvent_t b = c->take_event();
    if (b && hipEventRecord(b, s) == hipSuccess) c->krec.push_back({a, b, name, flop, bytes});
  }
};

const char* gemm_name(int layout, int epi) {
  static const char* n[3][7] = {
      {"gemm_nt_bf16", "gemm_nt_f32", "gemm_nt_resid", "gemm_nt_accum", "gemm_nt_swiglu", "gemm_nt_x",
       "gemm_nt_rope"},
      {"gemm_nn_bf16", "gemm_nn_f32", "gemm_nn_resid", "gemm_nn_accum", "gemm_nn_x", "gemm_nn_swiglu_bwd",
       "gemm_nn_x"},
      {"gemm_tn_bf16", "gemm_tn_f32", "gemm_tn_resid", "gemm_tn_accum", "gemm_tn_x", "gemm_tn_x",
       "gemm_tn_x"}};
  return n[layout][epi];
}

hipError_t gemm(mt_ctx* c, hipStream_t s, int layout, int epi, int64_t M, int64_t N, int64_t K,
                const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, void* C,
                int64_t ldc, const float* R = nullptr, int64_t ldr = 0, uint16_t* gu = nullptr,
                int64_t ldgu = 0, int64_t ffn = 0) {
  mt_gemm_args a{layout, epi, M, N, K, A, lda, B, ldb, C, ldc, R, ldr, gu, ldgu, ffn,
                 nullptr, nullptr, 0, 0, 0};
  // the SwiGLU product computes both the gate and the up projection
  const double nn = (epi == MT_EPI_SWIGLU) ? 2.0 * N : (double)N;
  KScope k(c, s, gemm_name(layout, epi), 2.0 * M * nn * K, 2.0 * (M * K + nn * K));
  return launch_gemm(a, s);
}

// The fused QKV projection: qkv = n1 [Wq; Wk; Wv]^T with RoPE applied to the
// q and k columns in fp32 in the epilogue, so q and k are rounded to bf16 once.
hipError_t gemm_qkv_rope(mt_ctx* c, hipStream_t s, int64_t T, const uint16_t* n1,
                         const uint16_t* Wqkv, uint16_t* qkv) {
  const Plan& p = c->p;
  const int64_t h = p.c.hidden;
  mt_gemm_args a{MT_GEMM_NT, MT_EPI_ROPE, T, p.ldq, h, n1, h, Wqkv, h, qkv, p.ldq,
                 nullptr, 0, nullptr, 0, 0,
                 c->wsp<float>(p.ws.cos_t), c->wsp<float>(p.ws.sin_t), p.qd + p.kvd,
                 p.c.seq_len, p.c.head_dim};
  KScope k(c, s, "gemm_nt_rope", 2.0 * T * p.ldq * h, 2.0 * (T * h + (double)p.ldq * h));
  return launch_gemm(a, s);
}

// A grouped product over the experts of an MoE block (one launch): rows of
// the expert-major row space belong to experts by off[] (device); the
// algorithmic work counts the real token-expert pairs, not the padding.
hipError_t gemm_grouped(mt_ctx* c, hipStream_t s, int layout, int epi, int64_t M, int64_t N,
                        int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                        void* C, int64_t ldc, const int32_t* off, int64_t stride_b,
                        int64_t stride_c, uint16_t* gu = nullptr, int64_t ldgu = 0,
                        int64_t ffn = 0) {
  const Plan& p = c->p;
  mt_gemm_args a{layout, epi, M, N, K, A, lda, B, ldb, C, ldc, nullptr, 0, gu, ldgu, ffn,
                 nullptr, nullptr, 0, 0, 0, off, p.c.n_experts, 0, stride_b, stride_c};
  const double pairs = (double)p.T * p.c.top_k;
  const double nn = (epi == MT_EPI_SWIGLU) ? 2.0 * N : (double)N;
  const double work = layout == MT_GEMM_TN ? 2.0 * M * N * pairs : 2.0 * pairs * nn * K;
  KScope k(c, s, layout == MT_GEMM_TN ? "gemm_tn_grouped" : layout == MT_GEMM_NN
                                                             ? "gemm_nn_grouped" : "gemm_nt_grouped",
           work, 0);
  return launch_gemm(a, s);
}

// Algorithmic work of the other kernels.
double attn_pairs(const mt_config& g) {
  return (double)g.micro_batch * g.micro_batches_per_pass * g.n_heads * 0.5 * (double)g.seq_len *
         (g.seq_len + 1.0);
}

#define CK(expr)                            \
  do {                                      \
    hipError_t e_ = (expr);                 \
    if (e_ != hipSuccess) return e_;        \
  } while (0)

// One decoder block forward on weights W (flat bf16 layer).  y == nullptr
// skips the down projection (its output is not needed).
hipError_t moe_forward(mt_ctx* c, const uint16_t* W, const Acts& a, float* y, int layer);

hipError_t block_forward(mt_ctx* c, const uint16_t* W, const Acts& a, float* y, int layer) {
  const Plan& p = c->p;
  const mt_config& g = p.c;
  const int64_t T = p.T, h = g.hidden, F = g.ffn;
  hipStream_t s = c->sc;
  const TensorOff* L = p.block_layout(layer);
  const double nb_fwd = (double)T * h * 6 + h * 2 + T * 4;   // rmsnorm: x in, bf16 out
  {
    KScope k(c, s, "rmsnorm_fwd", 0, nb_fwd);
    CK(launch_rmsnorm_fwd(a.x, W + L[T_ATTN_NORM].off, a.n1, a.rstd1, T, (int)h, g.rms_eps, s));
  }
  CK(gemm_qkv_rope(c, s, T, a.n1, W + L[T_WQ].off, a.qkv));
  {
    KScope k(c, s, "attn_fwd", 4.0 * g.head_dim * attn_pairs(g), 0);
    CK(launch_attn_fwd(a.qkv, a.o, a.lse, (int)(T / g.seq_len), g.seq_len, g.n_heads, g.n_kv_heads,
                       g.head_dim, s));
  }
  CK(gemm(c, s, MT_GEMM_NT, MT_EPI_F32_RESID, T, h, p.qd, a.o, p.qd, W + L[T_WO].off, p.qd, a.h1, h,
          a.x, h));
  {
    KScope k(c, s, "rmsnorm_fwd", 0, nb_fwd);
    CK(launch_rmsnorm_fwd(a.h1, W + L[T_MLP_NORM].off, a.n2, a.rstd2, T, (int)h, g.rms_eps, s));
  }
  if (p.is_moe(layer)) return moe_forward(c, W, a, y, layer);
  CK(gemm(c, s, MT_GEMM_NT, MT_EPI_SWIGLU, T, F, h, a.n2, h, W + L[T_WGATE].off, h, a.m, F, nullptr,
          0, a.gu, 2 * F, F));
  if (y)
    CK(gemm(c, s, MT_GEMM_NT, MT_EPI_F32_RESID, T, h, F, a.m, F, W + L[T_WDOWN].off, F, y, h, a.h1,
            h));
  return hipSuccess;
}

// FFN of a mixture-of-experts block (after n2): router logits, top-k and
// gates, the expert-major row plan, the experts' SwiGLU and down products as
// grouped GEMMs, and (y != nullptr) y = h1 + sum_j g_j expert_j(n2).  The
// expert outputs are kept in the window even when y is not needed: the
// gates' backward reads them.
hipError_t moe_forward(mt_ctx* c, const uint16_t* W, const Acts& a, float* y, int layer) {
  const Plan& p = c->p;
  const mt_config& g = p.c;
  const int64_t T = p.T, h = g.hidden, Fe = g.expert_ffn, R = p.moe_rows;
  const int E = g.n_experts, k = g.top_k;
  hipStream_t s = c->sc;
  const TensorOff* Mo = p.moe;
  CK(gemm(c, s, MT_GEMM_NT, MT_EPI_F32, T, E, h, a.n2, h, W + Mo[M_ROUTER].off, h, a.mlog, E));
  {
    KScope ks(c, s, "moe_route", 0, (double)T * (E * 4 + k * 8) + (double)R * h * 4);
    CK(launch_moe_route(a.mlog, E, T, E, k, a.msel, a.mgate, s));
    // keep this block's selection for mt_moe_routing (a recompute writes the same)
    CK(launch_copy(c->wsp<int32_t>(p.ws.mroute) + (int64_t)(layer / g.moe_every) * T * k, a.msel,
                   (size_t)T * k * 4, 8, s));
    CK(launch_moe_plan(a.msel, T, E, k, a.moff, a.mpos, a.mrowtok, s));
    CK(launch_moe_gather(a.n2, (int)h, a.mrowtok, a.moff, E, R, a.mx, s));
  }
  CK(gemm_grouped(c, s, MT_GEMM_NT, MT_EPI_SWIGLU, R, Fe, h, a.mx, h, W + Mo[M_GU].off, h, a.mm, Fe,
                  a.moff, 2 * Fe * h, 0, a.mgu, 2 * Fe, Fe));
  CK(gemm_grouped(c, s, MT_GEMM_NT, MT_EPI_F32, R, h, Fe, a.mm, Fe, W + Mo[M_DOWN].off, Fe, a.myo,
                  h, a.moff, h * Fe, 0));
  if (y) {
    KScope ks(c, s, "moe_combine", 0, (double)T * h * 8 + (double)T * k * h * 4);
    CK(launch_moe_combine(a.h1, a.myo, a.mpos, a.mgate, k, (int)h, T, y, s));
  }
  return hipSuccess;
}

// Backward of the mixture-of-experts FFN down to dn (the gradient of n2):
// gates and combine, the experts' products (grouped), their weight gradients
// into the slab, the router's.
hipError_t moe_backward(mt_ctx* c, const uint16_t* W, const Acts& a, const float* dy, float* dn,
                        const std::function<void*(int)>& slab, int wepi) {
  const Plan& p = c->p;
  const mt_config& g = p.c;
  const int64_t T = p.T, h = g.hidden, Fe = g.expert_ffn, R = p.moe_rows, ldl = p.moe_ldl;
  const int E = g.n_experts, k = g.top_k;
  hipStream_t s = c->sc;
  const TensorOff* Mo = p.moe;
  uint16_t* dout = c->wsp<uint16_t>(p.ws.mdout);
  float* dX = c->wsp<float>(p.ws.mdx);
  uint16_t* dlog = c->wsp<uint16_t>(p.ws.mdlog);
  uint16_t* dgu = c->wsp<uint16_t>(p.ws.dgu);
  {
    KScope ks(c, s, "moe_route_bwd", 0, (double)T * h * 4 + (double)T * k * h * 6);
    CK(launch_moe_bwd_gates(dy, a.myo, a.mpos, a.msel, a.mgate, k, E, (int)h, T, dout, dlog, ldl,
                            s));
    CK(launch_moe_zero_pad(a.mrowtok, a.moff, E, (int)h, R, dout, s));
  }
  CK(gemm_grouped(c, s, MT_GEMM_NN, MT_EPI_SWIGLU_BWD, R, Fe, h, dout, h, W + Mo[M_DOWN].off, Fe,
                  dgu, 2 * Fe, a.moff, h * Fe, 0, a.mgu, 2 * Fe, Fe));
  CK(gemm_grouped(c, s, MT_GEMM_TN, wepi, h, Fe, R, dout, h, a.mm, Fe, slab(M_DOWN), Fe, a.moff, 0,
                  h * Fe));
  CK(gemm_grouped(c, s, MT_GEMM_TN, wepi, 2 * Fe, h, R, dgu, 2 * Fe, a.mx, h, slab(M_GU), h, a.moff,
                  0, 2 * Fe * h));
  CK(gemm_grouped(c, s, MT_GEMM_NN, MT_EPI_F32, R, h, 2 * Fe, dgu, 2 * Fe, W + Mo[M_GU].off, h, dX,
                  h, a.moff, 2 * Fe * h, 0));
  CK(gemm(c, s, MT_GEMM_TN, wepi, E, h, T, dlog, ldl, a.n2, h, slab(M_ROUTER), h));
  {
    KScope ks(c, s, "moe_combine", 0, (double)T * k * h * 4 + (double)T * h * 4);
    CK(launch_moe_bwd_combine(dX, a.mpos, k, (int)h, T, dn, s));
  }
  CK(gemm(c, s, MT_GEMM_NN, MT_EPI_F32_ACCUM, T, h, E, dlog, ldl, W + Mo[M_ROUTER].off, h, dn, h));
  return hipSuccess;
}

// One decoder block backward.  dy/dyb: gradient of the block output (fp32 and
// bf16); writes dx/dxb (gradient of the block input) and every weight
// gradient into `slab` at the layer's flat offsets.
hipError_t block_backward(mt_ctx* c, const uint16_t* W, const Acts& a, const float* dy,
                          uint16_t* dyb, float* dx, void* slab_base, int layer) {
  const Plan& p = c->p;
  const mt_config& g = p.c;
  const int64_t T = p.T, h = g.hidden, F = g.ffn;
  hipStream_t s = c->sc;
  const TensorOff* L = p.block_layout(layer);
  uint16_t* dgu = c->wsp<uint16_t>(p.ws.dgu);
  float* dn = c->wsp<float>(p.ws.dn);
  float* dh1 = c->wsp<float>(p.ws.dh1);
  uint16_t* dh1b = c->wsp<uint16_t>(p.ws.dh1b);
  uint16_t* dout = c->wsp<uint16_t>(p.ws.dout);
  uint16_t* dqkv = c->wsp<uint16_t>(p.ws.dqkv);
  float* partial = c->wsp<float>(p.ws.partial);
  // weight gradients land in the slab at the layer's flat offsets, fp32 or bf16
  const bool sb = p.slab_bf16;
  const int wepi = sb ? MT_EPI_BF16 : MT_EPI_F32;
  const std::function<void*(int)> slab = [&](int t) -> void* {
    return static_cast<uint8_t*>(slab_base) + (size_t)L[t].off * (sb ? 2 : 4);
  };
  auto dg32 = [&](int t) { return sb ? nullptr : static_cast<float*>(slab(t)); };
  auto dg16 = [&](int t) { return sb ? static_cast<uint16_t*>(slab(t)) : nullptr; };
  if (p.is_moe(layer)) {
    CK(moe_backward(c, W, a, dy, dn, slab, wepi));
  } else {
    // MLP: dm = dy Wd, fused SwiGLU backward -> dgu = [da | du]
    CK(gemm(c, s, MT_GEMM_NN, MT_EPI_SWIGLU_BWD, T, F, h, dyb, h, W + L[T_WDOWN].off, F, dgu, 2 * F,
            nullptr, 0, a.gu, 2 * F, F));
    CK(gemm(c, s, MT_GEMM_TN, wepi, h, F, T, dyb, h, a.m, F, slab(T_WDOWN), F));
    CK(gemm(c, s, MT_GEMM_TN, wepi, 2 * F, h, T, dgu, 2 * F, a.n2, h, slab(T_WGATE), h));
    CK(gemm(c, s, MT_GEMM_NN, MT_EPI_F32, T, h, 2 * F, dgu, 2 * F, W + L[T_WGATE].off, h, dn, h));
  }
  const double nb_bwd = (double)T * h * 18;  // dn, x, resid in; dx (fp32 + bf16) out
  {
    KScope k(c, s, "rmsnorm_bwd", 0, nb_bwd);
    CK(launch_rmsnorm_bwd(dn, a.h1, a.rstd2, W + L[T_MLP_NORM].off, dy, dh1, dh1b,
                          dg32(T_MLP_NORM), dg16(T_MLP_NORM), partial, T, (int)h, s));
  }
  // attention
  CK(gemm(c, s, MT_GEMM_NN, MT_EPI_BF16, T, p.qd, h, dh1b, h, W + L[T_WO].off, p.qd, dout, p.qd));
  CK(gemm(c, s, MT_GEMM_TN, wepi, h, p.qd, T, dh1b, h, a.o, p.qd, slab(T_WO), p.qd));
  {
    KScope k(c, s, "attn_bwd", 10.0 * g.head_dim * attn_pairs(g), 0);
    // dq and dk come out rotated back to the pre-RoPE q and k (inverse RoPE fused)
    CK(launch_attn_bwd(a.qkv, a.o, dout, a.lse, c->wsp<char>(p.ws.dsum), dqkv, (int)(T / g.seq_len),
                       g.seq_len, g.n_heads, g.n_kv_heads, g.head_dim, c->wsp<float>(p.ws.cos_t),
                       c->wsp<float>(p.ws.sin_t), s));
  }
  CK(gemm(c, s, MT_GEMM_TN, wepi, p.ldq, h, T, dqkv, p.ldq, a.n1, h, slab(T_WQ), h));
  CK(gemm(c, s, MT_GEMM_NN, MT_EPI_F32, T, h, p.ldq, dqkv, p.ldq, W + L[T_WQ].off, h, dn, h));
  {
    KScope k(c, s, "rmsnorm_bwd", 0, nb_bwd);
    CK(launch_rmsnorm_bwd(dn, a.x, a.rstd1, W + L[T_ATTN_NORM].off, dh1, dx, dyb,
                          dg32(T_ATTN_NORM), dg16(T_ATTN_NORM), partial, T, (int)h, s));
  }
  return hipSuccess;
}

// ------------------------------------------------------------- schedule
void build_steps(mt_ctx* c) {
  const Plan& p = c->p;
  const int L = p.c.n_layers, K = p.c.ckpt_interval, nseg = p.n_segments;
  const int last0 = (nseg - 1) * K;
  std::vector<Step>& st = c->steps;
  st.clear();
  for (int l = 0; l < L; ++l) {
    Step s{K_FWD};
    s.layer = l;
    s.slot = l % K;
    s.unit = l;
    st.push_back(s);
  }
  for (int ch = 0; ch < p.n_chunks; ++ch) {
    Step s{K_HEAD_LOGITS};
    s.chunk = ch;
    s.unit = L + ch;
    st.push_back(s);
  }
  st.push_back(Step{K_CE});
  c->split = st.size();
  for (int ch = p.n_chunks - 1; ch >= 0; --ch) {
    Step s{K_HEAD_GRAD};
    s.chunk = ch;
    s.unit = L + ch;
    st.push_back(s);
  }
  for (int seg = nseg - 1; seg >= 0; --seg) {
    const int lo = seg * K, hi = std::min(L, lo + K);
    if (lo != last0) {
      for (int l = lo; l < hi; ++l) {
        Step s{K_RECOMP};
        s.layer = l;
        s.slot = l - lo;
        s.unit = l;
        s.write_y = (l + 1 < hi);
        st.push_back(s);
      }
    }
    for (int l = hi - 1; l >= lo; --l) {
      Step s{K_BWD};
      s.layer = l;
      s.slot = l - lo;
      s.unit = l;
      st.push_back(s);
    }
  }
  st.push_back(Step{K_EMBED_GRAD});

  // Two-buffer simulation: reuse a resident unit; otherwise evict the buffer
  // whose content is needed latest (or never), and issue the copy right after
  // the last step that reads that buffer.
  c->loads.clear();
  int content[2] = {c->buf_unit[0], c->buf_unit[1]};
  int last_use[2] = {-1, -1};
  const int n = (int)st.size();
  for (int i = 0; i < n; ++i) {
    Step& s = st[i];
    if (s.unit < 0) continue;
    int b = -1;
    for (int k = 0; k < 2; ++k)
      if (content[k] == s.unit) b = k;
    if (b < 0) {
      int nu[2];
      for (int k = 0; k < 2; ++k) {
        nu[k] = n + 1;
        for (int j = i; j < n; ++j)
          if (st[j].unit >= 0 && st[j].unit == content[k]) {
            nu[k] = j;
            break;
          }
      }
      // never evict the buffer the previous step uses (it may still run)
      int prev = -1;
      for (int j = i - 1; j >= 0; --j)
        if (st[j].unit >= 0) {
          prev = st[j].buf;
          break;
        }
      if (prev >= 0)
        b = 1 - prev;
      else
        b = (nu[0] >= nu[1]) ? 0 : 1;
      c->loads.push_back(Load{s.unit, b, last_use[b]});
      s.load = (int)c->loads.size() - 1;
      content[b] = s.unit;
    }
    s.buf = b;
    last_use[b] = i;
  }
  c->buf_unit[0] = content[0];
  c->buf_unit[1] = content[1];
  c->next_load = 0;
  c->next_step = 0;
}

mt_status issue_load(mt_ctx* c, const Load& ld) {
  const uint16_t* src;
  int64_t n;
  c->unit_src(ld.unit, &src, &n);
  {  // an overlapped optimizer step may still be refreshing this unit's copy
    std::unique_lock<std::mutex> lk(c->mu);
    c->idle_cv.wait(lk, [&] { return !c->upd_pending[ld.unit] || c->poisoned.load(); });
    if (c->poisoned) return MT_E_ABORTED;
  }
  MT_HIP(c, hipStreamWaitEvent(c->sp, c->ev_free[ld.buf], 0));
  {
    KScope k(c, c->sp, "h2d_load", 0, (double)n * 2);
    MT_HIP(c, hipMemcpyAsync(c->wbuf[ld.buf], src, (size_t)n * 2, hipMemcpyHostToDevice, c->sp));
  }
  MT_HIP(c, hipEventRecord(c->ev_ready[ld.buf], c->sp));
  c->st.h2d_bytes += n * 2;
  c->st.weight_loads += 1;
  return MT_OK;
}

mt_status issue_ready_loads(mt_ctx* c, int enqueued_upto) {
  while (c->next_load < c->loads.size() && c->loads[c->next_load].after <= enqueued_upto) {
    mt_status r = issue_load(c, c->loads[c->next_load]);
    if (r != MT_OK) return r;
    ++c->next_load;
  }
  return MT_OK;
}

// --------------------------------------------------------------- slabs
int acquire_slab(mt_ctx* c) {
  std::unique_lock<std::mutex> lk(c->mu);
  if (c->free_slabs.empty()) {
    c->st.slab_waits += 1;
    const double t0 = now_s();
    c->slab_cv.wait(lk, [&] { return !c->free_slabs.empty() || c->poisoned.load(); });
    c->st.slab_wait_s += now_s() - t0;
  }
  if (c->free_slabs.empty()) return -1;
  int s = c->free_slabs.back();
  c->free_slabs.pop_back();
  return s;
}

// Device -> pinned host copy on the offload stream, by the DMA engine or by
// a copy kernel (mt_config.drain_workgroups).
hipError_t drain(mt_ctx* c, void* host, const void* dev, size_t bytes) {
  const int wgs = c->p.c.drain_workgroups;
  if (wgs == 0) return hipMemcpyAsync(host, dev, bytes, hipMemcpyDeviceToHost, c->so);
  return launch_copy(host, dev, bytes, wgs, c->so);
}

// Gradient of a unit is complete in device slab s: copy it out and hand it to
// the worker.
mt_status offload_slab(mt_ctx* c, int s, int group, int64_t e0, int64_t n, int unit) {
  MT_HIP(c, hipEventRecord(c->ev_written[s], c->sc));
  MT_HIP(c, hipStreamWaitEvent(c->so, c->ev_written[s], 0));
  const size_t bytes = (size_t)n * (c->p.slab_bf16 ? 2 : 4);
  {
    KScope k(c, c->so, "drain_d2h", 0, (double)bytes);
    MT_HIP(c, drain(c, c->hslab[s], c->dslab[s], bytes));
  }
  MT_HIP(c, hipEventRecord(c->ev_copied[s], c->so));
  c->st.d2h_bytes += (int64_t)bytes;
  Job j;
  j.kind = Job::SLAB;
  j.slab = s;
  j.group = group;
  j.e0 = e0;
  j.n = n;
  j.add = c->accumulate != 0;
  j.adamw = c->fused;
  j.unit = unit;
  {
    std::lock_guard<std::mutex> g(c->mu);
    if (j.adamw) c->upd_pending[unit] = 1;
    c->jobs.push_back(std::move(j));
    c->outstanding += 1;
  }
  c->cv.notify_all();
  return MT_OK;
}

void worker_main(mt_ctx* c) {
  (void)hipSetDevice(c->device);
  for (;;) {
    Job j;
    {
      std::unique_lock<std::mutex> lk(c->mu);
      c->cv.wait(lk, [&] { return c->stop || !c->jobs.empty(); });
      if (c->jobs.empty()) return;
      j = std::move(c->jobs.front());
      c->jobs.pop_front();
    }
    hipError_t e = hipEventSynchronize(j.kind == Job::SLAB ? c->ev_copied[j.slab]
                                                           : c->ev_dx0_copied[j.parity]);
    if (e != hipSuccess) {
      c->set_err("worker: hipEventSynchronize: %s", hipGetErrorString(e));
      c->poisoned = true;
    } else {
      if (c->delay_us > 0) std::this_thread::sleep_for(std::chrono::microseconds(c->delay_us));
      const double t0 = now_s();
      const mt_ctx::Bind& b = c->bind_of(j.kind == Job::SLAB ? j.group : MT_GROUP_EMBED);
      // A slab holding a unit's last gradient of the step goes to the
      // optimizer thread as is: it adds the slab and steps in one pass over
      // the host state, then returns the slab.
      const bool fused = j.adamw && j.kind == Job::SLAB;
      if (fused) {
      } else if (j.kind == Job::SLAB) {
        if (c->p.slab_bf16)
          accumulate_bf16(*c->pool, b.grad + j.e0, reinterpret_cast<const uint16_t*>(c->hslab[j.slab]),
                          j.n, j.add);
        else
          accumulate(*c->pool, b.grad + j.e0, c->hslab[j.slab], j.n, j.add);
      } else {
        const int64_t h = c->p.c.hidden;
        embed_scatter(*c->pool, c->embed.grad, c->embed.n / h, j.tok.data(),
                      (int64_t)j.tok.size(), h, c->dx0_stage[j.parity], j.add);
      }
      const double t1 = now_s();
      if (!fused) {  // the staging memory is consumed: hand it back before the optimizer runs
        std::lock_guard<std::mutex> g(c->mu);
        c->st.accumulate_s += t1 - t0;
        if (j.kind == Job::SLAB)
          c->free_slabs.push_back(j.slab);
        else
          c->embed_busy[j.parity] = 0;
      }
      c->slab_cv.notify_all();
      c->idle_cv.notify_all();
      if (j.adamw) {  // the optimizer thread takes it from here
        std::lock_guard<std::mutex> g(c->mu);
        Job o;
        o.kind = j.kind;
        o.group = j.kind == Job::SLAB ? j.group : MT_GROUP_EMBED;
        o.e0 = j.kind == Job::SLAB ? j.e0 : 0;
        o.n = j.kind == Job::SLAB ? j.n : b.n;
        o.unit = j.unit;
        o.slab = fused ? j.slab : -1;
        o.add = j.add;
        c->opt_jobs.push_back(std::move(o));
        c->outstanding += 1;
        c->opt_cv.notify_all();
      }
    }
    {
      std::lock_guard<std::mutex> g(c->mu);
      if (e != hipSuccess) {
        if (j.kind == Job::SLAB)
          c->free_slabs.push_back(j.slab);
        else
          c->embed_busy[j.parity] = 0;
      }
      c->outstanding -= 1;
    }
    c->slab_cv.notify_all();
    c->idle_cv.notify_all();
  }
}

// AdamW on groups (or head chunks) whose last-micro-batch gradient is complete,
// on its own thread and pool so that slab draining never waits behind it.
void opt_main(mt_ctx* c) {
  for (;;) {
    Job j;
    {
      std::unique_lock<std::mutex> lk(c->mu);
      c->opt_cv.wait(lk, [&] { return c->stop || !c->opt_jobs.empty(); });
      if (c->opt_jobs.empty()) return;
      // Serve pending units in the order the next forward reads them
      // (embedding, blocks 0..L-1, head chunks): the backward hands them over
      // last-block-first, and any backlog would otherwise hold up block 0.
      auto key = [](const Job& x) { return x.kind == Job::SLAB ? x.unit : -1; };
      auto it = std::min_element(c->opt_jobs.begin(), c->opt_jobs.end(),
                                 [&](const Job& a, const Job& b) { return key(a) < key(b); });
      j = std::move(*it);
      c->opt_jobs.erase(it);
    }
    const double t0 = now_s();
    const mt_ctx::Bind& b = c->bind_of(j.group);
    if (j.slab >= 0)  // last gradient still in its slab: add it and step in one pass
      adamw_slab(*c->opt_pool, b.master + j.e0, b.grad + j.e0, b.m + j.e0, b.v + j.e0,
                 b.pinned ? b.pinned + j.e0 : nullptr, c->hslab[j.slab], c->p.slab_bf16, j.add,
                 j.n, c->hp, c->opt_step);
    else
      adamw(*c->opt_pool, b.master + j.e0, b.grad + j.e0, b.m + j.e0, b.v + j.e0,
            b.pinned ? b.pinned + j.e0 : nullptr, j.n, c->hp, c->opt_step);
    {
      std::lock_guard<std::mutex> g(c->mu);
      c->st.adamw_s += now_s() - t0;
      if (j.slab >= 0) {
        c->free_slabs.push_back(j.slab);
        c->slab_cv.notify_all();
      }
      if (j.kind == Job::SLAB)
        c->upd_pending[j.unit] = 0;
      else
        c->embed_upd_pending = false;
      c->outstanding -= 1;
    }
    c->idle_cv.notify_all();
  }
}

// ---------------------------------------------------------- step bodies
mt_status run_step(mt_ctx* c, const Step& s) {
  const Plan& p = c->p;
  const mt_config& g = p.c;
  const int L = g.n_layers, K = g.ckpt_interval;
  const int64_t T = p.T, h = g.hidden;
  hipStream_t cs = c->sc;
  const uint16_t* W = s.buf >= 0 ? c->wbuf[s.buf] : nullptr;
  if (s.load >= 0) MT_HIP(c, hipStreamWaitEvent(cs, c->ev_ready[s.buf], 0));

  switch (s.kind) {
    case K_FWD:
    case K_RECOMP: {
      const int l = s.layer;
      const int w = s.slot;
      float* x = (l % K == 0) ? c->ckpt_ptr(l / K) : c->slot_x(w);
      float* y = nullptr;
      if (s.kind == K_FWD) {
        if (l == L - 1)
          y = c->wsp<float>(p.ws.xL);
        else if ((l + 1) % K == 0)
          y = c->ckpt_ptr((l + 1) / K);
        else
          y = c->slot_x(w + 1);
      } else if (s.write_y) {
        y = c->slot_x(w + 1);
      }
      MT_HIP(c, block_forward(c, W, acts_of(c, w, x), y, l));
      c->st.layer_forwards += 1;
      break;
    }
    case K_HEAD_LOGITS: {
      // the chunk's logits, one token chunk at a time, reduced at once to
      // softmax statistics merged into each token's running log-sum-exp
      const int ch = s.chunk;
      const uint16_t* Wr = W + (ch == 0 ? p.head[1].off : 0);
      const int64_t r0 = p.chunk_row0[ch], nr = p.chunk_row0[ch + 1] - r0;
      if (ch == 0)
        MT_HIP(c, launch_rmsnorm_fwd(c->wsp<float>(p.ws.xL), W + p.head[0].off,
                                     c->wsp<uint16_t>(p.ws.xf), c->wsp<float>(p.ws.rstd_f), T,
                                     (int)h, g.rms_eps, cs));
      const int32_t* lab = c->wsp<int32_t>(p.ws.labels[c->parity]);
      for (int64_t t0 = 0; t0 < T; t0 += p.head_tc) {
        const int64_t tn = std::min<int64_t>(p.head_tc, T - t0);
        MT_HIP(c, gemm(c, cs, MT_GEMM_NT, MT_EPI_F32, tn, nr, h, c->wsp<uint16_t>(p.ws.xf) + t0 * h,
                       h, Wr, h, c->wsp<float>(p.ws.logits), p.head_rows));
        KScope k(c, cs, "cross_entropy", 0, (double)tn * nr * 4);
        MT_HIP(c, launch_ce_stats(c->wsp<float>(p.ws.logits), p.head_rows, tn, (int)nr, r0, lab + t0,
                                  ch == 0, c->wsp<float>(p.ws.ce_m) + t0,
                                  c->wsp<float>(p.ws.ce_s) + t0, c->wsp<float>(p.ws.ce_lab) + t0,
                                  cs));
      }
      break;
    }
    case K_CE: {
      break;  // launched by mt_forward, which knows the labels
    }
    case K_HEAD_GRAD: {
      const int ch = s.chunk;
      const int sl = acquire_slab(c);
      if (sl < 0) return MT_E_ABORTED;
      const bool sb = p.slab_bf16;
      const size_t es = sb ? 2 : 4;
      uint8_t* slab = reinterpret_cast<uint8_t*>(c->dslab[sl]);
      const int64_t e0 = p.chunk_e0[ch], ne = p.chunk_e0[ch + 1] - e0;
      const uint16_t* Wr = W + (ch == 0 ? p.head[1].off : 0);
      void* dWr = slab + (ch == 0 ? p.head[1].off : 0) * es;
      const int64_t r0 = p.chunk_row0[ch], nr = p.chunk_row0[ch + 1] - r0;
      if (ch == 0 && p.head[1].off > p.head[0].numel)
        MT_HIP(c, hipMemsetAsync(slab, 0, (size_t)p.head[1].off * es, cs));
      // per token chunk: recompute the chunk's logits, form dlogits from the
      // forward's log-sum-exp, then dxf (+)= dl W and dW (+)= dl^T xf
      const int32_t* lab = c->wsp<int32_t>(p.ws.labels[c->parity]);
      CeCoef cf;
      cf.T_mb = p.T_mb;
      for (int mb = 0; mb < 32; ++mb)
        cf.c[mb] = (mb < p.n_mb && c->n_valid[mb] > 0) ? c->grad_scale / (float)c->n_valid[mb] : 0.0f;
      uint16_t* dl = c->wsp<uint16_t>(p.ws.dlogits);
      const bool multi = p.n_tchunks > 1;
      float* acc32 = sb ? c->wsp<float>(p.ws.dw_acc) : static_cast<float*>(dWr);
      for (int64_t t0 = 0; t0 < T; t0 += p.head_tc) {
        const int64_t tn = std::min<int64_t>(p.head_tc, T - t0);
        const uint16_t* xf = c->wsp<uint16_t>(p.ws.xf) + t0 * h;
        MT_HIP(c, gemm(c, cs, MT_GEMM_NT, MT_EPI_F32, tn, nr, h, xf, h, Wr, h,
                       c->wsp<float>(p.ws.logits), p.head_rows));
        {
          KScope k(c, cs, "cross_entropy", 0, (double)tn * nr * 6);
          MT_HIP(c, launch_ce_grad(c->wsp<float>(p.ws.logits), p.head_rows, tn, (int)nr, r0,
                                   lab + t0, c->wsp<float>(p.ws.ce_lse) + t0, t0, cf, dl,
                                   p.head_rows, cs));
        }
        MT_HIP(c, gemm(c, cs, MT_GEMM_NN, c->head_grad_first ? MT_EPI_F32 : MT_EPI_F32_ACCUM, tn, h,
                       nr, dl, p.head_rows, Wr, h, c->wsp<float>(p.ws.dxf) + t0 * h, h));
        if (!multi)
          MT_HIP(c, gemm(c, cs, MT_GEMM_TN, sb ? MT_EPI_BF16 : MT_EPI_F32, nr, h, tn, dl,
                         p.head_rows, xf, h, dWr, h));
        else
          MT_HIP(c, gemm(c, cs, MT_GEMM_TN, t0 == 0 ? MT_EPI_F32 : MT_EPI_F32_ACCUM, nr, h, tn, dl,
                         p.head_rows, xf, h, acc32, h));
      }
      if (multi && sb) {
        KScope k(c, cs, "cast_bf16", 0, (double)nr * h * 6);
        MT_HIP(c, launch_cast_bf16(acc32, static_cast<uint16_t*>(dWr), nr * h, cs));
      }
      c->head_grad_first = false;
      if (ch == 0) {
        c->dy_idx = 0;
        MT_HIP(c, launch_rmsnorm_bwd(c->wsp<float>(p.ws.dxf), c->wsp<float>(p.ws.xL),
                                     c->wsp<float>(p.ws.rstd_f), W + p.head[0].off, nullptr,
                                     c->wsp<float>(p.ws.dy0), c->wsp<uint16_t>(p.ws.dyb),
                                     sb ? nullptr : reinterpret_cast<float*>(slab),
                                     sb ? reinterpret_cast<uint16_t*>(slab) : nullptr,
                                     c->wsp<float>(p.ws.partial), T, (int)h, cs));
      }
      mt_status r = offload_slab(c, sl, MT_GROUP_HEAD, e0, ne, p.c.n_layers + ch);
      if (r != MT_OK) return r;
      break;
    }
    case K_BWD: {
      const int l = s.layer, w = s.slot;
      const int sl = acquire_slab(c);
      if (sl < 0) return MT_E_ABORTED;
      void* slab = c->dslab[sl];
      {  // padding between tensors (absent at the supported widths) must read as zero
        const TensorOff* BL = p.block_layout(l);
        bool gaps = BL[T_COUNT - 1].off + BL[T_COUNT - 1].numel != p.block_elems(l);
        for (int t = 1; t < T_COUNT; ++t) gaps = gaps || BL[t].off != BL[t - 1].off + BL[t - 1].numel;
        if (gaps)
          MT_HIP(c, hipMemsetAsync(slab, 0, (size_t)p.block_elems(l) * (p.slab_bf16 ? 2 : 4), cs));
      }
      float* x = (l % K == 0) ? c->ckpt_ptr(l / K) : c->slot_x(w);
      float* dy = c->wsp<float>(c->dy_idx ? p.ws.dy1 : p.ws.dy0);
      float* dx = c->wsp<float>(c->dy_idx ? p.ws.dy0 : p.ws.dy1);
      MT_HIP(c, block_backward(c, W, acts_of(c, w, x), dy, c->wsp<uint16_t>(p.ws.dyb), dx, slab, l));
      c->dy_idx ^= 1;
      c->st.layer_backwards += 1;
      mt_status r = offload_slab(c, sl, l, 0, p.block_elems(l), l);
      if (r != MT_OK) return r;
      break;
    }
    case K_EMBED_GRAD: {
      const int par = c->parity;
      {  // the staging buffer of two micro-batches ago must be consumed
        std::unique_lock<std::mutex> lk(c->mu);
        c->idle_cv.wait(lk, [&] { return c->embed_busy[par] == 0 || c->poisoned.load(); });
        if (c->poisoned) return MT_E_ABORTED;
        c->embed_busy[par] = 1;
      }
      float* dx0 = c->wsp<float>(c->dy_idx ? p.ws.dy1 : p.ws.dy0);
      MT_HIP(c, hipEventRecord(c->ev_dx0[par], cs));
      MT_HIP(c, hipStreamWaitEvent(c->so, c->ev_dx0[par], 0));
      {
        KScope k(c, c->so, "drain_d2h", 0, (double)T * h * 4);
        MT_HIP(c, drain(c, c->dx0_stage[par], dx0, (size_t)T * h * 4));
      }
      MT_HIP(c, hipEventRecord(c->ev_dx0_copied[par], c->so));
      c->st.d2h_bytes += T * h * 4;
      Job j;
      j.kind = Job::EMBED;
      j.parity = par;
      j.add = c->accumulate != 0;
      j.adamw = c->fused;
      j.tok = c->tok_cur;
      {
        std::lock_guard<std::mutex> gd(c->mu);
        if (j.adamw) c->embed_upd_pending = true;
        c->jobs.push_back(std::move(j));
        c->outstanding += 1;
      }
      c->cv.notify_all();
      MT_HIP(c, hipEventRecord(c->ev_bwd_done[par], cs));
      c->bwd_used[par] = true;
      break;
    }
  }
  if (s.buf >= 0) MT_HIP(c, hipEventRecord(c->ev_free[s.buf], cs));
  return MT_OK;
}

// Enqueue steps [next_step, end), issuing each copy as soon as the step that
// frees its buffer is enqueued.
mt_status run_until(mt_ctx* c, size_t end, const int64_t* n_valid, float grad_scale) {
  mt_status r = issue_ready_loads(c, (int)c->next_step - 1);
  if (r != MT_OK) return r;
  for (; c->next_step < end; ++c->next_step) {
    const Step& s = c->steps[c->next_step];
    if (s.load >= 0 && (size_t)s.load >= c->next_load) {
      c->set_err("internal: copy for step %zu not issued", c->next_step);
      c->poisoned = true;
      return MT_E_STATE;
    }
    if (s.kind == K_CE) {
      // per-token loss from the merged log-sum-exp; one mean per micro-batch
      // of the pass, each over its own labelled tokens; the pass loss (slot
      // 0) is the mean of theirs
      const Plan& p = c->p;
      const int64_t Tm = p.T_mb;
      float* loss = c->wsp<float>(p.ws.loss);
      for (int mb = 0; mb < p.n_mb; ++mb) {
        c->n_valid[mb] = n_valid[mb];
      }
      c->grad_scale = grad_scale;
      {
        KScope k(c, c->sc, "cross_entropy", 0, (double)p.T * 20);
        MT_HIP(c, launch_ce_finish(c->wsp<float>(p.ws.ce_m), c->wsp<float>(p.ws.ce_s),
                                   c->wsp<float>(p.ws.ce_lab),
                                   c->wsp<int32_t>(p.ws.labels[c->parity]), p.T,
                                   c->wsp<float>(p.ws.ce_lse), c->wsp<float>(p.ws.loss_rows), c->sc));
      }
      for (int mb = 0; mb < p.n_mb; ++mb)
        MT_HIP(c, launch_loss_mean(c->wsp<float>(p.ws.loss_rows) + mb * Tm, Tm,
                                   n_valid[mb] > 0 ? 1.0f / (float)n_valid[mb] : 0.0f,
                                   p.n_mb == 1 ? loss : loss + 1 + mb, c->sc));
      if (p.n_mb > 1) MT_HIP(c, launch_mean(loss + 1, p.n_mb, loss, c->sc));
    } else {
      r = run_step(c, s);
      if (r != MT_OK) return r;
    }
    r = issue_ready_loads(c, (int)c->next_step);
    if (r != MT_OK) return r;
  }
  return MT_OK;
}

mt_status check_live(const mt_ctx* c) {
  if (!c) return MT_E_ARG;
  if (c->poisoned) return MT_E_ABORTED;
  return MT_OK;
}

}  // namespace

// =================================================================== C ABI
extern "C" mt_status mt_create(const mt_config* cfg, const mt_device_arena* a, mt_ctx** out) {
  if (!cfg || !a || !out) return MT_E_ARG;
  *out = nullptr;
  std::unique_ptr<mt_ctx> c(new (std::nothrow) mt_ctx());
  if (!c) return MT_E_NOMEM;
  if (!make_plan(*cfg, &c->p).empty()) return MT_E_ARG;
  const Plan& p = c->p;
  c->nslab = cfg->n_grad_slabs;
  auto al = [](const void* q) { return q && ((uintptr_t)q % 256) == 0; };
  if (!al(a->weight_buf[0]) || !al(a->weight_buf[1]) || !al(a->window) || !al(a->workspace))
    return MT_E_ARG;
  if (p.n_segments > 1 && !al(a->checkpoints)) return MT_E_ARG;
  for (int i = 0; i < c->nslab; ++i)
    if (!al(a->grad_slab[i])) return MT_E_ARG;
  if (!a->stream_prefetch || !a->stream_compute || !a->stream_offload ||
      a->stream_prefetch == a->stream_compute || a->stream_prefetch == a->stream_offload ||
      a->stream_compute == a->stream_offload)
    return MT_E_ARG;
  if (a->weight_buf_bytes < p.weight_buf_bytes || a->grad_slab_bytes < p.slab_bytes ||
      a->window_bytes < p.window_bytes || a->workspace_bytes < p.ws.bytes ||
      (p.n_segments > 1 && a->checkpoints_bytes < p.ckpt_bytes))
    return MT_E_NOMEM;

  hipError_t e = hipGetDevice(&c->device);
  if (e != hipSuccess) return MT_E_HIP;
  c->sp = (hipStream_t)a->stream_prefetch;
  c->sc = (hipStream_t)a->stream_compute;
  c->so = (hipStream_t)a->stream_offload;
  c->wbuf[0] = (uint16_t*)a->weight_buf[0];
  c->wbuf[1] = (uint16_t*)a->weight_buf[1];
  for (int i = 0; i < c->nslab; ++i) c->dslab[i] = (float*)a->grad_slab[i];
  c->window = (uint8_t*)a->window;
  c->ckpt = (uint8_t*)a->checkpoints;
  c->ws = (uint8_t*)a->workspace;
  c->layers.resize(cfg->n_layers);
  c->upd_pending.assign(cfg->n_layers + p.n_chunks, 0);

  auto ev = [&](hipEvent_t* x) { return hipEventCreateWithFlags(x, hipEventDisableTiming); };
  for (int i = 0; i < 2; ++i) {
    if (ev(&c->ev_ready[i]) || ev(&c->ev_free[i]) || ev(&c->ev_x0[i]) || ev(&c->ev_bwd_done[i]) ||
        ev(&c->ev_dx0[i]) || ev(&c->ev_dx0_copied[i]))
      return MT_E_HIP;
  }
  for (int i = 0; i < c->nslab; ++i)
    if (ev(&c->ev_written[i]) || ev(&c->ev_copied[i])) return MT_E_HIP;
  if (ev(&c->ev_loss)) return MT_E_HIP;
  if (hipEventCreate(&c->ev_origin) != hipSuccess) return MT_E_HIP;

  const size_t T = (size_t)p.T, h = (size_t)cfg->hidden;
  for (int i = 0; i < c->nslab; ++i)
    if (hipHostMalloc((void**)&c->hslab[i], p.slab_bytes, hipHostMallocDefault) != hipSuccess)
      return MT_E_NOMEM;
  for (int i = 0; i < 2; ++i) {
    if (hipHostMalloc((void**)&c->x0_stage[i], T * h * 4, hipHostMallocDefault) != hipSuccess ||
        hipHostMalloc((void**)&c->dx0_stage[i], T * h * 4, hipHostMallocDefault) != hipSuccess ||
        hipHostMalloc((void**)&c->lab_stage[i], T * 4, hipHostMallocDefault) != hipSuccess)
      return MT_E_NOMEM;
  }
  if (hipHostMalloc((void**)&c->loss_pin, mt_ctx::kLossRing * 4, hipHostMallocDefault) !=
      hipSuccess)
    return MT_E_NOMEM;

  // RoPE table: angles in float64, stored fp32 (host-computed once).
  {
    const size_t n = (size_t)cfg->seq_len * (cfg->head_dim / 2);
    std::vector<float> cs(n), sn(n);
    rope_table(cfg->seq_len, cfg->head_dim, cfg->rope_base, cs.data(), sn.data());
    if (hipMemcpy(c->ws + p.ws.cos_t, cs.data(), n * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(c->ws + p.ws.sin_t, sn.data(), n * 4, hipMemcpyHostToDevice) != hipSuccess)
      return MT_E_HIP;
  }

  c->pool.reset(new ThreadPool(cfg->host_threads > 0 ? cfg->host_threads : default_threads()));
  c->opt_pool.reset(new ThreadPool(cfg->host_threads > 0 ? cfg->host_threads : default_threads()));
  c->io_pool.reset(new ThreadPool(4));
  if (const char* d = getenv("MT_TEST_WORKER_DELAY_US")) c->delay_us = atoi(d);
  for (int i = c->nslab - 1; i >= 0; --i) c->free_slabs.push_back(i);
  c->worker = std::thread(worker_main, c.get());
  c->opt_worker = std::thread(opt_main, c.get());
  *out = c.release();
  return MT_OK;
}

extern "C" void mt_destroy(mt_ctx* c) {
  if (!c) return;
  (void)hipStreamSynchronize(c->sp);
  (void)hipStreamSynchronize(c->sc);
  (void)hipStreamSynchronize(c->so);
  {
    std::lock_guard<std::mutex> g(c->mu);
    c->stop = true;
  }
  c->cv.notify_all();
  c->opt_cv.notify_all();
  if (c->worker.joinable()) c->worker.join();
  if (c->opt_worker.joinable()) c->opt_worker.join();
  for (auto& b : c->layers)
    if (b.pinned) (void)hipHostFree(b.pinned);
  if (c->head.pinned) (void)hipHostFree(c->head.pinned);
  for (int i = 0; i < c->nslab; ++i)
    if (c->hslab[i]) (void)hipHostFree(c->hslab[i]);
  for (int i = 0; i < 2; ++i) {
    if (c->x0_stage[i]) (void)hipHostFree(c->x0_stage[i]);
    if (c->dx0_stage[i]) (void)hipHostFree(c->dx0_stage[i]);
    if (c->lab_stage[i]) (void)hipHostFree(c->lab_stage[i]);
  }
  if (c->loss_pin) (void)hipHostFree(c->loss_pin);
  hipEvent_t* evs[] = {c->ev_ready, c->ev_free, c->ev_x0, c->ev_bwd_done, c->ev_dx0,
                       c->ev_dx0_copied};
  for (auto* e : evs)
    for (int i = 0; i < 2; ++i)
      if (e[i]) (void)hipEventDestroy(e[i]);
  if (c->ev_loss) (void)hipEventDestroy(c->ev_loss);
  if (c->ev_origin) (void)hipEventDestroy(c->ev_origin);
  for (auto& r : c->krec) {
    c->ev_pool.push_back(r.a);
    c->ev_pool.push_back(r.b);
  }
  for (hipEvent_t e : c->ev_pool) (void)hipEventDestroy(e);
  for (int i = 0; i < c->nslab; ++i) {
    if (c->ev_written[i]) (void)hipEventDestroy(c->ev_written[i]);
    if (c->ev_copied[i]) (void)hipEventDestroy(c->ev_copied[i]);
  }
  delete c;
}

extern "C" const char* mt_last_error(const mt_ctx* c) {
  if (!c) return "null context";
  return c->err.c_str();
}

extern "C" mt_status mt_bind_layer(mt_ctx* c, int32_t group, float* master, float* grad,
                                   float* adam_m, float* adam_v, int64_t numel) {
  mt_status r = check_live(c);
  if (r != MT_OK) return r;
  if (!master || !grad || !adam_m || !adam_v) return MT_E_ARG;
  const Plan& p = c->p;
  int64_t want;
  mt_ctx::Bind* b;
  if (group == MT_GROUP_EMBED) {
    want = p.embed_elems;
    b = &c->embed;
  } else if (group == MT_GROUP_HEAD) {
    want = p.head_elems;
    b = &c->head;
  } else if (group >= 0 && group < p.c.n_layers) {
    want = p.block_elems(group);
    b = &c->layers[group];
  } else {
    return MT_E_ARG;
  }
  if (numel != want) {
    c->set_err("group %d: numel %lld, layout needs %lld", group, (long long)numel,
               (long long)want);
    return MT_E_ARG;
  }
  if (c->state == ST_FWD || c->state == ST_BWD) return MT_E_STATE;
  b->master = master;
  b->grad = grad;
  b->m = adam_m;
  b->v = adam_v;
  b->n = numel;
  if (group != MT_GROUP_EMBED) {
    if (!b->pinned &&
        hipHostMalloc((void**)&b->pinned, (size_t)numel * 2, hipHostMallocDefault) != hipSuccess) {
      b->pinned = nullptr;
      return MT_E_NOMEM;
    }
    cast_bf16(*c->pool, master, b->pinned, numel);
  }
  c->buf_unit[0] = c->buf_unit[1] = -1;
  bool all = c->embed.master && c->head.master;
  for (auto& x : c->layers) all = all && x.master;
  if (all && c->state == ST_UNBOUND) c->state = ST_IDLE;
  return MT_OK;
}

extern "C" mt_status mt_forward(mt_ctx* c, const int32_t* tokens, const int32_t* labels,
                                float grad_scale, float* loss_out) {
  mt_status r = check_live(c);
  if (r != MT_OK) return r;
  if (c->state == ST_UNBOUND) return MT_E_UNBOUND;
  if (c->state == ST_FWD) return MT_E_STATE;
  if (!tokens || !labels || !(grad_scale == grad_scale)) return MT_E_ARG;
  const Plan& p = c->p;
  const int64_t T = p.T, h = p.c.hidden;
  int64_t n_valid[32] = {0};  // per micro-batch of the pass
  for (int64_t t = 0; t < T; ++t) {
    if (tokens[t] < 0 || tokens[t] >= p.c.vocab) return MT_E_ARG;
    if (labels[t] >= p.c.vocab || labels[t] < -1) return MT_E_ARG;
    n_valid[t / p.T_mb] += labels[t] >= 0;
  }
  {  // an overlapped optimizer step may still be updating the embedding
    std::unique_lock<std::mutex> lk(c->mu);
    c->idle_cv.wait(lk, [&] { return !c->embed_upd_pending || c->poisoned.load(); });
    if (c->poisoned) return MT_E_ABORTED;
  }
  c->parity = (int)(c->mb & 1);
  const int par = c->parity;
  // staging of two micro-batches ago must have reached the device
  if (c->x0_used[par]) MT_HIP(c, hipEventSynchronize(c->ev_x0[par]));
  embed_gather(*c->io_pool, c->embed.master, tokens, T, h, c->x0_stage[par]);
  memcpy(c->lab_stage[par], labels, (size_t)T * 4);
  c->tok_cur.assign(tokens, tokens + T);
  // the device copies of x0 / labels of two micro-batches ago are free once
  // that micro-batch's backward has finished
  if (c->bwd_used[par]) MT_HIP(c, hipStreamWaitEvent(c->sp, c->ev_bwd_done[par], 0));
  {
    KScope k(c, c->sp, "h2d_input", 0, (double)T * (h + 1) * 4);
    MT_HIP(c, hipMemcpyAsync(c->ws + p.ws.x0[par], c->x0_stage[par], (size_t)T * h * 4,
                             hipMemcpyHostToDevice, c->sp));
    MT_HIP(c, hipMemcpyAsync(c->ws + p.ws.labels[par], c->lab_stage[par], (size_t)T * 4,
                             hipMemcpyHostToDevice, c->sp));
  }
  MT_HIP(c, hipEventRecord(c->ev_x0[par], c->sp));
  c->x0_used[par] = true;
  MT_HIP(c, hipStreamWaitEvent(c->sc, c->ev_x0[par], 0));

  build_steps(c);
  c->head_grad_first = true;
  c->dy_idx = 0;
  r = run_until(c, c->split, n_valid, grad_scale);
  if (r != MT_OK) return r;
  // loss -> pinned ring, resolved at flush or mt_sync_loss; if this forward's
  // slot still holds an unresolved loss (a whole ring of forwards without
  // either call), the pending losses are resolved first
  if (!c->pending_loss.empty() && c->pending_loss.front().second == c->loss_next) {
    MT_HIP(c, hipEventSynchronize(c->ev_loss));
    for (auto& pl : c->pending_loss) *pl.first = c->loss_pin[pl.second];
    c->pending_loss.clear();
  }
  const int slot = c->loss_next;
  c->loss_next = (c->loss_next + 1) % mt_ctx::kLossRing;
  MT_HIP(c, hipMemcpyAsync(c->loss_pin + slot, c->ws + p.ws.loss, 4, hipMemcpyDeviceToHost, c->sc));
  MT_HIP(c, hipEventRecord(c->ev_loss, c->sc));
  if (loss_out) c->pending_loss.emplace_back(loss_out, slot);
  c->step_slots.push_back(slot);
  c->state = ST_FWD;
  return MT_OK;
}

static mt_status backward_impl(mt_ctx* c, int32_t accumulate_flag, const mt_adamw_hparams* hp,
                               int64_t step) {
  mt_status r = check_live(c);
  if (r != MT_OK) return r;
  if (c->state != ST_FWD) return MT_E_STATE;
  if (accumulate_flag != 0 && accumulate_flag != 1) return MT_E_ARG;
  c->accumulate = accumulate_flag;
  c->fused = hp != nullptr;
  if (c->fused) {
    // A unit is marked "update pending" only when its gradient job is queued
    // (offload_slab / the embedding job): that is its last use in this step,
    // so no copy of it issued by this backward can wait on its own update.
    std::lock_guard<std::mutex> g(c->mu);
    c->hp = *hp;
    c->opt_step = step;
  }
  // The previous micro-batch's embedding gradient may still be draining from
  // dy0/dy1 on the offload stream; this backward overwrites both (the final
  // norm's backward and the first block backward), so the compute stream
  // waits for that drain first (write after read across streams).
  if (c->bwd_used[c->parity ^ 1])
    MT_HIP(c, hipStreamWaitEvent(c->sc, c->ev_dx0_copied[c->parity ^ 1], 0));
  r = run_until(c, c->steps.size(), nullptr, 0.0f);
  c->fused = false;
  if (r != MT_OK) return r;
  if (hp) {
    c->buf_unit[0] = c->buf_unit[1] = -1;  // working copies are being rewritten
    c->last_step_slots.swap(c->step_slots);
    c->step_slots.clear();
  }
  c->mb += 1;
  c->st.microbatches += 1;
  c->state = hp ? ST_IDLE : ST_BWD;
  return MT_OK;
}

extern "C" mt_status mt_backward(mt_ctx* c, int32_t accumulate_flag) {
  return backward_impl(c, accumulate_flag, nullptr, 0);
}

extern "C" mt_status mt_backward_step(mt_ctx* c, int32_t accumulate_flag,
                                      const mt_adamw_hparams* hp, int64_t step) {
  if (!c || !hp || step < 1) return MT_E_ARG;
  return backward_impl(c, accumulate_flag, hp, step);
}

extern "C" mt_status mt_flush_grads(mt_ctx* c) {
  mt_status r = check_live(c);
  if (r != MT_OK) return r;
  if (c->state == ST_FWD) return MT_E_STATE;
  {
    std::unique_lock<std::mutex> lk(c->mu);
    c->idle_cv.wait(lk, [&] { return c->outstanding == 0 || c->poisoned.load(); });
  }
  if (c->poisoned) return MT_E_ABORTED;
  MT_HIP(c, hipStreamSynchronize(c->sp));
  MT_HIP(c, hipStreamSynchronize(c->sc));
  MT_HIP(c, hipStreamSynchronize(c->so));
  MT_HIP(c, c->collect_kernel_times());
  for (auto& pl : c->pending_loss) *pl.first = c->loss_pin[pl.second];
  c->pending_loss.clear();
  if (c->state == ST_BWD) c->state = ST_FLUSHED;
  return MT_OK;
}

extern "C" mt_status mt_sync_loss(mt_ctx* c) {
  mt_status r = check_live(c);
  if (r != MT_OK) return r;
  if (c->pending_loss.empty()) return MT_OK;
  // every loss copy is on the compute stream, so the last one's event covers them all
  MT_HIP(c, hipEventSynchronize(c->ev_loss));
  for (auto& pl : c->pending_loss) *pl.first = c->loss_pin[pl.second];
  c->pending_loss.clear();
  return MT_OK;
}

extern "C" mt_status mt_step_loss(mt_ctx* c, float* loss_out) {
  mt_status r = check_live(c);
  if (r != MT_OK) return r;
  if (!loss_out) return MT_E_ARG;
  const std::vector<int>& sl = c->step_slots.empty() ? c->last_step_slots : c->step_slots;
  if (sl.empty()) return MT_E_STATE;
  // every loss copy is on the compute stream, so the last one's event covers them all
  MT_HIP(c, hipEventSynchronize(c->ev_loss));
  double sum = 0.0;
  for (int s : sl) sum += (double)c->loss_pin[s];
  *loss_out = (float)(sum / (double)sl.size());
  return MT_OK;
}

extern "C" mt_status mt_moe_routing(mt_ctx* c, int32_t layer, int32_t* sel_out) {
  mt_status r = check_live(c);
  if (r != MT_OK) return r;
  const Plan& p = c->p;
  if (!sel_out || layer < 0 || layer >= p.c.n_layers || !p.is_moe(layer)) return MT_E_ARG;
  const size_t n = (size_t)p.T * p.c.top_k;
  MT_HIP(c, hipStreamSynchronize(c->sc));
  MT_HIP(c, hipMemcpy(sel_out, c->wsp<int32_t>(p.ws.mroute) + (layer / p.c.moe_every) * n, n * 4,
                      hipMemcpyDeviceToHost));
  return MT_OK;
}

extern "C" mt_status mt_adamw_step(mt_ctx* c, const mt_adamw_hparams* hp, int64_t step) {
  mt_status r = check_live(c);
  if (r != MT_OK) return r;
  if (!hp || step < 1) return MT_E_ARG;
  if (c->state != ST_FLUSHED) return MT_E_STATE;
  const double t0 = now_s();
  adamw(*c->pool, c->embed.master, c->embed.grad, c->embed.m, c->embed.v, nullptr, c->embed.n,
        *hp, step);
  for (auto& b : c->layers) adamw(*c->pool, b.master, b.grad, b.m, b.v, b.pinned, b.n, *hp, step);
  adamw(*c->pool, c->head.master, c->head.grad, c->head.m, c->head.v, c->head.pinned, c->head.n,
        *hp, step);
  c->buf_unit[0] = c->buf_unit[1] = -1;  // working copies changed
  c->last_step_slots.swap(c->step_slots);
  c->step_slots.clear();
  c->st.adamw_s += now_s() - t0;
  c->state = ST_IDLE;
  return MT_OK;
}

extern "C" mt_status mt_get_stats(mt_ctx* c, mt_stats* out) {
  if (!c || !out) return MT_E_ARG;
  std::lock_guard<std::mutex> g(c->mu);
  *out = c->st;
  return MT_OK;
}

extern "C" mt_status mt_kernel_timing(mt_ctx* c, int32_t enable) {
  mt_status r = check_live(c);
  if (r != MT_OK) return r;
  if (enable != 0 && enable != 1) return MT_E_ARG;
  if (enable) {
    c->ktot.clear();
    for (auto& k : c->krec) {  // records of an earlier window are dropped unread
      c->ev_pool.push_back(k.a);
      c->ev_pool.push_back(k.b);
    }
    c->krec.clear();
    MT_HIP(c, hipEventRecord(c->ev_origin, c->sc));
  }
  c->ktiming = enable != 0;
  return MT_OK;
}

extern "C" mt_status mt_get_kernel_times(mt_ctx* c, mt_kernel_time* out, int32_t cap,
                                         int32_t* n_out) {
  if (!c || !n_out || cap < 0 || (cap > 0 && !out)) return MT_E_ARG;
  std::vector<std::pair<std::string, mt_ctx::KTot>> v(c->ktot.begin(), c->ktot.end());
  std::sort(v.begin(), v.end(), [](const auto& a, const auto& b) { return a.second.ms > b.second.ms; });
  int32_t n = 0;
  for (auto& kv : v) {
    if (n < cap) {
      memset(out[n].name, 0, sizeof(out[n].name));
      strncpy(out[n].name, kv.first.c_str(), sizeof(out[n].name) - 1);
      out[n].launches = kv.second.n;
      out[n].ms = kv.second.ms;
      out[n].flop = kv.second.flop;
      out[n].bytes = kv.second.bytes;
    }
    ++n;
  }
  *n_out = n;
  return MT_OK;
}
