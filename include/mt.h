/*
 * mt.h -- C ABI of libmt: host-memory-centric, layer-streamed training of a
 * Llama-style decoder on one MI355X (gfx950).
 *
 * The method (MegaTrain, as described on the pages cited below):
 *   - fp32 master weights, gradients and Adam m/v live in host memory; the GPU
 *     is a transient compute engine (zhichai.net "MegaTrain：单卡训百亿大模型的突破与实践",
 *     design point 1; m.lqnn.cn MegaTrain article, section 二 "ParameterState").
 *   - layers are streamed in one at a time into a ping-pong pair of flat
 *     device buffers from pinned, pre-flattened host copies (zhichai design
 *     point 2; lqnn 三.1 "gpu_flat_buffers" / "layer_pinned_flats").
 *   - prefetch, compute and gradient offload run on three streams ordered by
 *     events ("no compute before the data is there, no write before the
 *     buffer is free") (zhichai design point 4; lqnn 三.2).
 *   - each layer's gradients land in one of a pool of flat gradient slabs
 *     (default 12) and a CPU thread adds them into the fp32 host gradient
 *     (lqnn 三.3).
 *   - an activation checkpoint every K layers; backward recomputes each
 *     K-layer segment (zhichai design point 3; lqnn 三.4, default K = 4).
 *   - a stateless layer template: the kernels of one block bound at run
 *     time to whatever flat buffer holds the layer (zhichai design point 4;
 *     blog.travelaiplan.net "單卡也能練 100B+：MegaTrain 實戰", 核心功能 3).
 *   - the optimizer step runs on the CPU over the host state (lqnn 二).
 *
 * Conventions
 *   - Every call returns mt_status; no C++ exception crosses the ABI.
 *   - Arguments are validated before anything is enqueued on the GPU.
 *   - The first HIP error poisons the context: later calls return
 *     MT_E_ABORTED; mt_last_error() holds the message.
 *   - A context is used by one caller thread at a time.
 *   - bf16 values are passed as uint16_t bit patterns.
 */
#ifndef MT_H
#define MT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MT_OK = 0,
  MT_E_ARG = -1,      /* invalid argument (null pointer, wrong size, bad value)      */
  MT_E_STATE = -2,    /* call out of order (see the call order below)                */
  MT_E_HIP = -3,      /* a HIP runtime call failed                                   */
  MT_E_NOMEM = -4,    /* host or pinned allocation failed, or an arena is too small  */
  MT_E_UNBOUND = -5,  /* forward called before every group was bound                 */
  MT_E_ABORTED = -6   /* the context was poisoned by an earlier HIP error            */
} mt_status;

/* Parameter groups: 0..n_layers-1 are decoder blocks. */
enum { MT_GROUP_EMBED = -1, MT_GROUP_HEAD = -2 };

typedef struct mt_config {
  int32_t n_layers;       /* decoder blocks                                     */
  int32_t hidden;         /* h, multiple of 256                                 */
  int32_t n_heads;        /* query heads                                        */
  int32_t n_kv_heads;     /* key/value heads, divides n_heads                   */
  int32_t head_dim;       /* d: 64 or 128                                       */
  int32_t ffn;            /* SwiGLU width F, multiple of 16                     */
  int32_t vocab;          /* V, multiple of 256                                 */
  float rms_eps;          /* RMSNorm epsilon (inside the square root)           */
  float rope_base;        /* RoPE base (10000)                                  */
  int32_t micro_batch;    /* b sequences per micro-batch                        */
  int32_t seq_len;        /* s tokens per sequence, multiple of 128             */
  int32_t ckpt_interval;  /* K: checkpoint every K layers (>= 1)                */
  int32_t n_grad_slabs;   /* gradient slab pool size (1..64), 12 by default     */
  int32_t host_threads;   /* CPU threads for accumulate / AdamW (0 = automatic) */
  int32_t slab_bf16;      /* 1: gradient slabs carry bf16 (half the device->host
                             bytes; rounded once per micro-batch, accumulated in
                             fp32 on the host); 0: fp32 slabs                   */
  int32_t drain_workgroups; /* device->host copy of each slab: 0 = the DMA
                             engine (hipMemcpyAsync on the offload stream);
                             n in 1..256 = a copy kernel of n workgroups that
                             writes the pinned host slab directly            */
  int32_t micro_batches_per_pass; /* 1..32: micro-batches that share each
                             weight residency.  mt_forward then takes this
                             many micro-batches of micro_batch sequences at
                             once (tokens [n][micro_batch][seq_len]); each is
                             normalised by its own valid-label count, and
                             their weight gradients are summed on the device
                             before the slab drains: gradient accumulation in
                             layer-major order, with weights crossing the host
                             link once per pass instead of once per
                             micro-batch.  1 = one micro-batch per pass.      */
  int32_t head_token_chunk; /* tokens per LM-head token chunk (a multiple of 8;
                             0 = 8192).  The head's fp32 logits and bf16
                             dlogits exist on the device for one token chunk
                             and one vocabulary chunk at a time: the forward
                             merges each chunk's softmax statistics into a
                             per-token log-sum-exp, the backward recomputes
                             the chunk's logits for its gradient.           */
  /* Mixture-of-experts blocks, a second parameter-structure group (m.lqnn.cn
   * MegaTrain article, 四: layers are grouped by structure, MoE layers form
   * their own group with their own flat layout).  Block l is an MoE block when
   * n_experts > 0 and l % moe_every == moe_every - 1.  Its FFN: router logits
   * r = n2 W_router^T; the top_k experts by logit (ties to the lower index);
   * gates = softmax over the selected logits; each expert a SwiGLU of width
   * expert_ffn; the block adds sum_j gate_j * expert_j(n2).  Flat layout of an
   * MoE block: attn_norm, wq, wk, wv, wo, mlp_norm, w_router [E, h], w_gu
   * [E * 2 expert_ffn, h] (expert e's gate rows, then its up rows), w_down
   * [E * h, expert_ffn]. */
  int32_t n_experts;      /* E: 0 (no MoE block) or a multiple of 8, <= 64      */
  int32_t top_k;          /* experts per token, 1..min(8, E)                    */
  int32_t expert_ffn;     /* F_e, a multiple of 128                             */
  int32_t moe_every;      /* >= 1                                               */
} mt_config;

/* One tensor of a group's flat layout. */
typedef struct mt_tensor_desc {
  char name[16];
  int64_t offset;         /* elements from the start of the group's flat array  */
  int64_t numel;
  int32_t rows, cols;     /* matrices are row-major [out, in]; gains are [1, h] */
} mt_tensor_desc;

/* Device and host memory the library needs for a configuration. */
typedef struct mt_device_req {
  size_t weight_buf;      /* bytes of EACH of the two bf16 ping-pong buffers    */
  size_t grad_slab;       /* bytes of EACH gradient slab (bf16 or fp32)         */
  size_t window;          /* activations of one K-layer recompute window        */
  size_t checkpoints;     /* max(1, ceil(L/K) - 1) fp32 [T, h] inputs of layers
                             K, 2K, ... (layer 0's input is the x0 staging in
                             the workspace)                                     */
  size_t workspace;       /* head logits of one token chunk, gradients in
                             flight, RoPE table, ...                            */
  size_t device_total;    /* 2*weight_buf + n_slabs*grad_slab + the rest        */
  size_t pinned_host;     /* pinned host bytes the library allocates itself     */
  size_t host_state;      /* caller-owned fp32 master+grad+m+v: 16 B/parameter  */
  int64_t unit_elems;     /* elements of the largest streamed unit              */
  int32_t head_chunks;    /* vocabulary chunks the LM head is streamed in       */
  int32_t reserved;
} mt_device_req;

/* Device memory and streams, owned by the caller (PyTorch allocates them).
 * Each pointer must be 256-byte aligned and at least the size given by
 * mt_device_requirements.  Streams are hipStream_t handles at default
 * priority; the three must be distinct. */
typedef struct mt_device_arena {
  void* weight_buf[2];
  void* grad_slab[64];    /* first n_grad_slabs entries used                    */
  void* window;
  void* checkpoints;
  void* workspace;
  void* stream_prefetch;  /* host -> device weight copies                       */
  void* stream_compute;   /* kernels                                            */
  void* stream_offload;   /* device -> host gradient copies                     */
  /* bytes actually allocated for each region (checked against the needs) */
  size_t weight_buf_bytes, grad_slab_bytes, window_bytes, checkpoints_bytes, workspace_bytes;
} mt_device_arena;

/* AdamW hyper-parameters (double so that derived coefficients such as
 * 1 - beta1^t are formed from the exact values the caller holds). */
typedef struct mt_adamw_hparams {
  double lr, beta1, beta2, eps, weight_decay;
} mt_adamw_hparams;

/* Per-context counters, cumulative since mt_create. */
typedef struct mt_stats {
  int64_t h2d_bytes;          /* weight bytes copied host -> device            */
  int64_t d2h_bytes;          /* gradient bytes copied device -> host          */
  int64_t weight_loads;       /* streamed units loaded                         */
  int64_t layer_forwards;     /* block forwards incl. recompute                */
  int64_t layer_backwards;
  int64_t slab_waits;         /* times the enqueue thread waited for a slab    */
  double slab_wait_s;         /* host seconds spent waiting for slabs          */
  double accumulate_s;        /* worker seconds adding slabs into host grads   */
  double adamw_s;             /* seconds in mt_adamw_step                      */
  int64_t microbatches;
  /* While mt_kernel_timing is enabled, from the same HIP timing events, added
   * up at each mt_flush_grads: device time with a host-link copy in flight
   * (weight and input loads, gradient and dx0 drains), with a compute kernel
   * running, and with both at once (union measures, milliseconds). */
  double timed_copy_ms;
  double timed_kernel_ms;
  double timed_overlap_ms;
} mt_stats;

typedef struct mt_ctx mt_ctx;

/* Flat layout of one group (pure, no GPU).  Tensors start at multiples of 256
 * elements; order: attn_norm, wq, wk, wv, wo, mlp_norm, w_gate, w_up, w_down
 * for blocks; final_norm, w_head for MT_GROUP_HEAD; emb for MT_GROUP_EMBED
 * (lqnn 三.1: pre-flattened per-layer weights).  Writes up to cap descriptors
 * into out (out may be NULL when cap == 0), the count into *n_out and the
 * flat length in elements into *flat_numel.  MT_E_ARG for a bad config/group. */
mt_status mt_layout(const mt_config* cfg, int32_t group, mt_tensor_desc* out, int32_t cap,
                    int32_t* n_out, int64_t* flat_numel);

/* Memory needed for cfg (pure, no GPU): the device holds only the two layer
 * buffers, one checkpoint window of activations, the checkpoints and the slab
 * pool, so device memory does not grow with depth (zhichai design point 2:
 * only the current layer's parameters and gradients on the GPU; lqnn 三.4:
 * one checkpoint window, "1-2 layers of weights plus a few activations").
 * MT_E_ARG for an unsupported config. */
mt_status mt_device_requirements(const mt_config* cfg, mt_device_req* out);

/* Create a context on the current HIP device (lqnn 三.1-三.3: one GPU context
 * with its two flat layer buffers, three streams and the gradient slab pool;
 * the slabs' CPU worker thread starts here).  The arena must satisfy
 * mt_device_requirements(cfg) (MT_E_NOMEM if a region is smaller); it is
 * borrowed, not freed, by the library.  Allocates pinned host slabs and
 * staging buffers, events and the worker threads.  The library allocates no
 * device memory. */
mt_status mt_create(const mt_config* cfg, const mt_device_arena* arena, mt_ctx** out);

/* Bind the host state of one group (lqnn 二: per parameter an fp32 master,
 * its gradient and Adam m / v, all in host memory; lqnn 三.1: a pinned,
 * pre-flattened copy per layer for the fastest DMA path): fp32 master, grad,
 * adam_m, adam_v flat arrays of exactly mt_layout's flat_numel elements
 * (64-byte aligned,
 * pageable memory is fine).  The caller keeps ownership; the arrays must
 * outlive the context.  For blocks and the head the library makes a pinned
 * bf16 working copy (round-to-nearest-even of master) that is what streams
 * to the GPU.  Rebinding a group replaces its pointers and refreshes the copy.
 * The caller must not write master except through mt_adamw_step, and must not
 * touch grad between mt_forward and the return of mt_flush_grads. */
mt_status mt_bind_layer(mt_ctx* ctx, int32_t group, float* master, float* grad, float* adam_m,
                        float* adam_v, int64_t numel);

/* Enqueue the forward pass of one pass of micro_batches_per_pass
 * micro-batches (zhichai design point 2: each layer's parameters are
 * prefetched, the layer runs and its buffer is released; design point 3: a
 * checkpoint every K layers): embedding gather on the host, streamed block
 * forwards with a
 * checkpoint every K layers, the LM head in vocabulary chunks, cross-entropy
 * and its gradient, scaled for each micro-batch by grad_scale / (labelled
 * tokens of that micro-batch).  tokens and labels are host int32 arrays of
 * micro_batches_per_pass*micro_batch*seq_len entries (micro-batch-major, then
 * sequence-major); label -1 is ignored; tokens must be in [0, vocab).  The
 * mean over the pass's micro-batches of their mean losses is written to
 * *loss_out when mt_flush_grads returns (loss_out may be NULL).  Returns
 * without waiting for the GPU. */
mt_status mt_forward(mt_ctx* ctx, const int32_t* tokens, const int32_t* labels, float grad_scale,
                     float* loss_out);

/* Enqueue the backward pass of the last forward (zhichai design point 2:
 * backward streams like forward and each layer's gradients go back to host
 * memory, never accumulated on the GPU; design point 3 / lqnn 三.4: each
 * K-layer segment is recomputed from its checkpoint; lqnn 三.3: gradients land
 * in a free slab of the pool and a CPU thread adds them into the fp32 master
 * gradients): LM head gradients, then per segment (last to first) recompute
 * from the checkpoint and block backwards.  Each unit's gradient is written
 * into a free slab (bf16 or fp32, mt_config.slab_bf16), copied to pinned host
 * memory on the offload stream and added in fp32 by the worker into the host
 * grad:
 * accumulate = 0 sets grad = g, accumulate = 1 adds grad += g.  The embedding
 * gradient is scattered into the embedding grad on the host.  May block while
 * every slab is in flight. */
mt_status mt_backward(mt_ctx* ctx, int32_t accumulate);

/* mt_backward for the LAST micro-batch of an optimizer step, with the
 * optimizer overlapped: as soon as a group's (or LM-head chunk's) gradient is
 * complete in host memory the CPU worker runs AdamW on it (same arithmetic as
 * mt_adamw_step) and refreshes its pinned bf16 working copy, while the GPU
 * keeps working on the remaining layers.  A later mt_forward waits, per
 * streamed unit, for that unit's update before copying it; mt_flush_grads
 * waits for all of them.  mt_adamw_step must not be called for this step.
 * Built from the optimizer running where the state lives (m.lqnn.cn MegaTrain
 * article, 二) and the pipelined slab worker (三.3). */
mt_status mt_backward_step(mt_ctx* ctx, int32_t accumulate, const mt_adamw_hparams* hp,
                           int64_t step);

/* Wait until every gradient of every enqueued backward is in the host grads
 * (and, after mt_backward_step, every group is updated) and all streams are
 * idle; writes pending losses.  The end of lqnn 三.3's three-stage pipeline
 * (GPU backward -> gradient copy -> CPU accumulation): its last stage drained. */
mt_status mt_flush_grads(mt_ctx* ctx);

/* Wait only until the loss of every enqueued forward has been computed and
 * write the pending losses (the *loss_out pointers given to mt_forward), so
 * that the host optimizer of one step overlaps the next step's streaming
 * (lqnn 二: the optimizer runs on the CPU where its state lives; 三.3: the
 * stages are pipelined rather than serialised).
 * Unlike mt_flush_grads it does not wait for slab drains, host accumulation
 * or the overlapped optimizer, so a training loop of mt_backward_step steps
 * can read each step's loss while the host is still updating that step's
 * units (the next mt_forward waits per unit for its update).  Gradients and
 * master weights may be read only after mt_flush_grads.  MT_E_ABORTED on a
 * poisoned context; MT_E_HIP if the wait fails. */
mt_status mt_sync_loss(mt_ctx* ctx);

/* AdamW on every bound group (decoupled weight decay, bias correction, step is
 * 1-based), then refresh the pinned bf16 working copies.  Allowed only after
 * mt_flush_grads.  zhichai design point 1: the optimizer step runs on the
 * CPU, so optimizer state never crosses to the GPU; lqnn 二: the in-memory
 * fp32 master is updated and the GPU only ever sees a use-and-discard copy. */
mt_status mt_adamw_step(mt_ctx* ctx, const mt_adamw_hparams* hp, int64_t step);

/* Counters of the pipeline (bytes each way over the host link, loads, slab
 * waits, host seconds), the quantities the pages' link-bound argument is about
 * (zhichai design point 2 and 存储层次: the CPU-GPU link is the bottleneck).
 * MT_E_ARG for null pointers. */
mt_status mt_get_stats(mt_ctx* ctx, mt_stats* out);

/* Live per-kernel timing.  While enabled, the library records a pair of HIP
 * timing events around every kernel it launches (on the stream the kernel
 * runs on) and, at each mt_flush_grads, adds the elapsed times to per-kind
 * totals together with each launch's algorithmic work: flop for the bf16 MFMA
 * kernels (2*M*N*K for a GEMM; 4*d*(causal score pairs) per head forward and
 * 10*d*pairs backward for attention) and bytes each kernel must read and
 * write once for the memory-bound ones.  Enabling resets the totals. */
typedef struct mt_kernel_time {
  char name[32];
  int64_t launches;
  double ms;       /* summed device time */
  double flop;     /* summed algorithmic floating-point operations */
  double bytes;    /* summed algorithmic HBM (or host-link) bytes */
} mt_kernel_time;
mt_status mt_kernel_timing(mt_ctx* ctx, int32_t enable);
/* Kinds seen since timing was enabled, by descending device time. */
mt_status mt_get_kernel_times(mt_ctx* ctx, mt_kernel_time* out, int32_t cap, int32_t* n_out);

/* The loss of an optimizer step built by gradient accumulation
 * (travelaiplan 怎麼開始: the global batch is reached by accumulating
 * micro-batches): the mean over the step's passes of the pass losses
 * mt_forward computed (each the mean over its micro-batches), summed in
 * float64 in pass order.  The step is the one still open (passes enqueued
 * since the last mt_backward_step or mt_adamw_step), or, if none is open, the
 * last one completed.  Waits for those losses on the GPU.  MT_E_STATE if no
 * pass has run yet; MT_E_ARG for null pointers. */
mt_status mt_step_loss(mt_ctx* ctx, float* loss_out);

/* The expert selection of MoE block `layer` in the last forward pass: top_k
 * expert indices per token, [T, top_k] int32 (T = tokens of the pass), the
 * largest router logit first.  Waits for the compute stream.  MT_E_ARG if
 * `layer` is not an MoE block.  (lqnn 四: the MoE group's routing is the
 * state a caller inspects for expert load; parity checks hand it to the
 * oracle, since a selection is a discontinuous function of the logits.) */
mt_status mt_moe_routing(mt_ctx* ctx, int32_t layer, int32_t* sel_out);

/* Message of the last error of the context (a string owned by it). */
const char* mt_last_error(const mt_ctx* ctx);
/* Waits for the streams, stops the worker threads and frees what the library
 * allocated (pinned copies and slabs, events); the caller's arena and host
 * state are untouched. */
void mt_destroy(mt_ctx* ctx);

/* ---- host kernels, usable without a GPU (the same code the context runs) ---- */

/* fp32 -> bf16 round-to-nearest-even (NaN stays NaN), n elements: how the
 * pinned working copy is made from the fp32 master (lqnn 二: the GPU only sees
 * a use-and-discard copy; round-to-nearest-even is the reading taken, the
 * pages fix no rounding). */
mt_status mt_host_cast_bf16(const float* src, uint16_t* dst, int64_t n, int32_t threads);

/* One AdamW step over n elements in place (lqnn 二: the optimizer named is
 * PyTorch AdamW, run on the CPU; decoupled decay, bias correction); bf16_out
 * (may be NULL) receives RNE(master) after the update. */
mt_status mt_host_adamw(float* master, const float* grad, float* m, float* v, uint16_t* bf16_out,
                        int64_t n, const mt_adamw_hparams* hp, int64_t step, int32_t threads);

/* The optimizer thread's pass for a unit's last gradient slab of a step:
 * grad = (accumulate ? grad : 0) + slab, then one AdamW step on that gradient
 * (as mt_host_accumulate followed by mt_host_adamw, bit for bit).  slab holds
 * n bf16 values (slab_bf16 = 1) or n fp32 values (0). */
mt_status mt_host_adamw_slab(float* master, float* grad, float* m, float* v, uint16_t* bf16_out,
                             const void* slab, int32_t slab_bf16, int32_t accumulate, int64_t n,
                             const mt_adamw_hparams* hp, int64_t step, int32_t threads);

/* grad = src (accumulate = 0) or grad += src (accumulate = 1): the CPU
 * worker's accumulation of a drained slab into the fp32 master gradient
 * (lqnn 三.3). */
mt_status mt_host_accumulate(float* grad, const float* src, int64_t n, int32_t accumulate,
                             int32_t threads);

/* Host-memory bandwidth probe, the roofline of the host optimizer and
 * accumulation loops: a[i] = b[i] + s * c[i] for i < n (the STREAM triad), reps
 * passes on `threads` threads (0: the library's default count, as for its
 * own pools).  Writes the fastest pass's seconds to *best_s.  MT_E_ARG for
 * n < 1, reps < 1 or a NULL pointer.  Arrays are the caller's, 64-byte
 * aligned for full speed. */
mt_status mt_host_triad(float* a, const float* b, const float* c, float s, int64_t n, int32_t reps,
                        int32_t threads, double* best_s);

/* RoPE cos/sin tables [seq_len, head_dim/2] from float64 angles
 * pos * base^(-2i/head_dim), rounded to fp32 (the block's RoPE is a reading:
 * the pages name "Llama" layers, lqnn 四, and give no formula). */
mt_status mt_host_rope_table(int32_t seq_len, int32_t head_dim, float base, float* cos_out,
                             float* sin_out);

#ifdef __cplusplus
}
#endif
#endif /* MT_H */
