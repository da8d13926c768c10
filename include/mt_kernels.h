/*
 * mt_kernels.h -- C ABI of the individual gfx950 kernels of one streamed
 * decoder block (the "stateless layer template": zhichai.net
 * "MegaTrain：单卡训百亿大模型的突破与实践", design point 4; blog.travelaiplan.net
 * "單卡也能練 100B+：MegaTrain 實戰", 核心功能 3 -- a custom forward and a
 * dedicated backward per layer instead of an autograd graph).
 *
 * These are the kernels mt_forward / mt_backward launch, exposed one by one so
 * that each can be checked against the CPU oracle.  All pointers are device
 * pointers (caller-owned), bf16 is passed as uint16_t bit patterns, matrices
 * are row-major with the given leading dimension in elements, and every call
 * enqueues on `stream` (a hipStream_t) and returns without waiting.  Shapes
 * are validated on the host first: MT_E_ARG for a shape the kernel does not
 * support, MT_E_HIP if the launch fails.  Activations are [T, features] with
 * T = batch * seq tokens, sequence-major.
 */
#ifndef MT_KERNELS_H
#define MT_KERNELS_H

#include "mt.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Operand layouts of C[M,N] = sum_k A(m,k) * B(n,k):
 *   NT: A(m,k) = A[m*lda + k],  B(n,k) = B[n*ldb + k]   (forward projections, y = x W^T)
 *   NN: A(m,k) = A[m*lda + k],  B(n,k) = B[k*ldb + n]   (input gradients, dx = dy W)
 *   TN: A(m,k) = A[k*lda + m],  B(n,k) = B[k*ldb + n]   (weight gradients, dW = dy^T x) */
enum { MT_GEMM_NT = 0, MT_GEMM_NN = 1, MT_GEMM_TN = 2 };

/* Epilogues (fp32 accumulation in all cases):
 *   BF16       C (bf16) = acc
 *   F32        C (fp32) = acc
 *   F32_RESID  C (fp32) = R + acc                              (residual add)
 *   F32_ACCUM  C (fp32) += acc
 *   SWIGLU     NT only.  B holds [gate; up] rows (up row f at B + ffn*ldb);
 *              N = ffn.  gu[m, f] = bf16(a), gu[m, ffn+f] = bf16(u),
 *              C (bf16) [m, f] = silu(a) * u, a = gate acc, u = up acc.
 *   SWIGLU_BWD NN only.  acc = dm[m, f], N = ffn; reads a, u from gu;
 *              C (bf16) [m, f] = dm*u*s*(1+a*(1-s)),  C[m, ffn+f] = dm*a*s,
 *              s = sigmoid(a).
 *   ROPE       NT only, the fused QKV projection.  C (bf16) = acc, except that
 *              in the columns below rope_cols every head of rope_dim columns
 *              is rotated in fp32 before its single bf16 rounding: the pair
 *              (a, b) = (c0 + i, c0 + i + rope_dim/2) becomes
 *              (a cos - b sin, b cos + a sin), cos/sin = rope_cos/rope_sin
 *              [pos * rope_dim/2 + i], pos = m mod rope_seq (rotate-half RoPE
 *              with a host-made fp32 table).  Requires rope_dim in {16, 32,
 *              64, 128} and N, rope_cols multiples of rope_dim. */
enum { MT_EPI_BF16 = 0, MT_EPI_F32 = 1, MT_EPI_F32_RESID = 2, MT_EPI_F32_ACCUM = 3,
       MT_EPI_SWIGLU = 4, MT_EPI_SWIGLU_BWD = 5, MT_EPI_ROPE = 6 };

/* Requirements (MT_E_ARG otherwise): M, N, K, lda, ldb, ldc, ldgu multiples of
 * 8, ldr a multiple of 4; C, R and gu 16-byte aligned (the epilogue moves
 * 16-byte vectors); the operands readable over their whole extent. */
typedef struct mt_gemm_args {
  int32_t layout, epilogue;
  int64_t M, N, K;          /* all multiples of 8                                 */
  const uint16_t* A; int64_t lda;
  const uint16_t* B; int64_t ldb;
  void* C; int64_t ldc;
  const float* R; int64_t ldr;
  uint16_t* gu; int64_t ldgu;
  int64_t ffn;
  const float* rope_cos;    /* ROPE only: fp32 [rope_seq, rope_dim/2] tables      */
  const float* rope_sin;
  int64_t rope_cols;        /* ROPE only: columns [0, rope_cols) are rotated      */
  int32_t rope_seq, rope_dim;
  /* Grouped products (the experts of an MoE block, one launch for all of
   * them).  groups = 0: an ordinary product.  groups = G > 0: group_off is a
   * device int32 array [G + 1] of row offsets, multiples of 256, increasing;
   * the rows of group g are [group_off[g], group_off[g+1]) of a row space of
   * at most M (NT, NN) or K (TN) rows, known only on the device.
   *   NT, NN: rows of A and C belong to groups; group g multiplies by
   *           B + g * group_stride_b (elements).  M is the row space's size.
   *   TN:     group g reduces over its own rows (the k index):
   *           C + g * group_stride_c (elements) = sum over those rows of
   *           A(row, m) B(row, n); K is the row space's size; an empty group
   *           writes zeros. */
  const int32_t* group_off;
  int32_t groups, group_reserved;
  int64_t group_stride_b, group_stride_c;
} mt_gemm_args;

mt_status mtk_gemm(const mt_gemm_args* args, void* stream);

/* RMSNorm forward: out[t,:] = bf16(x[t,:] * r_t * g), rstd[t] = r_t =
 * 1/sqrt(mean(x[t,:]^2) + eps).  x fp32 [T,h], g bf16 [h]. h multiple of 256, <= 16384. */
mt_status mtk_rmsnorm_fwd(const float* x, const uint16_t* g, uint16_t* out, float* rstd,
                          int64_t T, int32_t h, float eps, void* stream);

/* Bytes of scratch mtk_rmsnorm_bwd needs for T rows of width h. */
size_t mtk_rmsnorm_bwd_workspace(int64_t T, int32_t h);

/* RMSNorm backward with residual: xhat = x r, dx = resid + r*(dn*g - xhat*mean(dn*g*xhat)),
 * dg[h] = sum_t dn*xhat (fixed-order reduction, deterministic).  resid may be NULL
 * (treated as 0); dx_bf16 may be NULL.  dx may alias resid. */
mt_status mtk_rmsnorm_bwd(const float* dn, const float* x, const float* rstd, const uint16_t* g,
                          const float* resid, float* dx, uint16_t* dx_bf16, float* dg,
                          void* workspace, int64_t T, int32_t h, void* stream);

/* mtk_rmsnorm_bwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight training loops,
 * harnesses that forbid hipMalloc).  It allocates nothing: the column
 * partials live in a fixed device array of mtk_noalloc_scratch_bytes() bytes
 * (48 MiB) per GPU, held until the process ends.  Same arguments and results
 * as mtk_rmsnorm_bwd (bit for bit: the same kernels).  MT_E_NOMEM when
 * mtk_rmsnorm_bwd_workspace(T, h) exceeds that size (nothing is launched);
 * MT_E_ARG as mtk_rmsnorm_bwd.  Calls that overlap in time on one GPU (other
 * streams or threads) race on the shared array; calls ordered on one stream
 * do not. */
mt_status mtk_rmsnorm_bwd_noalloc(const float* dn, const float* x, const float* rstd,
                                  const uint16_t* g, const float* resid, float* dx,
                                  uint16_t* dx_bf16, float* dg, int64_t T, int32_t h,
                                  void* stream);
/* Size of that fixed per-GPU scratch array, in bytes. */
size_t mtk_noalloc_scratch_bytes(void);

/* RoPE in place on the q and k columns of qkv [T, (n_heads + 2 n_kv_heads) * d]:
 * pairs (i, i+d/2) of every head rotated by +angle (inverse = 0) or -angle,
 * angle table cos/sin fp32 [seq_len, d/2], position = t mod seq_len. */
mt_status mtk_rope(uint16_t* qkv, int64_t T, int32_t seq_len, int32_t n_heads,
                   int32_t n_kv_heads, int32_t head_dim, const float* cos_t, const float* sin_t,
                   int32_t inverse, void* stream);

/* Causal grouped-query flash attention forward.  q, k, v are column blocks of
 * qkv [T, (nq + 2 nkv) d]; o bf16 [T, nq d]; lse fp32 [nq, T] (natural-log
 * log-sum-exp of the scaled scores).  seq_len multiple of 128, d 64 or 128,
 * (seq_len / 128) * nq * batch <= 2^24; qkv and o 16-byte aligned (MT_E_ARG
 * otherwise). */
mt_status mtk_attention_fwd(const uint16_t* qkv, uint16_t* o, float* lse, int32_t batch,
                            int32_t seq_len, int32_t n_heads, int32_t n_kv_heads,
                            int32_t head_dim, void* stream);

/* Bytes of device scratch mtk_attention_bwd needs for these sizes (0 for sizes
 * it rejects): fp32 [nq, T] row statistics, plus, when n_kv_heads < n_heads,
 * fp32 [nq, T, d] per-query-head shares of dK and dV. */
size_t mtk_attention_bwd_workspace(int32_t batch, int32_t seq_len, int32_t n_heads,
                                   int32_t n_kv_heads, int32_t head_dim);

/* Flash attention backward.  dout bf16 [T, nq d]; writes dq, dk, dv into the
 * matching column blocks of dqkv (same layout as qkv).  workspace: device
 * scratch of mtk_attention_bwd_workspace(...) bytes, owned by the caller, no
 * contents kept between calls.  Deterministic (no float atomics; dk/dv summed
 * over the query heads of a group in fixed order).  MT_E_ARG for null
 * pointers, sizes attention_fwd rejects, or qkv, o, dout, dqkv not 16-byte
 * aligned. */
mt_status mtk_attention_bwd(const uint16_t* qkv, const uint16_t* o, const uint16_t* dout,
                            const float* lse, void* workspace, uint16_t* dqkv, int32_t batch,
                            int32_t seq_len, int32_t n_heads, int32_t n_kv_heads,
                            int32_t head_dim, void* stream);

/* mtk_attention_bwd for q and k that were rotated by RoPE after the
 * projection (the MT_EPI_ROPE product): qkv holds the rotated q and k, and dq
 * and dk are written as gradients with respect to the pre-rotation q and k,
 * i.e. rotated back by -angle in fp32 before their single bf16 rounding.
 * cos_t/sin_t: the fp32 [seq_len, head_dim/2] tables the forward used,
 * 16-byte aligned.  The backward of RoPE is the transpose of a rotation (the
 * oracle's RoPE reading: rotate-half pairs, angles from a float64 table). */
mt_status mtk_attention_bwd_rope(const uint16_t* qkv, const uint16_t* o, const uint16_t* dout,
                                 const float* lse, void* workspace, uint16_t* dqkv, int32_t batch,
                                 int32_t seq_len, int32_t n_heads, int32_t n_kv_heads,
                                 int32_t head_dim, const float* cos_t, const float* sin_t,
                                 void* stream);

/* Cross-entropy over fp32 logits [T, V] (row stride ld): loss_rows[t] =
 * lse_t - logits[t, label_t] (0 for label < 0); dlogits bf16 [T, V] (row stride
 * ld_d) = (softmax - onehot) * grad_scale / n_valid (0 rows for ignored labels);
 * *loss_out (device fp32) = sum(loss_rows) / n_valid, fixed-order sum.
 * labels: device int32 [T]; n_valid: labelled rows (host value). */
mt_status mtk_cross_entropy(const float* logits, int64_t ld, const int32_t* labels, int64_t T,
                            int32_t V, float grad_scale, int64_t n_valid, uint16_t* dlogits,
                            int64_t ld_d, float* loss_rows, float* loss_out, void* stream);

/* MFMA ceiling probe (measurement only, not part of a training step):
 * `workgroups` workgroups of 4 waves, each wave running C =
 * mtk_mfma_peak_chains() independent chains of `iters`
 * v_mfma_f32_32x32x16_bf16 on register operands of 1.0.  Writes
 * out[4 * workgroups] (device fp32), every element C * 16 * iters, so the
 * caller can check the work was done.  Algorithmic work: workgroups * 4 * C *
 * iters * 32768 flop.  MT_E_ARG for workgroups outside 1..65535 or iters
 * outside 1..2^19. */
mt_status mtk_mfma_peak(float* out, int32_t workgroups, int32_t iters, void* stream);
int32_t mtk_mfma_peak_chains(void);

/* Copy `bytes` (multiple of 16, both pointers 16-byte aligned) with a copy
 * kernel of `workgroups` 256-thread workgroups instead of the copy engine.
 * Either side may be pinned host memory (hipHostMalloc), which the kernel
 * reads or writes across the host link.  Used to drain gradient slabs to the
 * host while the copy engine streams the next layer in (the pages' three
 * overlapped stages, m.lqnn.cn MegaTrain article 三.2-三.3). */
mt_status mtk_copy(void* dst, const void* src, size_t bytes, int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MT_KERNELS_H */
