// C-ABI wrappers of the individual block kernels: validate on the host, then
// launch on the caller's stream.
#include "common.h"

using namespace mt;

static mt_status hip_status(hipError_t e) { return e == hipSuccess ? MT_OK : MT_E_HIP; }

extern "C" mt_status mtk_gemm(const mt_gemm_args* a, void* stream) {
  if (!a || !gemm_shape_ok(*a, nullptr)) return MT_E_ARG;
  return hip_status(launch_gemm(*a, (hipStream_t)stream));
}

extern "C" mt_status mtk_rmsnorm_fwd(const float* x, const uint16_t* g, uint16_t* out,
                                     float* rstd, int64_t T, int32_t h, float eps, void* stream) {
  if (!x || !g || !out || !rstd || T < 1 || h < 4 || h % 4 || h > 16384 || !(eps >= 0.0f))
    return MT_E_ARG;
  return hip_status(launch_rmsnorm_fwd(x, g, out, rstd, T, h, eps, (hipStream_t)stream));
}

extern "C" size_t mtk_rmsnorm_bwd_workspace(int64_t T, int32_t h) {
  if (T < 1 || h < 4) return 0;
  return rmsnorm_bwd_partial_bytes(T, h);
}

extern "C" mt_status mtk_rmsnorm_bwd(const float* dn, const float* x, const float* rstd,
                                     const uint16_t* g, const float* resid, float* dx,
                                     uint16_t* dx_bf16, float* dg, void* workspace, int64_t T,
                                     int32_t h, void* stream) {
  if (!dn || !x || !rstd || !g || !dx || !dg || !workspace || T < 1 || h < 4 || h % 4 ||
      h > 16384)
    return MT_E_ARG;
  return hip_status(launch_rmsnorm_bwd(dn, x, rstd, g, resid, dx, dx_bf16, dg, nullptr,
                                       static_cast<float*>(workspace), T, h,
                                       (hipStream_t)stream));
}

extern "C" mt_status mtk_rope(uint16_t* qkv, int64_t T, int32_t seq_len, int32_t n_heads,
                              int32_t n_kv_heads, int32_t head_dim, const float* cos_t,
                              const float* sin_t, int32_t inverse, void* stream) {
  if (!qkv || !cos_t || !sin_t || T < 1 || seq_len < 1 || T % seq_len || n_heads < 1 ||
      n_kv_heads < 1 || head_dim < 2 || head_dim % 2)
    return MT_E_ARG;
  return hip_status(launch_rope(qkv, T, seq_len, n_heads, n_kv_heads, head_dim, cos_t, sin_t,
                                inverse, (hipStream_t)stream));
}

// The kernels launch (seq / 128) x heads x batch workgroups in one grid
// dimension (at most 2^24 of them).
static bool attn_ok(int32_t batch, int32_t seq, int32_t nq, int32_t nkv, int32_t d) {
  return batch >= 1 && seq >= 128 && seq % 128 == 0 && nq >= 1 && nkv >= 1 && nq % nkv == 0 &&
         (d == 64 || d == 128) && nq <= 65535 && batch <= 65535 &&
         (int64_t)(seq / 128) * nq * batch <= (int64_t)1 << 24;
}
// Rows are moved in 16-byte vectors (and K/V tiles by 16-byte direct loads).
static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

extern "C" mt_status mtk_attention_fwd(const uint16_t* qkv, uint16_t* o, float* lse,
                                       int32_t batch, int32_t seq_len, int32_t n_heads,
                                       int32_t n_kv_heads, int32_t head_dim, void* stream) {
  if (!qkv || !o || !lse || !attn_ok(batch, seq_len, n_heads, n_kv_heads, head_dim) ||
      !aligned16(qkv) || !aligned16(o))
    return MT_E_ARG;
  return hip_status(launch_attn_fwd(qkv, o, lse, batch, seq_len, n_heads, n_kv_heads, head_dim,
                                    (hipStream_t)stream));
}

extern "C" size_t mtk_attention_bwd_workspace(int32_t batch, int32_t seq_len, int32_t n_heads,
                                              int32_t n_kv_heads, int32_t head_dim) {
  if (!attn_ok(batch, seq_len, n_heads, n_kv_heads, head_dim)) return 0;
  return attn_bwd_workspace_bytes(batch, seq_len, n_heads, n_kv_heads, head_dim);
}

extern "C" mt_status mtk_attention_bwd(const uint16_t* qkv, const uint16_t* o,
                                       const uint16_t* dout, const float* lse, void* workspace,
                                       uint16_t* dqkv, int32_t batch, int32_t seq_len,
                                       int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                       void* stream) {
  if (!qkv || !o || !dout || !lse || !workspace || !dqkv ||
      !attn_ok(batch, seq_len, n_heads, n_kv_heads, head_dim) || !aligned16(qkv) ||
      !aligned16(o) || !aligned16(dout) || !aligned16(dqkv))
    return MT_E_ARG;
  return hip_status(launch_attn_bwd(qkv, o, dout, lse, workspace, dqkv, batch, seq_len, n_heads,
                                    n_kv_heads, head_dim, nullptr, nullptr, (hipStream_t)stream));
}

extern "C" mt_status mtk_attention_bwd_rope(const uint16_t* qkv, const uint16_t* o,
                                            const uint16_t* dout, const float* lse,
                                            void* workspace, uint16_t* dqkv, int32_t batch,
                                            int32_t seq_len, int32_t n_heads, int32_t n_kv_heads,
                                            int32_t head_dim, const float* cos_t,
                                            const float* sin_t, void* stream) {
  if (!qkv || !o || !dout || !lse || !workspace || !dqkv || !cos_t || !sin_t ||
      (((uintptr_t)cos_t | (uintptr_t)sin_t) & 15) ||
      !attn_ok(batch, seq_len, n_heads, n_kv_heads, head_dim) || !aligned16(qkv) ||
      !aligned16(o) || !aligned16(dout) || !aligned16(dqkv))
    return MT_E_ARG;
  return hip_status(launch_attn_bwd(qkv, o, dout, lse, workspace, dqkv, batch, seq_len, n_heads,
                                    n_kv_heads, head_dim, cos_t, sin_t, (hipStream_t)stream));
}

extern "C" mt_status mtk_cross_entropy(const float* logits, int64_t ld, const int32_t* labels,
                                       int64_t T, int32_t V, float grad_scale, int64_t n_valid,
                                       uint16_t* dlogits, int64_t ld_d, float* loss_rows,
                                       float* loss_out, void* stream) {
  if (!logits || !labels || !dlogits || !loss_rows || !loss_out || T < 1 || V < 4 || V % 4 ||
      ld < V || ld % 4 || ld_d < V || ld_d % 4 || n_valid < 0 || n_valid > T)
    return MT_E_ARG;
  return hip_status(launch_cross_entropy(logits, ld, labels, T, V, grad_scale, n_valid, dlogits,
                                         ld_d, loss_rows, loss_out, (hipStream_t)stream));
}

extern "C" mt_status mtk_copy(void* dst, const void* src, size_t bytes, int32_t workgroups,
                              void* stream) {
  if (!dst || !src || bytes % 16 || workgroups < 1 || workgroups > 65535 ||
      ((uintptr_t)dst % 16) || ((uintptr_t)src % 16))
    return MT_E_ARG;
  return hip_status(launch_copy(dst, src, bytes, workgroups, (hipStream_t)stream));
}
