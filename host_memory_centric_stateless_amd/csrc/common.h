// Internal helpers shared by the libmt sources (device and host).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mt.h"
#include "../../include/mt_kernels.h"

namespace mt {

// ---------------------------------------------------------------- bf16 bits
// Round-to-nearest-even fp32 -> bf16; NaN stays a (quiet) NaN.  On the GPU
// this is gfx950's conversion instruction (v_cvt_pk_bf16_f32, two values per
// instruction), which rounds the same way; the host spells the rounding out.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));

__host__ __device__ inline uint16_t f2bf(float f) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_bit_cast(uint16_t, (__bf16)f);
#else
  uint32_t u;
  __builtin_memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
#endif
}

__host__ __device__ inline float bf2f(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
#if defined(__HIP_DEVICE_COMPILE__)
  return __uint_as_float(u);
#else
  float f;
  __builtin_memcpy(&f, &u, 4);
  return f;
#endif
}

__host__ __device__ inline uint32_t pack_bf2(float lo, float hi) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_hw){lo, hi}, bf16x2_hw));
#else
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
#endif
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; shapes are validated by the
// C-ABI wrappers before these are called.
hipError_t launch_gemm(const mt_gemm_args& a, hipStream_t s);
hipError_t launch_rmsnorm_fwd(const float* x, const uint16_t* g, uint16_t* out, float* rstd,
                              int64_t T, int h, float eps, hipStream_t s);
// dg receives the gain gradient in fp32, or in bf16 via dg_bf16 when dg is null.
hipError_t launch_rmsnorm_bwd(const float* dn, const float* x, const float* rstd,
                              const uint16_t* g, const float* resid, float* dx,
                              uint16_t* dx_bf16, float* dg, uint16_t* dg_bf16, float* partial,
                              int64_t T, int h, hipStream_t s);
size_t rmsnorm_bwd_partial_bytes(int64_t T, int h);
hipError_t launch_rope(uint16_t* qkv, int64_t T, int seq, int nq, int nkv, int d,
                       const float* cos_t, const float* sin_t, int inverse, hipStream_t s);
hipError_t launch_attn_fwd(const uint16_t* qkv, uint16_t* o, float* lse, int batch, int seq,
                           int nq, int nkv, int d, hipStream_t s);
size_t attn_bwd_workspace_bytes(int batch, int seq, int nq, int nkv, int d);
// cos_t/sin_t (both or neither): RoPE tables [seq, d/2]; dq and dk are then
// rotated back from the rotated q/k to the pre-rotation ones before rounding.
hipError_t launch_attn_bwd(const uint16_t* qkv, const uint16_t* o, const uint16_t* dout,
                           const float* lse, void* workspace, uint16_t* dqkv, int batch, int seq,
                           int nq, int nkv, int d, const float* cos_t, const float* sin_t,
                           hipStream_t s);
// out[0] = mean of v[0..n) (one workgroup, fixed order).
hipError_t launch_mean(const float* v, int64_t n, float* out, hipStream_t s);
hipError_t launch_cross_entropy(const float* logits, int64_t ld, const int32_t* labels, int64_t T,
                                int V, float grad_scale, int64_t n_valid, uint16_t* dlogits,
                                int64_t ld_d, float* loss_rows, float* loss_out, hipStream_t s);

// Cross-entropy in token x vocabulary chunks (the LM head never holds a whole
// [T, V] logits matrix).  CeCoef: the dlogits coefficient of each micro-batch
// of the pass (grad_scale / labelled tokens), rows t of micro-batch t / T_mb.
struct CeCoef {
  float c[32];
  int64_t T_mb;
};
// Merge the softmax statistics of `rows` rows of one logits chunk (columns
// r0 .. r0+nr of the vocabulary, row stride ld) into m_run / s_run (first:
// overwrite) and keep the label's logit when it is in the chunk.  Pointers
// labels, m_run, s_run, lab_logit are offset to the chunk's first row.
hipError_t launch_ce_stats(const float* logits, int64_t ld, int64_t rows, int nr, int64_t r0,
                           const int32_t* labels, int first, float* m_run, float* s_run,
                           float* lab_logit, hipStream_t s);
// lse = m + log(s) and loss_rows = lse - label logit (0 where label < 0) for T rows.
hipError_t launch_ce_finish(const float* m_run, const float* s_run, const float* lab_logit,
                            const int32_t* labels, int64_t T, float* lse, float* loss_rows,
                            hipStream_t s);
// dlogits (bf16, row stride ldd) of `rows` rows of one logits chunk; labels
// and lse offset to the chunk's first row, which is row t0 of the pass.
hipError_t launch_ce_grad(const float* logits, int64_t ld, int64_t rows, int nr, int64_t r0,
                          const int32_t* labels, const float* lse, int64_t t0, const CeCoef& cf,
                          uint16_t* dl, int64_t ldd, hipStream_t s);
// fp32 -> bf16 round-to-nearest-even, n a multiple of 4.
hipError_t launch_cast_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s);
// out[0] = inv_n * sum of rows[0..n) (one workgroup, fixed order).
hipError_t launch_loss_mean(const float* rows, int64_t n, float inv_n, float* out, hipStream_t s);

// 16-byte-vector copy by `wgs` workgroups (bytes multiple of 16; either side
// may be host-mapped pinned memory).
hipError_t launch_copy(void* dst, const void* src, size_t bytes, int wgs, hipStream_t s);

// Shape checks shared by the C-ABI wrappers and the engine.
bool gemm_shape_ok(const mt_gemm_args& a, const char** why);

}  // namespace mt
