// MFMA ceiling probe: the dense bf16 MFMA rate one launch sustains with
// operands in registers and no memory traffic in the loop.  It measures the
// ceiling the GEMM and attention kernels are measured against next to the
// nominal 2.5 PFLOP/s, on the same clock as they run.
#include "common.h"

namespace mt {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Independent accumulators per wave.  Two (with the other waves of the SIMD)
// keep the pipe full; a single dependent chain issues at about 0.6 of the
// rate when it is the only wave on its SIMD.
constexpr int CHAINS = 2;

// Every operand element is 1.0, so each v_mfma_f32_32x32x16_bf16 adds 16 to
// every accumulator element: after `iters` rounds each element is 16 iters
// (exact in fp32 while 16 iters < 2^24).  out[wave] = sum over the chains of
// lane 0's first element = CHAINS * 16 * iters (mtk_mfma_peak_chains()).
__global__ __launch_bounds__(256) void mfma_peak_kernel(float* __restrict__ out, int iters) {
  const __bf16 one = (__bf16)1.0f;
  const bf16x8_t a = {one, one, one, one, one, one, one, one};
  bf16x8_t b = a;
  f32x16_t acc[CHAINS];
#pragma unroll
  for (int c = 0; c < CHAINS; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    // keep b opaque to the compiler so the chain is not folded
    asm volatile("" : "+v"(b));
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < CHAINS; ++c) s += acc[c][0];
  if ((threadIdx.x & 63) == 0) out[(int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace
}  // namespace mt

extern "C" int32_t mtk_mfma_peak_chains(void) { return mt::CHAINS; }

extern "C" mt_status mtk_mfma_peak(float* out, int32_t workgroups, int32_t iters, void* stream) {
  if (!out || workgroups < 1 || workgroups > 65535 || iters < 1 || iters > (1 << 19))
    return MT_E_ARG;
  hipLaunchKernelGGL(mt::mfma_peak_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, out,
                     iters);
  return hipGetLastError() == hipSuccess ? MT_OK : MT_E_HIP;
}
