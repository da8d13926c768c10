// Routing kernels of the mixture-of-experts block, the second parameter-
// structure group (m.lqnn.cn MegaTrain article, 四: layers grouped by structure,
// MoE layers forming their own group on the same streaming machinery).
//
// The expert products themselves are grouped bf16 MFMA GEMMs (gemm.hip with
// mt_gemm_args.groups): the token rows routed to each expert are laid out
// expert-major, each expert's block padded with zero rows to a multiple of
// 256, so one launch covers every expert and a 256-row tile never straddles
// two experts.  The row offsets exist only on the device, so no step waits
// for the host.  Everything here is deterministic: rows are ordered by token
// within an expert, and every sum runs in a fixed order.
#include "common.h"
#include "moe.h"

namespace mt {
namespace {

constexpr int NT = 256;

__device__ inline float block_sum256(float v, float* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

// Top-k of the router logits (ties to the lower expert index) and the gates,
// a softmax over the selected logits.  One thread per token.
__global__ __launch_bounds__(NT) void moe_route_kernel(const float* __restrict__ logits,
                                                       int64_t ld, int64_t T, int E, int k,
                                                       int32_t* __restrict__ sel,
                                                       float* __restrict__ gates) {
  const int64_t t = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (t >= T) return;
  const float* r = logits + t * ld;
  uint64_t taken = 0;
  float sl[8];
  for (int j = 0; j < k; ++j) {
    int bi = -1;
    float best = 0.0f;
    for (int e = 0; e < E; ++e) {
      if ((taken >> e) & 1) continue;
      const float v = r[e];
      if (bi < 0 || v > best) {
        best = v;
        bi = e;
      }
    }
    taken |= 1ull << bi;
    sel[t * k + j] = bi;
    sl[j] = best;
  }
  float z = 0.0f;
  for (int j = 0; j < k; ++j) z += expf(sl[j] - sl[0]);
  for (int j = 0; j < k; ++j) gates[t * k + j] = expf(sl[j] - sl[0]) / z;
}

// Expert-major row plan, one workgroup: off[e] (padded to 256), the row of
// each (token, slot) pair and the token of each row (-1 for padding rows).
// Rows of an expert follow token order: for each chunk of 256 tokens a
// workgroup-wide prefix count per expert gives each token its rank.
__global__ __launch_bounds__(NT) void moe_plan_kernel(const int32_t* __restrict__ sel, int64_t T,
                                                      int E, int k, int32_t* __restrict__ off,
                                                      int32_t* __restrict__ pos,
                                                      int32_t* __restrict__ rowtok) {
  __shared__ int cnt[64], run[64], wtot[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid < 64) cnt[tid] = 0;
  __syncthreads();
  for (int64_t i = tid; i < T * k; i += NT) atomicAdd(&cnt[sel[i]], 1);  // integer counts
  __syncthreads();
  if (tid == 0) {
    int b = 0;
    for (int e = 0; e < E; ++e) {
      off[e] = b;
      run[e] = b;
      b += (cnt[e] + 255) / 256 * 256;
    }
    off[E] = b;
    cnt[0] = b;  // total rows, read below
  }
  __syncthreads();
  const int total = cnt[0];
  for (int r = tid; r < total; r += NT) rowtok[r] = -1;
  __syncthreads();
  for (int64_t c0 = 0; c0 < T; c0 += NT) {
    const int64_t t = c0 + tid;
    int mine[8];
    for (int j = 0; j < k; ++j) mine[j] = t < T ? sel[t * k + j] : -1;
    for (int e = 0; e < E; ++e) {
      int slot = -1;
      for (int j = 0; j < k; ++j)
        if (mine[j] == e) slot = j;
      const unsigned long long b = __ballot(slot >= 0);
      const int before = __popcll(b & ((1ull << lane) - 1ull));
      if (lane == 0) wtot[w] = __popcll(b);
      __syncthreads();
      int wbase = 0;
      for (int v = 0; v < w; ++v) wbase += wtot[v];
      if (slot >= 0) {
        const int row = run[e] + wbase + before;
        pos[t * k + slot] = row;
        rowtok[row] = (int32_t)t;
      }
      __syncthreads();
      if (tid == 0) run[e] += wtot[0] + wtot[1] + wtot[2] + wtot[3];
      __syncthreads();
    }
  }
}

// X[row] = n2[token of row] (bf16), zero rows for padding; one workgroup per
// row, rows past the last expert's block untouched.
__global__ __launch_bounds__(NT) void moe_gather_kernel(const uint16_t* __restrict__ n2, int h,
                                                        const int32_t* __restrict__ rowtok,
                                                        const int32_t* __restrict__ off, int E,
                                                        uint16_t* __restrict__ X) {
  const int64_t row = blockIdx.x;
  if (row >= off[E]) return;
  const int64_t t = rowtok[row];
  uint4* dst = reinterpret_cast<uint4*>(X + row * h);
  const uint4* src = reinterpret_cast<const uint4*>(n2 + t * h);
  for (int c = threadIdx.x; c < h / 8; c += NT) dst[c] = t >= 0 ? src[c] : make_uint4(0, 0, 0, 0);
}

// y[t] = h1[t] + sum_j g_j Yo[pos_j] (fp32, slots in order); one workgroup
// per token.
__global__ __launch_bounds__(NT) void moe_combine_kernel(const float* __restrict__ h1,
                                                         const float* __restrict__ Yo,
                                                         const int32_t* __restrict__ pos,
                                                         const float* __restrict__ gates, int k,
                                                         int h, float* __restrict__ y) {
  const int64_t t = blockIdx.x;
  for (int c = threadIdx.x; c < h / 4; c += NT) {
    float4 a = reinterpret_cast<const float4*>(h1 + t * h)[c];
    for (int j = 0; j < k; ++j) {
      const float g = gates[t * k + j];
      const float4 o = reinterpret_cast<const float4*>(Yo + (int64_t)pos[t * k + j] * h)[c];
      a.x += g * o.x;
      a.y += g * o.y;
      a.z += g * o.z;
      a.w += g * o.w;
    }
    reinterpret_cast<float4*>(y + t * h)[c] = a;
  }
}

// Backward of the combine and the gates, one workgroup per token: each
// expert row receives g_j dy (bf16, its output gradient); dg_j = <dy, Yo>;
// the router logits' gradient g_j (dg_j - sum_i g_i dg_i) at the selected
// experts, 0 elsewhere (bf16 [T, ldl]).
__global__ __launch_bounds__(NT) void moe_bwd_gates_kernel(
    const float* __restrict__ dy, const float* __restrict__ Yo, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ sel, const float* __restrict__ gates, int k, int E, int h,
    uint16_t* __restrict__ dout, uint16_t* __restrict__ dlog, int64_t ldl) {
  __shared__ float sh[4];
  __shared__ float dg[8];
  const int64_t t = blockIdx.x;
  const float* d = dy + t * h;
  for (int j = 0; j < k; ++j) {
    const int64_t r = pos[t * k + j];
    const float g = gates[t * k + j];
    float acc = 0.0f;
    for (int c = threadIdx.x; c < h / 4; c += NT) {
      const float4 v = reinterpret_cast<const float4*>(d)[c];
      const float4 o = reinterpret_cast<const float4*>(Yo + r * h)[c];
      acc += v.x * o.x + v.y * o.y + v.z * o.z + v.w * o.w;
      reinterpret_cast<uint2*>(dout + r * h)[c] =
          make_uint2(pack_bf2(g * v.x, g * v.y), pack_bf2(g * v.z, g * v.w));
    }
    acc = block_sum256(acc, sh);
    if (threadIdx.x == 0) dg[j] = acc;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.0f;
    for (int j = 0; j < k; ++j) s += gates[t * k + j] * dg[j];
    for (int e = 0; e < (int)ldl; ++e) dlog[t * ldl + e] = 0;
    for (int j = 0; j < k; ++j)
      dlog[t * ldl + sel[t * k + j]] = f2bf(gates[t * k + j] * (dg[j] - s));
  }
}

// Zero the padding rows of an expert-major bf16 matrix [rows, h].
__global__ __launch_bounds__(NT) void moe_zero_pad_kernel(const int32_t* __restrict__ rowtok,
                                                          const int32_t* __restrict__ off, int E,
                                                          int h, uint16_t* __restrict__ X) {
  const int64_t row = blockIdx.x;
  if (row >= off[E] || rowtok[row] >= 0) return;
  uint4* dst = reinterpret_cast<uint4*>(X + row * h);
  for (int c = threadIdx.x; c < h / 8; c += NT) dst[c] = make_uint4(0, 0, 0, 0);
}

// dn[t] = sum_j dX[pos_j] (fp32, slots in order); one workgroup per token.
__global__ __launch_bounds__(NT) void moe_bwd_combine_kernel(const float* __restrict__ dX,
                                                             const int32_t* __restrict__ pos, int k,
                                                             int h, float* __restrict__ dn) {
  const int64_t t = blockIdx.x;
  for (int c = threadIdx.x; c < h / 4; c += NT) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const float4 o = reinterpret_cast<const float4*>(dX + (int64_t)pos[t * k + j] * h)[c];
      a.x += o.x;
      a.y += o.y;
      a.z += o.z;
      a.w += o.w;
    }
    reinterpret_cast<float4*>(dn + t * h)[c] = a;
  }
}

}  // namespace

hipError_t launch_moe_route(const float* logits, int64_t ld, int64_t T, int E, int k, int32_t* sel,
                            float* gates, hipStream_t s) {
  hipLaunchKernelGGL(moe_route_kernel, dim3((unsigned)((T + NT - 1) / NT)), dim3(NT), 0, s, logits,
                     ld, T, E, k, sel, gates);
  return hipGetLastError();
}

hipError_t launch_moe_plan(const int32_t* sel, int64_t T, int E, int k, int32_t* off, int32_t* pos,
                           int32_t* rowtok, hipStream_t s) {
  hipLaunchKernelGGL(moe_plan_kernel, dim3(1), dim3(NT), 0, s, sel, T, E, k, off, pos, rowtok);
  return hipGetLastError();
}

hipError_t launch_moe_gather(const uint16_t* n2, int h, const int32_t* rowtok, const int32_t* off,
                             int E, int64_t rows, uint16_t* X, hipStream_t s) {
  hipLaunchKernelGGL(moe_gather_kernel, dim3((unsigned)rows), dim3(NT), 0, s, n2, h, rowtok, off, E,
                     X);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const float* h1, const float* Yo, const int32_t* pos,
                              const float* gates, int k, int h, int64_t T, float* y,
                              hipStream_t s) {
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)T), dim3(NT), 0, s, h1, Yo, pos, gates, k,
                     h, y);
  return hipGetLastError();
}

hipError_t launch_moe_bwd_gates(const float* dy, const float* Yo, const int32_t* pos,
                                const int32_t* sel, const float* gates, int k, int E, int h,
                                int64_t T, uint16_t* dout, uint16_t* dlog, int64_t ldl,
                                hipStream_t s) {
  hipLaunchKernelGGL(moe_bwd_gates_kernel, dim3((unsigned)T), dim3(NT), 0, s, dy, Yo, pos, sel,
                     gates, k, E, h, dout, dlog, ldl);
  return hipGetLastError();
}

hipError_t launch_moe_zero_pad(const int32_t* rowtok, const int32_t* off, int E, int h,
                               int64_t rows, uint16_t* X, hipStream_t s) {
  hipLaunchKernelGGL(moe_zero_pad_kernel, dim3((unsigned)rows), dim3(NT), 0, s, rowtok, off, E, h,
                     X);
  return hipGetLastError();
}

hipError_t launch_moe_bwd_combine(const float* dX, const int32_t* pos, int k, int h, int64_t T,
                                  float* dn, hipStream_t s) {
  hipLaunchKernelGGL(moe_bwd_combine_kernel, dim3((unsigned)T), dim3(NT), 0, s, dX, pos, k, h, dn);
  return hipGetLastError();
}

}  // namespace mt
