// HBM-bound kernels of the streamed decoder block: RMSNorm forward/backward,
// RoPE, and the LM-head cross-entropy with its gradient.
//
// Each reads and writes its operands once; statistics and reductions are in
// fp32 and every reduction runs in a fixed order, so recomputed activations
// are bit-identical to the forward's (the segment recompute of m.lqnn.cn
// MegaTrain article, 三.4, relies on that) and the results do not depend on
// timing.
#include "common.h"

namespace mt {
namespace {

constexpr int NT = 256;

__device__ inline float block_sum(float v, float* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

// ------------------------------------------------------------- RMSNorm fwd
// One row per workgroup; h/4 float4 vectors spread over 256 threads.
// MAXV: float4 vectors per thread (h <= 1024 * MAXV).
template <int MAXV>
__global__ __launch_bounds__(NT) void rmsnorm_fwd_kernel(const float* __restrict__ x,
                                                         const uint16_t* __restrict__ g,
                                                         uint16_t* __restrict__ out,
                                                         float* __restrict__ rstd, int h,
                                                         float eps) {
  __shared__ float sh[4];
  const int64_t row = blockIdx.x;
  const float* xr = x + row * h;
  const int nv = h / 4;
  float4 v[MAXV];
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = threadIdx.x + i * NT;
    if (c < nv) {
      v[i] = *reinterpret_cast<const float4*>(xr + c * 4);
      ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    }
  }
  ss = block_sum(ss, sh);
  const float r = 1.0f / sqrtf(ss / (float)h + eps);
  uint16_t* orow = out + row * h;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = threadIdx.x + i * NT;
    if (c < nv) {
      const uint2 gg = *reinterpret_cast<const uint2*>(g + c * 4);
      const float g0 = bf2f(gg.x & 0xffff), g1 = bf2f(gg.x >> 16);
      const float g2 = bf2f(gg.y & 0xffff), g3 = bf2f(gg.y >> 16);
      uint2 o;
      o.x = pack_bf2(v[i].x * r * g0, v[i].y * r * g1);
      o.y = pack_bf2(v[i].z * r * g2, v[i].w * r * g3);
      *reinterpret_cast<uint2*>(orow + c * 4) = o;
    }
  }
  if (threadIdx.x == 0) rstd[row] = r;
}

// ------------------------------------------------------------- RMSNorm bwd
// Workgroup b handles rows [b*R, (b+1)*R) in order and keeps per-column
// partial sums of dn*xhat in registers; a second kernel adds the partials in
// a fixed order.
template <int MAXV>
__global__ __launch_bounds__(NT) void rmsnorm_bwd_kernel(
    const float* __restrict__ dn, const float* __restrict__ x, const float* __restrict__ rstd,
    const uint16_t* __restrict__ g, const float* resid, float* dx, uint16_t* __restrict__ dxb,
    float* __restrict__ partial, int64_t T, int h, int64_t rows_per_block) {
  __shared__ float sh[4];
  const int nv = h / 4;
  float gv[MAXV][4];
  float acc[MAXV][4];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = threadIdx.x + i * NT;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[i][e] = 0.0f;
    if (c < nv) {
      const uint2 gg = *reinterpret_cast<const uint2*>(g + c * 4);
      gv[i][0] = bf2f(gg.x & 0xffff);
      gv[i][1] = bf2f(gg.x >> 16);
      gv[i][2] = bf2f(gg.y & 0xffff);
      gv[i][3] = bf2f(gg.y >> 16);
    }
  }
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  const int64_t r1 = r0 + rows_per_block < T ? r0 + rows_per_block : T;
  for (int64_t row = r0; row < r1; ++row) {
    const float r = rstd[row];
    float xh[MAXV][4], dh[MAXV][4];
    float dot = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int c = threadIdx.x + i * NT;
      if (c < nv) {
        const float4 xv = *reinterpret_cast<const float4*>(x + row * h + c * 4);
        const float4 dv = *reinterpret_cast<const float4*>(dn + row * h + c * 4);
        const float xs[4] = {xv.x, xv.y, xv.z, xv.w};
        const float ds[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xh[i][e] = xs[e] * r;
          dh[i][e] = ds[e] * gv[i][e];
          dot += dh[i][e] * xh[i][e];
          acc[i][e] += ds[e] * xh[i][e];
        }
      }
    }
    dot = block_sum(dot, sh) / (float)h;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int c = threadIdx.x + i * NT;
      if (c < nv) {
        float o[4];
        float4 rv = resid ? *reinterpret_cast<const float4*>(resid + row * h + c * 4)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        const float rs[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = rs[e] + r * (dh[i][e] - xh[i][e] * dot);
        *reinterpret_cast<float4*>(dx + row * h + c * 4) = make_float4(o[0], o[1], o[2], o[3]);
        if (dxb) {
          uint2 ob;
          ob.x = pack_bf2(o[0], o[1]);
          ob.y = pack_bf2(o[2], o[3]);
          *reinterpret_cast<uint2*>(dxb + row * h + c * 4) = ob;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = threadIdx.x + i * NT;
    if (c < nv)
      *reinterpret_cast<float4*>(partial + (int64_t)blockIdx.x * h + c * 4) =
          make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
  }
}

// Column sums of the [nblk][h] partials: a workgroup owns 64 columns; wave w
// adds the block rows b = w (mod 4) in four interleaved chains, and the four
// waves' sums are then added in wave order (a fixed order for any launch).
__global__ __launch_bounds__(NT) void colsum_kernel(const float* __restrict__ partial,
                                                    float* __restrict__ out,
                                                    uint16_t* __restrict__ out16, int nblk, int h) {
  __shared__ float sh[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (c < h) {
    int b = w;
    for (; b + 12 < nblk; b += 16)
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] += partial[(int64_t)(b + 4 * u) * h + c];
#pragma unroll
    for (int u = 0; u < 3; ++u)
      if (b + 4 * u < nblk) a[u] += partial[(int64_t)(b + 4 * u) * h + c];
  }
  sh[w][lane] = (a[0] + a[1]) + (a[2] + a[3]);
  __syncthreads();
  if (w != 0 || c >= h) return;
  const float s = ((sh[0][lane] + sh[1][lane]) + sh[2][lane]) + sh[3][lane];
  if (out16)
    out16[c] = f2bf(s);
  else
    out[c] = s;
}

// Four rows per workgroup (up to 2048 workgroups), so that several
// workgroups share each CU and their row loads overlap.
int64_t bwd_blocks(int64_t T) {
  int64_t nb = (T + 3) / 4;
  return nb < 2048 ? nb : 2048;
}

// -------------------------------------------------------------------- RoPE
// One thread per (token, head, pair i); pairs (i, i + d/2).
__global__ void rope_kernel(uint16_t* __restrict__ qkv, int64_t T, int seq, int nheads_rot,
                            int ld, int d, const float* __restrict__ cos_t,
                            const float* __restrict__ sin_t, float sign) {
  const int half = d / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = T * nheads_rot * half;
  if (idx >= total) return;
  const int i = (int)(idx % half);
  const int64_t th = idx / half;
  const int hd = (int)(th % nheads_rot);
  const int64_t t = th / nheads_rot;
  const int pos = (int)(t % seq);
  uint16_t* p = qkv + t * ld + (int64_t)hd * d;
  const float c = cos_t[(int64_t)pos * half + i];
  const float s = sign * sin_t[(int64_t)pos * half + i];
  const float a = bf2f(p[i]), b = bf2f(p[i + half]);
  p[i] = f2bf(a * c - b * s);
  p[i + half] = f2bf(b * c + a * s);
}

// The same rotation, eight pairs (i0..i0+7 with their partners i0+d/2..) per
// thread with 16-byte accesses, when d is a multiple of 16 and the rows and
// tables are 16-byte aligned: one index decomposition per eight pairs instead
// of per pair.
__global__ void rope8_kernel(uint16_t* __restrict__ qkv, int64_t n8, int seq, int nheads_rot,
                             int ld, int d, const float* __restrict__ cos_t,
                             const float* __restrict__ sin_t, float sign) {
  const int half = d / 2, per = half / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n8) return;
  const int j = (int)(idx % per);
  const int64_t th = idx / per;
  const int hd = (int)(th % nheads_rot);
  const int64_t t = th / nheads_rot;
  const int pos = (int)(t % seq);
  uint16_t* p = qkv + t * ld + (int64_t)hd * d + j * 8;
  const float* cp = cos_t + (int64_t)pos * half + j * 8;
  const float* sp = sin_t + (int64_t)pos * half + j * 8;
  const uint4 lo = *reinterpret_cast<const uint4*>(p);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + half);
  const float4 c0 = *reinterpret_cast<const float4*>(cp), c1 = *reinterpret_cast<const float4*>(cp + 4);
  const float4 s0 = *reinterpret_cast<const float4*>(sp), s1 = *reinterpret_cast<const float4*>(sp + 4);
  const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  const uint32_t lw[4] = {lo.x, lo.y, lo.z, lo.w}, hw[4] = {hi.x, hi.y, hi.z, hi.w};
  uint32_t ol[4], oh[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint16_t rl[2], rh[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = 2 * e + h;
      const float a = bf2f((uint16_t)(lw[e] >> (16 * h))), b = bf2f((uint16_t)(hw[e] >> (16 * h)));
      const float si = sign * sn[i];
      rl[h] = f2bf(a * c[i] - b * si);
      rh[h] = f2bf(b * c[i] + a * si);
    }
    ol[e] = (uint32_t)rl[0] | ((uint32_t)rl[1] << 16);
    oh[e] = (uint32_t)rh[0] | ((uint32_t)rh[1] << 16);
  }
  *reinterpret_cast<uint4*>(p) = make_uint4(ol[0], ol[1], ol[2], ol[3]);
  *reinterpret_cast<uint4*>(p + half) = make_uint4(oh[0], oh[1], oh[2], oh[3]);
}

// ---------------------------------------------------------- cross-entropy
// One row per workgroup: online max / sum of exp over the row, then
// dlogits = (exp(l - lse) - onehot) * coef.
__global__ __launch_bounds__(NT) void ce_kernel(const float* __restrict__ logits, int64_t ld,
                                                const int32_t* __restrict__ labels, int V,
                                                float coef, uint16_t* __restrict__ dl,
                                                int64_t ldd, float* __restrict__ loss_rows) {
  __shared__ float shm[4], shs[4];
  const int64_t row = blockIdx.x;
  const float* lr = logits + row * ld;
  uint16_t* dr = dl + row * ldd;
  const int label = labels[row];
  if (label < 0) {
    for (int c = threadIdx.x * 4; c < V; c += NT * 4)
      *reinterpret_cast<uint2*>(dr + c) = make_uint2(0u, 0u);
    if (threadIdx.x == 0) loss_rows[row] = 0.0f;
    return;
  }
  float m = -INFINITY, s = 0.0f;
  for (int c = threadIdx.x * 4; c < V; c += NT * 4) {
    const float4 v = *reinterpret_cast<const float4*>(lr + c);
    const float mx = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
    const float mn = fmaxf(m, mx);
    s = s * expf(m - mn) + expf(v.x - mn) + expf(v.y - mn) + expf(v.z - mn) + expf(v.w - mn);
    m = mn;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float mo = __shfl_xor(m, o), so = __shfl_xor(s, o);
    const float mn = fmaxf(m, mo);
    s = (m == -INFINITY ? 0.0f : s * expf(m - mn)) + (mo == -INFINITY ? 0.0f : so * expf(mo - mn));
    m = mn;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    shm[w] = m;
    shs[w] = s;
  }
  __syncthreads();
  float M = fmaxf(fmaxf(shm[0], shm[1]), fmaxf(shm[2], shm[3]));
  float S = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) S += shs[k] * expf(shm[k] - M);
  const float lse = M + logf(S);
  for (int c = threadIdx.x * 4; c < V; c += NT * 4) {
    const float4 v = *reinterpret_cast<const float4*>(lr + c);
    float p0 = expf(v.x - lse), p1 = expf(v.y - lse), p2 = expf(v.z - lse), p3 = expf(v.w - lse);
    if (label >= c && label < c + 4) {
      const int k = label - c;
      if (k == 0) p0 -= 1.0f;
      if (k == 1) p1 -= 1.0f;
      if (k == 2) p2 -= 1.0f;
      if (k == 3) p3 -= 1.0f;
    }
    *reinterpret_cast<uint2*>(dr + c) = make_uint2(pack_bf2(p0 * coef, p1 * coef),
                                                   pack_bf2(p2 * coef, p3 * coef));
  }
  if (threadIdx.x == 0) loss_rows[row] = lse - lr[label];
}

// ---------------------------------------- cross-entropy in token x vocab chunks
// The LM head's logits exist one token chunk x one vocabulary chunk at a time.
// Forward: each chunk's softmax statistics (row maximum m_c and sum of
// exp(l - m_c)) are merged into the token's running (m, s), and the label's
// logit is kept when the label falls in the chunk.  After the last chunk
// lse = m + log(s).  Backward: each chunk's logits are recomputed and
// dlogits = (exp(l - lse) - onehot) * coef follows without the whole row.

// Chunk statistics of one row, one workgroup per row of the token chunk.
__global__ __launch_bounds__(NT) void ce_stats_kernel(const float* __restrict__ logits, int64_t ld,
                                                      int nr, int64_t r0,
                                                      const int32_t* __restrict__ labels, int first,
                                                      float* __restrict__ m_run,
                                                      float* __restrict__ s_run,
                                                      float* __restrict__ lab_logit) {
  __shared__ float shm[4], shs[4];
  const int64_t row = blockIdx.x;
  const float* lr = logits + row * ld;
  float m = -INFINITY, s = 0.0f;
  for (int c = threadIdx.x * 4; c < nr; c += NT * 4) {
    const float4 v = *reinterpret_cast<const float4*>(lr + c);
    const float mx = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
    const float mn = fmaxf(m, mx);
    s = s * expf(m - mn) + expf(v.x - mn) + expf(v.y - mn) + expf(v.z - mn) + expf(v.w - mn);
    m = mn;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float mo = __shfl_xor(m, o), so = __shfl_xor(s, o);
    const float mn = fmaxf(m, mo);
    s = (m == -INFINITY ? 0.0f : s * expf(m - mn)) + (mo == -INFINITY ? 0.0f : so * expf(mo - mn));
    m = mn;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    shm[w] = m;
    shs[w] = s;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  const float M = fmaxf(fmaxf(shm[0], shm[1]), fmaxf(shm[2], shm[3]));
  float S = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) S += shs[k] * expf(shm[k] - M);
  if (first) {
    m_run[row] = M;
    s_run[row] = S;
  } else {
    const float mo = m_run[row], so = s_run[row];
    const float mn = fmaxf(mo, M);
    s_run[row] = so * expf(mo - mn) + S * expf(M - mn);
    m_run[row] = mn;
  }
  const int64_t label = labels[row];
  if (label >= r0 && label < r0 + nr) lab_logit[row] = lr[label - r0];
}

// lse and the per-row loss (0 for ignored rows), one thread per row.
__global__ __launch_bounds__(NT) void ce_finish_kernel(const float* __restrict__ m_run,
                                                       const float* __restrict__ s_run,
                                                       const float* __restrict__ lab_logit,
                                                       const int32_t* __restrict__ labels,
                                                       int64_t T, float* __restrict__ lse,
                                                       float* __restrict__ loss_rows) {
  const int64_t t = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (t >= T) return;
  const float l = m_run[t] + logf(s_run[t]);
  lse[t] = l;
  loss_rows[t] = labels[t] >= 0 ? l - lab_logit[t] : 0.0f;
}

// dlogits of one token chunk x vocabulary chunk, one workgroup per row:
// rows t0 + row of the pass; coefficient of the row's micro-batch.
__global__ __launch_bounds__(NT) void ce_grad_kernel(const float* __restrict__ logits, int64_t ld,
                                                     int nr, int64_t r0,
                                                     const int32_t* __restrict__ labels,
                                                     const float* __restrict__ lse, int64_t t0,
                                                     CeCoef cf, uint16_t* __restrict__ dl,
                                                     int64_t ldd) {
  const int64_t row = blockIdx.x;
  const float* lr = logits + row * ld;
  uint16_t* dr = dl + row * ldd;
  const int64_t label = labels[row];
  if (label < 0) {
    for (int c = threadIdx.x * 4; c < nr; c += NT * 4)
      *reinterpret_cast<uint2*>(dr + c) = make_uint2(0u, 0u);
    return;
  }
  const float l = lse[row];
  const float coef = cf.c[(t0 + row) / cf.T_mb];
  const int64_t lc = label - r0;  // label column inside the chunk (may be outside)
  for (int c = threadIdx.x * 4; c < nr; c += NT * 4) {
    const float4 v = *reinterpret_cast<const float4*>(lr + c);
    float p[4] = {expf(v.x - l), expf(v.y - l), expf(v.z - l), expf(v.w - l)};
    if (lc >= c && lc < c + 4) p[lc - c] -= 1.0f;
    *reinterpret_cast<uint2*>(dr + c) =
        make_uint2(pack_bf2(p[0] * coef, p[1] * coef), pack_bf2(p[2] * coef, p[3] * coef));
  }
}

// fp32 -> bf16 (round to nearest even), n a multiple of 4.
__global__ void cast_bf16_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                 int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4 v = reinterpret_cast<const float4*>(src)[i];
    reinterpret_cast<uint2*>(dst)[i] = make_uint2(pack_bf2(v.x, v.y), pack_bf2(v.z, v.w));
  }
}

// Fixed-order sum of loss_rows: thread t adds rows t, t+256, ...; then the
// block sum.
__global__ __launch_bounds__(NT) void loss_reduce_kernel(const float* __restrict__ rows, int64_t T,
                                                         float inv_n, float* __restrict__ out) {
  __shared__ float sh[4];
  float s = 0.0f;
  for (int64_t t = threadIdx.x; t < T; t += NT) s += rows[t];
  s = block_sum(s, sh);
  if (threadIdx.x == 0) *out = s * inv_n;
}

// ------------------------------------------------------------- host copy
// Streams 16-byte vectors from device memory into host-mapped pinned memory
// (or back): the GPU's own stores cross the host link, so a gradient slab can
// drain while the copy engine is busy bringing the next layer in.
__global__ void copy16_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

}  // namespace

hipError_t launch_copy(void* dst, const void* src, size_t bytes, int wgs, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 > 0)
    hipLaunchKernelGGL(copy16_kernel, dim3(wgs), dim3(NT), 0, s,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_fwd(const float* x, const uint16_t* g, uint16_t* out, float* rstd,
                              int64_t T, int h, float eps, hipStream_t s) {
  const int vpt = (h / 4 + NT - 1) / NT;
#define MT_FWD(V) \
  if (vpt <= V) { \
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<V>, dim3((unsigned)T), dim3(NT), 0, s, x, g, out, rstd, \
                       h, eps); \
    return hipGetLastError(); \
  }
  MT_FWD(1) MT_FWD(2) MT_FWD(4) MT_FWD(5) MT_FWD(8) MT_FWD(16)
#undef MT_FWD
  return hipErrorInvalidValue;
}

size_t rmsnorm_bwd_partial_bytes(int64_t T, int h) {
  return (size_t)bwd_blocks(T) * (size_t)h * sizeof(float);
}

hipError_t launch_rmsnorm_bwd(const float* dn, const float* x, const float* rstd,
                              const uint16_t* g, const float* resid, float* dx,
                              uint16_t* dx_bf16, float* dg, uint16_t* dg_bf16, float* partial,
                              int64_t T, int h, hipStream_t s) {
  const int64_t nb = bwd_blocks(T);
  const int64_t rpb = (T + nb - 1) / nb;
  const int64_t nblk = (T + rpb - 1) / rpb;
  const int vpt = (h / 4 + NT - 1) / NT;
  bool done = false;
#define MT_BWD(V) \
  if (!done && vpt <= V) { \
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<V>, dim3((unsigned)nblk), dim3(NT), 0, s, dn, x, rstd, \
                       g, resid, dx, dx_bf16, partial, T, h, rpb); \
    done = true; \
  }
  MT_BWD(1) MT_BWD(2) MT_BWD(4) MT_BWD(5) MT_BWD(8) MT_BWD(16)
#undef MT_BWD
  if (!done) return hipErrorInvalidValue;
  hipLaunchKernelGGL(colsum_kernel, dim3((h + 63) / 64), dim3(NT), 0, s, partial, dg, dg_bf16,
                     (int)nblk, h);
  return hipGetLastError();
}

hipError_t launch_rope(uint16_t* qkv, int64_t T, int seq, int nq, int nkv, int d,
                       const float* cos_t, const float* sin_t, int inverse, hipStream_t s) {
  const int nrot = nq + nkv;  // q heads then k heads are contiguous in a qkv row
  const int ld = (nq + 2 * nkv) * d;
  const int64_t total = T * nrot * (d / 2);
  const bool vec = d % 16 == 0 && (((uintptr_t)qkv | (uintptr_t)cos_t | (uintptr_t)sin_t) & 15) == 0;
  if (vec)
    hipLaunchKernelGGL(rope8_kernel, dim3((unsigned)((total / 8 + NT - 1) / NT)), dim3(NT), 0, s,
                       qkv, total / 8, seq, nrot, ld, d, cos_t, sin_t, inverse ? -1.0f : 1.0f);
  else
    hipLaunchKernelGGL(rope_kernel, dim3((unsigned)((total + NT - 1) / NT)), dim3(NT), 0, s, qkv, T,
                       seq, nrot, ld, d, cos_t, sin_t, inverse ? -1.0f : 1.0f);
  return hipGetLastError();
}

hipError_t launch_ce_stats(const float* logits, int64_t ld, int64_t rows, int nr, int64_t r0,
                           const int32_t* labels, int first, float* m_run, float* s_run,
                           float* lab_logit, hipStream_t s) {
  hipLaunchKernelGGL(ce_stats_kernel, dim3((unsigned)rows), dim3(NT), 0, s, logits, ld, nr, r0,
                     labels, first, m_run, s_run, lab_logit);
  return hipGetLastError();
}

hipError_t launch_ce_finish(const float* m_run, const float* s_run, const float* lab_logit,
                            const int32_t* labels, int64_t T, float* lse, float* loss_rows,
                            hipStream_t s) {
  hipLaunchKernelGGL(ce_finish_kernel, dim3((unsigned)((T + NT - 1) / NT)), dim3(NT), 0, s, m_run,
                     s_run, lab_logit, labels, T, lse, loss_rows);
  return hipGetLastError();
}

hipError_t launch_ce_grad(const float* logits, int64_t ld, int64_t rows, int nr, int64_t r0,
                          const int32_t* labels, const float* lse, int64_t t0, const CeCoef& cf,
                          uint16_t* dl, int64_t ldd, hipStream_t s) {
  hipLaunchKernelGGL(ce_grad_kernel, dim3((unsigned)rows), dim3(NT), 0, s, logits, ld, nr, r0,
                     labels, lse, t0, cf, dl, ldd);
  return hipGetLastError();
}

hipError_t launch_cast_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s) {
  const int64_t n4 = n / 4;
  if (n4 > 0)
    hipLaunchKernelGGL(cast_bf16_kernel, dim3(1024), dim3(NT), 0, s, src, dst, n4);
  return hipGetLastError();
}

hipError_t launch_loss_mean(const float* rows, int64_t n, float inv_n, float* out, hipStream_t s) {
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(NT), 0, s, rows, n, inv_n, out);
  return hipGetLastError();
}

hipError_t launch_mean(const float* v, int64_t n, float* out, hipStream_t s) {
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(NT), 0, s, v, n, 1.0f / (float)n, out);
  return hipGetLastError();
}

hipError_t launch_cross_entropy(const float* logits, int64_t ld, const int32_t* labels, int64_t T,
                                int V, float grad_scale, int64_t n_valid, uint16_t* dlogits,
                                int64_t ld_d, float* loss_rows, float* loss_out, hipStream_t s) {
  const float coef = n_valid > 0 ? grad_scale / (float)n_valid : 0.0f;
  hipLaunchKernelGGL(ce_kernel, dim3((unsigned)T), dim3(NT), 0, s, logits, ld, labels, V, coef,
                     dlogits, ld_d, loss_rows);
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(NT), 0, s, loss_rows, T,
                     n_valid > 0 ? 1.0f / (float)n_valid : 0.0f, loss_out);
  return hipGetLastError();
}

}  // namespace mt
