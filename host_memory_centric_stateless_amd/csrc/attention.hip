// Causal grouped-query flash attention, forward and backward, for gfx950.
//
// The block's attention (q head j reads kv head j / (nq/nkv)) computed tile by
// tile with an online softmax, so memory is linear in the sequence length --
// what lets one GPU train long contexts once weights and optimizer state live
// on the host (zhichai.net "MegaTrain：单卡训百亿大模型的突破与实践", 性能与能力:
// long context as a by-product of the layer-wise memory design).
//
// MFMA orientation.  v_mfma_f32_32x32x16_bf16 leaves C[row][col] in lane
// col = lane%32, rows 8*(r/4) + 4*(lane/32) + r%4 of accumulator element r.
// Computing the transposed scores S^T = K Q^T puts one query per lane, so the
// softmax statistics of a query are lane-local (plus the partner lane
// lane^32).  The probabilities then feed the next product directly as the B
// operand: element e of a lane's 8-value fragment for k-step (i, hh) is row
// i*32 + 16*hh + 8*(e/4) + 4*(lane/32) + e%4 -- a permutation of the 16
// reduction indices that the A operand (read from a transposed LDS tile with
// two 8-byte reads) follows exactly, so the sum is unchanged.
//
// Backward is two deterministic kernels: dK/dV with the key block outer
// (loops over every query head of the group and every later query tile, so
// grouped heads are summed in a fixed order) and dQ with the query block
// outer.  No floating-point atomics.
#include "common.h"

namespace mt {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ inline bf16x8_t as_frag(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ inline bf16x8_t ld_frag(const uint16_t* p) {
  return as_frag(*reinterpret_cast<const u32x4*>(p));
}
// Two 4-element halves (8 bytes each) -> one fragment.
__device__ inline bf16x8_t ld_frag2(const uint16_t* p0, const uint16_t* p1) {
  u32x2 a = *reinterpret_cast<const u32x2*>(p0);
  u32x2 b = *reinterpret_cast<const u32x2*>(p1);
  return as_frag(u32x4{a[0], a[1], b[0], b[1]});
}
__device__ inline bf16x8_t pack_frag(const float* v) {
  return as_frag(u32x4{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]),
                       pack_bf2(v[6], v[7])});
}
__device__ inline f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ inline void zero(f32x16_t& a) {
#pragma unroll
  for (int r = 0; r < 16; ++r) a[r] = 0.0f;
}

// Copy a [ROWS][D] bf16 tile (global row stride ld) into LDS: normal copy
// [ROWS][D+8] and/or transposed copy [D][ROWS+8].  Work is split into 8x8
// blocks handled by threads t0..t0+nthr-1 (t = threadIdx.x - t0).
template <int ROWS, int D>
__device__ inline void load_tile(const uint16_t* src, int64_t ld, uint16_t* nrm, uint16_t* trn,
                                 int t, int nthr) {
  constexpr int DB = D / 8, NB = (ROWS / 8) * DB;
  for (int blk = t; blk < NB; blk += nthr) {
    const int rb = blk / DB, db = blk % DB;
    u32x4 r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      r[i] = *reinterpret_cast<const u32x4*>(src + (int64_t)(rb * 8 + i) * ld + db * 8);
    if (nrm) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4*>(nrm + (rb * 8 + i) * (D + 8) + db * 8) = r[i];
    }
    if (trn) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        u32x4 o;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          uint32_t w0 = r[2 * p][jj >> 1], w1 = r[2 * p + 1][jj >> 1];
          uint32_t lo = (jj & 1) ? (w0 >> 16) : (w0 & 0xffffu);
          uint32_t hi = (jj & 1) ? (w1 & 0xffff0000u) : (w1 << 16);
          o[p] = lo | hi;
        }
        *reinterpret_cast<u32x4*>(trn + (db * 8 + jj) * (ROWS + 8) + rb * 8) = o;
      }
    }
  }
}

// --------------------------------------------------------------- forward
template <int D>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const uint16_t* __restrict__ qkv,
                                                       uint16_t* __restrict__ out,
                                                       float* __restrict__ lse, int seq, int nq,
                                                       int nkv, int64_t T) {
  constexpr int BKV = 64, KS = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BKV * (D + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * (BKV + 8)];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5;
  const int qb = gridDim.x - 1 - blockIdx.x;
  const int j = blockIdx.y, b = blockIdx.z;
  const int kvh = j / (nq / nkv);
  const int64_t ld = (int64_t)(nq + 2 * nkv) * D;
  const int64_t row0 = (int64_t)b * seq;
  const uint16_t* Qp = qkv + j * D;
  const uint16_t* Kp = qkv + (int64_t)nq * D + kvh * D;
  const uint16_t* Vp = qkv + (int64_t)(nq + nkv) * D + kvh * D;
  const float sl2 = LOG2E / sqrtf((float)D);

  const int q0 = qb * 128 + w * 32;
  const int q = q0 + (lane & 31);
  bf16x8_t qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = ld_frag(Qp + (row0 + q) * ld + ks * 16 + g * 8);

  f32x16_t acc[DT];
#pragma unroll
  for (int dd = 0; dd < DT; ++dd) zero(acc[dd]);
  float m_run = -INFINITY, l_run = 0.0f;

  const int nkb = (qb * 128 + 127) / BKV + 1;
  for (int kb = 0; kb < nkb; ++kb) {
    const int kv0 = kb * BKV;
    if (tid < 128)
      load_tile<BKV, D>(Kp + (row0 + kv0) * ld, ld, Ks, nullptr, tid, 128);
    else
      load_tile<BKV, D>(Vp + (row0 + kv0) * ld, ld, nullptr, Vt, tid - 128, 128);
    __syncthreads();
    if (kv0 <= q0 + 31) {
      f32x16_t s[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        zero(s[i]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          s[i] = mfma(ld_frag(Ks + (i * 32 + (lane & 31)) * (D + 8) + ks * 16 + g * 8), qf[ks],
                      s[i]);
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kv = kv0 + i * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
          float v = (kv <= q) ? s[i][r] * sl2 : -INFINITY;
          s[i][r] = v;
          mloc = fmaxf(mloc, v);
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dd = 0; dd < DT; ++dd)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dd][r] *= alpha;
      float pv[2][16];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pr = exp2f(s[i][r] - m_new);
          pv[i][r] = pr;
          l_run += pr;
        }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          bf16x8_t pf = pack_frag(&pv[i][hh * 8]);
          const int kvo = i * 32 + hh * 16 + g * 4;
#pragma unroll
          for (int dd = 0; dd < DT; ++dd) {
            const uint16_t* vr = Vt + (dd * 32 + (lane & 31)) * (BKV + 8) + kvo;
            acc[dd] = mfma(ld_frag2(vr, vr + 8), pf, acc[dd]);
          }
        }
    }
    __syncthreads();
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  uint16_t* op = out + (row0 + q) * (int64_t)nq * D + j * D;
#pragma unroll
  for (int dd = 0; dd < DT; ++dd)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int d = dd * 32 + rr * 8 + g * 4;
      u32x2 v{pack_bf2(acc[dd][rr * 4 + 0] * inv, acc[dd][rr * 4 + 1] * inv),
              pack_bf2(acc[dd][rr * 4 + 2] * inv, acc[dd][rr * 4 + 3] * inv)};
      *reinterpret_cast<u32x2*>(op + d) = v;
    }
  if (g == 0) lse[(int64_t)j * T + row0 + q] = (m_run + log2f(l_tot)) * LN2;
}

// ------------------------------------------------- backward: D = rowsum(dO*O)
template <int D>
__global__ void attn_dsum_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                                 float* __restrict__ dsum, int nq, int64_t T) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // t * nq + j
  if (idx >= T * nq) return;
  const int64_t t = idx / nq;
  const int j = (int)(idx % nq);
  const uint16_t* a = o + t * nq * D + j * D;
  const uint16_t* c = dout + t * nq * D + j * D;
  float s = 0.0f;
#pragma unroll
  for (int d = 0; d < D; d += 8) {
    u32x4 x = *reinterpret_cast<const u32x4*>(a + d);
    u32x4 y = *reinterpret_cast<const u32x4*>(c + d);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      s += bf2f((uint16_t)(x[p] & 0xffff)) * bf2f((uint16_t)(y[p] & 0xffff));
      s += bf2f((uint16_t)(x[p] >> 16)) * bf2f((uint16_t)(y[p] >> 16));
    }
  }
  dsum[(int64_t)j * T + t] = s;
}

// ------------------------------------------------------- backward: dQ
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ dsum, uint16_t* __restrict__ dqkv,
    int seq, int nq, int nkv, int64_t T) {
  constexpr int BKV = 64, KS = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BKV * (D + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BKV * (D + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[D * (BKV + 8)];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5;
  const int qb = gridDim.x - 1 - blockIdx.x;
  const int j = blockIdx.y, b = blockIdx.z;
  const int kvh = j / (nq / nkv);
  const int64_t ld = (int64_t)(nq + 2 * nkv) * D;
  const int64_t row0 = (int64_t)b * seq;
  const uint16_t* Qp = qkv + j * D;
  const uint16_t* Kp = qkv + (int64_t)nq * D + kvh * D;
  const uint16_t* Vp = qkv + (int64_t)(nq + nkv) * D + kvh * D;
  const float sl2 = LOG2E / sqrtf((float)D);

  const int q0 = qb * 128 + w * 32;
  const int q = q0 + (lane & 31);
  bf16x8_t qf[KS], df[KS];
  const uint16_t* dop = dout + (row0 + q) * (int64_t)nq * D + j * D;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = ld_frag(Qp + (row0 + q) * ld + ks * 16 + g * 8);
    df[ks] = ld_frag(dop + ks * 16 + g * 8);
  }
  const float lse2 = lse[(int64_t)j * T + row0 + q] * LOG2E;
  const float dq_sum = dsum[(int64_t)j * T + row0 + q];

  f32x16_t acc[DT];
#pragma unroll
  for (int dd = 0; dd < DT; ++dd) zero(acc[dd]);

  const int nkb = (qb * 128 + 127) / BKV + 1;
  for (int kb = 0; kb < nkb; ++kb) {
    const int kv0 = kb * BKV;
    if (tid < 128)
      load_tile<BKV, D>(Kp + (row0 + kv0) * ld, ld, Ks, Kt, tid, 128);
    else
      load_tile<BKV, D>(Vp + (row0 + kv0) * ld, ld, Vs, nullptr, tid - 128, 128);
    __syncthreads();
    if (kv0 <= q0 + 31) {
      f32x16_t s[2], dp[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        zero(s[i]);
        zero(dp[i]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int ro = (i * 32 + (lane & 31)) * (D + 8) + ks * 16 + g * 8;
          s[i] = mfma(ld_frag(Ks + ro), qf[ks], s[i]);
          dp[i] = mfma(ld_frag(Vs + ro), df[ks], dp[i]);
        }
      }
      float ds[2][16];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kv = kv0 + i * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
          float pr = (kv <= q) ? exp2f(s[i][r] * sl2 - lse2) : 0.0f;
          ds[i][r] = pr * (dp[i][r] - dq_sum);
        }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          bf16x8_t sf = pack_frag(&ds[i][hh * 8]);
          const int kvo = i * 32 + hh * 16 + g * 4;
#pragma unroll
          for (int dd = 0; dd < DT; ++dd) {
            const uint16_t* kr = Kt + (dd * 32 + (lane & 31)) * (BKV + 8) + kvo;
            acc[dd] = mfma(ld_frag2(kr, kr + 8), sf, acc[dd]);
          }
        }
    }
    __syncthreads();
  }
  const float scale = 1.0f / sqrtf((float)D);
  uint16_t* dq = dqkv + (row0 + q) * ld + j * D;
#pragma unroll
  for (int dd = 0; dd < DT; ++dd)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int d = dd * 32 + rr * 8 + g * 4;
      u32x2 v{pack_bf2(acc[dd][rr * 4 + 0] * scale, acc[dd][rr * 4 + 1] * scale),
              pack_bf2(acc[dd][rr * 4 + 2] * scale, acc[dd][rr * 4 + 3] * scale)};
      *reinterpret_cast<u32x2*>(dq + d) = v;
    }
}

// ---------------------------------------------------- backward: dK, dV
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ dsum, uint16_t* __restrict__ dqkv,
    int seq, int nq, int nkv, int64_t T) {
  constexpr int BQ = 64, KS = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[BQ * (D + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[D * (BQ + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t Os[BQ * (D + 8)];  // dO, normal
  __shared__ __attribute__((aligned(16))) uint16_t Ot[D * (BQ + 8)];  // dO, transposed
  __shared__ __attribute__((aligned(16))) float Ls[BQ];
  __shared__ __attribute__((aligned(16))) float Ds[BQ];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5;
  const int kvb = gridDim.x - 1 - blockIdx.x;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int grp = nq / nkv;
  const int64_t ld = (int64_t)(nq + 2 * nkv) * D;
  const int64_t ldo = (int64_t)nq * D;
  const int64_t row0 = (int64_t)b * seq;
  const uint16_t* Kp = qkv + (int64_t)nq * D + kvh * D;
  const uint16_t* Vp = qkv + (int64_t)(nq + nkv) * D + kvh * D;
  const float sl2 = LOG2E / sqrtf((float)D);

  const int kw0 = kvb * 128 + w * 32;
  const int kv = kw0 + (lane & 31);
  bf16x8_t kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = ld_frag(Kp + (row0 + kv) * ld + ks * 16 + g * 8);
    vf[ks] = ld_frag(Vp + (row0 + kv) * ld + ks * 16 + g * 8);
  }
  f32x16_t adk[DT], adv[DT];
#pragma unroll
  for (int dd = 0; dd < DT; ++dd) {
    zero(adk[dd]);
    zero(adv[dd]);
  }
  const int nqt = seq / BQ;
  for (int hq = 0; hq < grp; ++hq) {
    const int j = kvh * grp + hq;
    const uint16_t* Qp = qkv + j * D;
    const uint16_t* dOp = dout + j * D;
    for (int qt = (kvb * 128) / BQ; qt < nqt; ++qt) {
      const int q0 = qt * BQ;
      if (tid < 128)
        load_tile<BQ, D>(Qp + (row0 + q0) * ld, ld, Qs, Qt, tid, 128);
      else
        load_tile<BQ, D>(dOp + (row0 + q0) * ldo, ldo, Os, Ot, tid - 128, 128);
      if (tid < BQ) {
        Ls[tid] = lse[(int64_t)j * T + row0 + q0 + tid] * LOG2E;
        Ds[tid] = dsum[(int64_t)j * T + row0 + q0 + tid];
      }
      __syncthreads();
      if (q0 + BQ - 1 >= kw0) {
        f32x16_t s[2], dp[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          zero(s[i]);
          zero(dp[i]);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const int ro = (i * 32 + (lane & 31)) * (D + 8) + ks * 16 + g * 8;
            s[i] = mfma(ld_frag(Qs + ro), kf[ks], s[i]);
            dp[i] = mfma(ld_frag(Os + ro), vf[ks], dp[i]);
          }
        }
        float pv[2][16], ds[2][16];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int ql = i * 32 + rr * 8 + g * 4;
            const float4 l4 = *reinterpret_cast<const float4*>(Ls + ql);
            const float4 d4 = *reinterpret_cast<const float4*>(Ds + ql);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
            const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = rr * 4 + e;
              const int qq = q0 + ql + e;
              float pr = (kv <= qq) ? exp2f(s[i][r] * sl2 - lv[e]) : 0.0f;
              pv[i][r] = pr;
              ds[i][r] = pr * (dp[i][r] - dv[e]);
            }
          }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            bf16x8_t pf = pack_frag(&pv[i][hh * 8]);
            bf16x8_t sf = pack_frag(&ds[i][hh * 8]);
            const int qo = i * 32 + hh * 16 + g * 4;
#pragma unroll
            for (int dd = 0; dd < DT; ++dd) {
              const int ro = (dd * 32 + (lane & 31)) * (BQ + 8) + qo;
              adv[dd] = mfma(ld_frag2(Ot + ro, Ot + ro + 8), pf, adv[dd]);
              adk[dd] = mfma(ld_frag2(Qt + ro, Qt + ro + 8), sf, adk[dd]);
            }
          }
      }
      __syncthreads();
    }
  }
  const float scale = 1.0f / sqrtf((float)D);
  uint16_t* dk = dqkv + (row0 + kv) * ld + (int64_t)nq * D + kvh * D;
  uint16_t* dv = dqkv + (row0 + kv) * ld + (int64_t)(nq + nkv) * D + kvh * D;
#pragma unroll
  for (int dd = 0; dd < DT; ++dd)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int d = dd * 32 + rr * 8 + g * 4;
      u32x2 k2{pack_bf2(adk[dd][rr * 4 + 0] * scale, adk[dd][rr * 4 + 1] * scale),
               pack_bf2(adk[dd][rr * 4 + 2] * scale, adk[dd][rr * 4 + 3] * scale)};
      u32x2 v2{pack_bf2(adv[dd][rr * 4 + 0], adv[dd][rr * 4 + 1]),
               pack_bf2(adv[dd][rr * 4 + 2], adv[dd][rr * 4 + 3])};
      *reinterpret_cast<u32x2*>(dk + d) = k2;
      *reinterpret_cast<u32x2*>(dv + d) = v2;
    }
}

template <int D>
hipError_t fwd_d(const uint16_t* qkv, uint16_t* o, float* lse, int batch, int seq, int nq, int nkv,
                 hipStream_t s) {
  const int64_t T = (int64_t)batch * seq;
  hipLaunchKernelGGL(attn_fwd_kernel<D>, dim3(seq / 128, nq, batch), dim3(256), 0, s, qkv, o, lse,
                     seq, nq, nkv, T);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_d(const uint16_t* qkv, const uint16_t* o, const uint16_t* dout, const float* lse,
                 float* dsum, uint16_t* dqkv, int batch, int seq, int nq, int nkv, hipStream_t s) {
  const int64_t T = (int64_t)batch * seq;
  const int64_t n = T * nq;
  hipLaunchKernelGGL(attn_dsum_kernel<D>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, o,
                     dout, dsum, nq, T);
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel<D>, dim3(seq / 128, nkv, batch), dim3(256), 0, s, qkv,
                     dout, lse, dsum, dqkv, seq, nq, nkv, T);
  hipLaunchKernelGGL(attn_bwd_dq_kernel<D>, dim3(seq / 128, nq, batch), dim3(256), 0, s, qkv,
                     dout, lse, dsum, dqkv, seq, nq, nkv, T);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const uint16_t* qkv, uint16_t* o, float* lse, int batch, int seq,
                           int nq, int nkv, int d, hipStream_t s) {
  if (d == 128) return fwd_d<128>(qkv, o, lse, batch, seq, nq, nkv, s);
  if (d == 64) return fwd_d<64>(qkv, o, lse, batch, seq, nq, nkv, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_bwd(const uint16_t* qkv, const uint16_t* o, const uint16_t* dout,
                           const float* lse, float* dsum, uint16_t* dqkv, int batch, int seq,
                           int nq, int nkv, int d, hipStream_t s) {
  if (d == 128) return bwd_d<128>(qkv, o, dout, lse, dsum, dqkv, batch, seq, nq, nkv, s);
  if (d == 64) return bwd_d<64>(qkv, o, dout, lse, dsum, dqkv, batch, seq, nq, nkv, s);
  return hipErrorInvalidValue;
}

}  // namespace mt
