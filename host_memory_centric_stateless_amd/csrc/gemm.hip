// bf16 MFMA GEMM for gfx950 with fp32 accumulation and fused epilogues.
//
// Every projection of the decoder block and its two gradients go through here
// (the block's dedicated forward/backward replaces an autograd graph:
// zhichai.net "MegaTrain：单卡训百亿大模型的突破与实践", design point 4).
//
// Tiling: 128x128 output tile per 256-thread workgroup (4 waves as 2x2, each
// wave 64x64 = 2x2 v_mfma_f32_32x32x16_bf16 tiles), K step 64, LDS double
// buffered.  LDS holds both operands as [row][k] (k contiguous, row stride 72
// elements so 16-byte fragment reads are conflict-free).  Operands whose
// reduction dimension is the slow one in memory (the transposed layouts of
// the input- and weight-gradient products) are transposed in registers on the
// way into LDS: each thread reads an 8(k) x 4(row) block with 8-byte loads and
// writes four 16-byte rows.
#include "common.h"

namespace mt {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDSK = BK + 8;  // elements per LDS row
constexpr int NT = 256;

__device__ inline bf16x8_t frag(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(p));
}

// Row r (0..127) of a B tile in the SwiGLU product: rows 0..63 are gate rows
// f0..f0+63, rows 64..127 the matching up rows.
struct RowMap {
  int64_t row0, nrows;   // plain: global row = row0 + r, valid if < nrows
  int64_t ffn;           // swiglu: > 0
  __device__ inline int64_t map(int r, bool& ok) const {
    if (ffn > 0) {
      int64_t f = row0 + (r & 63);
      ok = f < nrows;
      return (r < 64) ? f : ffn + f;
    }
    int64_t g = row0 + r;
    ok = g < nrows;
    return g;
  }
};

// Operand stored [row][k] (k contiguous): 128 rows x 64 k, 4 x 16 B per thread.
struct LoadK {
  u32x4 r[4];
  __device__ inline void load(const uint16_t* base, int64_t ld, const RowMap& rm, int64_t k0,
                              int64_t K, int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int idx = tid + NT * i;
      int row = idx >> 3;
      int64_t k = k0 + (idx & 7) * 8;
      bool ok;
      int64_t g = rm.map(row, ok);
      if (ok && k < K)
        r[i] = *reinterpret_cast<const u32x4*>(base + g * ld + k);
      else
        r[i] = u32x4{0, 0, 0, 0};
    }
  }
  __device__ inline void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int idx = tid + NT * i;
      *reinterpret_cast<u32x4*>(lds + (idx >> 3) * LDSK + (idx & 7) * 8) = r[i];
    }
  }
};

// Operand stored [k][row] (row contiguous): 64 k x 128 rows.  Thread owns the
// 8 x 4 block k = kb*8.., rows mb*4.. and writes it transposed into LDS.
struct LoadT {
  u32x2 r[8];
  __device__ inline void load(const uint16_t* base, int64_t ld, int64_t row0, int64_t nrows,
                              int64_t k0, int64_t K, int tid) {
    const int kb = tid >> 5, mb = tid & 31;
    const int64_t g = row0 + mb * 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int64_t k = k0 + kb * 8 + i;
      if (k < K && g < nrows)
        r[i] = *reinterpret_cast<const u32x2*>(base + k * ld + g);
      else
        r[i] = u32x2{0, 0};
    }
  }
  __device__ inline void store(uint16_t* lds, int tid) const {
    const int kb = tid >> 5, mb = tid & 31;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 o;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint32_t w0 = r[2 * p][j >> 1], w1 = r[2 * p + 1][j >> 1];
        uint32_t lo = (j & 1) ? (w0 >> 16) : (w0 & 0xffffu);
        uint32_t hi = (j & 1) ? (w1 & 0xffff0000u) : (w1 << 16);
        o[p] = lo | hi;
      }
      *reinterpret_cast<u32x4*>(lds + (mb * 4 + j) * LDSK + kb * 8) = o;
    }
  }
};

__device__ inline float silu_f(float a) { return a / (1.0f + expf(-a)); }

template <int LAYOUT, int EPI>
__global__ __launch_bounds__(NT) void gemm_kernel(mt_gemm_args p) {
  constexpr bool A_T = (LAYOUT == MT_GEMM_TN);
  constexpr bool B_T = (LAYOUT != MT_GEMM_NT);
  constexpr bool SWI = (EPI == MT_EPI_SWIGLU);
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDSK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDSK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t n0 = (int64_t)blockIdx.x * (SWI ? BN / 2 : BN);
  const int64_t K = p.K;
  const uint16_t* A = p.A;
  const uint16_t* B = p.B;

  RowMap ra{m0, p.M, 0};
  RowMap rb{n0, p.N, SWI ? p.ffn : 0};

  typename std::conditional<A_T, LoadT, LoadK>::type la;
  typename std::conditional<B_T, LoadT, LoadK>::type lb;

  auto load_tiles = [&](int64_t k0) {
    if constexpr (A_T) la.load(A, p.lda, m0, p.M, k0, K, tid);
    else la.load(A, p.lda, ra, k0, K, tid);
    if constexpr (B_T) lb.load(B, p.ldb, n0, p.N, k0, K, tid);
    else lb.load(B, p.ldb, rb, k0, K, tid);
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (int)((K + BK - 1) / BK);
  load_tiles(0);
  la.store(As[0], tid);
  lb.store(Bs[0], tid);
  __syncthreads();

  const int arow = wm * 64 + (lane & 31);
  const int brow0 = SWI ? (wn * 32 + (lane & 31)) : (wn * 64 + (lane & 31));
  const int bstep = SWI ? 64 : 32;  // LDS row distance between the wave's two N sub-tiles
  const int kofs = (lane >> 5) * 8;

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tiles((int64_t)(kt + 1) * BK);
    const uint16_t* as = As[cur];
    const uint16_t* bs = Bs[cur];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t a0 = frag(as + arow * LDSK + ks * 16 + kofs);
      bf16x8_t a1 = frag(as + (arow + 32) * LDSK + ks * 16 + kofs);
      bf16x8_t b0 = frag(bs + brow0 * LDSK + ks * 16 + kofs);
      bf16x8_t b1 = frag(bs + (brow0 + bstep) * LDSK + ks * 16 + kofs);
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      la.store(As[cur ^ 1], tid);
      lb.store(Bs[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogue
  // acc[i][j][r] is C[row, col] with row = 8*(r/4) + 4*(lane/32) + r%4 and
  // col = lane%32 inside the 32x32 sub-tile (i, j).
  const int g4 = (lane >> 5) * 4;
  if constexpr (SWI) {
    const int64_t f = n0 + wn * 32 + (lane & 31);
    if (f < p.N) {
      uint16_t* C = static_cast<uint16_t*>(p.C);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int64_t row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + g4 + (r & 3);
          if (row < p.M) {
            float a = acc[i][0][r], u = acc[i][1][r];
            p.gu[row * p.ldgu + f] = f2bf(a);
            p.gu[row * p.ldgu + p.ffn + f] = f2bf(u);
            C[row * p.ldc + f] = f2bf(silu_f(a) * u);
          }
        }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= p.N) continue;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int64_t row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + g4 + (r & 3);
          if (row >= p.M) continue;
          float v = acc[i][j][r];
          if constexpr (EPI == MT_EPI_BF16) {
            static_cast<uint16_t*>(p.C)[row * p.ldc + col] = f2bf(v);
          } else if constexpr (EPI == MT_EPI_F32) {
            static_cast<float*>(p.C)[row * p.ldc + col] = v;
          } else if constexpr (EPI == MT_EPI_F32_RESID) {
            static_cast<float*>(p.C)[row * p.ldc + col] = p.R[row * p.ldr + col] + v;
          } else if constexpr (EPI == MT_EPI_F32_ACCUM) {
            static_cast<float*>(p.C)[row * p.ldc + col] += v;
          } else if constexpr (EPI == MT_EPI_SWIGLU_BWD) {
            float a = bf2f(p.gu[row * p.ldgu + col]);
            float u = bf2f(p.gu[row * p.ldgu + p.ffn + col]);
            float s = 1.0f / (1.0f + expf(-a));
            uint16_t* C = static_cast<uint16_t*>(p.C);
            C[row * p.ldc + col] = f2bf(v * u * s * (1.0f + a * (1.0f - s)));
            C[row * p.ldc + p.ffn + col] = f2bf(v * a * s);
          }
        }
    }
  }
}

template <int LAYOUT, int EPI>
hipError_t launch_one(const mt_gemm_args& a, hipStream_t s) {
  const int64_t nt = (EPI == MT_EPI_SWIGLU) ? (a.N + 63) / 64 : (a.N + BN - 1) / BN;
  dim3 grid((unsigned)nt, (unsigned)((a.M + BM - 1) / BM));
  hipLaunchKernelGGL((gemm_kernel<LAYOUT, EPI>), grid, dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool gemm_shape_ok(const mt_gemm_args& a, const char** why) {
  auto bad = [&](const char* w) { if (why) *why = w; return false; };
  if (a.layout < 0 || a.layout > 2) return bad("layout");
  if (a.epilogue < 0 || a.epilogue > 5) return bad("epilogue");
  if (a.M <= 0 || a.N <= 0 || a.K <= 0) return bad("empty or negative dimension");
  if (a.M % 8 || a.N % 8 || a.K % 8) return bad("M, N, K must be multiples of 8");
  if (a.M / 128 >= 65535) return bad("M too large");
  if (!a.A || !a.B || !a.C) return bad("null operand");
  if (a.lda % 8 || a.ldb % 8) return bad("lda/ldb must be multiples of 8");
  const bool at = a.layout == MT_GEMM_TN, bt = a.layout != MT_GEMM_NT;
  if ((at ? a.lda < a.M : a.lda < a.K) || (bt ? a.ldb < a.N : a.ldb < a.K)) return bad("lda/ldb");
  if (a.epilogue == MT_EPI_SWIGLU) {
    if (a.layout != MT_GEMM_NT) return bad("SWIGLU needs the NT layout");
    if (a.ffn != a.N || !a.gu || a.ldgu < 2 * a.ffn || a.ldc < a.N) return bad("SWIGLU args");
  } else if (a.epilogue == MT_EPI_SWIGLU_BWD) {
    if (a.layout != MT_GEMM_NN) return bad("SWIGLU_BWD needs the NN layout");
    if (a.ffn != a.N || !a.gu || a.ldgu < 2 * a.ffn || a.ldc < 2 * a.ffn) return bad("SWIGLU_BWD args");
  } else {
    if (a.ldc < a.N) return bad("ldc");
    if (a.epilogue == MT_EPI_F32_RESID && (!a.R || a.ldr < a.N)) return bad("residual");
  }
  return true;
}

hipError_t launch_gemm(const mt_gemm_args& a, hipStream_t s) {
#define MT_GEMM_CASE(L, E) \
  if (a.layout == L && a.epilogue == E) return launch_one<L, E>(a, s);
  MT_GEMM_CASE(MT_GEMM_NT, MT_EPI_BF16)
  MT_GEMM_CASE(MT_GEMM_NT, MT_EPI_F32)
  MT_GEMM_CASE(MT_GEMM_NT, MT_EPI_F32_RESID)
  MT_GEMM_CASE(MT_GEMM_NT, MT_EPI_F32_ACCUM)
  MT_GEMM_CASE(MT_GEMM_NT, MT_EPI_SWIGLU)
  MT_GEMM_CASE(MT_GEMM_NN, MT_EPI_BF16)
  MT_GEMM_CASE(MT_GEMM_NN, MT_EPI_F32)
  MT_GEMM_CASE(MT_GEMM_NN, MT_EPI_F32_RESID)
  MT_GEMM_CASE(MT_GEMM_NN, MT_EPI_F32_ACCUM)
  MT_GEMM_CASE(MT_GEMM_NN, MT_EPI_SWIGLU_BWD)
  MT_GEMM_CASE(MT_GEMM_TN, MT_EPI_BF16)
  MT_GEMM_CASE(MT_GEMM_TN, MT_EPI_F32)
  MT_GEMM_CASE(MT_GEMM_TN, MT_EPI_F32_RESID)
  MT_GEMM_CASE(MT_GEMM_TN, MT_EPI_F32_ACCUM)
#undef MT_GEMM_CASE
  return hipErrorInvalidValue;
}

}  // namespace mt
