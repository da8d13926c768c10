// bf16 MFMA GEMM for gfx950 with fp32 accumulation and fused epilogues.
//
// Every projection of the decoder block and its two gradients go through here
// (the block's dedicated forward/backward replaces an autograd graph:
// zhichai.net "MegaTrain：单卡训百亿大模型的突破与实践", design point 4).
//
// Two kernels share one epilogue (store_tile):
//   * gemm_direct_kernel: 256x256 output tiles, 8 waves of 128x64 (two waves
//     per SIMD), K step 64 in two LDS stages.  Operand tiles go from global
//     memory straight into LDS with buffer_load ... lds into unpadded,
//     XOR-swizzled tiles; [k][row] operands (the transposed layouts of the
//     gradient products) are read as MFMA fragments with ds_read_b64_tr_b16.
//     Used for every product large enough to fill the chip whose K is a
//     multiple of 128.
//   * gemm_kernel: the same tiling staged through registers (128x128 tiles of
//     4 waves for small products, or 256x256 when K has a tail).
// v_mfma_f32_32x32x16_bf16 throughout; blockIdx -> tile is XCD-aware so that
// neighbouring tiles share an L2.  Epilogues: bf16 / fp32 stores, residual
// add, fp32 accumulate, SwiGLU forward and backward, and the fused QKV RoPE.
#include "common.h"

namespace mt {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 64;
constexpr int LDSK = BK + 8;  // elements per LDS row

__device__ inline bf16x8_t frag(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(p));
}

// Global row of tile row r, clamped into the matrix (out-of-range rows are
// loaded from a valid row and zeroed, so the loads carry no branches).  In the
// SwiGLU product the B tile holds gate rows f0..f0+H-1 followed by the
// matching up rows (H = half the tile).
template <int H, bool SWI>
struct RowMap {
  int64_t row0, nrows;   // rows valid below nrows (SwiGLU: gate/up index below ffn)
  int64_t ffn;
  __device__ inline int64_t map(int r, bool& ok) const {
    if constexpr (SWI) {
      const int64_t f = row0 + (r % H);
      ok = f < nrows;
      const int64_t fc = ok ? f : nrows - 1;
      return (r < H) ? fc : ffn + fc;
    } else {
      const int64_t g = row0 + r;
      ok = g < nrows;
      return ok ? g : nrows - 1;
    }
  }
};

// B rows of the RoPE product (the fused QKV projection).  Inside every head
// of d rows the tile's local row l = 16 g + w (w < 16) holds head row
// 8 g + w for w < 8 and d/2 + 8 g + w - 8 otherwise.  The epilogue gives a
// lane 16 consecutive local columns, so it then holds eight whole rotation
// pairs (i, i + d/2), i = 8 g .. 8 g + 7, and rotates them in fp32 before the
// single bf16 rounding.  Heads never straddle a tile (tiles are 128 or 256
// columns wide, d divides 128).
struct RopeRowMap {
  int64_t row0, nrows;
  int d;
  __device__ inline int64_t map(int r, bool& ok) const {
    const int l = r % d, g = l >> 4, w = l & 15;
    const int hr = (w < 8) ? 8 * g + w : (d >> 1) + 8 * g + (w - 8);
    const int64_t gr = row0 + (r - l) + hr;
    ok = gr < nrows;
    return ok ? gr : nrows - 1;
  }
};

// Operand loads are raw buffer loads.  Each thread's byte offsets from the
// tile's first row (or k-row) are fixed for the whole K loop, so a load is a
// wave-uniform resource, rebuilt per tile in scalar registers, plus one
// 32-bit VGPR that is never rewritten (no per-tile 64-bit address arithmetic,
// and no address register that must outlive its load).  The resource ends
// where the matrix ends: a read past it returns zeros instead of faulting.
// Out-of-range vectors are zeroed when written to LDS, not when loaded, so no
// wait on the loads is needed until after the MFMAs.
constexpr int BUF_FLAGS = 0x00020000;  // word 3 of a raw buffer resource (gfx9 family)

// Resource from element `off` of an operand to its end (`extent` bytes from
// the operand's start).  The prefetch after the last tile starts past the end
// (left <= 0): its resource is empty, so those loads return zeros and touch no
// memory.  Offsets and extents are multiples of 16 bytes, so a 16-byte load
// is either wholly inside or wholly outside.
__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base, int64_t off,
                                                   int64_t extent) {
  const int64_t left = extent - off * 2;
  const uint32_t n = left <= 0 ? 0u : left > 0xffffffffLL ? 0xffffffffu : (uint32_t)left;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base + off), (short)0, (int)n,
                                           BUF_FLAGS);
}

// Operand stored [row][k] (k contiguous): R rows x 64 k, R*8/NTH vectors of
// 16 B per thread.  The tile's rows are fixed, so their offsets (out-of-range
// rows clamped to the last valid one) are computed once.
template <int R, int NTH>
struct LoadK {
  static constexpr int V = R * 8 / NTH;
  static_assert(NTH % 8 == 0, "a thread keeps one k chunk");
  u32x4 r[V];
  uint32_t off[V];
  uint32_t rok = 0;  // bit i: vector i's row is inside the matrix
  uint32_t ok = 0;   // bit i: vector i of the current tile is inside the matrix
  int64_t row_base = 0;
  template <class Map>
  __device__ inline void init(int64_t ld, const Map& rm, int tid) {
    row_base = rm.row0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int idx = tid + NTH * i;
      bool in;
      const int64_t g = rm.map(idx >> 3, in);
      rok |= (uint32_t)in << i;
      off[i] = (uint32_t)(((g - row_base) * ld + (idx & 7) * 8) * 2);
    }
  }
  __device__ inline void load(const uint16_t* base, int64_t ld, int64_t extent, int64_t k0,
                              int64_t K, int tid) {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(base, row_base * ld + k0, extent);
    ok = (k0 + (tid & 7) * 8 < K) ? rok : 0u;
#pragma unroll
    for (int i = 0; i < V; ++i)
      r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off[i], 0, 0));
  }
  __device__ inline void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int idx = tid + NTH * i;
      *reinterpret_cast<u32x4*>(lds + (idx >> 3) * LDSK + (idx & 7) * 8) =
          ((ok >> i) & 1) ? r[i] : u32x4{0, 0, 0, 0};
    }
  }
};

// Operand stored [k][row] (row contiguous): the 64 (k) x R (row) tile is
// copied unchanged into a k-major LDS tile of pitch PT with 16-byte vectors;
// MFMA fragments are then taken from it with LDS transpose reads (frag_t).
// The pitch is R + 32 elements (64 bytes past a multiple of 256): the four
// k-rows that one transpose read touches fall on disjoint banks.
template <int R, int NTH>
struct LoadKT {
  static constexpr int PT = R + 32;
  static constexpr int VPR = R / 8;          // 16-byte vectors per k-row
  static constexpr int V = 64 * VPR / NTH;   // vectors per thread
  static constexpr int LDS_ELEMS = 64 * PT;
  static_assert(NTH % VPR == 0, "a thread keeps one row chunk");
  u32x4 r[V];
  uint32_t off[V];
  bool rin = false;  // this thread's 8 rows are inside the matrix (nrows is a multiple of 8)
  uint32_t ok = 0;
  int64_t row0 = 0;
  __device__ inline void init(int64_t ld, int64_t row0_, int64_t nrows, int tid) {
    row0 = row0_;
    rin = row0 + (tid % VPR) * 8 < nrows;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int idx = tid + NTH * i;
      off[i] = (uint32_t)(((int64_t)(idx / VPR) * ld + (idx % VPR) * 8) * 2);
    }
  }
  __device__ inline void load(const uint16_t* base, int64_t ld, int64_t extent, int64_t k0,
                              int64_t K, int tid) {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(base, k0 * ld + row0, extent);
    ok = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      ok |= (uint32_t)(rin && k0 + (tid + NTH * i) / VPR < K) << i;
      r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off[i], 0, 0));
    }
  }
  __device__ inline void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int idx = tid + NTH * i;
      *reinterpret_cast<u32x4*>(lds + (idx / VPR) * PT + (idx % VPR) * 8) =
          ((ok >> i) & 1) ? r[i] : u32x4{0, 0, 0, 0};
    }
  }
};

// MFMA fragment (rows row_base..+31, k-step ks) from a k-major LDS tile.  One
// ds_read_b64_tr_b16 over a 16-lane group returns, to lane i, element i%4 of
// the 8-byte chunks addressed by lanes i/4, i/4+4, i/4+8, i/4+12.  Lane s of
// the group addresses k-row kb + s/4 at row offset r0 + 4*(s%4), so lane i
// receives row r0 + i at k-rows kb..kb+3; a second read at kb+4 completes the
// eight k values of the 32x32x16 operand layout (row = lane%32,
// k = 8*(lane/32) + 0..7).
__device__ inline bf16x8_t frag_t(const uint16_t* lds, int pitch, int row_base, int ks,
                                  int lane) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4 lds_s4;
  const int g = lane >> 4, sl = lane & 15;
  const int k = ks * 16 + 8 * (g >> 1) + (sl >> 2);
  const int row = row_base + 16 * (g & 1) + 4 * (sl & 3);
  const uint16_t* q = lds + k * pitch + row;
  const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)q);
  const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(q + 4 * pitch));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8_t, u32x4{a[0], a[1], b[0], b[1]});
}

__device__ inline float silu_f(float a) { return a / (1.0f + expf(-a)); }

// Tile order.  Workgroup i of a launch goes to XCD i % 8 and each XCD has its
// own L2, so the linear id is first regrouped per XCD (XCD x gets the x-th
// contiguous share of the tile list), and inside a share tiles run down
// groups of GROUP_M row tiles before moving to the next column tile, so the
// workgroups an XCD runs at once cover a compact block of tiles and share
// their A row-panels and B column-panels in that XCD's L2.
constexpr int NXCD = 8, GROUP_M = 8;

__device__ inline bool tile_of(int bid, int nm, int nn, int& tm, int& tn) {
  const int total = nm * nn;
  const int per = (total + NXCD - 1) / NXCD;
  const int t = (bid % NXCD) * per + bid / NXCD;
  if (t >= total) return false;
  const int group = t / (GROUP_M * nn);
  const int first = group * GROUP_M;
  const int gsize = min(GROUP_M, nm - first);
  const int r = t - group * GROUP_M * nn;
  tm = first + r % gsize;
  tn = r / gsize;
  return true;
}

// Epilogue of a BM x BN tile: acc[i][j][r] is C[row, col] with
// row = 8*(r/4) + 4*(lane/32) + r%4 and col = lane%32 inside the 32x32
// sub-tile (i, j).  tb: this wave's 32 x EPI_TP floats of LDS scratch.
constexpr int EPI_TP = 40;  // floats per LDS row: lanes l and l+32 write disjoint banks

template <int EPI, int BM, int BN, int WVM, int WVN>
__device__ __forceinline__ void store_tile(const mt_gemm_args& p,
                                           f32x16_t (&acc)[BM / WVM / 32][BN / WVN / 32],
                                           int64_t m0, int64_t n0, int wm, int wn, int lane,
                                           float* tb) {
  constexpr bool SWI = (EPI == MT_EPI_SWIGLU);
  constexpr int WM = BM / WVM, WN = BN / WVN, TM = WM / 32, TN = WN / 32;
  constexpr int TP = EPI_TP;
  const int g4 = (lane >> 5) * 4;
  // The block is private to the wave, and LDS executes one wave's accesses in
  // issue order, so a compiler-only barrier is enough between its writes and
  // the reads of other lanes' values.  (A memory fence would also wait for
  // the wave's outstanding global stores.)
  auto lds_order = []() {
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
  };
  auto turn = [&](const f32x16_t& v, float (&out)[16]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) tb[(8 * (r >> 2) + g4 + (r & 3)) * TP + (lane & 31)] = v[r];
    lds_order();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 x = *reinterpret_cast<const float4*>(tb + (lane >> 1) * TP + (lane & 1) * 16 + 4 * q);
      out[4 * q + 0] = x.x; out[4 * q + 1] = x.y; out[4 * q + 2] = x.z; out[4 * q + 3] = x.w;
    }
    lds_order();
  };
  auto pack8 = [](const float* v) {
    return u32x4{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]),
                 pack_bf2(v[6], v[7])};
  };
  auto unpack8 = [](const u32x4 w, float* v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf2f((uint16_t)(w[e] & 0xffffu));
      v[2 * e + 1] = bf2f((uint16_t)(w[e] >> 16));
    }
  };
  if constexpr (SWI) {
    uint16_t* C = static_cast<uint16_t*>(p.C);
#pragma unroll
    for (int j = 0; j < TN / 2; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        float a[16], u[16];
        turn(acc[i][j], a);
        turn(acc[i][j + TN / 2], u);
        const int64_t row = m0 + wm * WM + i * 32 + (lane >> 1);
        const int64_t f0 = n0 + wn * (WN / 2) + j * 32 + (lane & 1) * 16;
        if (row >= p.M) continue;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int64_t f = f0 + 8 * h;
          if (f >= p.N) continue;
          float y[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = silu_f(a[8 * h + e]) * u[8 * h + e];
          *reinterpret_cast<u32x4*>(p.gu + row * p.ldgu + f) = pack8(a + 8 * h);
          *reinterpret_cast<u32x4*>(p.gu + row * p.ldgu + p.ffn + f) = pack8(u + 8 * h);
          *reinterpret_cast<u32x4*>(C + row * p.ldc + f) = pack8(y);
        }
      }
  } else {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        float v[16];
        turn(acc[i][j], v);
        const int64_t row = m0 + wm * WM + i * 32 + (lane >> 1);
        const int64_t c0 = n0 + wn * WN + j * 32 + (lane & 1) * 16;
        if (row >= p.M) continue;
        const bool in[2] = {c0 < p.N, c0 + 8 < p.N};
        // every load of the sub-tile is issued before its first store, so the
        // loads overlap (C may alias R, which forbids moving a load past a store)
        if constexpr (EPI == MT_EPI_BF16) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
            if (in[h])
              *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.C) + row * p.ldc + c0 + 8 * h) =
                  pack8(v + 8 * h);
        } else if constexpr (EPI == MT_EPI_ROPE) {
          // v[0..7] and v[8..15] are head columns i0.. and d/2 + i0.. (RopeRowMap);
          // N is a multiple of d, so the 16 columns are all inside or all outside
          if (!in[0]) continue;
          const int hd = p.rope_dim >> 1;
          const int64_t l = c0 % p.rope_dim;
          const int i0 = (int)(l >> 1);
          uint16_t* C = static_cast<uint16_t*>(p.C) + row * p.ldc + (c0 - l) + i0;
          if (c0 < p.rope_cols) {
            const int64_t t = (int64_t)(row % p.rope_seq) * hd + i0;
            const float4 c4[2] = {*reinterpret_cast<const float4*>(p.rope_cos + t),
                                  *reinterpret_cast<const float4*>(p.rope_cos + t + 4)};
            const float4 s4[2] = {*reinterpret_cast<const float4*>(p.rope_sin + t),
                                  *reinterpret_cast<const float4*>(p.rope_sin + t + 4)};
            const float cs[8] = {c4[0].x, c4[0].y, c4[0].z, c4[0].w, c4[1].x, c4[1].y, c4[1].z, c4[1].w};
            const float sn[8] = {s4[0].x, s4[0].y, s4[0].z, s4[0].w, s4[1].x, s4[1].y, s4[1].z, s4[1].w};
            float a[8], b[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              a[e] = v[e] * cs[e] - v[8 + e] * sn[e];
              b[e] = v[8 + e] * cs[e] + v[e] * sn[e];
            }
            *reinterpret_cast<u32x4*>(C) = pack8(a);
            *reinterpret_cast<u32x4*>(C + hd) = pack8(b);
          } else {
            *reinterpret_cast<u32x4*>(C) = pack8(v);
            *reinterpret_cast<u32x4*>(C + hd) = pack8(v + 8);
          }
        } else if constexpr (EPI == MT_EPI_SWIGLU_BWD) {
          u32x4 ga[2], gu_[2];
#pragma unroll
          for (int h = 0; h < 2; ++h)
            if (in[h]) {
              ga[h] = *reinterpret_cast<const u32x4*>(p.gu + row * p.ldgu + c0 + 8 * h);
              gu_[h] = *reinterpret_cast<const u32x4*>(p.gu + row * p.ldgu + p.ffn + c0 + 8 * h);
            }
          uint16_t* C = static_cast<uint16_t*>(p.C);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            if (!in[h]) continue;
            float a[8], u[8], d0[8], d1[8];
            unpack8(ga[h], a);
            unpack8(gu_[h], u);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float x = v[8 * h + e];
              const float sg = 1.0f / (1.0f + expf(-a[e]));
              d0[e] = x * u[e] * sg * (1.0f + a[e] * (1.0f - sg));
              d1[e] = x * a[e] * sg;
            }
            *reinterpret_cast<u32x4*>(C + row * p.ldc + c0 + 8 * h) = pack8(d0);
            *reinterpret_cast<u32x4*>(C + row * p.ldc + p.ffn + c0 + 8 * h) = pack8(d1);
          }
        } else {
          float* C = static_cast<float*>(p.C) + row * p.ldc + c0;
          float4 add[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            add[q] = make_float4(0.f, 0.f, 0.f, 0.f);
            if constexpr (EPI == MT_EPI_F32_RESID) {
              if (in[q >> 1]) add[q] = *reinterpret_cast<const float4*>(p.R + row * p.ldr + c0 + 4 * q);
            } else if constexpr (EPI == MT_EPI_F32_ACCUM) {
              if (in[q >> 1]) add[q] = *reinterpret_cast<const float4*>(C + 4 * q);
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (in[q >> 1])
              *reinterpret_cast<float4*>(C + 4 * q) =
                  make_float4(v[4 * q] + add[q].x, v[4 * q + 1] + add[q].y, v[4 * q + 2] + add[q].z,
                              v[4 * q + 3] + add[q].w);
        }
      }
  }
}

// BM x BN output tile per workgroup; each of the 4 waves owns a
// (BM/2) x (BN/2) quadrant = TM x TN tiles of 32 x 32.  Larger tiles issue
// fewer LDS fragment reads per MFMA (TM + TN reads feed TM * TN MFMAs).
template <int LAYOUT, int EPI, int BM, int BN, int WVM, int WVN>
__global__ __launch_bounds__(64 * WVM * WVN) void gemm_kernel(mt_gemm_args p, int nm, int nn) {
  constexpr int NTH = 64 * WVM * WVN;  // WVM x WVN waves, each a (BM/WVM) x (BN/WVN) block
  constexpr bool A_T = (LAYOUT == MT_GEMM_TN);
  constexpr bool B_T = (LAYOUT != MT_GEMM_NT);
  constexpr bool SWI = (EPI == MT_EPI_SWIGLU);
  static_assert(!(SWI && B_T), "the SwiGLU product takes B as [rows][k]");
  constexpr int WM = BM / WVM, WN = BN / WVN, TM = WM / 32, TN = WN / 32;
  static_assert(TM >= 1 && TN >= 1 && (!SWI || TN % 2 == 0), "wave block too small");
  constexpr int HALF = BN / 2;  // SwiGLU: gate rows, then up rows
  constexpr int SA = A_T ? LoadKT<BM, NTH>::LDS_ELEMS : BM * LDSK;
  constexpr int SB = B_T ? LoadKT<BN, NTH>::LDS_ELEMS : BN * LDSK;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][SA];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][SB];

  int tm, tn;
  if (!tile_of(blockIdx.x, nm, nn, tm, tn)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WVN, wn = wave % WVN;
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * (SWI ? HALF : BN);
  const int64_t K = p.K;
  const uint16_t* A = p.A;
  const uint16_t* B = p.B;

  RowMap<BM, false> ra{m0, p.M, 0};
  RowMap<HALF, SWI> rb{n0, p.N, SWI ? p.ffn : 0};

  typename std::conditional<A_T, LoadKT<BM, NTH>, LoadK<BM, NTH>>::type la;
  typename std::conditional<B_T, LoadKT<BN, NTH>, LoadK<BN, NTH>>::type lb;
  if constexpr (A_T) la.init(p.lda, m0, p.M, tid);
  else la.init(p.lda, ra, tid);
  if constexpr (B_T) lb.init(p.ldb, n0, p.N, tid);
  else if constexpr (EPI == MT_EPI_ROPE) lb.init(p.ldb, RopeRowMap{n0, p.N, p.rope_dim}, tid);
  else lb.init(p.ldb, rb, tid);
  // bytes from each operand's start to the end of its last row
  const int64_t ext_a = A_T ? ((K - 1) * p.lda + p.M) * 2 : ((p.M - 1) * p.lda + K) * 2;
  const int64_t ext_b = B_T ? ((K - 1) * p.ldb + p.N) * 2
                            : (((SWI ? p.ffn : 0) + p.N - 1) * p.ldb + K) * 2;

  auto load_tiles = [&](int64_t k0) {
    la.load(A, p.lda, ext_a, k0, K, tid);
    lb.load(B, p.ldb, ext_b, k0, K, tid);
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (int)((K + BK - 1) / BK);
  load_tiles(0);
  la.store(As[0], tid);
  lb.store(Bs[0], tid);
  __syncthreads();

  // LDS row of the wave's j-th B sub-tile: plain tiles are contiguous; in the
  // SwiGLU product sub-tiles 0..TN/2-1 are gate columns and TN/2.. the
  // matching up columns.
  auto brow = [&](int j) {
    if constexpr (SWI)
      return (j < TN / 2) ? wn * (WN / 2) + j * 32 : HALF + wn * (WN / 2) + (j - TN / 2) * 32;
    else
      return wn * WN + j * 32;
  };
  const int arow = wm * WM + (lane & 31);
  const int kofs = (lane >> 5) * 8;

  // MFMA operands are double-buffered in registers: the fragments of k-step
  // s+1 are read from LDS while the MFMAs of k-step s run.  The last k-step
  // of a tile runs after the barrier, under the reads of the next tile's
  // first fragments, so the matrix cores never wait on LDS at a tile edge.
  bf16x8_t fa[2][TM], fb[2][TN];
  auto read_frags = [&](const uint16_t* as, const uint16_t* bs, int ks, int slot) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if constexpr (A_T)
        fa[slot][i] = frag_t(as, LoadKT<BM, NTH>::PT, wm * WM + i * 32, ks, lane);
      else
        fa[slot][i] = frag(as + (arow + i * 32) * LDSK + ks * 16 + kofs);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if constexpr (B_T)
        fb[slot][j] = frag_t(bs, LoadKT<BN, NTH>::PT, wn * WN + j * 32, ks, lane);
      else
        fb[slot][j] = frag(bs + (brow(j) + (lane & 31)) * LDSK + ks * 16 + kofs);
    }
  };
  auto mfmas = [&](int slot) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j], acc[i][j], 0,
                                                            0, 0);
  };
  // Within a k-step the next k-step's fragment reads are interleaved with
  // this k-step's MFMAs (one MFMA, then RPM reads), so the LDS reads are
  // spread over the matrix work instead of bunched just ahead of the MFMAs
  // that use them (group masks: 0x008 MFMA, 0x100 LDS read).  Spreading them
  // over all of the k-step rather than its first half keeps every 256 x 256
  // instance at most 248 VGPRs: two waves per SIMD then still leave room for
  // a wave of the gradient-drain copy kernel, so a GEMM workgroup can still
  // start on a CU that the drain occupies (at 256 VGPRs a 256-tile product
  // lost those CUs and ran a second round).
  constexpr int NREAD = (A_T ? 2 : 1) * TM + (B_T ? 2 : 1) * TN;
  constexpr int RPM = (NREAD + TM * TN - 1) / (TM * TN);
  auto interleave = [&]() {
#pragma unroll
    for (int j = 0; j < TM * TN; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
    }
  };
  constexpr int KS = BK / 16;  // k-steps per tile (even, so slots alternate 0,1,0,1)
  static_assert(KS % 2 == 0, "k-steps per tile must be even");

  // The loop body has no branches, so that each half of it is one scheduling
  // region (in the last iteration the loads fall past K; every vector is
  // masked, so zeros go to the idle LDS buffer and are never read).
  // Scheduling barriers keep the next tile's global loads ahead of the MFMAs,
  // where three k-steps hide their latency, and the LDS stores after them.
  read_frags(As[0], Bs[0], 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    load_tiles((int64_t)(kt + 1) * BK);
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* as = As[cur];
    const uint16_t* bs = Bs[cur];
#pragma unroll
    //
    // Each k-step's MFMA block runs at raised wave priority: of the two waves
    // sharing a SIMD, the one inside its matrix block keeps issuing, while the
    // other's global loads, LDS stores and barrier run in its gaps (1.6 %
    // faster over the block products of the 7B shape; same results).
    for (int ks = 0; ks < KS - 1; ++ks) {
      __builtin_amdgcn_s_setprio(1);
      read_frags(as, bs, ks + 1, (ks + 1) & 1);
      mfmas(ks & 1);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
    }
    la.store(As[cur ^ 1], tid);
    lb.store(Bs[cur ^ 1], tid);
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);
    read_frags(As[cur ^ 1], Bs[cur ^ 1], 0, 0);
    mfmas((KS - 1) & 1);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  }

  // ------------------------------------------------------------ epilogue
  // acc[i][j][r] is C[row, col] with row = 8*(r/4) + 4*(lane/32) + r%4 and
  // col = lane%32 inside the 32x32 sub-tile (i, j): one column per lane.  Each
  // sub-tile is turned around through a wave-private LDS block so that a lane
  // holds 16 consecutive columns of one row (row = lane/2, columns
  // 16*(lane%2)..+15), and every global access of the epilogue is a 16-byte
  // vector (N and the leading dimensions are multiples of 8, so each 8-column
  // half is wholly inside or outside the matrix).
  __syncthreads();  // the K loop's last fragment reads are done in every wave
  static_assert(NTH / 64 * 32 * EPI_TP * 4 <= (int)sizeof(As), "epilogue scratch");
  store_tile<EPI, BM, BN, WVM, WVN>(p, acc, m0, n0, wm, wn, lane,
                                    reinterpret_cast<float*>(&As[0][0]) + (tid >> 6) * 32 * EPI_TP);
}

// ------------------------------------------------- direct-to-LDS variant
// The 256 x 256 tile when K is a multiple of 128 (every product of the model
// shapes).  Operand tiles go from global memory straight into LDS with
// buffer_load_dwordx4 ... lds: no VGPR staging and no ds_write, which in
// timing probes of the register-staged kernel cost about a third of its time.
// One such load moves 64 lanes x 16 bytes into 1 KB of LDS in lane order, so
// the LDS tiles are unpadded and conflict-free fragment reads come from an
// XOR swizzle of 16-byte chunks chosen on the global side.  The two stages
// are separate LDS arrays and the K loop is unrolled by two, so that the
// compiler can tell a DMA into one stage from fragment reads of the other.
typedef __attribute__((address_space(3))) void lds_void;

__device__ inline void dma16(__amdgpu_buffer_rsrc_t rs, uint16_t* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, voff, 0, 0, 0);
}

// [row][k] operand, R rows x 64 k: LDS row r holds its eight 16-byte k
// chunks with chunk c at slot c ^ ((r >> 1) & 7).  Load i of wave w fills
// rows 8 (w V + i) .. +7; lane l writes row 8 (w V + i) + l/8, slot l%8.
template <int R, int NTH>
struct DLoadK {
  static constexpr int V = R * 8 / NTH;  // loads per wave and tile
  uint32_t off[V];
  int64_t row_base = 0;
  template <class Map>
  __device__ inline void init(int64_t ld, const Map& rm, int wave, int lane) {
    row_base = rm.row0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int r = 8 * (wave * V + i) + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      bool in;
      const int64_t g = rm.map(r, in);  // out-of-range rows read a valid row; their results are not stored
      off[i] = (uint32_t)(((g - row_base) * ld + c * 8) * 2);
    }
  }
  __device__ inline void load(const uint16_t* base, int64_t ld, int64_t extent, int64_t k0,
                              uint16_t* lds, int wave) const {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(base, row_base * ld + k0, extent);
#pragma unroll
    for (int i = 0; i < V; ++i) dma16(rs, lds + (wave * V + i) * 512, off[i]);
  }
};

// [k][row] operand, 64 k x R rows (R = 256: two k-rows per load): LDS k-row
// k holds its R/8 row chunks with chunk c at slot c ^ (4 (k & 3)).  Half a
// wave's transpose read touches four k-rows (k & 3 = 0..3, same bank offset:
// a k-row is 512 bytes) times four consecutive chunks (c & 3 = 0..3), and
// the swizzle sends these 16 chunks to 16 distinct 16-byte bank groups.
template <int R, int NTH>
struct DLoadKT {
  static constexpr int VPR = R / 8;            // chunks per k-row
  static constexpr int V = 64 * VPR / NTH;     // loads per wave and tile
  static_assert(512 % R == 0 && 64 % VPR == 0 && VPR >= 16, "whole k-rows per load");
  uint32_t off[V];
  int64_t row0 = 0;
  __device__ inline void init(int64_t ld, int64_t row0_, int wave, int lane) {
    row0 = row0_;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = 64 * (wave * V + i) + lane;  // chunk index in the tile
      const int k = e / VPR;
      const int c = (e % VPR) ^ (4 * (k & 3));
      off[i] = (uint32_t)(((int64_t)k * ld + c * 8) * 2);
    }
  }
  __device__ inline void load(const uint16_t* base, int64_t ld, int64_t extent, int64_t k0,
                              uint16_t* lds, int wave) const {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(base, k0 * ld + row0, extent);
#pragma unroll
    for (int i = 0; i < V; ++i) dma16(rs, lds + (wave * V + i) * 512, off[i]);
  }
};

// MFMA fragment (rows row..row+31 over the lanes, k-step ks) of a swizzled
// [row][64] tile.
__device__ inline bf16x8_t frag_sw(const uint16_t* lds, int row, int ks, int lane) {
  const int kc = ks * 2 + (lane >> 5);
  return frag(lds + row * 64 + ((kc ^ ((row >> 1) & 7)) << 3));
}

// As frag_t, from a swizzled [64][R] tile.
template <int R>
__device__ inline bf16x8_t frag_tsw(const uint16_t* lds, int row_base, int ks, int lane) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4 lds_s4;
  const int g = lane >> 4, sl = lane & 15;
  const int k = ks * 16 + 8 * (g >> 1) + (sl >> 2);
  const int row = row_base + 16 * (g & 1) + 4 * (sl & 3);
  const uint16_t* q = lds + k * R + ((((row >> 3) ^ (4 * (k & 3))) << 3) | (row & 7));
  const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)q);
  const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(q + 4 * R));  // k + 4: same swizzle
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8_t, u32x4{a[0], a[1], b[0], b[1]});
}

template <int LAYOUT, int EPI>
__global__ __launch_bounds__(512) void gemm_direct_kernel(mt_gemm_args pa, int nm, int nn) {
  constexpr int BM = 256, BN = 256, WVM = 2, WVN = 4, NTH = 512;
  mt_gemm_args p = pa;
  constexpr bool A_T = (LAYOUT == MT_GEMM_TN);
  constexpr bool B_T = (LAYOUT != MT_GEMM_NT);
  constexpr bool SWI = (EPI == MT_EPI_SWIGLU);
  static_assert(!(SWI && B_T), "the SwiGLU product takes B as [rows][k]");
  constexpr int WM = BM / WVM, WN = BN / WVN, TM = WM / 32, TN = WN / 32;
  constexpr int HALF = BN / 2;
  constexpr int TILE = 256 * 64;  // elements of one operand tile
  __shared__ __attribute__((aligned(16))) uint16_t A0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t A1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t B0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t B1[TILE];

  int tm, tn;
  if (!tile_of(blockIdx.x, nm, nn, tm, tn)) return;
  if (p.groups > 0) {
    // grouped product: this workgroup's group and its operands (uniform values)
    if constexpr (LAYOUT == MT_GEMM_TN) {
      const int g = blockIdx.y;
      const int64_t r0 = p.group_off[g], r1 = p.group_off[g + 1];
      p.A += r0 * p.lda;
      p.B += r0 * p.ldb;
      p.K = r1 - r0;
      p.C = static_cast<char*>(p.C) +
            g * p.group_stride_c * (EPI == MT_EPI_BF16 ? 2 : 4);
    } else {
      const int64_t mt0 = (int64_t)tm * BM;
      if (mt0 >= p.group_off[p.groups]) return;  // past the last group's rows
      int g = 0;
      while (g + 1 < p.groups && p.group_off[g + 1] <= mt0) ++g;
      p.B += g * p.group_stride_b;
    }
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WVN, wn = wave % WVN;
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * (SWI ? HALF : BN);
  const int64_t K = p.K;
  const uint16_t* A = p.A;
  const uint16_t* B = p.B;

  RowMap<BM, false> ra{m0, p.M, 0};
  RowMap<HALF, SWI> rb{n0, p.N, SWI ? p.ffn : 0};
  typename std::conditional<A_T, DLoadKT<BM, NTH>, DLoadK<BM, NTH>>::type la;
  typename std::conditional<B_T, DLoadKT<BN, NTH>, DLoadK<BN, NTH>>::type lb;
  if constexpr (A_T) la.init(p.lda, m0, wave, lane);
  else la.init(p.lda, ra, wave, lane);
  if constexpr (B_T) lb.init(p.ldb, n0, wave, lane);
  else if constexpr (EPI == MT_EPI_ROPE) lb.init(p.ldb, RopeRowMap{n0, p.N, p.rope_dim}, wave, lane);
  else lb.init(p.ldb, rb, wave, lane);
  const int64_t ext_a = A_T ? ((K - 1) * p.lda + p.M) * 2 : ((p.M - 1) * p.lda + K) * 2;
  const int64_t ext_b = B_T ? ((K - 1) * p.ldb + p.N) * 2
                            : (((SWI ? p.ffn : 0) + p.N - 1) * p.ldb + K) * 2;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto brow = [&](int j) {
    if constexpr (SWI)
      return (j < TN / 2) ? wn * (WN / 2) + j * 32 : HALF + wn * (WN / 2) + (j - TN / 2) * 32;
    else
      return wn * WN + j * 32;
  };
  const int arow = wm * WM + (lane & 31);

  bf16x8_t fa[2][TM], fb[2][TN];
  auto read_frags = [&](const uint16_t* as, const uint16_t* bs, int ks, int slot) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if constexpr (A_T)
        fa[slot][i] = frag_tsw<BM>(as, wm * WM + i * 32, ks, lane);
      else
        fa[slot][i] = frag_sw(as, arow + i * 32, ks, lane);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if constexpr (B_T)
        fb[slot][j] = frag_tsw<BN>(bs, wn * WN + j * 32, ks, lane);
      else
        fb[slot][j] = frag_sw(bs, brow(j) + (lane & 31), ks, lane);
    }
  };
  auto mfmas = [&](int slot) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j], acc[i][j], 0,
                                                            0, 0);
  };
  constexpr int NREAD = (A_T ? 2 : 1) * TM + (B_T ? 2 : 1) * TN;
  constexpr int RPM = (NREAD + TM * TN - 1) / (TM * TN);
  auto interleave = [&]() {
#pragma unroll
    for (int j = 0; j < TM * TN; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
    }
  };
  constexpr int KS = BK / 16;
  // this wave's loads into LDS are complete (the barrier then covers every wave's)
  auto wait_dma = []() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // One tile: the k-steps of the tile in (ca, cb) while the next tile's loads
  // fill (na, nb); the last k-step runs after the barrier, under the reads of
  // the next tile's first fragments (as in gemm_kernel).
  auto tile = [&](const uint16_t* ca, const uint16_t* cb, uint16_t* na, uint16_t* nb,
                  int64_t knext) {
    la.load(A, p.lda, ext_a, knext, na, wave);
    lb.load(B, p.ldb, ext_b, knext, nb, wave);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) {
      __builtin_amdgcn_s_setprio(1);
      read_frags(ca, cb, ks + 1, (ks + 1) & 1);
      mfmas(ks & 1);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
    }
    wait_dma();
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);
    read_frags(na, nb, 0, 0);
    mfmas((KS - 1) & 1);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };

  const int nk = (int)(K / BK);  // even: K is a multiple of 128
  la.load(A, p.lda, ext_a, 0, A0, wave);
  lb.load(B, p.ldb, ext_b, 0, B0, wave);
  wait_dma();
  __syncthreads();
  read_frags(A0, B0, 0, 0);
  for (int kt = 0; kt < nk; kt += 2) {
    tile(A0, B0, A1, B1, (int64_t)(kt + 1) * BK);
    tile(A1, B1, A0, B0, (int64_t)(kt + 2) * BK);  // past the end: empty resource, zeros
  }

  __syncthreads();  // the K loop's last fragment reads are done in every wave
  // 8 waves x 32 x EPI_TP floats of scratch: waves 0..5 in A0, 6..7 in B0
  static_assert(6 * 32 * EPI_TP * 4 <= (int)sizeof(A0) && 2 * 32 * EPI_TP * 4 <= (int)sizeof(B0),
                "epilogue scratch");
  float* tb = wave < 6 ? reinterpret_cast<float*>(A0) + wave * 32 * EPI_TP
                       : reinterpret_cast<float*>(B0) + (wave - 6) * 32 * EPI_TP;
  store_tile<EPI, BM, BN, WVM, WVN>(p, acc, m0, n0, wm, wn, lane, tb);
}

template <int LAYOUT, int EPI, int BM, int BN, int WVM, int WVN>
hipError_t launch_tiles(const mt_gemm_args& a, hipStream_t s) {
  const int nn = (int)((EPI == MT_EPI_SWIGLU) ? (a.N + BN / 2 - 1) / (BN / 2) : (a.N + BN - 1) / BN);
  const int nm = (int)((a.M + BM - 1) / BM);
  const int per = (nm * nn + NXCD - 1) / NXCD;
  hipLaunchKernelGGL((gemm_kernel<LAYOUT, EPI, BM, BN, WVM, WVN>), dim3((unsigned)(per * NXCD)),
                     dim3(64 * WVM * WVN), 0, s, a, nm, nn);
  return hipGetLastError();
}

// 256 x 256 tiles (8 waves of 128 x 64: two waves per SIMD) when the product
// has enough of them to fill the chip, 128 x 128 (4 waves) otherwise.
template <int LAYOUT, int EPI>
hipError_t launch_direct(const mt_gemm_args& a, hipStream_t s) {
  const int nn = (int)((EPI == MT_EPI_SWIGLU) ? (a.N + 127) / 128 : (a.N + 255) / 256);
  const int nm = (int)((a.M + 255) / 256);
  const int per = (nm * nn + NXCD - 1) / NXCD;
  // grouped weight-gradient products: one grid row of tiles per group
  const unsigned gy = (a.groups > 0 && LAYOUT == MT_GEMM_TN) ? (unsigned)a.groups : 1u;
  hipLaunchKernelGGL((gemm_direct_kernel<LAYOUT, EPI>), dim3((unsigned)(per * NXCD), gy), dim3(512),
                     0, s, a, nm, nn);
  return hipGetLastError();
}

template <int LAYOUT, int EPI>
hipError_t launch_one(const mt_gemm_args& a, hipStream_t s) {
  if (a.groups > 0) return launch_direct<LAYOUT, EPI>(a, s);  // shapes checked by gemm_shape_ok
  const int64_t nbig = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  if (a.M >= 1024 && a.N >= 1024 && nbig >= 128) {
    // the direct loads move 16-byte chunks: operand bases must be 16-byte aligned
    if (a.K % 128 == 0 && (((uintptr_t)a.A | (uintptr_t)a.B) & 15) == 0)
      return launch_direct<LAYOUT, EPI>(a, s);
    return launch_tiles<LAYOUT, EPI, 256, 256, 2, 4>(a, s);
  }
  return launch_tiles<LAYOUT, EPI, 128, 128, 2, 2>(a, s);
}

}  // namespace

bool gemm_shape_ok(const mt_gemm_args& a, const char** why) {
  auto bad = [&](const char* w) { if (why) *why = w; return false; };
  if (a.layout < 0 || a.layout > 2) return bad("layout");
  if (a.epilogue < 0 || a.epilogue > 6) return bad("epilogue");
  if (a.M <= 0 || a.N <= 0 || a.K <= 0) return bad("empty or negative dimension");
  if (a.M % 8 || a.N % 8 || a.K % 8) return bad("M, N, K must be multiples of 8");
  if ((a.M / 128 + 1) * (a.N / 64 + 1) >= (1LL << 31)) return bad("too many tiles");
  if (!a.A || !a.B || !a.C) return bad("null operand");
  if (a.lda % 8 || a.ldb % 8) return bad("lda/ldb must be multiples of 8");
  if (a.ldc % 8 || a.ldr % 4 || a.ldgu % 8) return bad("ldc, ldgu must be multiples of 8, ldr of 4");
  if (((uintptr_t)a.C | (uintptr_t)a.R | (uintptr_t)a.gu) & 15)
    return bad("C, R and gu must be 16-byte aligned");
  const bool at = a.layout == MT_GEMM_TN, bt = a.layout != MT_GEMM_NT;
  if ((at ? a.lda < a.M : a.lda < a.K) || (bt ? a.ldb < a.N : a.ldb < a.K)) return bad("lda/ldb");
  if (a.groups != 0) {
    // grouped products run on the direct-to-LDS kernel: 16-byte aligned
    // operands, per-group row blocks of 256, k steps of 128
    if (a.groups < 0 || a.groups > 64 || !a.group_off) return bad("groups / group_off");
    if (((uintptr_t)a.A | (uintptr_t)a.B) & 15) return bad("grouped operands must be 16-byte aligned");
    if (a.layout == MT_GEMM_TN) {
      if (a.K % 256) return bad("grouped TN: K (row space) must be a multiple of 256");
      if (a.epilogue != MT_EPI_BF16 && a.epilogue != MT_EPI_F32)
        return bad("grouped TN: BF16 or F32 epilogue");
      if (a.group_stride_c < a.M * a.ldc) return bad("group_stride_c");
    } else {
      if (a.M % 256 || a.K % 128) return bad("grouped NT/NN: M multiple of 256, K of 128");
      if (a.epilogue == MT_EPI_F32_RESID || a.epilogue == MT_EPI_F32_ACCUM ||
          a.epilogue == MT_EPI_ROPE)
        return bad("grouped NT/NN: BF16, F32 or SwiGLU epilogues");
      if (a.group_stride_b <= 0) return bad("group_stride_b");
    }
  }
  if (a.epilogue == MT_EPI_SWIGLU) {
    if (a.layout != MT_GEMM_NT) return bad("SWIGLU needs the NT layout");
    if (a.ffn != a.N || !a.gu || a.ldgu < 2 * a.ffn || a.ldc < a.N) return bad("SWIGLU args");
  } else if (a.epilogue == MT_EPI_SWIGLU_BWD) {
    if (a.layout != MT_GEMM_NN) return bad("SWIGLU_BWD needs the NN layout");
    if (a.ffn != a.N || !a.gu || a.ldgu < 2 * a.ffn || a.ldc < 2 * a.ffn) return bad("SWIGLU_BWD args");
  } else {
    if (a.ldc < a.N) return bad("ldc");
    if (a.epilogue == MT_EPI_F32_RESID && (!a.R || a.ldr < a.N)) return bad("residual");
    if (a.epilogue == MT_EPI_ROPE) {
      if (a.layout != MT_GEMM_NT) return bad("ROPE needs the NT layout");
      const int d = a.rope_dim;
      if (!(d == 16 || d == 32 || d == 64 || d == 128)) return bad("rope_dim");
      if (!a.rope_cos || !a.rope_sin || a.rope_seq < 1) return bad("rope tables");
      if ((((uintptr_t)a.rope_cos | (uintptr_t)a.rope_sin) & 15)) return bad("rope table alignment");
      if (a.N % d || a.rope_cols % d || a.rope_cols < 0 || a.rope_cols > a.N) return bad("rope_cols");
    }
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
  MT_GEMM_CASE(MT_GEMM_NT, MT_EPI_ROPE)
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
