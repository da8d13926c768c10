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
// operand: element e of a lane's 8-value fragment for k-step hh of a 32-row
// tile is row 16*hh + 8*(e/4) + 4*(lane/32) + e%4 -- a permutation of the 16
// reduction indices that the A operand (read from a transposed LDS tile with
// two 8-byte reads) follows exactly, so the sum is unchanged.
//
// Tiles of 32 rows go from global memory straight into padded LDS stages
// (buffer_load ... lds), loaded two or three tiles ahead with partial waits
// and fence-free barriers; the grid runs the heaviest blocks first, each
// head's workgroups on one XCD.
//
// Backward is deterministic, with no floating-point atomics: D = rowsum(dO*O)
// and lse log2(e) per query (attn_dsum_kernel); dK and dV together in one
// launch with the key block outer (one workgroup per head, or with grouped
// heads one per query head writing fp32 shares that attn_gqa_reduce_kernel
// adds in query-head order); dQ with the query block outer.  Given RoPE
// tables, dQ and dK leave the kernels rotated back to the pre-rotation q and
// k in fp32, so each is rounded to bf16 once.
#include "common.h"

namespace mt {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
// Word 3 of a raw (unformatted, unswizzled) buffer resource on gfx9-family
// parts: 32-bit data format, no index stride.
constexpr int BUF_FLAGS = 0x00020000;
// log2 headroom of the forward's lazily updated running maximum
constexpr float RESCALE_SLACK = 8.0f;

__device__ inline bf16x8_t as_frag(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ inline bf16x8_t ld_frag(const uint16_t* p) {
  return as_frag(*reinterpret_cast<const u32x4*>(p));
}
// 2^x on the hardware exponential unit.  Arguments here are max-subtracted
// (<= 0) logits; results that would be denormal are negligible against the
// row sum, so the library's denormal-range scaling is not needed.
__device__ inline float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ inline void zero(f32x16_t& a) {
#pragma unroll
  for (int r = 0; r < 16; ++r) a[r] = 0.0f;
}

// Makes a value loaded before a loop count as used right here, so its load is
// waited for once, ahead of the loop.  Otherwise the compiler sinks such loads
// to the loop entry, and the wait counter, merged over the back edge, then has
// every iteration wait for the next tile's prefetch as well.
template <class T>
__device__ inline void settle(const T& v) {
  asm volatile("" ::"v"(v));
}

// LDS tiles are [ROWS][D] row-major copies of global rows (pitch PITCH
// elements), read two ways: 16-byte row reads (MFMA operand with rows = tile
// rows, k = d) and transpose reads (operand with rows = d, k = tile rows).
// PITCH = 152 elements = 304 bytes = 48 mod 256: the 16 rows of a row read hit
// distinct 16-byte bank slots, and the four tile rows of one transpose read
// (32 bytes each, two 16-lane groups side by side) fall on disjoint banks.
constexpr int PITCH = 152;

// Global -> registers -> LDS copy of one [ROWS][D] tile by 256 threads, split
// so that the global loads can be issued a tile ahead of the LDS stores.  The
// loads are buffer loads: a wave-uniform resource for the tile plus a 32-bit
// per-lane byte offset fixed for the whole kernel, so no address register is
// rewritten while a load is in flight and there is no per-tile 64-bit address
// arithmetic.
template <int ROWS, int D>
struct TileCopy {
  static constexpr int VPR = D / 8;                // 16-byte vectors per row
  static constexpr int V = ROWS * VPR / 256;       // vectors per thread
  static_assert(V >= 1 && ROWS * VPR % 256 == 0, "tile does not split over 256 threads");
  u32x4 r[V];
  uint32_t off[V];
  int span;  // bytes from the tile's first element to the end of its last row
  __device__ inline TileCopy(int64_t ld, int tid) {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int idx = tid + 256 * i;
      off[i] = (uint32_t)(((int64_t)(idx / VPR) * ld + (idx % VPR) * 8) * 2);
    }
    span = (int)(((int64_t)(ROWS - 1) * ld + D) * 2);
  }
  __device__ inline void load(const uint16_t* src) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(src), (short)0, span, BUF_FLAGS);
#pragma unroll
    for (int i = 0; i < V; ++i)
      r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off[i], 0, 0));
  }
  __device__ inline void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int idx = tid + 256 * i;
      *reinterpret_cast<u32x4*>(lds + (idx / VPR) * PITCH + (idx % VPR) * 8) = r[i];
    }
  }
};

// Row-read fragment: rows row0 + lane%32, k = d0 + 8*(lane/32) + 0..7.
__device__ inline bf16x8_t row_frag(const uint16_t* t, int row0, int d0, int lane) {
  return ld_frag(t + (row0 + (lane & 31)) * PITCH + d0 + (lane >> 5) * 8);
}

// One score block: acc += sum over k-steps of (tile rows row0.., k-step ks)
// x b[ks], for the k-steps [K0, K0 + G).  The G fragment reads are all issued
// before the first MFMA, so their LDS latencies overlap; left to itself the
// compiler issues each read just ahead of its MFMA, and the dependent chain
// then waits on LDS at every step.
template <int G, int K0, int N>
__device__ inline void score_group(f32x16_t& acc, const uint16_t* t, int row0,
                                   const bf16x8_t (&b)[N], int lane) {
  bf16x8_t a[G];
#pragma unroll
  for (int k = 0; k < G; ++k) a[k] = row_frag(t, row0, (K0 + k) * 16, lane);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < G; ++k) acc = mfma(a[k], b[K0 + k], acc);
}

// Transpose-read fragment: rows d = d0 + lane%32 of a [rows][d] tile, with
// the eight k values (tile rows) in the order the probabilities use as the B
// operand: k = r0 + 8*(e/4) + 4*(lane/32) + e%4 for element e.  One
// ds_read_b64_tr_b16 over a 16-lane group hands lane i element i%4 of the
// 8-byte chunks addressed by lanes i/4 + 4j (j = 0..3); lane s of the group
// addresses tile row kb + s/4 at column d0 + 16*(group&1) + 4*(s%4), so lane
// i receives column d0 + 16*(group&1) + i at tile rows kb..kb+3.
__device__ inline bf16x8_t tr_frag(const uint16_t* t, int r0, int d0, int lane) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4 lds_s4;
  const int grp = lane >> 4, sl = lane & 15;
  const int row = r0 + 4 * (grp >> 1) + (sl >> 2);
  const int col = d0 + 16 * (grp & 1) + 4 * (sl & 3);
  const uint16_t* q = t + row * PITCH + col;
  const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)q);
  const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(q + 8 * PITCH));
  const u32x2 x = __builtin_bit_cast(u32x2, lo), y = __builtin_bit_cast(u32x2, hi);
  return as_frag(u32x4{x[0], x[1], y[0], y[1]});
}

// Stores one lane's share of a transposed head row: acc[dd][4 rr + e] is
// element d = 32 dd + 8 rr + 4 g + e of the row of this lane's query (or
// key), g = lane / 32.  Values are scaled, then rounded once to bf16.  With
// RoPE tables the row is a gradient with respect to rotated q or k, and it
// is rotated back in fp32 first (the transpose of the forward rotation by the
// angle of position pos): the pair (d, d + D/2) sits in accumulators dd and
// dd + D/64 of the same lane.
template <int D>
__device__ inline void store_head_row(const f32x16_t (&acc)[D / 32], uint16_t* dst, float scale,
                                      const float* cos_t, const float* sin_t, int pos, int g) {
  constexpr int DT = D / 32, HD = D / 2;
  if (cos_t) {
#pragma unroll
    for (int dd = 0; dd < DT / 2; ++dd)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int i = dd * 32 + rr * 8 + g * 4;
        const float4 c4 = *reinterpret_cast<const float4*>(cos_t + (int64_t)pos * HD + i);
        const float4 s4 = *reinterpret_cast<const float4*>(sin_t + (int64_t)pos * HD + i);
        const float cs[4] = {c4.x, c4.y, c4.z, c4.w}, sn[4] = {s4.x, s4.y, s4.z, s4.w};
        float a[4], b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = acc[dd][rr * 4 + e] * scale, y = acc[dd + DT / 2][rr * 4 + e] * scale;
          a[e] = x * cs[e] + y * sn[e];
          b[e] = y * cs[e] - x * sn[e];
        }
        *reinterpret_cast<u32x2*>(dst + i) = u32x2{pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3])};
        *reinterpret_cast<u32x2*>(dst + i + HD) = u32x2{pack_bf2(b[0], b[1]), pack_bf2(b[2], b[3])};
      }
  } else {
#pragma unroll
    for (int dd = 0; dd < DT; ++dd)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d = dd * 32 + rr * 8 + g * 4;
        *reinterpret_cast<u32x2*>(dst + d) =
            u32x2{pack_bf2(acc[dd][rr * 4 + 0] * scale, acc[dd][rr * 4 + 1] * scale),
                  pack_bf2(acc[dd][rr * 4 + 2] * scale, acc[dd][rr * 4 + 3] * scale)};
      }
  }
}

// ------------------------------------------------------- grid order
// Workgroup id -> (block, batch x head).  Blocks go in decreasing order of
// work, heaviest first over all heads (under the causal mask a query block's
// work grows with its index and a key block's falls), so the grid drains
// evenly.  Workgroups are handed to the 8 XCDs in turn (id % 8); when
// nbh = batch x heads is a multiple of 8, the (batch, head) pairs are laid out
// so that all workgroups of one head run on one XCD and its K/V (or Q/dO)
// rows are read from that XCD's L2.
constexpr int NXCD = 8;
__device__ inline void attn_order(int id, int nblk, int nbh, bool high_first, int& blk, int& bh) {
  const int i = id / nbh, r = id - i * nbh;
  blk = high_first ? nblk - 1 - i : i;
  bh = (nbh % NXCD == 0) ? (r % NXCD) * (nbh / NXCD) + r / NXCD : r;
}

// ------------------------------------------------- padded LDS tiles
// Tiles go from global memory straight into LDS with buffer_load ... lds: one
// such load moves 64 lanes x 16 bytes into 1 KB of LDS in lane order, with no
// VGPR staging and no ds_write.  A tile of R rows of one head (D bf16 each)
// is laid out with a row pitch of 2D + PAD bytes; the lanes whose 16 bytes
// land in a pad (or past the last row) load a chunk of the tile that another
// lane loads too, and what they write is never read.  The pads make the
// fragment reads free of bank conflicts with addresses that are one
// per-lane base plus immediate offsets:
//   * PAD = 16 (a row starts one 16-byte slot further round the 256-byte
//     bank sweep): the 16 lanes of a ds_read_b128 read one chunk of 16
//     consecutive rows in 16 distinct slots;
//   * PAD = 64 (four slots): the 32 lanes of a ds_read_b64_tr_b16 read four
//     chunks of four consecutive rows in 16 distinct slots.
typedef __attribute__((address_space(3))) void lds_void;
__device__ inline void dma16(__amdgpu_buffer_rsrc_t rs, uint16_t* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, voff, 0, 0, 0);
}

template <int D, int R, int PAD>
struct PTile {
  static constexpr int PITCH = 2 * D + PAD;             // bytes
  static constexpr int N = (R * PITCH + 1023) / 1024;   // 1 KB loads per tile
  static constexpr int ELEMS = N * 512;                 // LDS elements a stage takes
  static constexpr int V = (N + 3) / 4;                 // loads per wave (at most)
};

// The loads of one tile by the 4 waves of a workgroup, rows of stride ld
// elements in global memory.  Every wave issues V loads per tile (wave w
// loads w, w + 4, ...); a wave's loads past the tile's N go to a 1 KB junk
// area, and a tile past the end of the sequence gets an empty buffer
// resource (its loads touch no memory and return zeros).  So every wave
// issues the same loads on every tile, and a wait can name how many of them
// may still be in flight.
template <int D, int R, int PAD>
struct TileDma {
  using P = PTile<D, R, PAD>;
  uint32_t off[P::V];
  int span;
  __device__ inline TileDma(int64_t ld, int wave, int lane) {
#pragma unroll
    for (int k = 0; k < P::V; ++k) {
      const int byte = (wave + 4 * k) * 1024 + lane * 16;
      int r = byte / P::PITCH, c = (byte % P::PITCH) >> 4;
      if (r >= R || c >= D / 8) {  // pad or past the tile: any chunk the tile loads anyway
        r = r < R ? r : R - 1;
        c = 0;
      }
      off[k] = (uint32_t)(((int64_t)r * ld + c * 8) * 2);
    }
    span = (int)(((R - 1) * ld + D) * 2);
  }
  __device__ inline void load(const uint16_t* src, bool valid, uint16_t* lds, uint16_t* junk,
                              int wave) const {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(src), (short)0, valid ? span : 0, BUF_FLAGS);
#pragma unroll
    for (int k = 0; k < P::V; ++k)
      dma16(rs, wave + 4 * k < P::N ? lds + (wave + 4 * k) * 512 : junk, off[k]);
  }
};
// this wave's loads into LDS have landed (a barrier then covers every wave's)
__device__ inline void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// all but this wave's N most recent loads have landed
template <int N>
__device__ inline void wait_dma_but() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier for LDS tiles with direct loads in flight: this wave's
// LDS reads have returned, then s_barrier, with no memory fence (a fence
// would wait for every load of the wave, including the prefetches; the
// caller has already waited for the loads the next tile reads).  The empty
// asm statements keep the compiler from moving memory accesses across it.
__device__ inline void tile_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per-lane element offset of the row read of a tile with a pad of PE
// elements per row: rows base + lane % 32, d = 16 ks + 8 (lane / 32) + 0..7
// at + 16 ks (ds_read_b128).
template <int D, int PE>
__device__ inline int row_base(int lane) {
  return (lane & 31) * (D + PE) + (lane >> 5) * 8;
}
// Per-lane element offset of the transpose read (pad PE elements): for the fragment
// of d = 32 dd + lane % 32 over tile rows base + 8 (e / 4) + 4 (lane / 32) +
// e % 4 (e = 0..7, the order the probabilities use as the B operand), add
// 32 dd for the low four rows and 8 rows more for the high four.  One
// ds_read_b64_tr_b16 over a 16-lane group hands lane i element i % 4 of the
// 8-byte chunks addressed by lanes i / 4 + 4 j (j = 0..3); lane s of group
// grp addresses row 4 (grp / 2) + s / 4 at d = 16 (grp & 1) + 4 (s % 4).
template <int D, int PE>
__device__ inline int tr_base(int lane) {
  const int grp = lane >> 4, sl = lane & 15;
  return (4 * (grp >> 1) + (sl >> 2)) * (D + PE) + 16 * (grp & 1) + 4 * (sl & 3);
}
__device__ inline bf16x8_t tr_read(const uint16_t* lo, const uint16_t* hi) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4 lds_s4;
  const s4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)lo);
  const s4 c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)hi);
  const u32x2 x = __builtin_bit_cast(u32x2, a), y = __builtin_bit_cast(u32x2, c);
  return as_frag(u32x4{x[0], x[1], y[0], y[1]});
}

// The value, opaque to the compiler.  A per-lane LDS offset passed through
// this inside a loop is added to its stage's base there, instead of one
// address register per stage being hoisted out of the loop.
__device__ inline int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Maximum and sum of a value over a lane and its partner lane ^ 32 (one VALU
// swap instead of an LDS permute).
__device__ inline float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// --------------------------------------------------------------- forward
// 256 threads = 4 waves x 32 queries; key/value tiles of 32 rows in padded
// LDS, four stages each, one barrier per tile.  Software pipelined per wave:
// while the probabilities of tile t are formed (VALU), the scores of tile
// t + 1 run on the matrix cores, and while P_t V_t runs, the row maxima of
// tile t + 1 are taken.  Tile t's step issues the loads of K and V tile t + 3
// and, before its barrier, waits only for those that step t + 1 reads (K tile
// t + 2 and V tile t + 1), so a load has about two tiles of work to land.
// The running maximum is updated lazily (only when a tile's maximum exceeds
// it by more than RESCALE_SLACK); the row sum adds the fp32 probabilities.
// Two workgroups per CU.
template <int D>
__device__ inline void fwd_scores(f32x16_t& s, const uint16_t* kt, const bf16x8_t (&qf)[D / 16]) {
  zero(s);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) s = mfma(ld_frag(kt + ks * 16), qf[ks], s);
}
__device__ inline float max16(const f32x16_t& s) {
  float m = fmaxf(s[0], s[1]);
#pragma unroll
  for (int r = 2; r < 16; r += 2) m = fmaxf(m, fmaxf(s[r], s[r + 1]));
  return m;
}

template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(const uint16_t* __restrict__ qkv,
                                                          uint16_t* __restrict__ out,
                                                          float* __restrict__ lse, int seq,
                                                          int nq, int nkv, int64_t T, int nbh) {
  constexpr int BKV = 32, KS = D / 16, DT = D / 32;
  using KT = PTile<D, BKV, 16>;
  using VT = PTile<D, BKV, 64>;
  constexpr int PV = D + 32;  // V row pitch, elements
  __shared__ __attribute__((aligned(16))) uint16_t K0[KT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t K1[KT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t K2[KT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t K3[KT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t V0[VT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t V1[VT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t V2[VT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t V3[VT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t junk[512];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, known uniform
  int qb, bh;
  attn_order(blockIdx.x, seq / 128, nbh, true, qb, bh);
  const int b = bh / nq, j = bh % nq;
  const int kvh = j / (nq / nkv);
  const int64_t ld = (int64_t)(nq + 2 * nkv) * D;
  const int64_t row0 = (int64_t)b * seq;
  const uint16_t* Qp = qkv + j * D;
  const uint16_t* Kp = qkv + (int64_t)nq * D + kvh * D + row0 * ld;
  const uint16_t* Vp = qkv + (int64_t)(nq + nkv) * D + kvh * D + row0 * ld;
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
  const int rb = row_base<D, 8>(lane), tb = tr_base<D, 32>(lane);
  const TileDma<D, BKV, 16> kdma(ld, w, lane);
  const TileDma<D, BKV, 64> vdma(ld, w, lane);

  const int nkt = 4 * qb + 4;  // key tiles up to the workgroup's last query (a multiple of 4)
  const int ntw = q0 / 32 + 1;  // tiles this wave needs; its last one is diagonal

  kdma.load(Kp, true, K0, junk, w);  // nkt >= 4
  kdma.load(Kp + BKV * ld, true, K1, junk, w);
  kdma.load(Kp + 2 * BKV * ld, true, K2, junk, w);
  vdma.load(Vp, true, V0, junk, w);
  vdma.load(Vp + BKV * ld, true, V1, junk, w);
  vdma.load(Vp + 2 * BKV * ld, true, V2, junk, w);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) settle(qf[ks]);
  wait_dma();
  __syncthreads();
  // The tiles carry x = S sl2 - m_run (log2 units relative to the running
  // maximum), formed while the previous tile's P V runs; mx is the lane's
  // maximum of x.  The first tile sets m_run to its row maximum.
  auto mask = [&](f32x16_t& x, int t) {  // keys after the lane's query
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (t * BKV + (r >> 2) * 8 + g * 4 + (r & 3) > q) x[r] = -INFINITY;
  };
  f32x16_t sA, sB;
  fwd_scores<D>(sA, K0 + rb, qf);
  if (ntw == 1) mask(sA, 0);
  m_run = pair_max(max16(sA)) * sl2;
#pragma unroll
  for (int r = 0; r < 16; ++r) sA[r] = fmaf(sA[r], sl2, -m_run);
  float mx = 0.0f;

  // Tile t: x holds its exponents and mx their lane maximum; kn is the K
  // stage of tile t + 1, vt the V stage of tile t; xn / mx receive tile t + 1.
  auto tile = [&](int t, f32x16_t& x, f32x16_t& xn, const uint16_t* kn, const uint16_t* vt) {
    if (t >= ntw) return;
    // The K fragments of tile t + 1 are read first (their LDS latency runs
    // under the mask and rescale below).  They are read and multiplied even
    // after the wave's last tile (whatever stage (t + 1) % 4 then holds; the
    // scores are never used): one straight-line path, so the accumulators
    // keep their registers.
    bf16x8_t kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = ld_frag(kn + rb + ks * 16);
    bf16x8_t vf[2][DT];  // the V fragments of P_t V_t
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int dd = 0; dd < DT; ++dd) {
        const uint16_t* p = vt + tb + hh * 16 * PV + dd * 32;
        vf[hh][dd] = tr_read(p, p + 8 * PV);
      }
    if (t == ntw - 1 && t > 0) {
      mask(x, t);
      mx = max16(x);
    }
    // The running maximum only has to bound the exponents: it moves (and the
    // accumulator is rescaled) only when a row's maximum exceeds it by more
    // than RESCALE_SLACK, so probabilities stay below 2^RESCALE_SLACK and
    // most tiles skip the rescale.
    const float rise = pair_max(mx);
    const bool grow = rise > RESCALE_SLACK;
    if (__ballot(grow)) {
      const float dm = grow ? rise : 0.0f;
      const float alpha = exp2_hw(-dm);
      m_run += dm;
      l_run *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] -= dm;
#pragma unroll
      for (int dd = 0; dd < DT; ++dd)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dd][r] *= alpha;
    }
    // S_{t+1} on the matrix cores while P_t (rounded to bf16: the B
    // fragments of P V) is formed on the VALU
    zero(xn);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) xn = mfma(kf[ks], qf[ks], xn);
    uint32_t u[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float a = exp2_hw(x[2 * k]), c = exp2_hw(x[2 * k + 1]);
      u[k] = pack_bf2(a, c);
      l_run += a;
      l_run += c;
    }
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 32 / KS, 0);  // its share of the VALU
    }
    __builtin_amdgcn_sched_barrier(0);
    const bf16x8_t pf[2] = {as_frag(u32x4{u[0], u[1], u[2], u[3]}),
                            as_frag(u32x4{u[4], u[5], u[6], u[7]})};
    // P_t V_t while the exponents of tile t + 1 and their maxima are formed
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int dd = 0; dd < DT; ++dd) acc[dd] = mfma(vf[hh][dd], pf[hh], acc[dd]);
    const float m = m_run;
#pragma unroll
    for (int r = 0; r < 16; ++r) xn[r] = fmaf(xn[r], sl2, -m);
    mx = max16(xn);
  };
  // Step t: K tile t + 1 is in stage kn, V tile t in stage vt; the step fills
  // stages kfill / vfill (those of tiles t - 1) with tiles t + 3.  Before its
  // barrier it waits for K tile t + 2 and V tile t + 1: V tile t + 2 and the
  // step's own loads may still be in flight.
  auto step = [&](int t, f32x16_t& s, f32x16_t& sn, const uint16_t* kn, const uint16_t* vt,
                  uint16_t* kfill, uint16_t* vfill) {
    const bool more = t + 3 < nkt;
    kdma.load(Kp + (int64_t)(t + 3) * BKV * ld, more, kfill, junk, w);
    vdma.load(Vp + (int64_t)(t + 3) * BKV * ld, more, vfill, junk, w);
    tile(t, s, sn, kn, vt);
    wait_dma_but<2 * VT::V + KT::V>();
    tile_barrier();
  };
  for (int t = 0; t < nkt; t += 4) {
    step(t, sA, sB, K1, V0, K3, V3);
    step(t + 1, sB, sA, K2, V1, K0, V0);
    step(t + 2, sA, sB, K3, V2, K1, V1);
    step(t + 3, sB, sA, K0, V3, K2, V2);
  }

  const float l_tot = pair_sum(l_run);
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
// Also writes lse2 = lse log2(e), the row statistic in the base-2 units the
// gradient kernels use.
template <int D>
__global__ void attn_dsum_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                                 const float* __restrict__ lse, float* __restrict__ dsum,
                                 float* __restrict__ lse2, int nq, int64_t T) {
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
  lse2[(int64_t)j * T + t] = lse[(int64_t)j * T + t] * LOG2E;
}

// ------------------------------------------------------- backward: dQ
// Query block outer (4 waves x 32 queries, one query per lane), key and value
// tiles of 32 rows in padded LDS, four stages each, one barrier per tile.
// Per key tile t a wave forms S_t = K_t q and dP_t = V_t dO on the matrix
// cores, then dS_t = P_t (dP_t - D) on the VALU while dQ += K_{t-1}^T dS_{t-1}
// (the previous tile's, K^T through transpose reads) runs on the matrix
// cores.  K tiles carry a 48-byte pad (row reads conflict-free, transpose
// reads at most two-way), V tiles a 16-byte one.  Tile t's step fills K stage
// (t + 2) % 4 (a K tile is read by two steps) and V stage (t + 3) % 4.
template <int D>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse2, const float* __restrict__ dsum, uint16_t* __restrict__ dqkv,
    const float* __restrict__ cos_t, const float* __restrict__ sin_t, int seq, int nq, int nkv,
    int64_t T, int nbh) {
  constexpr int BKV = 32, KS = D / 16, DT = D / 32;
  constexpr int KPE = 24, VPE = 8;  // row pads, elements
  using KT = PTile<D, BKV, 2 * KPE>;
  using VT = PTile<D, BKV, 2 * VPE>;
  constexpr int PK = D + KPE;
  __shared__ __attribute__((aligned(16))) uint16_t K0[KT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t K1[KT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t K2[KT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t K3[KT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t V0[VT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t V1[VT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t V2[VT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t V3[VT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t junk[512];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, known uniform
  int qb, bh;
  attn_order(blockIdx.x, seq / 128, nbh, true, qb, bh);
  const int b = bh / nq, j = bh % nq;
  const int kvh = j / (nq / nkv);
  const int64_t ld = (int64_t)(nq + 2 * nkv) * D;
  const int64_t row0 = (int64_t)b * seq;
  const uint16_t* Qp = qkv + j * D;
  const uint16_t* Kp = qkv + (int64_t)nq * D + kvh * D + row0 * ld;
  const uint16_t* Vp = qkv + (int64_t)(nq + nkv) * D + kvh * D + row0 * ld;
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
  const float lq = lse2[(int64_t)j * T + row0 + q];
  const float dq_sum = dsum[(int64_t)j * T + row0 + q];
  f32x16_t acc[DT];
#pragma unroll
  for (int dd = 0; dd < DT; ++dd) zero(acc[dd]);
  const int rbk = row_base<D, KPE>(lane), tbk = tr_base<D, KPE>(lane);
  const int rbv = row_base<D, VPE>(lane);
  const TileDma<D, BKV, 2 * KPE> kdma(ld, w, lane);
  const TileDma<D, BKV, 2 * VPE> vdma(ld, w, lane);

  const int nkt = 4 * qb + 4;   // key tiles up to the workgroup's last query (a multiple of 4)
  const int ntw = q0 / 32 + 1;  // tiles this wave needs; its last one is diagonal

  kdma.load(Kp, true, K0, junk, w);
  kdma.load(Kp + BKV * ld, true, K1, junk, w);
  kdma.load(Kp + 2 * BKV * ld, true, K2, junk, w);
  vdma.load(Vp, true, V0, junk, w);
  vdma.load(Vp + BKV * ld, true, V1, junk, w);
  vdma.load(Vp + 2 * BKV * ld, true, V2, junk, w);
  vdma.load(Vp + 3 * BKV * ld, true, V3, junk, w);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    settle(qf[ks]);
    settle(df[ks]);
  }
  settle(lq);
  settle(dq_sum);
  wait_dma();
  __syncthreads();

  f32x16_t sc, dp;
  bf16x8_t ds[2];
  // S_t and dP_t from K and V stages kt, vt (the causal mask on the wave's
  // diagonal tile)
  auto scores = [&](int t, const uint16_t* kt, const uint16_t* vt) {
    const uint16_t* ka = kt + opaque(rbk);
    const uint16_t* va = vt + opaque(rbv);
    bf16x8_t kf[KS], vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = ld_frag(ka + ks * 16);
      vf[ks] = ld_frag(va + ks * 16);
    }
    zero(sc);
    zero(dp);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      sc = mfma(kf[ks], qf[ks], sc);
      dp = mfma(vf[ks], df[ks], dp);
    }
    if (t == ntw - 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (t * BKV + (r >> 2) * 8 + g * 4 + (r & 3) > q) sc[r] = -INFINITY;
    }
  };
  // dS_t = P_t (dP_t - D), rounded to bf16: the B fragments of K^T dS^T
  auto grads = [&]() {
    uint32_t u[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float a = exp2_hw(fmaf(sc[2 * k], sl2, -lq)) * (dp[2 * k] - dq_sum);
      const float c = exp2_hw(fmaf(sc[2 * k + 1], sl2, -lq)) * (dp[2 * k + 1] - dq_sum);
      u[k] = pack_bf2(a, c);
    }
    ds[0] = as_frag(u32x4{u[0], u[1], u[2], u[3]});
    ds[1] = as_frag(u32x4{u[4], u[5], u[6], u[7]});
  };
  scores(0, K0, V0);
  grads();
  __syncthreads();  // every wave has read V0 before step 1 refills it

  // Step t (1 .. nkt): K tile t in stage kc, t - 1 in kp, V tile t in vc;
  // fills kfill with K tile t + 2 and vfill with V tile t + 3.  dQ of tile
  // t - 1 runs under dS of tile t (formed from stale scores, and never used,
  // on the step after the wave's last tile).  Before the barrier it waits for
  // K tile t + 1 and V tile t + 1.
  auto step = [&](int t, const uint16_t* kc, const uint16_t* kp, const uint16_t* vc,
                  uint16_t* kfill, uint16_t* vfill) {
    kdma.load(Kp + (int64_t)(t + 2) * BKV * ld, t + 2 < nkt, kfill, junk, w);
    vdma.load(Vp + (int64_t)(t + 3) * BKV * ld, t + 3 < nkt, vfill, junk, w);
    if (t <= ntw) {
      const bf16x8_t dsp[2] = {ds[0], ds[1]};
      if (t < ntw) scores(t, kc, vc);
      bf16x8_t kt[2][DT];
      const uint16_t* kpt = kp + opaque(tbk);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int dd = 0; dd < DT; ++dd) {
          const uint16_t* p = kpt + hh * 16 * PK + dd * 32;
          kt[hh][dd] = tr_read(p, p + 8 * PK);
        }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int dd = 0; dd < DT; ++dd) acc[dd] = mfma(kt[hh][dd], dsp[hh], acc[dd]);
      grads();
#pragma unroll
      for (int k = 0; k < 2 * DT; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 72 / (2 * DT), 0);  // its share of the VALU
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_dma_but<2 * VT::V + KT::V>();
    tile_barrier();
  };
  for (int t = 1; t <= nkt; t += 4) {
    step(t, K1, K0, V1, K3, V0);
    step(t + 1, K2, K1, V2, K0, V1);
    step(t + 2, K3, K2, V3, K1, V2);
    step(t + 3, K0, K3, V0, K2, V3);
  }
  store_head_row<D>(acc, dqkv + (row0 + q) * ld + j * D, 1.0f / sqrtf((float)D), cos_t, sin_t, q,
                    g);
}

// ------------------------------------------------ backward: dK and dV fused
// One launch for both: key block outer (4 waves x 32 keys, one key per lane,
// one wave per SIMD so that a wave holds K, V and both accumulators), the
// 32-row Q and dO tiles after the block (and their D and lse log2(e) rows)
// streaming through padded LDS, four stages, one barrier per tile.  Per tile a
// wave forms S = Q k and dP = dO v on the matrix cores (two chains), then P
// and dS = P (dP - D) on the VALU while the previous tile's dV^T += dO^T P and
// dK^T += Q^T dS (eight accumulator chains) run on the matrix cores.  A step
// issues its LDS fragment reads ahead of their MFMAs: this tile's row
// fragments first, then the previous tile's transposes, two per MFMA of the S
// and dP chains, so that no MFMA waits on a read issued just before it.  Both
// tiles are read by rows and by transposes: 48-byte pads.  Grouped heads
// (SPLIT): one workgroup per query head, writing fp32 shares of dK and dV.
template <int D, bool SPLIT>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ dout,
    const float* __restrict__ stats, int stat_off, uint16_t* __restrict__ dqkv,
    float* __restrict__ part_k, float* __restrict__ part_v, const float* __restrict__ cos_t,
    const float* __restrict__ sin_t, int seq, int nq, int nkv, int64_t T, int nbh) {
  constexpr int BQ = 32, KS = D / 16, DT = D / 32, PE = 24;
  using TT = PTile<D, BQ, 2 * PE>;
  constexpr int PT = D + PE;
  __shared__ __attribute__((aligned(16))) uint16_t Q0[TT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Q1[TT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Q2[TT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Q3[TT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t O0[TT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t O1[TT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t O2[TT::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t O3[TT::ELEMS];
  // per stage: D of the tile's 32 queries, then their lse log2(e)
  __shared__ __attribute__((aligned(16))) float S0[64];
  __shared__ __attribute__((aligned(16))) float S1[64];
  __shared__ __attribute__((aligned(16))) float S2[64];
  __shared__ __attribute__((aligned(16))) float S3[64];
  __shared__ __attribute__((aligned(16))) uint16_t junk[512];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, known uniform
  int kvb, bh;
  attn_order(blockIdx.x, seq / 128, nbh, false, kvb, bh);
  const int nh = SPLIT ? nq : nkv;
  const int b = bh / nh, hd = bh % nh;
  const int kvh = SPLIT ? hd / (nq / nkv) : hd;
  const int j = hd;  // the query head whose tiles the workgroup walks
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
  f32x16_t dk[DT], dv[DT];
#pragma unroll
  for (int dd = 0; dd < DT; ++dd) {
    zero(dk[dd]);
    zero(dv[dd]);
  }
  const int qt0 = kvb * 4, nqt = seq / BQ;
  const int n_it = nqt - qt0;  // query tiles from the block's first (a multiple of 4)
  const int first = qt0 + w;   // the wave's first query tile that sees one of its keys (diagonal)
  const int rb = row_base<D, PE>(lane), tb = tr_base<D, PE>(lane);
  const TileDma<D, BQ, 2 * PE> qdma(ld, w, lane);
  const TileDma<D, BQ, 2 * PE> odma(ldo, w, lane);
  // statistics: lane l < 32 loads D of query l of the tile, lane l >= 32 its lse log2(e)
  const uint32_t soff = (uint32_t)(((lane < 32) ? lane : stat_off + lane - 32) * 4);
  const int sspan = (stat_off + 32) * 4;

  // Loads of query tile it (of query head j) into (qs, os, st); past the
  // end: empty.
  auto load = [&](int it, uint16_t* qs, uint16_t* os, float* st) {
    const bool valid = it < n_it;
    const int q0 = (qt0 + (valid ? it : 0)) * BQ;
    qdma.load(qkv + j * D + (row0 + q0) * ld, valid, qs, junk, w);
    odma.load(dout + j * D + (row0 + q0) * ldo, valid, os, junk, w);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(stats + (int64_t)j * T + row0 + q0), (short)0, valid ? sspan : 0,
        BUF_FLAGS);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(w == 0 ? (void*)st : (void*)junk), 4,
                                             soff, 0, 0, 0);
  };
  load(0, Q0, O0, S0);  // n_it >= 4
  load(1, Q1, O1, S1);
  load(2, Q2, O2, S2);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    settle(kf[ks]);
    settle(vf[ks]);
  }
  wait_dma();
  __syncthreads();

  f32x16_t sc, dp;
  zero(sc);
  zero(dp);
  bf16x8_t pP[2], pS[2];  // P and dS of the latest tile, rounded to bf16 (B fragments)
  // S and dP of query tile it from stages qs, os, with the causal mask on
  // the wave's diagonal tile.  Tiles before the wave's first are skipped
  // (their P and dS become zeros).
  auto scores = [&](int it, const uint16_t* qs, const uint16_t* os) {
    const int i = qt0 + it;
    if (i < first) return;
    const uint16_t* qa = qs + opaque(rb);
    const uint16_t* oa = os + opaque(rb);
    bf16x8_t af[KS], bf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      af[ks] = ld_frag(qa + ks * 16);
      bf[ks] = ld_frag(oa + ks * 16);
    }
    zero(sc);
    zero(dp);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      sc = mfma(af[ks], kf[ks], sc);
      dp = mfma(bf[ks], vf[ks], dp);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (i == first) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kv > i * BQ + (r >> 2) * 8 + g * 4 + (r & 3)) sc[r] = -INFINITY;
    }
  };
  // Rows rr = 2 h, 2 h + 1 of the lane's P and dS, packed into up / us.
  uint32_t up[8], us[8];
  auto probs_half = [&](int h, const float* st) {
#pragma unroll
    for (int rr = 2 * h; rr < 2 * h + 2; ++rr) {
      const float4 l4 = *reinterpret_cast<const float4*>(st + 32 + rr * 8 + g * 4);
      const float4 d4 = *reinterpret_cast<const float4*>(st + rr * 8 + g * 4);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dvv[4] = {d4.x, d4.y, d4.z, d4.w};
      float pv[4], sv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = rr * 4 + e;
        pv[e] = exp2_hw(fmaf(sc[r], sl2, -lv[e]));
        sv[e] = pv[e] * (dp[r] - dvv[e]);
      }
      up[2 * rr] = pack_bf2(pv[0], pv[1]);
      up[2 * rr + 1] = pack_bf2(pv[2], pv[3]);
      us[2 * rr] = pack_bf2(sv[0], sv[1]);
      us[2 * rr + 1] = pack_bf2(sv[2], sv[3]);
    }
  };
  auto frags = [&](int it) {
    if (qt0 + it < first) {  // a tile before the wave's first: no contribution
#pragma unroll
      for (int k = 0; k < 8; ++k) up[k] = us[k] = 0u;
    }
    pP[0] = as_frag(u32x4{up[0], up[1], up[2], up[3]});
    pP[1] = as_frag(u32x4{up[4], up[5], up[6], up[7]});
    pS[0] = as_frag(u32x4{us[0], us[1], us[2], us[3]});
    pS[1] = as_frag(u32x4{us[4], us[5], us[6], us[7]});
  };
  scores(0, Q0, O0);
  probs_half(0, S0);
  probs_half(1, S0);
  frags(0);

  // Step it (1 .. n_it): tile it in stages (qc, oc, stc), it - 1 in (qp, op);
  // fills (qfill, ofill, sfill) with tile it + 2.  The accumulation of tile
  // it - 1 runs under the VALU of tile it (formed from stale scores, and never
  // used, on the last step).  Before the barrier it waits for tile it + 1.
  auto step = [&](int it, const uint16_t* qc, const uint16_t* oc, const float* stc,
                  const uint16_t* qp, const uint16_t* op, uint16_t* qfill, uint16_t* ofill,
                  float* sfill) {
    load(it + 2, qfill, ofill, sfill);
    const bf16x8_t pp[2] = {pP[0], pP[1]}, ps[2] = {pS[0], pS[1]};
    const uint16_t* qt = qp + opaque(tb);
    const uint16_t* ot = op + opaque(tb);
    bf16x8_t xq[2][DT], xo[2][DT];
    auto tr_all = [&]() {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int dd = 0; dd < DT; ++dd) {
          const int o = hh * 16 * PT + dd * 32;
          xq[hh][dd] = tr_read(qt + o, qt + o + 8 * PT);
          xo[hh][dd] = tr_read(ot + o, ot + o + 8 * PT);
        }
    };
    const int i = qt0 + it;
    if (it < n_it && i >= first) {
      // this tile's row fragments, then the previous tile's transposes, read
      // a few MFMAs ahead of their use under the S and dP chains
      const uint16_t* qa = qc + opaque(rb);
      const uint16_t* oa = oc + opaque(rb);
      bf16x8_t af[KS], bf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        af[ks] = ld_frag(qa + ks * 16);
        bf[ks] = ld_frag(oa + ks * 16);
      }
      tr_all();
      zero(sc);
      zero(dp);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sc = mfma(af[ks], kf[ks], sc);
        dp = mfma(bf[ks], vf[ks], dp);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int k = 0; k < 2 * KS; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (i == first) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kv > i * BQ + (r >> 2) * 8 + g * 4 + (r & 3)) sc[r] = -INFINITY;
      }
    } else {
      tr_all();
    }
#pragma unroll
    for (int dd = 0; dd < DT; ++dd) {
      dv[dd] = mfma(xo[0][dd], pp[0], dv[dd]);
      dk[dd] = mfma(xq[0][dd], ps[0], dk[dd]);
    }
    probs_half(0, stc);
#pragma unroll
    for (int k = 0; k < 2 * DT; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 48 / (2 * DT), 0);  // its VALU share
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dd = 0; dd < DT; ++dd) {
      dv[dd] = mfma(xo[1][dd], pp[1], dv[dd]);
      dk[dd] = mfma(xq[1][dd], ps[1], dk[dd]);
    }
    probs_half(1, stc);
#pragma unroll
    for (int k = 0; k < 2 * DT; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 48 / (2 * DT), 0);  // its VALU share
    }
    __builtin_amdgcn_sched_barrier(0);
    frags(it);
    wait_dma_but<2 * TT::V + 1>();
    tile_barrier();
  };
  for (int it = 1; it <= n_it; it += 4) {
    step(it, Q1, O1, S1, Q0, O0, Q3, O3, S3);
    step(it + 1, Q2, O2, S2, Q1, O1, Q0, O0, S0);
    step(it + 2, Q3, O3, S3, Q2, O2, Q1, O1, S1);
    step(it + 3, Q0, O0, S0, Q3, O3, Q2, O2, S2);
  }
  if constexpr (SPLIT) {
    // unscaled fp32 shares of query head hd: part_k, part_v [nq][T][D]
    float* dsk = part_k + ((int64_t)hd * T + row0 + kv) * D;
    float* dsv = part_v + ((int64_t)hd * T + row0 + kv) * D;
#pragma unroll
    for (int dd = 0; dd < DT; ++dd)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        *reinterpret_cast<float4*>(dsk + dd * 32 + rr * 8 + g * 4) =
            make_float4(dk[dd][rr * 4 + 0], dk[dd][rr * 4 + 1], dk[dd][rr * 4 + 2],
                        dk[dd][rr * 4 + 3]);
        *reinterpret_cast<float4*>(dsv + dd * 32 + rr * 8 + g * 4) =
            make_float4(dv[dd][rr * 4 + 0], dv[dd][rr * 4 + 1], dv[dd][rr * 4 + 2],
                        dv[dd][rr * 4 + 3]);
      }
  } else {
    // dK is a gradient with respect to rotated keys (rotated back here); dV is not
    uint16_t* base = dqkv + (row0 + kv) * ld;
    store_head_row<D>(dk, base + (int64_t)nq * D + kvh * D, 1.0f / sqrtf((float)D), cos_t, sin_t,
                      kv, g);
    store_head_row<D>(dv, base + (int64_t)(nq + nkv) * D + kvh * D, 1.0f, nullptr, nullptr, kv,
                      g);
  }
}

// dK or dV of a grouped kv head from its query heads' fp32 shares, added in
// query-head order (fixed for any launch), scaled, rounded to bf16 into the
// column block starting at head col0 of dqkv.  One thread per
// four consecutive d of one (row, kv head).
// With RoPE tables (dK) a thread instead takes four d of the first half and
// their rotation partners d + D/2, and rotates the scaled sums back in fp32
// before the rounding.
template <int D>
__global__ __launch_bounds__(256) void attn_gqa_reduce_kernel(const float* __restrict__ part,
                                                              uint16_t* __restrict__ dqkv,
                                                              int64_t T, int nq, int nkv,
                                                              int col0, float scale,
                                                              const float* __restrict__ cos_t,
                                                              const float* __restrict__ sin_t,
                                                              int seq) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int per_head = cos_t ? D / 8 : D / 4;
  const int64_t per_row = (int64_t)nkv * per_head;
  if (i >= T * per_row) return;
  const int64_t row = i / per_row;
  const int kvh = (int)((i % per_row) / per_head);
  const int d = (int)(i % per_head) * 4;
  const int grp = nq / nkv;
  const int64_t ld = (int64_t)(nq + 2 * nkv) * D;
  uint16_t* dst = dqkv + row * ld + (int64_t)(col0 + kvh) * D;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int g = 0; g < grp; ++g) {
    const float* src = part + ((int64_t)(kvh * grp + g) * T + row) * D;
    const float4 v = *reinterpret_cast<const float4*>(src + d);
    a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
    if (cos_t) {
      const float4 w = *reinterpret_cast<const float4*>(src + d + D / 2);
      b.x += w.x; b.y += w.y; b.z += w.z; b.w += w.w;
    }
  }
  if (cos_t) {
    const int64_t t = (row % seq) * (D / 2) + d;
    const float4 c = *reinterpret_cast<const float4*>(cos_t + t);
    const float4 s = *reinterpret_cast<const float4*>(sin_t + t);
    const float x[4] = {a.x * scale, a.y * scale, a.z * scale, a.w * scale};
    const float y[4] = {b.x * scale, b.y * scale, b.z * scale, b.w * scale};
    const float cs[4] = {c.x, c.y, c.z, c.w}, sn[4] = {s.x, s.y, s.z, s.w};
    float ra[4], rb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ra[e] = x[e] * cs[e] + y[e] * sn[e];
      rb[e] = y[e] * cs[e] - x[e] * sn[e];
    }
    *reinterpret_cast<u32x2*>(dst + d) = u32x2{pack_bf2(ra[0], ra[1]), pack_bf2(ra[2], ra[3])};
    *reinterpret_cast<u32x2*>(dst + d + D / 2) = u32x2{pack_bf2(rb[0], rb[1]), pack_bf2(rb[2], rb[3])};
  } else {
    *reinterpret_cast<u32x2*>(dst + d) =
        u32x2{pack_bf2(a.x * scale, a.y * scale), pack_bf2(a.z * scale, a.w * scale)};
  }
}

template <int D>
hipError_t fwd_d(const uint16_t* qkv, uint16_t* o, float* lse, int batch, int seq, int nq, int nkv,
                 hipStream_t s) {
  const int64_t T = (int64_t)batch * seq;
  const int nbh = nq * batch;
  hipLaunchKernelGGL(attn_fwd_kernel<D>, dim3((unsigned)(seq / 128 * nbh)), dim3(256), 0, s, qkv, o,
                     lse, seq, nq, nkv, T, nbh);
  return hipGetLastError();
}

// With grouped heads the dK/dV launches run one workgroup per query head (nq
// instead of nkv workgroups per key block, so the grid fills the chip) and
// the group's shares are added by attn_gqa_reduce_kernel.
template <int D>
hipError_t bwd_d(const uint16_t* qkv, const uint16_t* o, const uint16_t* dout, const float* lse,
                 float* dsum, float* lse2, float* part, uint16_t* dqkv, const float* cos_t,
                 const float* sin_t, int batch, int seq, int nq, int nkv, hipStream_t s) {
  const int64_t T = (int64_t)batch * seq;
  const int64_t n = T * nq;
  hipLaunchKernelGGL(attn_dsum_kernel<D>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, o,
                     dout, lse, dsum, lse2, nq, T);
  const int nblk = seq / 128;
  // dsum and lse2 are one allocation: lse2 starts stat_off floats after dsum
  const int stat_off = (int)(lse2 - dsum);
  if (nq == nkv) {
    const int nbh = nkv * batch;
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, false>), dim3((unsigned)(nblk * nbh)), dim3(256), 0,
                       s, qkv, dout, dsum, stat_off, dqkv, nullptr, nullptr, cos_t, sin_t, seq, nq,
                       nkv, T, nbh);
  } else {
    const int nbh = nq * batch;
    float* part_v = part + T * nq * D;
    const int64_t nv = T * nkv * (D / 4), nk = T * nkv * (cos_t ? D / 8 : D / 4);
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, true>), dim3((unsigned)(nblk * nbh)), dim3(256), 0,
                       s, qkv, dout, dsum, stat_off, dqkv, part, part_v, nullptr, nullptr, seq, nq,
                       nkv, T, nbh);
    hipLaunchKernelGGL(attn_gqa_reduce_kernel<D>, dim3((unsigned)((nv + 255) / 256)), dim3(256), 0,
                       s, part_v, dqkv, T, nq, nkv, nq + nkv, 1.0f, nullptr, nullptr, seq);
    hipLaunchKernelGGL(attn_gqa_reduce_kernel<D>, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0,
                       s, part, dqkv, T, nq, nkv, nq, 1.0f / sqrtf((float)D), cos_t, sin_t, seq);
  }
  hipLaunchKernelGGL(attn_bwd_dq_kernel<D>, dim3((unsigned)(nblk * nq * batch)), dim3(256), 0, s,
                     qkv, dout, lse2, dsum, dqkv, cos_t, sin_t, seq, nq, nkv, T, nq * batch);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const uint16_t* qkv, uint16_t* o, float* lse, int batch, int seq,
                           int nq, int nkv, int d, hipStream_t s) {
  if (d == 128) return fwd_d<128>(qkv, o, lse, batch, seq, nq, nkv, s);
  if (d == 64) return fwd_d<64>(qkv, o, lse, batch, seq, nq, nkv, s);
  return hipErrorInvalidValue;
}

// Workspace: the D rows and lse log2(e) (fp32 [nq, T] each), then with
// grouped heads the per-query-head dK and dV shares (fp32 [nq, T, d] each).
static size_t dsum_bytes(int64_t T, int nq) { return ((size_t)T * nq * 4 + 255) / 256 * 256; }

size_t attn_bwd_workspace_bytes(int batch, int seq, int nq, int nkv, int d) {
  const int64_t T = (int64_t)batch * seq;
  return 2 * dsum_bytes(T, nq) + (nq != nkv ? 2 * (size_t)T * nq * d * 4 : 0);
}

hipError_t launch_attn_bwd(const uint16_t* qkv, const uint16_t* o, const uint16_t* dout,
                           const float* lse, void* workspace, uint16_t* dqkv, int batch, int seq,
                           int nq, int nkv, int d, const float* cos_t, const float* sin_t,
                           hipStream_t s) {
  const size_t sb = dsum_bytes((int64_t)batch * seq, nq);
  float* dsum = static_cast<float*>(workspace);
  float* lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + sb);
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * sb);
  if (!cos_t != !sin_t) return hipErrorInvalidValue;
  if (d == 128)
    return bwd_d<128>(qkv, o, dout, lse, dsum, lse2, part, dqkv, cos_t, sin_t, batch, seq, nq,
                      nkv, s);
  if (d == 64)
    return bwd_d<64>(qkv, o, dout, lse, dsum, lse2, part, dqkv, cos_t, sin_t, batch, seq, nq, nkv,
                     s);
  return hipErrorInvalidValue;
}

}  // namespace mt
