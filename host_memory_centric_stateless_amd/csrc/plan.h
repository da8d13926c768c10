// Static plan of a configuration: flat layout, streamed units, device regions.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/mt.h"

namespace mt {

constexpr int64_t kAlign = 256;  // elements; every tensor starts at a multiple
inline int64_t round_up(int64_t n, int64_t a) { return (n + a - 1) / a * a; }
inline size_t round_bytes(size_t n) { return (n + 255) / 256 * 256; }

struct TensorOff {
  const char* name;
  int64_t off, numel;
  int32_t rows, cols;
};

// Byte offsets of one window slot (activations of one block kept for its
// backward).
struct SlotLayout {
  size_t x, rstd1, n1, qkv, o, lse, h1, rstd2, n2, gu, m;
  // mixture-of-experts blocks, after n2 (the same slot holds one block at a
  // time): router logits, selection, gates, row plan, expert-major rows
  size_t mlog, msel, mgate, mpos, moff, mrowtok, mx, mgu, mm, myo;
  size_t bytes;
};

// Byte offsets inside the workspace region.
struct WorkLayout {
  size_t xL, xf, rstd_f, logits, dlogits, ce_m, ce_s, ce_lab, ce_lse, dw_acc, loss_rows, loss, dxf,
      dy0, dy1, dyb, dgu, dn, dh1, dh1b, dout, dsum, dqkv, partial, cos_t, sin_t, labels[2], x0[2],
      mdout, mdx, mdlog, mroute, bytes;
};

// Indices into Plan::layer[] (dense blocks) and Plan::moe[] (mixture-of-
// experts blocks: the attention part shares the first six indices).
enum { T_ATTN_NORM = 0, T_WQ, T_WK, T_WV, T_WO, T_MLP_NORM, T_WGATE, T_WUP, T_WDOWN, T_COUNT };
enum { M_ROUTER = T_MLP_NORM + 1, M_GU, M_DOWN };

struct Plan {
  mt_config c;
  int64_t T;            // tokens per pass (n_mb micro-batches)
  int64_t T_mb;         // tokens per micro-batch
  int n_mb;             // micro-batches per pass
  int64_t qd, kvd, ldq; // q width, kv width, qkv row width
  TensorOff layer[T_COUNT];
  int64_t layer_elems;
  // mixture-of-experts blocks (a second structure group)
  TensorOff moe[T_COUNT];
  int64_t moe_elems;
  int64_t moe_rows;      // expert-major row space: T k rounded to 256, + 256 E
  int64_t moe_ldl;       // row stride of the router-logit gradient (E rounded to 8)
  bool any_moe;
  bool is_moe(int l) const {
    return c.n_experts > 0 && l % c.moe_every == c.moe_every - 1;
  }
  const TensorOff* block_layout(int l) const { return is_moe(l) ? moe : layer; }
  int64_t block_elems(int l) const { return is_moe(l) ? moe_elems : layer_elems; }
  TensorOff head[2];    // final_norm, w_head
  int64_t head_elems;
  int64_t embed_elems;
  // LM head streamed in vocabulary chunks: rows [row0[c], row0[c+1]).  Chunk c
  // covers flat elements [chunk_e0[c], chunk_e0[c+1]) of the head group; chunk
  // 0 starts at element 0 so it also carries final_norm.
  int n_chunks;
  std::vector<int64_t> chunk_row0, chunk_e0;
  int64_t head_rows;    // rows of the largest vocabulary chunk
  // The head's logits exist for one token chunk of head_tc tokens at a time.
  int64_t head_tc;
  int n_tchunks;
  int64_t unit_elems;
  bool slab_bf16;       // gradient slabs hold bf16 (else fp32)
  int n_segments;
  SlotLayout slot;
  WorkLayout ws;
  size_t weight_buf_bytes, slab_bytes, window_bytes, ckpt_bytes;
};

// Fills *p; returns an empty string or the reason the config is unsupported.
std::string make_plan(const mt_config& c, Plan* p);

}  // namespace mt
