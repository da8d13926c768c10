// Flat layout, streamed units and device-region sizes of a configuration.
//
// Flat layout: each layer's weights are one pre-flattened array so that one
// copy moves a whole layer, and the same element offsets index the fp32 host
// master/grad/m/v, the pinned bf16 working copy, the device weight buffer and
// the fp32 gradient slab (m.lqnn.cn MegaTrain article, 三.1: per-layer pinned
// flat copies and fixed-size flat GPU buffers; 三.3: flat gradient slabs).
// Tensor order follows the block's data flow and each tensor starts at a
// multiple of 256 elements, so wq|wk|wv and w_gate|w_up are contiguous and are
// read as one fused matrix.
#include "plan.h"

#include <algorithm>
#include <cstring>

#include "common.h"

namespace mt {

// every block is a mixture-of-experts block (no dense FFN tail needed)
static bool all_moe(const mt_config& c) { return c.n_experts > 0 && c.moe_every == 1; }

static void lay(TensorOff* t, int n, int64_t* total) {
  int64_t off = 0;
  for (int i = 0; i < n; ++i) {
    off = round_up(off, kAlign);
    t[i].off = off;
    t[i].numel = (int64_t)t[i].rows * t[i].cols;
    off += t[i].numel;
  }
  *total = round_up(off, kAlign);
}

std::string make_plan(const mt_config& c, Plan* p) {
  if (c.n_layers < 1) return "n_layers must be >= 1";
  if (c.hidden < 256 || c.hidden % 256) return "hidden must be a positive multiple of 256";
  if (c.hidden > 16384) return "hidden must be <= 16384";
  if (c.head_dim != 64 && c.head_dim != 128) return "head_dim must be 64 or 128";
  if (c.n_heads < 1 || c.n_kv_heads < 1 || c.n_heads % c.n_kv_heads)
    return "n_kv_heads must divide n_heads";
  if (c.ffn < 16 || c.ffn % 16) return "ffn must be a positive multiple of 16";
  if (c.vocab < 256 || c.vocab % 256) return "vocab must be a positive multiple of 256";
  if (c.micro_batch < 1) return "micro_batch must be >= 1";
  if (c.seq_len < 128 || c.seq_len % 128) return "seq_len must be a positive multiple of 128";
  if (c.ckpt_interval < 1) return "ckpt_interval must be >= 1";
  if (c.n_grad_slabs < 1 || c.n_grad_slabs > 64) return "n_grad_slabs must be in 1..64";
  if (!(c.rms_eps >= 0.0f) || !(c.rope_base > 1.0f)) return "rms_eps / rope_base";
  if (c.host_threads < 0) return "host_threads must be >= 0";
  if (c.slab_bf16 != 0 && c.slab_bf16 != 1) return "slab_bf16 must be 0 or 1";
  if (c.drain_workgroups < 0 || c.drain_workgroups > 256) return "drain_workgroups must be in 0..256";
  if (c.micro_batches_per_pass < 1 || c.micro_batches_per_pass > 32)
    return "micro_batches_per_pass must be in 1..32";
  if (c.head_token_chunk < 0 || c.head_token_chunk % 8)
    return "head_token_chunk must be 0 or a positive multiple of 8";
  if (c.n_experts != 0) {
    if (c.n_experts < 8 || c.n_experts > 64 || c.n_experts % 8)
      return "n_experts must be 0 or a multiple of 8 up to 64";
    if (c.top_k < 1 || c.top_k > 8 || c.top_k > c.n_experts) return "top_k must be in 1..min(8, E)";
    if (c.expert_ffn < 128 || c.expert_ffn % 128) return "expert_ffn must be a multiple of 128";
    if (c.moe_every < 1) return "moe_every must be >= 1";
  }

  p->c = c;
  const int64_t h = c.hidden, F = c.ffn, V = c.vocab;
  p->T_mb = (int64_t)c.micro_batch * c.seq_len;
  p->n_mb = c.micro_batches_per_pass;
  p->T = p->T_mb * p->n_mb;
  p->qd = (int64_t)c.n_heads * c.head_dim;
  p->kvd = (int64_t)c.n_kv_heads * c.head_dim;
  p->ldq = p->qd + 2 * p->kvd;
  if (p->T / 128 >= 65535) return "too many tokens per micro-batch";
  p->head_tc = std::min<int64_t>(p->T, c.head_token_chunk > 0 ? c.head_token_chunk : 8192);
  p->n_tchunks = (int)((p->T + p->head_tc - 1) / p->head_tc);

  TensorOff* L = p->layer;
  L[T_ATTN_NORM] = {"attn_norm", 0, 0, 1, (int32_t)h};
  L[T_WQ] = {"wq", 0, 0, (int32_t)p->qd, (int32_t)h};
  L[T_WK] = {"wk", 0, 0, (int32_t)p->kvd, (int32_t)h};
  L[T_WV] = {"wv", 0, 0, (int32_t)p->kvd, (int32_t)h};
  L[T_WO] = {"wo", 0, 0, (int32_t)h, (int32_t)p->qd};
  L[T_MLP_NORM] = {"mlp_norm", 0, 0, 1, (int32_t)h};
  L[T_WGATE] = {"w_gate", 0, 0, (int32_t)F, (int32_t)h};
  L[T_WUP] = {"w_up", 0, 0, (int32_t)F, (int32_t)h};
  L[T_WDOWN] = {"w_down", 0, 0, (int32_t)h, (int32_t)F};
  lay(L, T_COUNT, &p->layer_elems);
  // fused operands must be contiguous
  if (L[T_WK].off != L[T_WQ].off + L[T_WQ].numel || L[T_WV].off != L[T_WK].off + L[T_WK].numel ||
      L[T_WUP].off != L[T_WGATE].off + L[T_WGATE].numel)
    return "fused projections not contiguous";
  // mixture-of-experts block layout (used only when n_experts > 0)
  p->any_moe = false;
  for (int l = 0; l < c.n_layers; ++l) p->any_moe = p->any_moe || p->is_moe(l);
  const int64_t E = c.n_experts, Fe = c.expert_ffn;
  TensorOff* Mo = p->moe;
  for (int i = 0; i <= T_MLP_NORM; ++i) Mo[i] = L[i];
  Mo[M_ROUTER] = {"w_router", 0, 0, (int32_t)E, (int32_t)h};
  Mo[M_GU] = {"w_gu", 0, 0, (int32_t)(E * 2 * Fe), (int32_t)h};
  Mo[M_DOWN] = {"w_down", 0, 0, (int32_t)(E * h), (int32_t)Fe};
  lay(Mo, T_COUNT, &p->moe_elems);
  if (!p->any_moe) p->moe_elems = 0;
  p->moe_rows = round_up(p->T * c.top_k, 256) + 256 * E;
  p->moe_ldl = round_up(E, 8);

  p->head[0] = {"final_norm", 0, 0, 1, (int32_t)h};
  p->head[1] = {"w_head", 0, 0, (int32_t)V, (int32_t)h};
  lay(p->head, 2, &p->head_elems);
  p->embed_elems = round_up(V * h, kAlign);

  // Head chunks: as many whole rows (multiple of 256) as fit in a layer-sized
  // unit; at least 256 rows.
  const int64_t woff = p->head[1].off;
  int64_t rows_cap = (p->layer_elems - woff) / h / 256 * 256;
  if (rows_cap < 256) rows_cap = 256;
  p->n_chunks = (int)((V + rows_cap - 1) / rows_cap);
  p->chunk_row0.assign(p->n_chunks + 1, 0);
  p->chunk_e0.assign(p->n_chunks + 1, 0);
  for (int k = 0; k <= p->n_chunks; ++k) {
    int64_t r = std::min<int64_t>((int64_t)k * rows_cap, V);
    p->chunk_row0[k] = r;
    p->chunk_e0[k] = (k == 0) ? 0 : woff + r * h;
  }
  p->chunk_e0[p->n_chunks] = p->head_elems;
  p->head_rows = 0;
  for (int k = 0; k < p->n_chunks; ++k)
    p->head_rows = std::max(p->head_rows, p->chunk_row0[k + 1] - p->chunk_row0[k]);
  p->unit_elems = std::max(p->layer_elems, p->moe_elems);
  for (int k = 0; k < p->n_chunks; ++k)
    p->unit_elems = std::max(p->unit_elems, p->chunk_e0[k + 1] - p->chunk_e0[k]);
  p->n_segments = (c.n_layers + c.ckpt_interval - 1) / c.ckpt_interval;

  const size_t T = (size_t)p->T;
  // window slot
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += round_bytes(bytes); return r; };
  SlotLayout& s = p->slot;
  s.x = take(T * h * 4);
  s.rstd1 = take(T * 4);
  s.n1 = take(T * h * 2);
  s.qkv = take(T * p->ldq * 2);
  s.o = take(T * p->qd * 2);
  s.lse = take((size_t)c.n_heads * T * 4);
  s.h1 = take(T * h * 4);
  s.rstd2 = take(T * 4);
  s.n2 = take(T * h * 2);
  const size_t tail0 = o;
  s.gu = take(T * 2 * F * 2);
  s.m = take(T * F * 2);
  const size_t dense_end = o;
  size_t moe_end = tail0;
  if (p->any_moe) {
    const size_t R = (size_t)p->moe_rows, k = (size_t)c.top_k;
    o = tail0;
    s.mlog = take(T * (size_t)E * 4);
    s.msel = take(T * k * 4);
    s.mgate = take(T * k * 4);
    s.mpos = take(T * k * 4);
    s.moff = take(65 * 4);
    s.mrowtok = take(R * 4);
    s.mx = take(R * h * 2);
    s.mgu = take(R * 2 * Fe * 2);
    s.mm = take(R * Fe * 2);
    s.myo = take(R * h * 4);
    moe_end = o;
  }
  // a slot holds one block at a time: the larger of the two tails
  if (!p->any_moe)
    s.bytes = dense_end;
  else if (all_moe(c))
    s.bytes = moe_end;
  else
    s.bytes = std::max(dense_end, moe_end);

  // workspace
  o = 0;
  WorkLayout& w = p->ws;
  w.xL = take(T * h * 4);
  w.xf = take(T * h * 2);
  w.rstd_f = take(T * 4);
  // one token chunk x one vocabulary chunk of logits and dlogits, the
  // per-token softmax statistics, and (several token chunks, bf16 slabs) an
  // fp32 accumulator for the chunk's weight gradient
  const size_t tc = (size_t)p->head_tc, hr = (size_t)p->head_rows;
  w.logits = take(tc * hr * 4);
  w.dlogits = take(tc * hr * 2);
  w.ce_m = take(T * 4);
  w.ce_s = take(T * 4);
  w.ce_lab = take(T * 4);
  w.ce_lse = take(T * 4);
  w.dw_acc = take(p->n_tchunks > 1 && c.slab_bf16 ? hr * (size_t)h * 4 : 0);
  w.loss_rows = take(T * 4);
  w.loss = take(256);
  w.dxf = take(T * h * 4);
  w.dy0 = take(T * h * 4);
  w.dy1 = take(T * h * 4);
  w.dyb = take(T * h * 2);
  w.dgu = take(std::max(T * 2 * F * 2, p->any_moe ? (size_t)p->moe_rows * 2 * Fe * 2 : 0));
  w.dn = take(T * h * 4);
  w.dh1 = take(T * h * 4);
  w.dh1b = take(T * h * 2);
  w.dout = take(T * p->qd * 2);
  w.dsum = take(attn_bwd_workspace_bytes((int)(p->T / c.seq_len), c.seq_len, c.n_heads,
                                         c.n_kv_heads, c.head_dim));
  w.dqkv = take(T * p->ldq * 2);
  w.partial = take(rmsnorm_bwd_partial_bytes(p->T, (int)h));
  w.cos_t = take((size_t)c.seq_len * (c.head_dim / 2) * 4);
  w.sin_t = take((size_t)c.seq_len * (c.head_dim / 2) * 4);
  w.labels[0] = take(T * 4);
  w.labels[1] = take(T * 4);
  w.x0[0] = take(T * h * 4);
  w.x0[1] = take(T * h * 4);
  const size_t R = p->any_moe ? (size_t)p->moe_rows : 0;
  w.mdout = take(R * h * 2);
  w.mdx = take(R * h * 4);
  w.mdlog = take(p->any_moe ? T * (size_t)p->moe_ldl * 2 : 0);
  // the expert selection of every MoE block in the last forward (mt_moe_routing)
  w.mroute = take(p->any_moe ? (size_t)(c.n_layers / c.moe_every) * T * c.top_k * 4 : 0);
  w.bytes = o;

  p->weight_buf_bytes = round_bytes((size_t)p->unit_elems * 2);
  p->slab_bf16 = c.slab_bf16 != 0;
  p->slab_bytes = round_bytes((size_t)p->unit_elems * (p->slab_bf16 ? 2 : 4));
  p->window_bytes = (size_t)std::min(c.ckpt_interval, c.n_layers) * s.bytes;
  p->ckpt_bytes = (size_t)std::max(1, p->n_segments - 1) * round_bytes(T * h * 4);
  return "";
}

}  // namespace mt

// ---------------------------------------------------------------- C ABI
extern "C" mt_status mt_layout(const mt_config* cfg, int32_t group, mt_tensor_desc* out,
                               int32_t cap, int32_t* n_out, int64_t* flat_numel) {
  if (!cfg || !n_out || !flat_numel || cap < 0 || (cap > 0 && !out)) return MT_E_ARG;
  mt::Plan p;
  if (!mt::make_plan(*cfg, &p).empty()) return MT_E_ARG;
  const mt::TensorOff* t;
  int n;
  int64_t total;
  mt::TensorOff emb{"emb", 0, (int64_t)cfg->vocab * cfg->hidden, cfg->vocab, cfg->hidden};
  if (group == MT_GROUP_EMBED) {
    t = &emb;
    n = 1;
    total = p.embed_elems;
  } else if (group == MT_GROUP_HEAD) {
    t = p.head;
    n = 2;
    total = p.head_elems;
  } else if (group >= 0 && group < cfg->n_layers) {
    t = p.block_layout(group);
    n = mt::T_COUNT;
    total = p.block_elems(group);
  } else {
    return MT_E_ARG;
  }
  for (int i = 0; i < n && i < cap; ++i) {
    std::memset(out[i].name, 0, sizeof(out[i].name));
    std::strncpy(out[i].name, t[i].name, sizeof(out[i].name) - 1);
    out[i].offset = t[i].off;
    out[i].numel = t[i].numel;
    out[i].rows = t[i].rows;
    out[i].cols = t[i].cols;
  }
  *n_out = n;
  *flat_numel = total;
  return MT_OK;
}

extern "C" mt_status mt_device_requirements(const mt_config* cfg, mt_device_req* out) {
  if (!cfg || !out) return MT_E_ARG;
  mt::Plan p;
  if (!mt::make_plan(*cfg, &p).empty()) return MT_E_ARG;
  std::memset(out, 0, sizeof(*out));
  out->weight_buf = p.weight_buf_bytes;
  out->grad_slab = p.slab_bytes;
  out->window = p.window_bytes;
  out->checkpoints = p.ckpt_bytes;
  out->workspace = p.ws.bytes;
  out->device_total = 2 * p.weight_buf_bytes + (size_t)cfg->n_grad_slabs * p.slab_bytes +
                      p.window_bytes + p.ckpt_bytes + p.ws.bytes;
  int64_t nparams = (int64_t)cfg->vocab * cfg->hidden;  // embedding
  nparams += p.head[0].numel + p.head[1].numel;
  int64_t block_elems = 0;
  for (int l = 0; l < cfg->n_layers; ++l) {
    for (int i = 0; i < mt::T_COUNT; ++i) nparams += p.block_layout(l)[i].numel;
    block_elems += p.block_elems(l);
  }
  out->host_state = (size_t)nparams * 16;
  const size_t T = (size_t)p.T;
  out->pinned_host = (size_t)(block_elems + p.head_elems) * 2 +
                     (size_t)cfg->n_grad_slabs * p.slab_bytes + 4 * T * cfg->hidden * 4 +
                     2 * T * 4 + 4096 * 4;
  out->unit_elems = p.unit_elems;
  out->head_chunks = p.n_chunks;
  return MT_OK;
}
