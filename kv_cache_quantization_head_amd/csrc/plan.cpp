// Host-side plan of the qkv library (no HIP): configuration checks, arena
// layout, per-call argument validation and the context's bookkeeping entry
// points.  See include/qkv.h for the contract.
#include "plan.h"

#include <algorithm>
#include <cstring>

namespace qkv {

static bool valid_dtype(int32_t t) { return t == QKV_F32 || t == QKV_BF16; }

int make_plan(const qkv_config *cfg, Plan *plan) {
  if (!cfg || !plan) return QKV_E_INVAL;
  const qkv_config &c = *cfg;
  if (c.n_layers < 1 || c.n_heads < 1) return QKV_E_INVAL;
  if (c.head_dim != 64 && c.head_dim != 128) return QKV_E_INVAL;
  if (c.n_clusters < 1 || c.n_clusters > 65535) return QKV_E_INVAL;
  if (c.n_stages < 1 || c.n_stages > 4) return QKV_E_INVAL;
  if (c.bits != 2 && c.bits != 4) return QKV_E_INVAL;
  if (c.group_size != 32 && c.group_size != 64) return QKV_E_INVAL;
  if (c.head_dim % c.group_size) return QKV_E_INVAL;
  if (c.kmeans_iters < 0 || c.kmeans_iters > 64) return QKV_E_INVAL;
  if (c.max_tokens < 1 || c.max_tokens >= (int64_t(1) << 31)) return QKV_E_INVAL;
  if (c.max_chunk_tokens < 0 || c.max_chunk_tokens > c.max_tokens) return QKV_E_INVAL;
  if (c.max_chunks < 1 || c.max_chunks > kMaxChunks) return QKV_E_INVAL;
  if (!valid_dtype(c.kv_dtype)) return QKV_E_INVAL;
  if (c.max_query_tokens < 0 || c.max_query_tokens >= (int64_t(1) << 31)) return QKV_E_INVAL;
  if (c.xlayer != 0 && c.xlayer != 1) return QKV_E_INVAL;
  if (c.codebook_reuse != 0 && c.codebook_reuse != 1) return QKV_E_INVAL;
  if (c.xlayer_adapt != 0 && (c.xlayer_adapt != 1 || !c.xlayer)) return QKV_E_INVAL;
  if (c.outlier_channels != 0 && (c.outlier_channels != 1 || c.xlayer)) return QKV_E_INVAL;
  if (c.xlayer) {
    if (c.xlayer_rank < 1 || c.xlayer_rank > 64) return QKV_E_INVAL;
    if (c.kv_dtype != QKV_BF16) return QKV_E_INVAL;
  }
  // element counts that kernels index with 32-bit arithmetic per head
  if (int64_t(c.n_heads) * c.head_dim * 4 > (int64_t(1) << 30)) return QKV_E_INVAL;

  Plan p{};
  p.cfg = c;
  if (p.cfg.max_chunk_tokens == 0) p.cfg.max_chunk_tokens = c.max_tokens;
  const uint64_t H = c.n_heads, d = c.head_dim, T = c.max_tokens, S = c.n_stages;
  const uint64_t C = c.n_clusters, G = c.group_size, K = c.max_chunks;
  p.kv_elem_bytes = c.kv_dtype == QKV_BF16 ? 2 : 4;
  // one head's slice of one call's input is addressed with 32-bit offsets
  if (uint64_t(p.cfg.max_chunk_tokens) * uint64_t(c.head_dim) * p.kv_elem_bytes >= (uint64_t(1) << 31))
    return QKV_E_INVAL;

  StreamLayout &s = p.s;
  uint64_t off = 0;
  s.header_off = off;
  off = align_up(off + sizeof(StreamHeader));
  s.codes_token = d * c.bits / 8;
  s.codes_head = T * s.codes_token;
  s.codes_stage = H * s.codes_head;
  s.codes_off = off;
  off = align_up(off + S * s.codes_stage);
  const uint64_t outl = c.outlier_channels ? 1 : 0;
  s.meta_token = (d / G + outl) * 4;
  s.meta_head = T * s.meta_token;
  s.meta_stage = H * s.meta_head;
  s.meta_off = off;
  off = align_up(off + S * s.meta_stage);
  // the fused read addresses one head's codes and (sigma, z) of one stage
  // with 32-bit offsets
  if (s.codes_head >= (uint64_t(1) << 32) || s.meta_head >= (uint64_t(1) << 32)) return QKV_E_INVAL;
  s.id_bytes = C <= 256 ? 1 : 2;
  s.ids_head = T * s.id_bytes;
  s.ids_off = off;
  off = align_up(off + H * s.ids_head);
  // one snapshot per chunk, or one per stream (codebook reuse: stride 0)
  const uint64_t snaps = c.codebook_reuse ? 1 : K;
  s.cb_row = d * p.kv_elem_bytes;
  s.cb_head = C * s.cb_row;
  s.cb_chunk = c.codebook_reuse ? 0 : H * s.cb_head;
  s.cb_off = off;
  off = align_up(off + snaps * H * s.cb_head);
  s.cn_head = C * 4;
  s.cn_chunk = c.codebook_reuse ? 0 : H * s.cn_head;
  s.cn_off = off;
  off = align_up(off + snaps * H * s.cn_head);
  // outlier channel flags: one d-bit mask per head and encode call
  s.mask_head = outl ? d / 8 : 0;
  s.mask_chunk = H * s.mask_head;
  s.mask_off = outl ? off : 0;
  if (outl) off = align_up(off + K * s.mask_chunk);
  s.bytes = off;

  p.streams_bytes = 2 * uint64_t(c.n_layers) * s.bytes;
  // re-fitted predictor blocks (adapted cross-layer mode), kept between calls
  p.xl_refit_off = p.streams_bytes;
  const uint64_t refit_bytes = c.xlayer_adapt ? align_up(uint64_t(c.n_layers) * 2 * H * d * d * 2) : 0;
  // cross-layer read: one layer's bf16 K and V in blocks of the chunk size
  p.xl_sweep_slice = p.cfg.max_chunk_tokens;
  p.xl_sweep_off = p.streams_bytes + refit_bytes;
  p.xl_sweep_bytes = 0;
  if (c.xlayer && c.max_query_tokens > 0) {
    const uint64_t slices = (T + uint64_t(p.xl_sweep_slice) - 1) / uint64_t(p.xl_sweep_slice);
    p.xl_sweep_bytes = align_up(slices * 2 * H * uint64_t(p.xl_sweep_slice) * d * 2);
  }
  p.scratch_off = p.xl_sweep_off + p.xl_sweep_bytes;
  uint64_t attn = 0;
  if (c.max_query_tokens > 0) {
    const uint64_t Q = c.max_query_tokens;
    p.attn_part_o_off = 0;
    p.attn_part_lse_off = align_up(uint64_t(kMaxSplits) * H * Q * d * 4);
    attn = align_up(p.attn_part_lse_off + uint64_t(kMaxSplits) * H * Q * 4);
  }
  uint64_t xl = 0;
  if (c.xlayer) {
    const uint64_t M = p.cfg.max_chunk_tokens;
    p.xl_pred_off = 0;
    p.xl_chain_off = align_up(2 * H * M * d * 4);
    p.xl_proj_off = align_up(p.xl_chain_off + 2 * H * M * d * 2);
    xl = align_up(p.xl_proj_off + 2 * M * uint64_t(c.xlayer_rank) * 4);
  }
  // per-tile stable sort of a call's cluster ids (k-means update): for every
  // (layer of the call, K|V, head, 256-token tile) a permutation (u8 x 256)
  // and per-cluster offsets (u16 x (C+1)); placed after the cross-layer
  // buffers, which the encoder uses at the same time
  p.sort_tiles = (uint64_t(p.cfg.max_chunk_tokens) + 255) / 256;
  const uint64_t units = C <= uint64_t(kSortMaxClusters) ? 2 * uint64_t(c.n_layers) * H * p.sort_tiles : 0;
  p.sort_perm_off = xl;
  p.sort_off_off = align_up(p.sort_perm_off + units * 256);
  uint64_t enc = align_up(p.sort_off_off + units * (C + 1) * 2);
  // re-fit sums: [parts][2 kv][2 matrices][H][d][d] fp64 (adapted mode)
  p.xl_gram_off = enc;
  if (c.xlayer_adapt) enc = align_up(enc + uint64_t(kRefitParts) * 4 * H * d * d * 8);
  // outlier flags: per-range channel sums of squares of the residual
  p.chan_part_off = enc;
  if (outl) enc = align_up(enc + 2 * uint64_t(c.n_layers) * H * kChanParts * d * 8);
  p.scratch_bytes = std::max(attn, enc);
  p.total_bytes = p.scratch_off + p.scratch_bytes;
  *plan = p;
  return QKV_OK;
}

static bool layer_range_ok(const qkv_ctx *ctx, int32_t layer0, int32_t n_layers) {
  return layer0 >= 0 && n_layers >= 1 &&
         int64_t(layer0) + n_layers <= int64_t(ctx->plan.cfg.n_layers);
}

int check_encode(const qkv_ctx *ctx, int32_t layer0, int32_t n_layers, const void *k,
                 const void *v, int64_t n) {
  if (!ctx) return QKV_E_INVAL;
  if (!layer_range_ok(ctx, layer0, n_layers) || !k || !v || n < 1) return QKV_E_INVAL;
  const qkv_config &c = ctx->plan.cfg;
  if (n > c.max_chunk_tokens) return QKV_E_CAPACITY;
  const LayerState &first = ctx->layers[layer0];
  for (int l = layer0; l < layer0 + n_layers; ++l) {
    const LayerState &ls = ctx->layers[l];
    if (ls.n_tokens != first.n_tokens || ls.starts.size() != first.starts.size()) return QKV_E_STATE;
    if (ls.n_tokens + n > c.max_tokens) return QKV_E_CAPACITY;
    if (int64_t(ls.starts.size()) + 1 > c.max_chunks) return QKV_E_CAPACITY;
  }
  if (c.xlayer && layer0 > 0) {
    if (ctx->chain_layer != layer0 - 1 || ctx->chain_t0 != first.n_tokens || ctx->chain_n != n)
      return QKV_E_STATE;
  }
  return QKV_OK;
}

int check_attend(const qkv_ctx *ctx, int32_t layer, const void *q, int64_t n_q, int32_t q_dtype,
                 const void *out, int32_t out_dtype) {
  if (!ctx) return QKV_E_INVAL;
  if (layer < 0 || layer >= ctx->plan.cfg.n_layers) return QKV_E_INVAL;
  if (!valid_dtype(q_dtype) || !valid_dtype(out_dtype) || n_q < 0) return QKV_E_INVAL;
  if (n_q > 0 && (!q || !out)) return QKV_E_INVAL;
  if (n_q > ctx->plan.cfg.max_query_tokens) return QKV_E_CAPACITY;
  if (ctx->layers[layer].n_tokens == 0) return QKV_E_STATE;
  return check_sweep(ctx, layer);
}

int check_sweep(const qkv_ctx *ctx, int32_t layer) {
  if (!ctx->plan.cfg.xlayer || layer == 0) return QKV_OK;
  if (ctx->sweep_layer != layer - 1 || ctx->sweep_tokens != ctx->layers[layer].n_tokens) return QKV_E_STATE;
  return QKV_OK;
}

int check_attend_with_chunk(const qkv_ctx *ctx, int32_t layer, const void *q, int64_t n_q, int32_t q_dtype,
                            const void *k_new, const void *v_new, int64_t n_new, const void *out,
                            int32_t out_dtype) {
  if (!ctx) return QKV_E_INVAL;
  if (layer < 0 || layer >= ctx->plan.cfg.n_layers) return QKV_E_INVAL;
  if (!valid_dtype(q_dtype) || !valid_dtype(out_dtype) || n_q < 0) return QKV_E_INVAL;
  if (n_new < 0 || n_new >= (int64_t(1) << 31)) return QKV_E_INVAL;
  if (n_q > 0 && (!q || !out)) return QKV_E_INVAL;
  if (n_new > 0 && (!k_new || !v_new)) return QKV_E_INVAL;
  if (n_q > ctx->plan.cfg.max_query_tokens) return QKV_E_CAPACITY;
  if (ctx->layers[layer].n_tokens == 0 && n_new == 0) return QKV_E_STATE;
  if (ctx->layers[layer].n_tokens > 0) return check_sweep(ctx, layer);
  return QKV_OK;
}

int check_reconstruct(const qkv_ctx *ctx, int32_t layer0, int32_t n_layers, int32_t kv, int64_t t0,
                      int64_t t1, const void *out, int32_t out_dtype) {
  if (!ctx) return QKV_E_INVAL;
  if (!layer_range_ok(ctx, layer0, n_layers) || (kv != 0 && kv != 1)) return QKV_E_INVAL;
  if (!valid_dtype(out_dtype) || t0 < 0 || t1 < t0) return QKV_E_INVAL;
  if (t1 > t0 && !out) return QKV_E_INVAL;
  for (int l = layer0; l < layer0 + n_layers; ++l)
    if (t1 > ctx->layers[l].n_tokens) return QKV_E_STATE;
  if (ctx->plan.cfg.xlayer && t1 > t0) {
    // layers >= 1 are rebuilt through the chain from layer 0: every layer up to
    // the last requested one must hold the range
    for (int l = 0; l < layer0 + n_layers; ++l)
      if (t1 > ctx->layers[l].n_tokens) return QKV_E_STATE;
  }
  return QKV_OK;
}

int check_rewind(const qkv_ctx *ctx, int32_t layer0, int32_t n_layers, int64_t n_tokens) {
  if (!ctx) return QKV_E_INVAL;
  if (!layer_range_ok(ctx, layer0, n_layers) || n_tokens < 0) return QKV_E_INVAL;
  for (int l = layer0; l < layer0 + n_layers; ++l) {
    const LayerState &ls = ctx->layers[l];
    if (n_tokens > ls.n_tokens) return QKV_E_STATE;
    if (n_tokens == ls.n_tokens) continue;
    if (std::find(ls.starts.begin(), ls.starts.end(), n_tokens) == ls.starts.end())
      return QKV_E_STATE;
  }
  return QKV_OK;
}

uint64_t packed_key_bytes(const Plan &p) {
  const uint64_t S = p.cfg.n_stages;
  return 2 * uint64_t(p.cfg.n_heads) * (S * p.s.codes_token + S * p.s.meta_token + p.s.id_bytes);
}
uint64_t bf16_key_bytes(const Plan &p) { return 2 * uint64_t(p.cfg.n_heads) * p.cfg.head_dim * 2; }

AttnSplit attention_split(const Plan &p, int64_t n_keys, int64_t n_q, int n_cu, uint64_t key_bytes,
                          int max_splits) {
  AttnSplit w{};
  w.n_qblocks = (n_q + 255) / 256;
  w.n_ktiles = std::max<int64_t>(1, (n_keys + 63) / 64);
  const int64_t total = w.n_qblocks * w.n_ktiles * p.cfg.n_heads;
  const int64_t cus = std::max(n_cu, 1);
  // one run per compute unit, but no query block shared by more than
  // max_splits blocks (partial slots of the scratch region)
  const int64_t ms = std::max(2, std::min(max_splits, kMaxSplits));
  // Per-head split when the keys do not stay in the MALL and every query
  // block of a head can have a block of its own: head h gets B = n_cu / H
  // blocks; its n_qblocks query blocks sweep key tiles [0, M) side by side
  // (they read the same tiles at about the same time, and consecutive blocks
  // share an XCD's L2), and the other B - n_qblocks blocks take the tails
  // [M, T) of all its query blocks.
  const int64_t H = p.cfg.n_heads, B = cus / H;
  if (uint64_t(n_keys) * key_bytes > kHeadSplitMinBytes && H <= cus && B >= w.n_qblocks) {
    const int64_t U = (w.n_qblocks * w.n_ktiles + B - 1) / B;
    const int64_t M = std::min(U, w.n_ktiles), tail = w.n_ktiles - M;
    // a tail of `tail` units meets at most ceil(tail / U) + 1 runs
    const int64_t segs = M == w.n_ktiles ? 1 : 2 + (tail + U - 1) / U;
    if (segs <= ms) {
      w.head_blocks = B;
      w.main_tiles = M;
      w.units_per_block = U;
      w.n_blocks = (H * B + 7) / 8 * 8;
      w.max_segments = segs;
      return w;
    }
  }
  w.units_per_block = std::max((total + cus - 1) / cus, (w.n_ktiles + ms - 2) / (ms - 1));
  w.n_blocks = (total + w.units_per_block - 1) / w.units_per_block;
  // blocks meeting one query block: at most ceil((T - 1) / U) + 1
  w.max_segments = std::min<int64_t>(ms, (w.n_ktiles - 1 + w.units_per_block - 1) / w.units_per_block + 1);
  return w;
}

}  // namespace qkv

using namespace qkv;

extern "C" size_t qkv_workspace_bytes(const qkv_config *cfg) {
  Plan p;
  if (make_plan(cfg, &p) != QKV_OK) return 0;
  return size_t(p.total_bytes);
}

extern "C" int qkv_layout(const qkv_ctx *ctx, int32_t layer, int32_t kv, qkv_layout_desc *out) {
  if (!ctx || !out || layer < 0 || layer >= ctx->plan.cfg.n_layers || (kv != 0 && kv != 1))
    return QKV_E_INVAL;
  const Plan &p = ctx->plan;
  const uint64_t base = stream_offset(p, layer, kv);
  qkv_layout_desc d{};
  d.codes_off = base + p.s.codes_off;
  d.codes_stage_stride = p.s.codes_stage;
  d.codes_head_stride = p.s.codes_head;
  d.codes_token_stride = p.s.codes_token;
  d.meta_off = base + p.s.meta_off;
  d.meta_stage_stride = p.s.meta_stage;
  d.meta_head_stride = p.s.meta_head;
  d.meta_token_stride = p.s.meta_token;
  d.ids_off = base + p.s.ids_off;
  d.ids_head_stride = p.s.ids_head;
  d.id_bytes = p.s.id_bytes;
  d.codebook_off = base + p.s.cb_off;
  d.codebook_chunk_stride = p.s.cb_chunk;
  d.codebook_head_stride = p.s.cb_head;
  d.cnorm_off = base + p.s.cn_off;
  d.cnorm_chunk_stride = p.s.cn_chunk;
  d.cnorm_head_stride = p.s.cn_head;
  d.chmask_off = p.s.mask_off ? base + p.s.mask_off : 0;
  d.chmask_chunk_stride = p.s.mask_chunk;
  d.chmask_head_stride = p.s.mask_head;
  d.n_tokens = ctx->layers[layer].n_tokens;
  d.n_chunks = int32_t(ctx->layers[layer].starts.size());
  *out = d;
  return QKV_OK;
}

extern "C" int qkv_chunk_starts(const qkv_ctx *ctx, int32_t layer, int64_t *starts, int32_t max) {
  if (!ctx || layer < 0 || layer >= ctx->plan.cfg.n_layers || max < 0) return QKV_E_INVAL;
  const LayerState &ls = ctx->layers[layer];
  const int n = int(ls.starts.size());
  if (starts)
    for (int i = 0; i < n && i < max; ++i) starts[i] = ls.starts[i];
  return n;
}

extern "C" const char *qkv_status_string(const qkv_ctx *ctx, int status) {
  switch (status) {
    case QKV_OK: return "ok";
    case QKV_E_INVAL: return "invalid argument or configuration";
    case QKV_E_CAPACITY: return "capacity exceeded (tokens, chunk size, chunks or queries)";
    case QKV_E_STATE: return "call not valid in the current state";
    case QKV_E_ARENA: return "arena too small or not 256-byte aligned";
    case QKV_E_HIP:
      if (ctx && !ctx->last_error.empty()) return ctx->last_error.c_str();
      return "HIP error";
    case QKV_E_UNSUPPORTED: return "not supported";
    default: return "unknown status";
  }
}
