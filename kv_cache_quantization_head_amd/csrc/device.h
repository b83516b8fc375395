// Shared device-side definitions of the qkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace qkv {

// Layout of one (layer, K|V) stream passed by value to kernels.
struct DevLayout {
  uint64_t stream_bytes, header_off;
  uint64_t codes_off, codes_stage, codes_head, codes_token;
  uint64_t meta_off, meta_stage, meta_head, meta_token;
  uint64_t ids_off, ids_head;
  uint64_t cb_off, cb_chunk, cb_head, cb_row;
  uint64_t cn_off, cn_chunk, cn_head;
  uint64_t mask_off, mask_chunk, mask_head;   // outlier channel flags (mask_off 0: option off)
  int32_t H, D, C, S, bits, G, id_bytes, kv_bf16;
};

inline DevLayout dev_layout(const Plan &p) {
  DevLayout d{};
  const StreamLayout &s = p.s;
  d.stream_bytes = s.bytes;
  d.header_off = s.header_off;
  d.codes_off = s.codes_off; d.codes_stage = s.codes_stage; d.codes_head = s.codes_head;
  d.codes_token = s.codes_token;
  d.meta_off = s.meta_off; d.meta_stage = s.meta_stage; d.meta_head = s.meta_head;
  d.meta_token = s.meta_token;
  d.ids_off = s.ids_off; d.ids_head = s.ids_head;
  d.cb_off = s.cb_off; d.cb_chunk = s.cb_chunk; d.cb_head = s.cb_head; d.cb_row = s.cb_row;
  d.cn_off = s.cn_off; d.cn_chunk = s.cn_chunk; d.cn_head = s.cn_head;
  d.mask_off = s.mask_off; d.mask_chunk = s.mask_chunk; d.mask_head = s.mask_head;
  d.H = p.cfg.n_heads; d.D = p.cfg.head_dim; d.C = p.cfg.n_clusters; d.S = p.cfg.n_stages;
  d.bits = p.cfg.bits; d.G = p.cfg.group_size; d.id_bytes = int32_t(s.id_bytes);
  d.kv_bf16 = p.cfg.kv_dtype == QKV_BF16;
  return d;
}

// Arguments of the encode kernels.  Streams of one launch are the 2*n_layers
// (layer, K|V) pairs starting at layer0 (blockIdx.z = 2*layer_rel + kv) unless
// `single_kv_layer` >= 0 (cross-layer mode: one layer, blockIdx.z = kv).
struct EncodeArgs {
  DevLayout L;
  uint8_t *arena;
  const uint8_t *k_in, *v_in;   // [n_layers][H][n][D] cache dtype
  int32_t layer0;
  int32_t n;                    // tokens of this call
  int32_t t0;                   // first token of the chunk in every stream
  int32_t slot;                 // snapshot slot of this chunk
  int32_t prev_slot;            // warm-start slot, -1 for strided init
  // cross-layer coding: base = pred instead of the centroid, reconstruction
  // written to chain (both [2][H][n][D], f32 / bf16)
  const float *pred;
  uint16_t *chain;
  // k-means update: per-tile stable sort of the ids
  uint8_t *sort_perm;           // [streams][H][tiles][256] u8 token offsets sorted by (id, t)
  uint16_t *sort_off;           // [streams][H][tiles][C+1] start of each cluster in the tile
  int32_t sort_tiles;           // tile stride of the two arrays
  double *chan_part;            // outlier flags: [streams][H][kChanParts][D] sums of r^2
};

struct ReconArgs {
  DevLayout L;
  const uint8_t *arena;
  int32_t layer0, kv;
  int32_t t0, n;                // tokens [t0, t0+n) of each layer
  void *out;                    // [n_layers][H][n][D], or null
  int32_t out_bf16;
  const float *pred;            // cross-layer base [H][n][D] for this kv, or null
  uint16_t *chain;              // bf16 copy of the output [H][n][D], or null
};

struct AttnArgs {
  DevLayout L;
  const uint8_t *stream_k, *stream_v;   // stream bases of the layer
  const void *q;                        // [H][n_q][D]
  int32_t q_bf16;
  int32_t n_q, n_keys;
  // stream-K work split over (head, query block, key tile) units
  int32_t n_qblocks;                    // query blocks of 256
  int32_t n_ktiles;                     // key tiles of 64 (at least 1)
  int32_t units_per_block;              // consecutive units per block
  // per-head split (0: plain stream-K): head_blocks blocks per head; the
  // first n_qblocks each take key tiles [0, main_tiles) of one query block,
  // the others the remaining tiles of all its query blocks in runs of
  // units_per_block
  int32_t head_blocks, main_tiles;
  int32_t max_segments;                 // most blocks sharing one query block
  int32_t xcd_remap;                    // number blocks XCD by XCD (grid % 8 == 0)
  void *out;                            // final [H][n_q][D]
  int32_t out_bf16;
  float *lse;                           // final [H][n_q] or null
  float *part_o;                        // [max_segments][H][n_q][D] partials
  float *part_lse;                      // [max_segments][H][n_q]
  const uint16_t *k_new, *v_new;        // fresh keys/values [H][n_keys][D] bf16 (uncoded read)
  // uncoded read of the cross-layer sweep region instead: consecutive blocks
  // of fresh_slice tokens, block s = [2 (K, V)][H][n_s][D] bf16 at
  // k_new + s * 2 * H * fresh_slice * D (0: the plain layout above)
  int32_t fresh_slice;
};

// LSE merge of two complete attention results over disjoint key sets.
struct MergeArgs {
  int32_t H, D, n_q;
  const float *o1, *lse1, *o2, *lse2;   // [H][n_q][D], [H][n_q]
  void *out;                            // [H][n_q][D]
  int32_t out_bf16;
  float *lse;                           // [H][n_q] or null
};

struct XlArgs {
  int32_t H, D, r, n;
  const uint16_t *chain;       // [2][H][n][D] bf16 reconstruction of the source layer
  const uint16_t *weights;     // predictor block of the source layer: per kv B, U, V
  uint64_t kv_weight_stride;   // elements between the K and V blocks
  float *proj;                 // [2][n][r] bf16-rounded projections (as f32)
  float *pred;                 // [2][H][n][D]
  // adapted predictor: when set, B of head h of tensor kv is read from
  // b_weights + (kv*H + h)*D*D instead of the caller's block
  const uint16_t *b_weights;
  int32_t lowrank_only;        // pred = U w only (the block term left out)
  int32_t skip_project;        // proj already holds this call's projections
};

// Adapted-predictor re-fit of one target layer (all heads, K and V).
struct RefitArgs {
  int32_t H, D, n;
  const uint16_t *chain;       // [2][H][n][D] bf16 y (source layer reconstruction)
  const uint8_t *k_in, *v_in;  // [H][n][D] bf16 target layer tokens
  const float *low_rank;       // [2][H][n][D] U w (the pred buffer of a low-rank-only prediction)
  double *gram;                // [kRefitParts][2 kv][2 mats][H][D][D]: y y^T and y (x - U w)^T
  uint16_t *b_out;             // [2][H][D][D] bf16 re-fitted blocks
};

// Optional per-kernel timing (qkv_trace): while a sink is installed for the
// duration of a call, every kernel launch is bracketed by two HIP events
// recorded on the launch's stream.  `label` is the stringified kernel
// expression; the sink keeps the kernel's base name.
struct TraceSink {
  virtual void begin(const char *label, hipStream_t st) = 0;
  virtual void end(hipStream_t st) = 0;
};
extern thread_local TraceSink *t_trace;

#define QKV_LAUNCH(KERNEL, GRID, BLOCK, LDS, ST, ...)                         \
  do {                                                                        \
    if (::qkv::t_trace) ::qkv::t_trace->begin(#KERNEL, ST);                   \
    hipLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, ST, __VA_ARGS__);            \
    if (::qkv::t_trace) ::qkv::t_trace->end(ST);                              \
  } while (0)

}  // namespace qkv
