// Host-side plan of the qkv library: configuration checks, arena layout and
// per-layer stream state.  Contains no HIP code so that it can be compiled and
// tested on a machine without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/qkv.h"

namespace qkv {

constexpr int kMaxChunks = 256;      // snapshot slots per stream (header size)
constexpr int kMaxSplits = 8;        // split-KV partitions of one attention call
constexpr int kRefitParts = 8;       // adapted-predictor re-fit: token ranges summed apart, then in order
constexpr int kSortMaxClusters = 4096;  // k-means update through per-tile sorts up to this C
constexpr int kChanParts = 64;       // outlier flags: token ranges whose channel sums are kept apart
constexpr uint64_t kAlign = 256;
constexpr uint64_t kNoAllocScratchBytes = uint64_t(128) << 20;  // qkv_attend_noalloc partials, per GPU

inline uint64_t align_up(uint64_t v, uint64_t a = kAlign) { return (v + a - 1) / a * a; }

// Device-side header at the start of every (layer, K|V) stream region.
// start[c] is the first token of chunk c; entries at or beyond n_chunks are
// not read by any kernel.
struct StreamHeader {
  int32_t n_chunks;
  int32_t n_tokens;
  int32_t start[kMaxChunks + 1];
};

// Byte offsets and strides of one stream, relative to the stream's base.
struct StreamLayout {
  uint64_t header_off;
  uint64_t codes_off, codes_stage, codes_head, codes_token;
  uint64_t meta_off, meta_stage, meta_head, meta_token;
  uint64_t ids_off, ids_head, id_bytes;
  uint64_t cb_off, cb_chunk, cb_head, cb_row;
  uint64_t cn_off, cn_chunk, cn_head;
  uint64_t mask_off, mask_chunk, mask_head;   // outlier channel flags (0 when off)
  uint64_t bytes;      // whole stream, aligned
};

struct Plan {
  qkv_config cfg;
  StreamLayout s;
  uint64_t streams_bytes;     // 2 * L * s.bytes
  // scratch, shared by the calls of one context (they are ordered on the device)
  uint64_t scratch_off, scratch_bytes;
  uint64_t attn_part_o_off, attn_part_lse_off;     // relative to scratch
  uint64_t xl_pred_off, xl_chain_off, xl_proj_off; // relative to scratch
  uint64_t xl_refit_off;                           // absolute: [L][2][H][d][d] bf16 (adapted mode)
  uint64_t xl_gram_off;                            // relative to scratch (adapted mode re-fit)
  uint64_t sort_perm_off, sort_off_off;            // relative to scratch (encode)
  uint64_t sort_tiles;                             // 256-token tiles per call, max
  uint64_t chan_part_off;                          // relative to scratch: [2L][H][kChanParts][d] fp64
  // cross-layer read: bf16 reconstruction of one layer (the last one read),
  // in blocks of xl_sweep_slice tokens, each [2][H][n_s][d] (absolute offset;
  // 0 bytes when the mode or attention is off)
  uint64_t xl_sweep_off, xl_sweep_bytes;
  int64_t xl_sweep_slice;
  uint64_t total_bytes;
  int kv_elem_bytes;
};

// Returns QKV_OK and fills plan, or a negative status.
int make_plan(const qkv_config *cfg, Plan *plan);

struct LayerState {
  int64_t n_tokens = 0;
  std::vector<int64_t> starts;   // first token of each chunk
};

}  // namespace qkv

struct qkv_ctx {
  qkv::Plan plan;
  uint8_t *arena = nullptr;
  uint64_t arena_bytes = 0;
  const uint8_t *predictor = nullptr;
  std::vector<qkv::LayerState> layers;
  // cross-layer chain: bf16 reconstruction of layer `chain_layer` for tokens
  // [chain_t0, chain_t0 + chain_n) is held in scratch after an encode call
  int32_t chain_layer = -1;
  int64_t chain_t0 = 0, chain_n = 0;
  // cross-layer read: the sweep region holds the bf16 reconstruction of
  // layer sweep_layer over its first sweep_tokens tokens (-1: nothing valid)
  int32_t sweep_layer = -1;
  int64_t sweep_tokens = 0;
  int n_cu = 0;                  // compute units of the device, read at the first attention call
  void *noalloc_scratch = nullptr; // this device's fixed partials array (qkv_attend_noalloc), set at init
  // per-kernel timing (qkv_trace): HIP events (as void*) recorded around each
  // launch while tracing is on; the pool is reused after every read
  struct TraceMark { std::string name; void *begin, *end; };
  int trace = 0;
  std::vector<TraceMark> trace_marks;
  std::vector<void *> trace_pool;
  size_t trace_used = 0;
  int last_hip_error = 0;
  std::string last_error;
};

namespace qkv {

// Validation of each entry point's arguments against the context state.
// These run before anything is enqueued and never touch device memory.
int check_encode(const qkv_ctx *ctx, int32_t layer0, int32_t n_layers, const void *k,
                 const void *v, int64_t n);
int check_attend(const qkv_ctx *ctx, int32_t layer, const void *q, int64_t n_q, int32_t q_dtype,
                 const void *out, int32_t out_dtype);
// cross-layer mode, layer >= 1: the read of `layer` needs the sweep region to
// hold layer-1 over every token of `layer` (QKV_OK, else QKV_E_STATE)
int check_sweep(const qkv_ctx *ctx, int32_t layer);
int check_reconstruct(const qkv_ctx *ctx, int32_t layer0, int32_t n_layers, int32_t kv, int64_t t0,
                      int64_t t1, const void *out, int32_t out_dtype);
int check_rewind(const qkv_ctx *ctx, int32_t layer0, int32_t n_layers, int64_t n_tokens);
int check_attend_with_chunk(const qkv_ctx *ctx, int32_t layer, const void *q, int64_t n_q, int32_t q_dtype,
                            const void *k_new, const void *v_new, int64_t n_new, const void *out,
                            int32_t out_dtype);

// Work split of an attention call (stream-K): the (head, query block of
// 256, key tile of 64) units are dealt out in runs of units_per_block
// consecutive units, one run per block, about one block per compute unit.
struct AttnSplit {
  int64_t n_qblocks, n_ktiles, units_per_block, n_blocks, max_segments;
  int64_t head_blocks, main_tiles;      // per-head split (head_blocks = 0: plain stream-K)
};
// key_bytes: bytes one key costs the read over all heads, K and V (packed:
// packed_key_bytes; uncoded bf16 rows: bf16_key_bytes).  max_splits bounds the
// blocks sharing one query block (partial slots used).
AttnSplit attention_split(const Plan &p, int64_t n_keys, int64_t n_q, int n_cu, uint64_t key_bytes,
                          int max_splits = kMaxSplits);
uint64_t packed_key_bytes(const Plan &p);
uint64_t bf16_key_bytes(const Plan &p);
// The per-head split pays when the keys read by one call do not stay in the
// device's last-level (MALL, 256 MiB) cache.
constexpr uint64_t kHeadSplitMinBytes = uint64_t(256) << 20;

// Byte offset of stream (layer, kv) from the arena base.
inline uint64_t stream_offset(const Plan &p, int layer, int kv) {
  return (uint64_t(layer) * 2 + uint64_t(kv)) * p.s.bytes;
}

}  // namespace qkv
