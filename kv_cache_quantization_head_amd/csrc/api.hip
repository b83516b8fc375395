// C-ABI entry points of the qkv library (see include/qkv.h).  Each call
// validates its arguments on the host (plan.cpp), then enqueues the kernels
// of the kernel sources on the caller's stream and updates the host bookkeeping.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "device.h"
#include "launch.h"
#include "plan.h"

using namespace qkv;

static int hip_status(qkv_ctx *ctx) {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return QKV_OK;
  ctx->last_hip_error = int(e);
  ctx->last_error = std::string("HIP error: ") + hipGetErrorString(e);
  return QKV_E_HIP;
}

static uint8_t *scratch(qkv_ctx *ctx, uint64_t off) { return ctx->arena + ctx->plan.scratch_off + off; }

namespace qkv {
thread_local TraceSink *t_trace = nullptr;
}

// Records the launches of one call on ctx while tracing is on: installed as
// the thread's trace sink for the lifetime of the scope.
class TraceScope final : public TraceSink {
 public:
  explicit TraceScope(qkv_ctx *ctx) : ctx_(ctx) {
    if (ctx_->trace) t_trace = this;
  }
  ~TraceScope() {
    if (t_trace == this) t_trace = nullptr;
  }
  void begin(const char *label, hipStream_t st) override {
    // "(k_name<...>)" -> "k_name"
    const char *p = label;
    while (*p == '(' || *p == ' ') ++p;
    const char *e = p;
    while (*e && *e != '<' && *e != ')' && *e != ' ') ++e;
    name_.assign(p, size_t(e - p));
    open_ = event();
    if (open_) (void)hipEventRecord(static_cast<hipEvent_t>(open_), st);
  }
  void end(hipStream_t st) override {
    void *close = event();
    if (!open_ || !close) return;
    (void)hipEventRecord(static_cast<hipEvent_t>(close), st);
    ctx_->trace_marks.push_back({name_, open_, close});
    open_ = nullptr;
  }

 private:
  void *event() {
    if (ctx_->trace_used == ctx_->trace_pool.size()) {
      hipEvent_t ev = nullptr;
      if (hipEventCreate(&ev) != hipSuccess) return nullptr;
      ctx_->trace_pool.push_back(ev);
    }
    return ctx_->trace_pool[ctx_->trace_used++];
  }
  qkv_ctx *ctx_;
  void *open_ = nullptr;
  std::string name_;
};

extern "C" void qkv_destroy(qkv_ctx *ctx) {
  if (!ctx) return;
  for (void *ev : ctx->trace_pool) (void)hipEventDestroy(static_cast<hipEvent_t>(ev));
  delete ctx;
}

extern "C" int qkv_trace(qkv_ctx *ctx, int32_t enable) {
  if (!ctx || (enable != 0 && enable != 1)) return QKV_E_INVAL;
  ctx->trace = enable;
  return QKV_OK;
}

extern "C" int qkv_trace_read(qkv_ctx *ctx, qkv_trace_entry *out, int32_t max) {
  if (!ctx || max < 0) return QKV_E_INVAL;
  std::vector<std::string> names;
  std::vector<int64_t> counts;
  std::vector<double> sums;
  int rc = QKV_OK;
  for (const auto &m : ctx->trace_marks) {
    float ms = 0.0f;
    if (hipEventSynchronize(static_cast<hipEvent_t>(m.end)) != hipSuccess ||
        hipEventElapsedTime(&ms, static_cast<hipEvent_t>(m.begin), static_cast<hipEvent_t>(m.end)) != hipSuccess) {
      rc = QKV_E_HIP;
      break;
    }
    size_t i = 0;
    while (i < names.size() && names[i] != m.name) ++i;
    if (i == names.size()) {
      names.push_back(m.name);
      counts.push_back(0);
      sums.push_back(0.0);
    }
    counts[i] += 1;
    sums[i] += ms;
  }
  ctx->trace_marks.clear();
  ctx->trace_used = 0;
  if (rc != QKV_OK) {
    (void)hip_status(ctx);
    return rc;
  }
  for (size_t i = 0; out && i < names.size() && int32_t(i) < max; ++i) {
    qkv_trace_entry &e = out[i];
    const size_t n = std::min(names[i].size(), sizeof(e.name) - 1);
    std::copy(names[i].begin(), names[i].begin() + n, e.name);
    e.name[n] = 0;
    e.launches = counts[i];
    e.total_ms = sums[i];
  }
  return int(names.size());
}

// Device address of the fixed partials array on the current device, looked
// up once per device (with that device current) and kept; nullptr when the
// lookup fails (no usable device).
static void *noalloc_scratch_for_current_device() {
  static std::mutex mu;
  static std::vector<void *> ptrs;
  static std::vector<char> done;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (size_t(dev) >= ptrs.size()) {
    ptrs.resize(size_t(dev) + 1, nullptr);
    done.resize(size_t(dev) + 1, 0);
  }
  if (!done[dev]) {
    void *p = nullptr;
    if (noalloc_scratch_address(&p) == 0) ptrs[dev] = p;
    done[dev] = 1;
  }
  return ptrs[dev];
}

extern "C" int qkv_init(const qkv_config *cfg, void *d_arena, size_t arena_bytes,
                        const void *d_predictor, qkv_ctx **out) {
  if (!out) return QKV_E_INVAL;
  *out = nullptr;
  Plan p;
  const int rc = make_plan(cfg, &p);
  if (rc != QKV_OK) return rc;
  if (!d_arena) return QKV_E_INVAL;
  if (reinterpret_cast<uintptr_t>(d_arena) % kAlign) return QKV_E_ARENA;
  if (arena_bytes < p.total_bytes) return QKV_E_ARENA;
  if (p.cfg.xlayer && !d_predictor) return QKV_E_INVAL;
  qkv_ctx *ctx = new (std::nothrow) qkv_ctx;
  if (!ctx) return QKV_E_INVAL;
  ctx->plan = p;
  ctx->arena = static_cast<uint8_t *>(d_arena);
  ctx->arena_bytes = arena_bytes;
  ctx->predictor = static_cast<const uint8_t *>(d_predictor);
  ctx->layers.resize(size_t(p.cfg.n_layers));
  if (p.cfg.max_query_tokens > 0) {
    ctx->noalloc_scratch = noalloc_scratch_for_current_device();
    (void)hipGetLastError();  // a failed lookup only disables qkv_attend_noalloc
  }
  *out = ctx;
  return QKV_OK;
}

// compute units of the current device, looked up once per context (the
// attention's work split deals one run per compute unit)
static void ensure_cu_count(qkv_ctx *ctx) {
  if (ctx->n_cu > 0) return;
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n_cu > 0)
    ctx->n_cu = n_cu;
  else
    ctx->n_cu = 256;
}

// re-fitted blocks of the transition into layer l (adapted cross-layer mode)
static uint16_t *refit_blocks(qkv_ctx *ctx, int l) {
  const qkv_config &c = ctx->plan.cfg;
  return reinterpret_cast<uint16_t *>(ctx->arena + ctx->plan.xl_refit_off +
                                      uint64_t(l) * 2 * c.n_heads * c.head_dim * c.head_dim * 2);
}

extern "C" int qkv_adapted_blocks(const qkv_ctx *ctx, int32_t layer, uint64_t *offset) {
  if (!ctx || !offset) return QKV_E_INVAL;
  const qkv_config &c = ctx->plan.cfg;
  if (!c.xlayer_adapt || layer < 1 || layer >= c.n_layers) return QKV_E_INVAL;
  *offset = ctx->plan.xl_refit_off + uint64_t(layer) * 2 * c.n_heads * c.head_dim * c.head_dim * 2;
  return QKV_OK;
}

// SAS + PRQ for the 2*n_layers streams of `a` (k-means loop, then codes).
// iters < 0: assign to the stream's codebook as it stands (codebook reuse).
// With outlier channels the call's flags are found between the final
// assignment and the stages.
static void enqueue_sas(const EncodeArgs &a, int streams, int iters, hipStream_t st) {
  launch_header(a, streams, st);
  if (iters >= 0) {
    launch_init(a, streams, st);
    for (int it = 0; it < iters; ++it) {
      launch_assign(a, streams, st);
      launch_update(a, streams, st);
    }
  }
  launch_assign(a, streams, st);
  if (a.L.mask_off) launch_chan_flags(a, streams, st);
  launch_quantize(a, streams, st);
}

extern "C" int qkv_encode_chunk(qkv_ctx *ctx, int32_t layer0, int32_t n_layers, const void *d_k,
                                const void *d_v, int64_t n, void *stream) {
  const int rc = check_encode(ctx, layer0, n_layers, d_k, d_v, n);
  if (rc != QKV_OK) return rc;
  TraceScope trace(ctx);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Plan &p = ctx->plan;
  const qkv_config &c = p.cfg;
  const int64_t t0 = ctx->layers[layer0].n_tokens;
  const int slot = int(ctx->layers[layer0].starts.size());

  EncodeArgs a{};
  a.L = dev_layout(p);
  a.arena = ctx->arena;
  a.n = int32_t(n);
  a.t0 = int32_t(t0);
  a.slot = slot;
  a.prev_slot = slot - 1;
  a.sort_perm = scratch(ctx, p.sort_perm_off);
  a.sort_off = reinterpret_cast<uint16_t *>(scratch(ctx, p.sort_off_off));
  a.sort_tiles = int32_t(p.sort_tiles);
  a.chan_part = reinterpret_cast<double *>(scratch(ctx, p.chan_part_off));
  const uint64_t layer_bytes = uint64_t(c.n_heads) * uint64_t(n) * c.head_dim * p.kv_elem_bytes;
  const uint8_t *kin = static_cast<const uint8_t *>(d_k);
  const uint8_t *vin = static_cast<const uint8_t *>(d_v);

  // codebook reuse: calls after a stream's first only assign
  const int iters = c.codebook_reuse && slot > 0 ? -1 : c.kmeans_iters;
  (void)hipGetLastError();
  if (!c.xlayer) {
    a.layer0 = layer0;
    a.k_in = kin;
    a.v_in = vin;
    enqueue_sas(a, 2 * n_layers, iters, st);
  } else {
    const uint64_t HD = uint64_t(c.n_heads) * c.head_dim;
    const uint64_t kv_stride = HD * c.head_dim + 2 * HD * uint64_t(c.xlayer_rank);
    uint16_t *chain = reinterpret_cast<uint16_t *>(scratch(ctx, p.xl_chain_off));
    float *pred = reinterpret_cast<float *>(scratch(ctx, p.xl_pred_off));
    float *proj = reinterpret_cast<float *>(scratch(ctx, p.xl_proj_off));
    for (int l = layer0; l < layer0 + n_layers; ++l) {
      a.layer0 = l;
      a.k_in = kin + uint64_t(l - layer0) * layer_bytes;
      a.v_in = vin + uint64_t(l - layer0) * layer_bytes;
      a.chain = chain;
      if (l == 0) {
        a.pred = nullptr;
        enqueue_sas(a, 2, iters, st);
      } else {
        XlArgs x{};
        x.H = c.n_heads; x.D = c.head_dim; x.r = c.xlayer_rank; x.n = int32_t(n);
        x.chain = chain;
        x.weights = reinterpret_cast<const uint16_t *>(ctx->predictor) + uint64_t(l - 1) * 2 * kv_stride;
        x.kv_weight_stride = kv_stride;
        x.proj = proj;
        x.pred = pred;
        if (c.xlayer_adapt) {
          uint16_t *blocks = refit_blocks(ctx, l);
          if (ctx->layers[l].starts.empty()) {
            // first call of the video for this layer: re-fit the blocks on
            // its tokens against the low-rank part of the prediction
            x.lowrank_only = 1;
            launch_xl_predict(x, 0, 2, st);
            RefitArgs f{};
            f.H = c.n_heads; f.D = c.head_dim; f.n = int32_t(n);
            f.chain = chain;
            f.k_in = a.k_in;
            f.v_in = a.v_in;
            f.low_rank = pred;
            f.gram = reinterpret_cast<double *>(scratch(ctx, p.xl_gram_off));
            f.b_out = blocks;
            launch_xl_refit(f, st);
            x.lowrank_only = 0;
            x.skip_project = 1;
          }
          x.b_weights = blocks;
        }
        launch_xl_predict(x, 0, 2, st);
        a.pred = pred;
        launch_header(a, 2, st);
        launch_quantize(a, 2, st);
      }
    }
  }
  const int hs = hip_status(ctx);
  if (hs != QKV_OK) return hs;
  for (int l = layer0; l < layer0 + n_layers; ++l) {
    ctx->layers[l].starts.push_back(t0);
    ctx->layers[l].n_tokens = t0 + n;
  }
  if (c.xlayer) {
    ctx->chain_layer = layer0 + n_layers - 1;
    ctx->chain_t0 = t0;
    ctx->chain_n = n;
    ctx->sweep_layer = -1;   // the encoded layers hold more tokens now
  }
  return QKV_OK;
}

// Cross-layer read: bring the sweep region to `layer` over all its tokens,
// slice by slice.  Layer 0 (SAS-coded) is reconstructed into it; a layer
// l >= 1 is predicted from the region's layer l-1 and its reconstruction
// is written over the same slice (the prediction of a slice is complete
// before its slice is overwritten: both run in stream order).
static void sweep_to(qkv_ctx *ctx, int layer, hipStream_t st) {
  const Plan &p = ctx->plan;
  const qkv_config &c = p.cfg;
  const int64_t T = ctx->layers[layer].n_tokens, M = p.xl_sweep_slice;
  const uint64_t HD = uint64_t(c.n_heads) * c.head_dim;
  const uint64_t kv_stride = HD * c.head_dim + 2 * HD * uint64_t(c.xlayer_rank);
  uint16_t *sweep = reinterpret_cast<uint16_t *>(ctx->arena + p.xl_sweep_off);
  float *pred = reinterpret_cast<float *>(scratch(ctx, p.xl_pred_off));
  float *proj = reinterpret_cast<float *>(scratch(ctx, p.xl_proj_off));
  ReconArgs r{};
  r.L = dev_layout(p);
  r.arena = ctx->arena;
  r.out = nullptr;
  r.out_bf16 = 1;
  for (int64_t ts = 0, sl = 0; ts < T; ts += M, ++sl) {
    const int64_t ns = std::min(M, T - ts);
    uint16_t *blk = sweep + uint64_t(sl) * 2 * HD * uint64_t(M);   // [2][H][ns][d]
    if (layer >= 1) {
      XlArgs x{};
      x.H = c.n_heads; x.D = c.head_dim; x.r = c.xlayer_rank; x.n = int32_t(ns);
      x.chain = blk;
      x.weights = reinterpret_cast<const uint16_t *>(ctx->predictor) + uint64_t(layer - 1) * 2 * kv_stride;
      x.kv_weight_stride = kv_stride;
      x.proj = proj;
      x.pred = pred;
      x.b_weights = c.xlayer_adapt ? refit_blocks(ctx, layer) : nullptr;
      launch_xl_predict(x, 0, 2, st);
    }
    for (int kv = 0; kv < 2; ++kv) {
      r.layer0 = layer;
      r.kv = kv;
      r.t0 = int32_t(ts);
      r.n = int32_t(ns);
      r.pred = layer >= 1 ? pred + uint64_t(kv) * HD * ns : nullptr;
      r.chain = blk + uint64_t(kv) * HD * ns;
      launch_reconstruct(r, 1, ns, 0, st);
    }
  }
  ctx->sweep_layer = layer;
  ctx->sweep_tokens = T;
}

// Enqueue the attention of n_q queries over `layer` with the split partials
// at part_o / part_lse ([max_segments][H][n_q][d] and [max_segments][H][n_q]).
static void enqueue_attend(qkv_ctx *ctx, const AttnSplit &w, int32_t layer, const void *d_q, int64_t n_q,
                           int32_t q_dtype, void *d_out, int32_t out_dtype, float *d_lse, float *part_o,
                           float *part_lse, hipStream_t st) {
  const Plan &p = ctx->plan;
  AttnArgs a{};
  a.L = dev_layout(p);
  a.stream_k = ctx->arena + stream_offset(p, layer, 0);
  a.stream_v = ctx->arena + stream_offset(p, layer, 1);
  a.q = d_q;
  a.q_bf16 = q_dtype == QKV_BF16;
  a.n_q = int32_t(n_q);
  a.n_keys = int32_t(ctx->layers[layer].n_tokens);
  a.n_qblocks = int32_t(w.n_qblocks);
  a.n_ktiles = int32_t(w.n_ktiles);
  a.units_per_block = int32_t(w.units_per_block);
  a.head_blocks = int32_t(w.head_blocks);
  a.main_tiles = int32_t(w.main_tiles);
  a.max_segments = int32_t(w.max_segments);
  a.xcd_remap = w.n_blocks % 8 == 0;
  a.out = d_out;
  a.out_bf16 = out_dtype == QKV_BF16;
  a.lse = d_lse;
  a.part_o = part_o;
  a.part_lse = part_lse;
  if (p.cfg.xlayer && layer >= 1) {
    // cross-layer coded layer: the bf16 tiles of the sweep region
    a.k_new = a.v_new = reinterpret_cast<const uint16_t *>(ctx->arena + p.xl_sweep_off);
    a.fresh_slice = int32_t(p.xl_sweep_slice);
    launch_attend_fresh(a, st);
    return;
  }
  launch_attend(a, st);
}

extern "C" int qkv_attend(qkv_ctx *ctx, int32_t layer, const void *d_q, int64_t n_q, int32_t q_dtype,
                          void *d_out, int32_t out_dtype, float *d_lse, void *stream) {
  const int rc = check_attend(ctx, layer, d_q, n_q, q_dtype, d_out, out_dtype);
  if (rc != QKV_OK) return rc;
  if (n_q == 0) return QKV_OK;
  TraceScope trace(ctx);
  const Plan &p = ctx->plan;
  ensure_cu_count(ctx);
  // a cross-layer coded layer is read as uncoded bf16 rows
  const uint64_t kb = p.cfg.xlayer && layer >= 1 ? bf16_key_bytes(p) : packed_key_bytes(p);
  const AttnSplit w = attention_split(p, ctx->layers[layer].n_tokens, n_q, ctx->n_cu, kb);
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (p.cfg.xlayer && (layer >= 1 || p.cfg.n_layers > 1)) sweep_to(ctx, layer, st);
  enqueue_attend(ctx, w, layer, d_q, n_q, q_dtype, d_out, out_dtype, d_lse,
                 reinterpret_cast<float *>(scratch(ctx, p.attn_part_o_off)),
                 reinterpret_cast<float *>(scratch(ctx, p.attn_part_lse_off)), st);
  ctx->chain_layer = -1;  // scratch reused
  return hip_status(ctx);
}

extern "C" int qkv_attend_noalloc(qkv_ctx *ctx, int32_t layer, const void *d_q, int64_t n_q, int32_t q_dtype,
                                  void *d_out, int32_t out_dtype, float *d_lse, void *stream) {
  const int rc = check_attend(ctx, layer, d_q, n_q, q_dtype, d_out, out_dtype);
  if (rc != QKV_OK) return rc;
  if (n_q == 0) return QKV_OK;
  if (!ctx->noalloc_scratch || ctx->plan.cfg.xlayer) return QKV_E_UNSUPPORTED;
  const Plan &p = ctx->plan;
  ensure_cu_count(ctx);
  const AttnSplit w = attention_split(p, ctx->layers[layer].n_tokens, n_q, ctx->n_cu, packed_key_bytes(p));
  // partials of the slots this call can use, in the fixed array
  const uint64_t rows = uint64_t(w.max_segments) * p.cfg.n_heads * uint64_t(n_q);
  const uint64_t lse_off = align_up(rows * p.cfg.head_dim * 4);
  if (lse_off + rows * 4 > kNoAllocScratchBytes) return QKV_E_CAPACITY;
  uint8_t *base = static_cast<uint8_t *>(ctx->noalloc_scratch);
  (void)hipGetLastError();
  enqueue_attend(ctx, w, layer, d_q, n_q, q_dtype, d_out, out_dtype, d_lse, reinterpret_cast<float *>(base),
                 reinterpret_cast<float *>(base + lse_off), static_cast<hipStream_t>(stream));
  return hip_status(ctx);
}

extern "C" int qkv_attend_with_chunk(qkv_ctx *ctx, int32_t layer, const void *d_q, int64_t n_q, int32_t q_dtype,
                                     const void *d_k_new, const void *d_v_new, int64_t n_new, void *d_out,
                                     int32_t out_dtype, float *d_lse, void *stream) {
  const int rc = check_attend_with_chunk(ctx, layer, d_q, n_q, q_dtype, d_k_new, d_v_new, n_new, d_out, out_dtype);
  if (rc != QKV_OK) return rc;
  if (n_q == 0) return QKV_OK;
  const int64_t n_cache = ctx->layers[layer].n_tokens;
  if (n_new == 0) return qkv_attend(ctx, layer, d_q, n_q, q_dtype, d_out, out_dtype, d_lse, stream);
  TraceScope trace(ctx);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Plan &p = ctx->plan;
  const qkv_config &c = p.cfg;
  ensure_cu_count(ctx);
  // Each part may split a query block over at most kMaxSplits - 2 blocks;
  // the last two partial slots hold the two complete parts for the merge.
  const uint64_t HQ = uint64_t(c.n_heads) * uint64_t(n_q);
  float *part_o = reinterpret_cast<float *>(scratch(ctx, p.attn_part_o_off));
  float *part_lse = reinterpret_cast<float *>(scratch(ctx, p.attn_part_lse_off));
  float *o_part[2] = {part_o + (kMaxSplits - 2) * HQ * c.head_dim, part_o + (kMaxSplits - 1) * HQ * c.head_dim};
  float *l_part[2] = {part_lse + (kMaxSplits - 2) * HQ, part_lse + (kMaxSplits - 1) * HQ};
  auto args_for = [&](int64_t n_keys, uint64_t key_bytes) {
    const AttnSplit w = attention_split(p, n_keys, n_q, ctx->n_cu, key_bytes, kMaxSplits - 2);
    AttnArgs a{};
    a.L = dev_layout(p);
    a.q = d_q;
    a.q_bf16 = q_dtype == QKV_BF16;
    a.n_q = int32_t(n_q);
    a.n_keys = int32_t(n_keys);
    a.n_qblocks = int32_t(w.n_qblocks);
    a.n_ktiles = int32_t(w.n_ktiles);
    a.units_per_block = int32_t(w.units_per_block);
    a.head_blocks = int32_t(w.head_blocks);
    a.main_tiles = int32_t(w.main_tiles);
    a.max_segments = int32_t(w.max_segments);
    a.xcd_remap = w.n_blocks % 8 == 0;
    a.part_o = part_o;
    a.part_lse = part_lse;
    return a;
  };
  (void)hipGetLastError();
  // fresh part: straight into the output when the cache holds nothing
  AttnArgs f = args_for(n_new, bf16_key_bytes(p));
  f.k_new = static_cast<const uint16_t *>(d_k_new);
  f.v_new = static_cast<const uint16_t *>(d_v_new);
  if (n_cache == 0) {
    f.out = d_out;
    f.out_bf16 = out_dtype == QKV_BF16;
    f.lse = d_lse;
    launch_attend_fresh(f, st);
    ctx->chain_layer = -1;  // scratch reused
    return hip_status(ctx);
  }
  if (c.xlayer && (layer >= 1 || c.n_layers > 1)) sweep_to(ctx, layer, st);
  AttnArgs a = args_for(n_cache, c.xlayer && layer >= 1 ? bf16_key_bytes(p) : packed_key_bytes(p));
  a.out = o_part[0];
  a.out_bf16 = 0;
  a.lse = l_part[0];
  if (c.xlayer && layer >= 1) {
    // cross-layer coded layer: the bf16 tiles of the sweep region
    a.k_new = a.v_new = reinterpret_cast<const uint16_t *>(ctx->arena + p.xl_sweep_off);
    a.fresh_slice = int32_t(p.xl_sweep_slice);
    launch_attend_fresh(a, st);
  } else {
    a.stream_k = ctx->arena + stream_offset(p, layer, 0);
    a.stream_v = ctx->arena + stream_offset(p, layer, 1);
    launch_attend(a, st);
  }
  f.out = o_part[1];
  f.out_bf16 = 0;
  f.lse = l_part[1];
  launch_attend_fresh(f, st);
  MergeArgs m{};
  m.H = c.n_heads;
  m.D = c.head_dim;
  m.n_q = int32_t(n_q);
  m.o1 = o_part[0];
  m.lse1 = l_part[0];
  m.o2 = o_part[1];
  m.lse2 = l_part[1];
  m.out = d_out;
  m.out_bf16 = out_dtype == QKV_BF16;
  m.lse = d_lse;
  launch_attend_merge2(m, st);
  ctx->chain_layer = -1;  // scratch reused
  return hip_status(ctx);
}

extern "C" int qkv_reconstruct(qkv_ctx *ctx, int32_t layer0, int32_t n_layers, int32_t kv, int64_t t0,
                               int64_t t1, void *d_out, int32_t out_dtype, void *stream) {
  const int rc = check_reconstruct(ctx, layer0, n_layers, kv, t0, t1, d_out, out_dtype);
  if (rc != QKV_OK) return rc;
  if (t1 == t0) return QKV_OK;
  TraceScope trace(ctx);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Plan &p = ctx->plan;
  const qkv_config &c = p.cfg;
  ReconArgs r{};
  r.L = dev_layout(p);
  r.arena = ctx->arena;
  r.kv = kv;
  r.out_bf16 = out_dtype == QKV_BF16;
  (void)hipGetLastError();
  if (!c.xlayer) {
    r.layer0 = layer0;
    r.t0 = int32_t(t0);
    r.n = int32_t(t1 - t0);
    r.out = d_out;
    launch_reconstruct(r, n_layers, t1 - t0, 0, st);
    return hip_status(ctx);
  }
  // cross-layer: layer l >= 1 needs the bf16 reconstruction of layer l-1
  const int last = layer0 + n_layers - 1;
  const int64_t M = c.max_chunk_tokens;
  const uint64_t HD = uint64_t(c.n_heads) * c.head_dim;
  const uint64_t kv_stride = HD * c.head_dim + 2 * HD * uint64_t(c.xlayer_rank);
  const uint64_t out_eb = out_dtype == QKV_BF16 ? 2 : 4;
  uint16_t *chain = reinterpret_cast<uint16_t *>(scratch(ctx, p.xl_chain_off));
  float *pred = reinterpret_cast<float *>(scratch(ctx, p.xl_pred_off));
  float *proj = reinterpret_cast<float *>(scratch(ctx, p.xl_proj_off));
  for (int64_t ts = t0; ts < t1; ts += M) {
    const int64_t ns = std::min(t1, ts + M) - ts;
    for (int l = 0; l <= last; ++l) {
      r.layer0 = l;
      r.t0 = int32_t(ts);
      r.n = int32_t(ns);
      r.out = l >= layer0 ? static_cast<uint8_t *>(d_out) + uint64_t(l - layer0) * HD * uint64_t(t1 - t0) * out_eb
                          : nullptr;
      r.pred = l >= 1 ? pred + uint64_t(kv) * HD * ns : nullptr;
      r.chain = l < last ? chain + uint64_t(kv) * HD * ns : nullptr;
      launch_reconstruct(r, 1, t1 - t0, int32_t(ts - t0), st);
      if (l < last) {
        XlArgs x{};
        x.H = c.n_heads; x.D = c.head_dim; x.r = c.xlayer_rank; x.n = int32_t(ns);
        x.chain = chain;
        x.weights = reinterpret_cast<const uint16_t *>(ctx->predictor) + uint64_t(l) * 2 * kv_stride;
        x.kv_weight_stride = kv_stride;
        x.proj = proj;
        x.pred = pred;
        x.b_weights = c.xlayer_adapt ? refit_blocks(ctx, l + 1) : nullptr;
        launch_xl_predict(x, kv, 1, st);
      }
    }
  }
  ctx->chain_layer = -1;
  return hip_status(ctx);
}

extern "C" int qkv_rewind(qkv_ctx *ctx, int32_t layer0, int32_t n_layers, int64_t n_tokens, void *stream) {
  const int rc = check_rewind(ctx, layer0, n_layers, n_tokens);
  if (rc != QKV_OK) return rc;
  TraceScope trace(ctx);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const DevLayout L = dev_layout(ctx->plan);
  bool launched = false;
  for (int l = layer0; l < layer0 + n_layers; ++l) {
    const LayerState &ls = ctx->layers[l];
    if (n_tokens == ls.n_tokens) continue;
    int kept = 0;
    while (kept < int(ls.starts.size()) && ls.starts[kept] < n_tokens) ++kept;
    if (!launched) (void)hipGetLastError();
    launched = true;
    launch_set_header(ctx->arena, L, l, 1, kept, int(n_tokens), st);
  }
  if (launched) {
    const int hs = hip_status(ctx);
    if (hs != QKV_OK) return hs;
  }
  for (int l = layer0; l < layer0 + n_layers; ++l) {
    LayerState &ls = ctx->layers[l];
    while (!ls.starts.empty() && ls.starts.back() >= n_tokens) ls.starts.pop_back();
    ls.n_tokens = n_tokens;
  }
  ctx->chain_layer = -1;
  ctx->sweep_layer = -1;
  return QKV_OK;
}
