/*
 * qkv -- cluster-smoothed progressive residual quantization of an
 * autoregressive video model's KV cache, on AMD Instinct MI355X (gfx950).
 *
 * What the library computes (sources cited by page title and section):
 *
 *  - Semantic-Aware Smoothing: "Quant VideoGen: Auto-Regressive Long Video
 *    Generation via 2-Bit KV-Cache Quantization" (Italian explainer on
 *    gist.science), "Sommario tecnico" 2.A.  Per head, tokens are clustered
 *    with k-means along the sequence axis and each token's centroid is
 *    subtracted.  Section 3 (centroid caching): each call's k-means starts
 *    from the previous call's centroids.
 *  - Progressive Residual Quantization: same page, section 2.B.  The
 *    residual is quantized, then what remains is quantized again, stage after
 *    stage; decode dequantizes the stages and adds the centroid back.
 *  - Fused read: same page, section 3 (dequantization fused into the
 *    kernels) and the abstract of "KV Cache Quantization for Self-Forcing
 *    Video Generation: A 33-Method Empirical Study" (BF16 buffers rebuilt
 *    during attention defeat the compression): qkv_attend never stores the
 *    rebuilt K/V.
 *  - Cross-layer residual mode: Coral-KV news article (news.hamidun.com,
 *    section on cross-layer prediction): layer l+1's K/V are predicted from
 *    layer l with a block-diagonal plus low-rank matrix and only the
 *    prediction residual is quantized.
 *
 * Numerical definition (the pages leave these open; the library fixes them):
 *  - distance: squared Euclidean, fp64, channels summed in order; ties to the
 *    lowest cluster index.  Centroid = fp64 mean of the members (summed in
 *    token order), rounded once to the cache dtype; empty clusters keep
 *    their centroid.  First call of a stream: centroid k starts at token
 *    floor(k*n/C).  `kmeans_iters` Lloyd iterations, then a final assignment.
 *  - groups of `group_size` contiguous channels of one token; per group and
 *    stage z = fp16(min), sigma = fp16(fl32(fl32(max - z)/(2^bits - 1))),
 *    code = clamp(rint(fl32(fl32(r - z) * fl32(1/sigma))), 0, 2^bits - 1)
 *    (all codes 0 when sigma == 0), rhat = fmaf(code, sigma, z), next stage
 *    on fl32(r - rhat).  Reconstruction: fl32 sums base + rhat_1 + ... in
 *    stage order.
 *
 * Memory: the caller owns every device buffer (arena, inputs, outputs,
 * predictor weights).  The library owns only the host-side context.  All
 * device pointers must stay valid until the stream has run the work.
 *
 * Streams: every call enqueues on the given HIP stream (a hipStream_t passed
 * as void*, NULL = the default stream) and returns without synchronizing.
 * All device work of one context must be ordered: one stream, or event
 * dependencies between the streams used.  The attention's split partials,
 * the encoder's sort buffers and channel sums and the cross-layer chain
 * and prediction share one scratch region of the arena, so an encode and an
 * attention of one context running concurrently on two unordered streams
 * corrupt each other without any error being reported.
 *
 * Errors: every entry point returns a qkv_status.  Arguments are validated
 * before anything is enqueued; a call that fails validation enqueues nothing
 * and leaves the context unchanged.  QKV_E_HIP means a kernel launch failed
 * (the context is then in an undefined state and should be destroyed).
 */
#ifndef QKV_H
#define QKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct qkv_ctx qkv_ctx;

/* element types of caller buffers */
enum { QKV_F32 = 0, QKV_BF16 = 1 };

/* status codes */
enum {
  QKV_OK = 0,
  QKV_E_INVAL = -1,       /* bad argument or configuration */
  QKV_E_CAPACITY = -2,    /* token, chunk or query capacity exceeded */
  QKV_E_STATE = -3,       /* call not valid in the current state */
  QKV_E_ARENA = -4,       /* arena too small or misaligned */
  QKV_E_HIP = -5,         /* a HIP call failed */
  QKV_E_UNSUPPORTED = -6  /* valid request the library does not implement */
};

typedef struct {
  int32_t n_layers;        /* L >= 1 */
  int32_t n_heads;         /* H >= 1 (query heads = KV heads) */
  int32_t head_dim;        /* d in {64, 128} */
  int32_t n_clusters;      /* C in [1, 65535]; ids are u8 when C <= 256, else u16 */
  int32_t n_stages;        /* S in [1, 4] */
  int32_t bits;            /* b in {2, 4} */
  int32_t group_size;      /* G in {32, 64}, G divides d */
  int32_t kmeans_iters;    /* Lloyd iterations per call, in [0, 64] */
  int64_t max_tokens;      /* capacity of each (layer, K|V) stream, < 2^31 */
  int64_t max_chunk_tokens;/* largest n of one encode call (0 = max_tokens);
                              n * d * element bytes < 2^31 */
  int32_t max_chunks;      /* codebook snapshots per stream, in [1, 256] */
  int32_t kv_dtype;        /* QKV_F32 or QKV_BF16: the cache (and codebook) type */
  int64_t max_query_tokens;/* largest n_q of qkv_attend (0 = attention unused) */
  int32_t xlayer;          /* 0: SAS + PRQ on every layer; 1: cross-layer residual
                              coding for layers >= 1 (requires QKV_BF16) */
  int32_t xlayer_rank;     /* r of the low-rank term, in [1, 64] when xlayer = 1 */
  int32_t codebook_reuse;  /* 0: every encode call runs the k-means (warm start from the
                              previous snapshot) and stores its own snapshot; 1: only a
                              stream's first call (after a rewind to 0: the next call)
                              runs the k-means; later calls assign their tokens to that
                              codebook, which is the one snapshot of the stream (the
                              codebook-reuse reading of centroid caching, QVG explainer,
                              "Sommario tecnico" 3) */
  int32_t xlayer_adapt;    /* with xlayer = 1: 0 uses the caller's block-diagonal B_h as
                              given; 1 re-fits every B_h of layers >= 1 once per video, on
                              the first encode call of the layer (ridge least squares with
                              the low-rank term fixed, fp64, rounded to bf16), and uses the
                              re-fitted blocks for that and every later call and for
                              decoding (Coral-KV's adapted configuration) */
  int32_t outlier_channels;/* 0: plain groups; 1: every encode call flags, per head, the
                              channels whose residual L2 norm stands out (modified z-score
                              on the median absolute deviation: 0.6745 (n_j - med) > 3.5 MAD,
                              and n_j > 2 med, medians over the d channels) and quantizes
                              them as one extra group per token and stage with its own
                              fp16 (sigma, z); the normal groups leave them out (Q-ARVD
                              explainer, outlier-aware adaptive dual-scale quantization,
                              carried over from weights to the KV residual).  SAS mode only
                              (xlayer = 0) */
} qkv_config;

/* Offsets (bytes from the arena base) and strides of one (layer, K|V) stream,
 * for read-back and tests.  Layouts:
 *   codes    u8  [S][H][max_tokens][d*bits/8]  element j of a token at byte
 *                j*bits/8, bit (j*bits)%8 (least significant first)
 *   meta     u16 [S][H][max_tokens][d/G][2]    fp16 bit patterns (sigma, z); with
 *                outlier_channels = 1 [d/G + 1][2], the last entry the outlier group's
 *                ((0, 0) when a group has no channel)
 *   ids      u8|u16 [H][max_tokens]            cluster id of each token
 *   codebook kv_dtype [max_chunks][H][C][d]    snapshot of each encode call
 *   cnorm    f32 [max_chunks][H][C]            ||c||^2 of each snapshot row
 *   chmask   u32 [max_chunks][H][d/32]         outlier channels of each call (bit j%32
 *                of word j/32 = channel j); only with outlier_channels = 1
 * The codebook of a token is the snapshot of the chunk that encoded it.  With
 * codebook_reuse = 1 there is one snapshot ([1][H][C][d], [1][H][C]) and the
 * chunk strides are 0. */
typedef struct {
  uint64_t codes_off, codes_stage_stride, codes_head_stride, codes_token_stride;
  uint64_t meta_off, meta_stage_stride, meta_head_stride, meta_token_stride;
  uint64_t ids_off, ids_head_stride, id_bytes;
  uint64_t codebook_off, codebook_chunk_stride, codebook_head_stride;
  uint64_t cnorm_off, cnorm_chunk_stride, cnorm_head_stride;
  int64_t n_tokens;        /* tokens encoded so far in this layer */
  int32_t n_chunks;        /* encode calls so far in this layer */
  int32_t reserved;
  uint64_t chmask_off, chmask_chunk_stride, chmask_head_stride;  /* 0 when outlier_channels = 0 */
} qkv_layout_desc;

/* Device bytes the arena must provide for `cfg` (0 if cfg is invalid). */
size_t qkv_workspace_bytes(const qkv_config *cfg);

/* Create a context over a caller-owned device arena of `arena_bytes`
 * (>= qkv_workspace_bytes, 256-byte aligned).  `d_predictor` is NULL unless
 * cfg->xlayer: then it points to bf16 device weights, for each layer
 * l = 0..L-2 (predicting l+1) and each tensor (K then V): B [H][d][d]
 * (B_h maps head h's channels: pred[i] = sum_j B_h[i][j] y[j]),
 * U [H*d][r], V [H*d][r]; it must stay valid for the context's lifetime.
 * Enqueues nothing.  Returns QKV_E_INVAL / QKV_E_ARENA on bad input. */
int qkv_init(const qkv_config *cfg, void *d_arena, size_t arena_bytes,
             const void *d_predictor, qkv_ctx **out);

/* Encode one chunk of n new tokens into layers [layer0, layer0+n_layers).
 * d_k, d_v: device [n_layers][H][n][d] in kv_dtype.  Appends n tokens to each
 * of the 2*n_layers streams and stores one codebook snapshot per stream and
 * head (SAS + PRQ), or, in cross-layer mode for layers >= 1, codes of the
 * residual against the prediction from the previous layer's reconstruction.
 * Every layer in the range must hold the same number of tokens before the
 * call.  In cross-layer mode a call starting at layer0 > 0 must directly
 * follow the call that encoded layer0-1 for the same tokens.
 * Errors: QKV_E_INVAL (n < 1, null pointer, bad layer range),
 * QKV_E_CAPACITY (tokens, chunk size or chunk count), QKV_E_STATE. */
int qkv_encode_chunk(qkv_ctx *ctx, int32_t layer0, int32_t n_layers,
                     const void *d_k, const void *d_v, int64_t n, void *stream);

/* Attention of n_q queries over every token encoded in `layer`:
 * out = softmax(q k^T / sqrt(d)) v per head with keys/values rebuilt from the
 * packed cache in registers/LDS (never stored).  q: device [H][n_q][d] in
 * q_dtype; out: device [H][n_q][d] in out_dtype; d_lse: device [H][n_q] f32
 * natural-log softmax denominators, or NULL.  Operands enter the products in
 * bf16; softmax and accumulation are fp32.
 * Cross-layer mode (Coral-KV news article, section on cross-layer
 * prediction): a layer l >= 1 is coded against the prediction from layer
 * l-1's reconstruction, so its keys exist only through that chain.  The
 * library keeps a rolling bf16 reconstruction of one layer (the last one
 * read; arena region of one layer's K and V, 1/L of the cache in bf16):
 * reading layer 0 stores its reconstruction there; reading layer l >= 1
 * requires the region to hold layer l-1 over the same tokens (the layers
 * are read in order 0, 1, 2, ... after the last encode call, as a model's
 * forward pass does), predicts layer l from it, writes layer l's
 * reconstruction over it and attends to those bf16 rows.  An encode call
 * or a rewind empties the region.  Errors: QKV_E_INVAL, QKV_E_CAPACITY
 * (n_q > max_query_tokens), QKV_E_STATE (nothing encoded; in cross-layer
 * mode, layer l >= 1 read before layer l-1). */
int qkv_attend(qkv_ctx *ctx, int32_t layer, const void *d_q, int64_t n_q, int32_t q_dtype,
               void *d_out, int32_t out_dtype, float *d_lse, void *stream);

/* qkv_attend for callers that cannot allocate device memory or use the
 * arena's scratch region (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, kernels, result and
 * errors as qkv_attend, but the split partials go to a fixed 128 MiB device
 * array the library holds on every GPU it runs on until the process ends
 * (looked up at qkv_init).  The call allocates nothing.  Every call on one
 * GPU shares that array and finds it as the last call left it (nothing in
 * it needs to start at zero): calls that overlap on one GPU, from any
 * context or stream, race.  Extra errors: QKV_E_CAPACITY when the call's
 * partials (slots x H x n_q x (d + 1) floats, at most 8 slots) exceed 128
 * MiB; QKV_E_UNSUPPORTED when the array's address could not be found at
 * qkv_init (no usable device, or max_query_tokens = 0) and in cross-layer
 * mode (whose read also uses the arena's scratch for the prediction). */
int qkv_attend_noalloc(qkv_ctx *ctx, int32_t layer, const void *d_q, int64_t n_q, int32_t q_dtype,
                       void *d_out, int32_t out_dtype, float *d_lse, void *stream);

/* The read as a generating model issues it: attention of n_q queries over
 * every token encoded in `layer` followed by n_new fresh tokens of the chunk
 * being generated, which are not in the cache yet (QVG explainer, "Sommario
 * tecnico" 2.B and 3: the cached tokens are dequantized inside the attention
 * kernels; the 33-method study, abstract: no bf16 copy of the cache is made).
 * d_k_new, d_v_new: device [H][n_new][d] bf16, read as they are.  The result
 * is softmax over the concatenated keys (cache first, then the fresh keys):
 * the two parts are computed separately and combined by their log-sum-exps.
 * n_new = 0 is qkv_attend; an empty cache with n_new > 0 attends to the
 * fresh tokens alone.  Other arguments as qkv_attend.  Errors: QKV_E_INVAL,
 * QKV_E_CAPACITY (n_q > max_query_tokens), QKV_E_STATE (empty cache and
 * n_new = 0; in cross-layer mode, as qkv_attend). */
int qkv_attend_with_chunk(qkv_ctx *ctx, int32_t layer, const void *d_q, int64_t n_q, int32_t q_dtype,
                          const void *d_k_new, const void *d_v_new, int64_t n_new, void *d_out,
                          int32_t out_dtype, float *d_lse, void *stream);

/* Rebuild tokens [t0, t1) of tensor kv (0 = K, 1 = V) for layers
 * [layer0, layer0+n_layers) into d_out: device [n_layers][H][t1-t0][d] in
 * out_dtype (QKV_F32 is the exact reconstruction; QKV_BF16 its nearest-even
 * rounding).  Errors: QKV_E_INVAL, QKV_E_STATE (t1 beyond the encoded tokens
 * of a layer). */
int qkv_reconstruct(qkv_ctx *ctx, int32_t layer0, int32_t n_layers, int32_t kv,
                    int64_t t0, int64_t t1, void *d_out, int32_t out_dtype, void *stream);

/* Drop every chunk that starts at or after n_tokens in layers
 * [layer0, layer0+n_layers); n_tokens must be a chunk boundary of each layer.
 * The next encode warm-starts from the last remaining snapshot. */
int qkv_rewind(qkv_ctx *ctx, int32_t layer0, int32_t n_layers, int64_t n_tokens, void *stream);

/* Layout of one stream (layer, kv) and its current token/chunk counts. */
int qkv_layout(const qkv_ctx *ctx, int32_t layer, int32_t kv, qkv_layout_desc *out);

/* First token of each chunk of `layer` (up to max entries); returns the
 * number of chunks, or a negative status. */
int qkv_chunk_starts(const qkv_ctx *ctx, int32_t layer, int64_t *starts, int32_t max);

/* Cross-layer mode with xlayer_adapt = 1: byte offset from the arena base of
 * the re-fitted blocks of the transition into `layer` (1 <= layer <
 * n_layers), bf16 [2 (K, V)][H][d][d] (row i of B_h maps head h's channels
 * to output channel i), valid once that layer has been encoded since its
 * stream was last empty.  Errors: QKV_E_INVAL (not adapted mode, bad layer). */
int qkv_adapted_blocks(const qkv_ctx *ctx, int32_t layer, uint64_t *offset);

/* Per-kernel timing, for measurement.  With enable = 1 every later call on
 * ctx records a HIP event on its stream before and after each kernel it
 * launches (the events are created by the library and reused); enable = 0
 * stops recording.  Tracing adds a small gap between kernels, so timed
 * regions should run with it off.  Errors: QKV_E_INVAL. */
int qkv_trace(qkv_ctx *ctx, int32_t enable);

typedef struct {
  char name[64];           /* kernel base name, e.g. "k_attend3" */
  int64_t launches;        /* launches recorded since the last read */
  double total_ms;         /* sum of their event-to-event times */
} qkv_trace_entry;

/* Wait for every recorded event, add the intervals up per kernel name (in
 * order of first launch), write up to max entries to out (out may be NULL)
 * and forget the records.  Returns the number of distinct kernels, or a
 * negative status (QKV_E_INVAL, QKV_E_HIP). */
int qkv_trace_read(qkv_ctx *ctx, qkv_trace_entry *out, int32_t max);

/* Release the context (not the caller's device memory). */
void qkv_destroy(qkv_ctx *ctx);

/* Static description of a status code (the last HIP error string for
 * QKV_E_HIP when ctx is not NULL). */
const char *qkv_status_string(const qkv_ctx *ctx, int status);

#ifdef __cplusplus
}
#endif

#endif /* QKV_H */
