// Fused read of the qkv library: split-KV attention over the packed cache
// (tiles rebuilt in bf16 in LDS, bf16 MFMA products, online softmax), the
// uncoded read of a fresh chunk, and the LSE merges.
#include "common.h"

namespace qkv {

// -------------------------------------------------------------- attention
//
// Fused read of the packed cache.  Block = 8 waves (two per SIMD) = 256
// queries of one head, 32 per wave; the (head, query block, key tile) units
// are split stream-K style over the blocks.  Per 64-key tile the block
// rebuilds K and V in bf16 into a double-buffered LDS tile (both as
// [key][d]); each wave then computes S^T = K Q^T for its 32 queries with
// v_mfma_f32_32x32x16_bf16 (a lane's accumulators hold 32 keys of one query;
// lanes l and l^32 share the query, so the softmax statistics need one
// cross-lane exchange), runs the online softmax in fp32 and accumulates
// O^T += V^T P^T with the probabilities rounded to bf16.  V^T comes from
// the row-major V tile through transposing LDS loads.  The key order inside
// each 16-key MFMA step is permuted identically in both operands so that
// P^T comes straight from the S^T accumulators.
//
//  * Rebuild items: one (tensor, key, 32 channels) per thread, K on even and
//    V on odd threads (every wave runs the same code, stores included; the
//    threads of a key read one centroid row).  The rebuild is
//    bf16(fl32 chain: c + sum_s z_s, then fmaf(q_s, sigma_s, .) per stage);
//    2-bit codes are widened two at a time by the fp4 conversion.  A key
//    past the segment's end is rebuilt from the segment's last key (its
//    logit is masked, so it weighs 0): the loads have no data-dependent
//    path, and only a segment's last tile runs the masking code.
//  * Loads are software-pipelined: ids of tile i+3 and the packed data
//    (codes, scale/zero, centroid rows) of tile i+2 are in flight while tile
//    i+1 is rebuilt and tile i multiplied.  The rebuild's arithmetic is
//    spread between the S^T products of the wave's own tile: measured on
//    the device, a wave's back-to-back products and the vector work of the
//    other wave of its SIMD overlap little, vector instructions placed
//    between a wave's own products largely do.  The chunk table is cached in
//    LDS; each item follows its key's chunk with a cursor that only moves
//    forward, the next chunk start and the chunk's codebook in registers.
//  * The softmax scale is folded into the exponent's fma; the running max is
//    only raised (and O, l rescaled) when a tile's max exceeds it by more
//    than 8 (log2 units), so exponentials stay <= 256; row sums of P are
//    accumulated from the bf16 probabilities with v_dot2_f32_bf16.
constexpr int AT_WAVES = 8;
constexpr int AT_BQ = 32 * AT_WAVES;
constexpr int AT_BK = 64;

// Transposing LDS load (ds_read_b64_tr_b16): within each 16-lane group,
// lane l receives element l%4 of the 8-byte rows addressed by lanes
// l/4 + 4j (j = 0..3), as element j.
typedef short shortx4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 lds_read_tr16(const uint16_t *p) {
  const shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4 *)(p));
  return __builtin_bit_cast(bf16x4, v);
}

typedef float floatx16 __attribute__((ext_vector_type(16)));
// max / sum of the values of lanes l and l^32, identical on both lanes
// (v_permlane32_swap_b32 hands each half the other half's values)
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr float AT3_TAU = 8.0f;

// b where bit k of i is set, else a: a bitwise select of two values.  A
// conditional expression over two register words lets the compiler merge
// them into one load at a run-time offset, which forces the words into
// memory.
template <int K>
__device__ __forceinline__ uint32_t bit_sel(int i, uint32_t a, uint32_t b) {
  const uint32_t m = 0u - ((uint32_t(i) >> K) & 1u);
  return (b & m) | (a & ~m);
}
// w[i] for a run-time i < N (bitwise selects, no indexed register access)
template <int N>
__device__ __forceinline__ uint32_t pick_word(const uint32_t *w, int i) {
  if constexpr (N == 2) return bit_sel<0>(i, w[0], w[1]);
  else return bit_sel<1>(i, bit_sel<0>(i, w[0], w[1]), bit_sel<0>(i, w[2], w[3]));
}

// Item registers of the outlier option: the item's mask word in its key's
// chunk and, where it flags a channel, the outlier group's (sigma, z) of every
// stage.
template <int SMAX>
struct OutlierRegs {
  uint32_t fm;
  uint32_t mo[SMAX];
};
struct NoOutlierRegs {};

template <int D, int G, int BITS, bool CB_BF16, int SMAX, bool FRESH = false, bool OUTL = false>
__global__ __launch_bounds__(512, 1) void k_attend3(AttnArgs a) {
  // SMAX = the number of PRQ stages (a template parameter so that the staging
  // registers are sized exactly).  FRESH: the keys and values are the
  // uncoded bf16 rows a.k_new / a.v_new ([H][n_keys][D]) of the chunk being
  // generated; an item is then copied to LDS as read.  OUTL: channels flagged
  // in the mask of the key's chunk take the outlier group's (sigma, z)
  // (meta entry D/G).
  constexpr int IC = 32;                   // channels of one rebuild item
  constexpr int NI = D / IC;               // items per key and tensor
  constexpr int KP = D + 16;               // bf16 elements per K row in LDS (+16: measured
                                           // slightly faster than +8 and +32)
  constexpr int VP = D + 32;               // bf16 elements per V row in LDS (the 4 rows x
                                           // 64 bytes of a transposing read by 32 lanes
                                           // fall in distinct banks)
  constexpr int EB = CB_BF16 ? 2 : 4;
  constexpr int KW = IC * BITS / 32;       // code words of an item
  constexpr int KC = IC * EB / 16;         // uint4 of an item's centroid slice
  static_assert(2 * 64 * NI <= 512, "one item per thread");
  static_assert(G % IC == 0, "an item lies inside one quantization group");
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][AT_BK * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][AT_BK * VP];
  __shared__ int32_t starts_s[kMaxChunks + 1];
  __shared__ int32_t nch_s;
  // OUTL: the segment head's mask words of every chunk, per tensor
  __shared__ uint32_t masks_s[2][OUTL ? kMaxChunks * (D / 32) : 1];
  // OUTL: a thread's centroid slice, [uint4 i][thread], read back per flagged channel
  __shared__ uint4 cent_s[OUTL ? KC * 512 : 1];

  const DevLayout &L = a.L;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hh = lane >> 5, c32 = lane & 31;
  const float sc = 1.4426950408889634f / sqrtf(float(D));
  constexpr int NS = D / 16, NDB = D / 32;
  // lane's transposing-read address in a V tile: key 4*hh + (lane%16)/4 of a
  // 16-key step, channels 16*((lane/16)%2) + 4*(lane%4) .. +3 of a 32-channel block
  const int v_lane = (4 * hh + ((lane & 15) >> 2)) * VP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // Rebuild items: one (tensor, key, 32 channels) per thread, K on even and
  // V on odd threads, so every wave runs the same rebuild code and the
  // threads of one key read one centroid row.  K and V tiles are
  // both stored [key][d]; the PV step reads V with transposing LDS loads.
  const int it_kv = tid & 1, it_rem = tid >> 1;
  const bool has_item = 2 * 64 * NI == 512 || it_rem < 64 * NI;   // every thread for D = 128
  const int it_key = it_rem / NI;
  const int it_ch = (it_rem % NI) * IC, it_g = it_ch / G;
  const uint8_t *st = it_kv ? a.stream_v : a.stream_k;

  if constexpr (FRESH) {
    if (tid == 0) nch_s = 1;
  } else {
    if (tid == 0) nch_s = ((const StreamHeader *)(a.stream_k + L.header_off))->n_chunks;
    __syncthreads();
    for (int i = tid; i < nch_s; i += blockDim.x)
      starts_s[i] = ((const StreamHeader *)(a.stream_k + L.header_off))->start[i];
  }

  // Stream-K work split: the (head, query block, key tile) units are dealt
  // out in equal consecutive runs, one run per block; a block walks its run
  // segment by segment (one segment per query block it touches).  A segment
  // that covers all key tiles of its query block writes the result; the
  // others write a partial (O, LSE) into slot (block - first block of the
  // query block) for the merge kernel.  Blocks are numbered so that each XCD
  // (blocks are dealt to the 8 XCDs round robin) gets a consecutive range of
  // runs: the query blocks of one head then share that XCD's L2.
  //
  // Per-head split (head_blocks > 0): block j of head h takes, for j below
  // the number of query blocks, key tiles [0, main_tiles) of query block j
  // (partial slot 0), so a head's query blocks read the same tiles side by
  // side; the other blocks take runs of the tails [main_tiles, T) of the
  // head's query blocks in order (slot 1 + the run's index among the runs
  // meeting that query block's tail).
  const int lb = a.xcd_remap ? (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8 : blockIdx.x;
  const int64_t T = a.n_ktiles, U = a.units_per_block;
  const int64_t total = T * a.n_qblocks * L.H;
  const int HB = a.head_blocks;
  const int hb = HB ? lb / HB : 0, jb = HB ? lb % HB : 0;
  const int64_t TL = T - a.main_tiles;      // tail tiles of a query block (per-head split)
  int64_t u, u_end;                          // stream-K units, or the block's tail units
  if (!HB) {
    u = int64_t(lb) * U;
    u_end = min(total, u + U);
  } else if (hb >= L.H) {
    u = u_end = 0;
  } else if (jb < a.n_qblocks) {
    u = 0;
    u_end = 1;                               // the one main segment
  } else {
    u = int64_t(jb - a.n_qblocks) * U;
    u_end = min(TL * a.n_qblocks, u + U);
  }
  __syncthreads();  // chunk table in LDS
  const int nch = nch_s;
  while (u < u_end) {
    int h, qblk, t0, t1, slot;
    if (!HB) {
      const int64_t seg = u / T;
      h = int(seg / a.n_qblocks);
      qblk = int(seg % a.n_qblocks);
      t0 = int(u % T);
      t1 = int(min(T, t0 + (u_end - u)));
      slot = (t0 == 0 && t1 == T) ? -1 : int(lb - (seg * T) / U);
      u += t1 - t0;
    } else if (jb < a.n_qblocks) {
      h = hb;
      qblk = jb;
      t0 = 0;
      t1 = a.main_tiles;
      slot = t1 == T ? -1 : 0;
      u = u_end;
    } else {
      h = hb;
      qblk = int(u / TL);
      t0 = int(a.main_tiles + u % TL);
      t1 = int(min(T, t0 + (u_end - u)));
      slot = 1 + int((jb - a.n_qblocks) - (int64_t(qblk) * TL) / U);
      u += t1 - t0;
    }
    const uint8_t *ids_base = FRESH ? nullptr : st + L.ids_off;
    const int ks = t0 * AT_BK;
    const int ke = min(a.n_keys, t1 * AT_BK);
    const int n_tiles = ke > ks ? (ke - ks + AT_BK - 1) / AT_BK : 0;

    if constexpr (OUTL) {
      // written after the previous segment's last tile barrier, read after
      // the barrier before this segment's first rebuild
      constexpr int MW = D / 32;
      const int per = nch * MW;
      for (int i = tid; i < 2 * per; i += blockDim.x) {
        const int kv = i / per, c = (i % per) / MW, w = i % MW;
        masks_s[kv][c * MW + w] = *(const uint32_t *)((kv ? a.stream_v : a.stream_k) + L.mask_off +
                                                       uint64_t(c) * L.mask_chunk + uint64_t(h) * L.mask_head + 4 * w);
      }
    }
    const int q = qblk * AT_BQ + wave * 32 + c32;
    // B operand of S^T = K Q^T, k-step s: Q[q][16 s + 8 hh .. +8] in bf16
    bf16x8 qf[NS];
  #pragma unroll
    for (int s = 0; s < NS; ++s) {
      bf16x8 v;
      if (q < a.n_q) {
        const uint64_t off = (uint64_t(h) * a.n_q + q) * D + s * 16 + hh * 8;
        if (a.q_bf16) {
          v = *(const bf16x8 *)((const uint16_t *)a.q + off);
        } else {
          const float *qp = (const float *)a.q + off;
  #pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (__bf16)qp[e];
        }
      } else {
  #pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)0.0f;
      }
      qf[s] = v;
    }
    // the query loads complete before the tile pipeline starts, so that no
    // wait for them is left inside the tile loop (vmcnt(0))
    __builtin_amdgcn_s_waitcnt(0x0F70);
    bf16x2 ones2;
    ones2[0] = (__bf16)1.0f;
    ones2[1] = (__bf16)1.0f;
    floatx16 o[NDB];
  #pragma unroll
    for (int db = 0; db < NDB; ++db)
  #pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
    float l_part = 0.0f;       // this lane's share of the row sum
    float m_run = -INFINITY;

    // The item's key in a tile, clamped to the segment's last key: a key
    // past the end is rebuilt from the last key's data (finite values whose
    // logits the last tile masks to -inf, so they weigh 0 in P V), which
    // leaves no data-dependent path in the loads.
    auto item_key = [&](int tile) -> int { return min(ks + tile * AT_BK + it_key, ke - 1); };
    // id of the item's key in a tile (tiles past the segment load nothing)
    // The id of the item's key in a tile is read as the aligned dword of the
    // ids region (256-byte aligned) that holds it, for 1- and 2-byte ids
    // alike, with no condition on the load (a tile past the segment reads
    // the segment's last tile); the id is cut out of the word only where it
    // is used, a tile later.  A load per width, or a shift right after the
    // load, made the compiler wait there for every load in flight.
    auto id_off = [&](int tile) -> uint64_t {
      return uint64_t(h) * L.ids_head + uint64_t(item_key(min(tile, n_tiles - 1))) * uint64_t(L.id_bytes);
    };
    auto load_id_word = [&](int tile) -> uint32_t {
      if constexpr (FRESH) return 0u;
      return *(const uint32_t *)(ids_base + (id_off(tile) & ~uint64_t(3)));
    };
    auto id_of = [&](int tile, uint32_t w) -> int {
      return int((w >> (8 * uint32_t(id_off(tile) & 3))) & (L.id_bytes == 1 ? 0xffu : 0xffffu));
    };
    struct Regs : std::conditional_t<OUTL, OutlierRegs<SMAX>, NoOutlierRegs> {
      uint32_t codes[SMAX][KW];
      uint32_t meta[SMAX];
      uint4 cent[KC];
    } R{};   // zero for threads without an item (rebuilt, never stored)
    // per-item pointers of the segment (key t = ks + AT_BK * tile + it_key)
    // clamped like item_key, so that every key the item reads lies at or
    // after t_first (the offsets below are unsigned): an item past the end of
    // a segment shorter than a tile reads the segment's last key throughout
    const int t_first = max(ks, min(ks + it_key, ke - 1));
    const uint8_t *code_p = FRESH ? nullptr : st + L.codes_off + uint64_t(h) * L.codes_head +
                                              uint64_t(t_first) * L.codes_token + it_ch * BITS / 8;
    const uint8_t *meta_p = FRESH ? nullptr : st + L.meta_off + uint64_t(h) * L.meta_head +
                                              uint64_t(t_first) * L.meta_token + 4 * it_g;
    const uint8_t *cb_p = FRESH ? nullptr : st + L.cb_off + uint64_t(h) * L.cb_head + uint64_t(it_ch) * EB;
    // fresh rows: channels it_ch .. it_ch+31 of key t_first of head h
    const uint16_t *fresh_p = FRESH ? (it_kv ? a.v_new : a.k_new) + (uint64_t(h) * a.n_keys + t_first) * D + it_ch
                                    : nullptr;
    // chunk (snapshot slot) of the item's key, advanced tile by tile: keys
    // only grow, and a tile's keys rarely cross more than one chunk start.
    // The next chunk's first token and the chunk's codebook are kept in
    // registers, so a tile that stays in its chunk reads nothing from LDS.
    int c_cur = (FRESH || nch == 1) ? 0 : chunk_of_lds(starts_s, nch, t_first);
    int c_next = (FRESH || c_cur + 1 >= nch) ? INT_MAX : starts_s[c_cur + 1];
    const uint8_t *cb_cur = FRESH ? nullptr : cb_p + uint64_t(c_cur) * L.cb_chunk;
    // packed data of the item's key: centroid slice, codes, (sigma, z)
    auto load_data = [&](int tile, uint32_t id_word) {
      if (!has_item || tile >= n_tiles) return;   // wave-uniform
      const int t = item_key(tile);
      if constexpr (FRESH) {
        const uint16_t *row = fresh_p + uint64_t(t - t_first) * D;
        if (a.fresh_slice > 0) {
          // key t of tensor it_kv, head h in the block of fresh_slice tokens holding it
          const int M = a.fresh_slice, sl = t / M, ts = t - sl * M;
          const int ns = min(M, a.n_keys - sl * M);
          row = a.k_new + uint64_t(sl) * 2 * L.H * uint64_t(M) * D +
                (uint64_t(it_kv * L.H + h) * ns + ts) * D + it_ch;
        }
  #pragma unroll
        for (int i = 0; i < KC; ++i) R.cent[i] = *(const uint4 *)(row + 8 * i);
        return;
      }
      while (t >= c_next) {
        ++c_cur;
        c_next = c_cur + 1 < nch ? starts_s[c_cur + 1] : INT_MAX;
        cb_cur += L.cb_chunk;
      }
      if constexpr (OUTL) R.fm = masks_s[it_kv][c_cur * (D / 32) + (it_ch >> 5)];
      const uint8_t *crow = cb_cur + uint32_t(id_of(tile, id_word)) * uint32_t(D * EB);
  #pragma unroll
      for (int i = 0; i < KC; ++i) R.cent[i] = *(const uint4 *)(crow + 16 * i);
      // offsets inside one head's codes and (sigma, z) of a stage: below 2^32
      // (the layout refuses larger heads)
      const uint32_t dt = uint32_t(t - t_first);
      const uint8_t *cp = code_p + dt * uint32_t(L.codes_token);
      const uint8_t *mp = meta_p + dt * uint32_t(L.meta_token);
  #pragma unroll
      for (int s2 = 0; s2 < SMAX; ++s2) {
        if constexpr (KW == 2) {
          const uint2 v = *(const uint2 *)(cp + uint64_t(s2) * L.codes_stage);
          R.codes[s2][0] = v.x; R.codes[s2][1] = v.y;
        } else {
  #pragma unroll
          for (int w = 0; w < KW; w += 4) {
            const uint4 v = *(const uint4 *)(cp + uint64_t(s2) * L.codes_stage + 4 * w);
            R.codes[s2][w] = v.x; R.codes[s2][w + 1] = v.y; R.codes[s2][w + 2] = v.z; R.codes[s2][w + 3] = v.w;
          }
        }
        R.meta[s2] = *(const uint32_t *)(mp + uint64_t(s2) * L.meta_stage);
      }
      if constexpr (OUTL) {
        if (R.fm) {
  #pragma unroll
          for (int s2 = 0; s2 < SMAX; ++s2)
            R.mo[s2] = *(const uint32_t *)(mp + uint64_t(s2) * L.meta_stage + 4 * (D / G - it_g));
        }
      }
    };
    // one PRQ stage folded into 16 channels: xh[c] = fmaf(q_c, sigma, xh[c]) (the
    // zero points of all stages are added to the centroid beforehand)
    auto stage16 = [&](const uint32_t *cw, float sf, float *xh) {
      float q[16];
      if constexpr (BITS == 2) {
        widen_codes2(cw[0], q);
      } else {
        widen_codes4(cw[0], q);
        widen_codes4(cw[1], q + 8);
      }
  #pragma unroll
      for (int c = 0; c < 16; ++c) xh[c] = fmaf(q[c], sf, xh[c]);
    };
    // centroid channel e of the item as fp32
    auto cent_f32 = [&](int e) -> float {
      if constexpr (CB_BF16) {
        const uint4 v = R.cent[e >> 3];
        const uint32_t w = ((e & 7) >> 1) == 0 ? v.x : ((e & 7) >> 1) == 1 ? v.y : ((e & 7) >> 1) == 2 ? v.z : v.w;
        return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
      } else {
        const uint4 v = R.cent[e >> 2];
        const uint32_t w = (e & 3) == 0 ? v.x : (e & 3) == 1 ? v.y : (e & 3) == 2 ? v.z : v.w;
        return __uint_as_float(w);
      }
    };
    // Rebuild the item for the products: xh = fmaf(q_S, sigma_S, ... fmaf(q_1,
    // sigma_1, c + (z_1 + ... + z_S))), then nearest-even bf16.  This differs
    // from the stage-by-stage reconstruction (c + rhat_1) + rhat_2 ... by a few
    // fp32 ulps, which changes the bf16 operand only for values within those
    // ulps of a bf16 rounding boundary.  It runs in steps, so that it can be
    // spread between the S^T products of a tile: per half of the item (16
    // channels) one step for c + (z_1 + ... + z_S), one per stage, one that
    // packs the half to bf16 and stores it into LDS tile buf.
    constexpr int RB_STEPS = FRESH ? 0 : 2 * (SMAX + 2);
    // Spread between the products where the registers allow it (packed
    // tiles, bf16 codebook, D = 128, no outlier fix-up, at most 3 INT4
    // stages); else the whole rebuild runs before the tile's products, while
    // no S^T accumulator is live (spreading it spilled registers there).
    constexpr bool RB_SPREAD = !FRESH && D == 128 && CB_BF16 && !OUTL && (BITS == 2 || SMAX <= 3);
    float xh[16];
    float zs = 0.0f;
    auto rebuild_step = [&](int c, int buf) {
      if constexpr (!FRESH) {
        const int half = c / (SMAX + 2), j = c % (SMAX + 2);
        if (j == 0) {
          if (half == 0) {
            zs = 0.0f;
  #pragma unroll
            for (int s2 = 0; s2 < SMAX; ++s2) zs += f16_bits_to_f32(uint16_t(R.meta[s2] >> 16));
          }
  #pragma unroll
          for (int e = 0; e < 16; ++e) xh[e] = cent_f32(16 * half + e) + zs;
        } else if (j <= SMAX) {
          stage16(&R.codes[j - 1][half * (BITS / 2)], f16_bits_to_f32(uint16_t(R.meta[j - 1] & 0xffffu)), xh);
        } else if (has_item) {
          uint16_t *dst = (it_kv ? &Vs[buf][it_key * VP + it_ch] : &Ks[buf][it_key * KP + it_ch]) + 16 * half;
          *(uint4 *)(dst) = make_uint4(pack_bf16x2(xh[0], xh[1]), pack_bf16x2(xh[2], xh[3]),
                                       pack_bf16x2(xh[4], xh[5]), pack_bf16x2(xh[6], xh[7]));
          *(uint4 *)(dst + 8) = make_uint4(pack_bf16x2(xh[8], xh[9]), pack_bf16x2(xh[10], xh[11]),
                                           pack_bf16x2(xh[12], xh[13]), pack_bf16x2(xh[14], xh[15]));
        }
      }
    };
    // Finish an item in LDS tile buf: the uncoded rows of a fresh tile are
    // copied as read (four explicit stores: a copy loop kept the item in
    // scratch); with the outlier option, the item's flagged channels (mask
    // word of the key's chunk, the outlier group's (sigma, z), both loaded
    // with the rest of the item's data) are rebuilt again with those and
    // stored over the plain result, the channel's centroid value read back
    // from the thread's copy of its slice in LDS.  A key past the segment's
    // end carries the last key's data, like the plain rebuild.
    auto finish_item = [&](int buf) {
      if (!has_item) return;
      uint16_t *dst = it_kv ? &Vs[buf][it_key * VP + it_ch] : &Ks[buf][it_key * KP + it_ch];
      if constexpr (FRESH) {
        static_assert(KC == 4, "a fresh item is 32 bf16 channels");
        const uint4 c0 = R.cent[0], c1 = R.cent[1], c2 = R.cent[2], c3 = R.cent[3];
        *(uint4 *)(dst) = c0;
        *(uint4 *)(dst + 8) = c1;
        *(uint4 *)(dst + 16) = c2;
        *(uint4 *)(dst + 24) = c3;
      }
      if constexpr (OUTL) {
        uint32_t fm = R.fm;
        if (fm) {
  #pragma unroll
          for (int i = 0; i < KC; ++i) cent_s[i * 512 + tid] = R.cent[i];
          float so[SMAX];
          float zso = 0.0f;
  #pragma unroll
          for (int s2 = 0; s2 < SMAX; ++s2) {
            so[s2] = f16_bits_to_f32(uint16_t(R.mo[s2] & 0xffffu));
            zso += f16_bits_to_f32(uint16_t(R.mo[s2] >> 16));
          }
          while (fm) {
            const int e = __builtin_ctz(fm);
            fm &= fm - 1u;
            constexpr int EPV = 16 / EB;   // centroid elements per uint4
            const uint8_t *cw = (const uint8_t *)&cent_s[(e / EPV) * 512 + tid] + (e % EPV) * EB;
            float v = (CB_BF16 ? bf16_to_f32(*(const uint16_t *)cw) : *(const float *)cw) + zso;
  #pragma unroll
            for (int s2 = 0; s2 < SMAX; ++s2) {
              const uint32_t w = pick_word<KW>(R.codes[s2], (e * BITS) >> 5);
              const float qv = float((w >> ((e * BITS) & 31)) & ((1u << BITS) - 1u));
              v = fmaf(qv, so[s2], v);
            }
            dst[e] = f32_to_bf16_bits(v);
          }
        }
      }
    };

    // a tile that reaches past the segment's last key (its last tile only)
    auto partial_tile = [&](int tile) { return ks + (tile + 1) * AT_BK > ke; };
    // One tile: S^T = K Q^T, the rebuild of the next tile (its registers are
    // ready: loaded during the previous tile), the online softmax and O^T +=
    // V^T P^T.  Each wave mixes its own vector work between its products:
    // the rebuild's arithmetic between the S^T products, the exponentials
    // beside the P V products.  On a segment's last tile the rebuild works on
    // the last data loaded; its result lands in the idle buffer and is never
    // read.
    auto compute_tile = [&](int tile) {
      const int buf = tile & 1;
      const int kt0 = ks + tile * AT_BK;
      // S^T for keys 32*kb + (8*(r/4) + 4*hh + r%4) of the tile, query c32
      floatx16 s0, s1;
  #pragma unroll
      for (int r = 0; r < 16; ++r) { s0[r] = 0.0f; s1[r] = 0.0f; }
      const uint16_t *kp = &Ks[buf][c32 * KP + 8 * hh];
      // k-step s issues its two products, then rebuild steps
      // [RB_STEPS s / NS, RB_STEPS (s+1) / NS) of the next tile; the K
      // fragments of step s+1 are loaded a step ahead.  Scheduling barriers
      // keep this order (the compiler would otherwise issue the 16 products
      // back to back).
      bf16x8 k0 = *(const bf16x8 *)(kp), k1 = *(const bf16x8 *)(kp + 32 * KP);
  #pragma unroll
      for (int s = 0; s < NS; ++s) {
        bf16x8 n0, n1;
        if (s + 1 < NS) {
          n0 = *(const bf16x8 *)(kp + 16 * (s + 1));
          n1 = *(const bf16x8 *)(kp + 32 * KP + 16 * (s + 1));
        }
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[s], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[s], s1, 0, 0, 0);
        if constexpr (RB_SPREAD) {
  #pragma unroll
          for (int c = RB_STEPS * s / NS; c < RB_STEPS * (s + 1) / NS; ++c) rebuild_step(c, buf ^ 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (s + 1 < NS) { k0 = n0; k1 = n1; }
      }
      if constexpr (RB_SPREAD) finish_item(buf ^ 1);
      if (partial_tile(tile)) {
        // an empty volatile asm keeps this a branch taken on the last tile
        // only (speculated, its selects would run on every tile)
        asm volatile("");
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt0 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key >= ke) s0[r] = -INFINITY;
          if (key + 32 >= ke) s1[r] = -INFINITY;
        }
      }
      // tile max: a tree of three-way maxima (v_maximum3_f32) over the 32 values
      // (finite or -inf)
      float vv[32];
  #pragma unroll
      for (int r = 0; r < 16; ++r) { vv[r] = s0[r]; vv[16 + r] = s1[r]; }
      int nv = 32;
  #pragma unroll
      for (int lvl = 0; lvl < 4; ++lvl) {
        if (nv == 1) break;
        int o = 0;
  #pragma unroll
        for (int i = 0; i + 3 <= nv; i += 3)
          vv[o++] = __builtin_elementwise_maximum(vv[i], __builtin_elementwise_maximum(vv[i + 1], vv[i + 2]));
        if (nv % 3 == 2) vv[o++] = __builtin_elementwise_maximum(vv[nv - 2], vv[nv - 1]);
        else if (nv % 3 == 1) vv[o++] = vv[nv - 1];
        nv = o;
      }
      float tmax = pair_max(vv[0]);
      const float mt = tmax * sc;
      const bool need = mt > m_run + AT3_TAU;
      if (__any(need)) {
        const float mnew = need ? mt : m_run;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mnew) : 1.0f;
        m_run = mnew;
  #pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] *= alpha;
        l_part *= alpha;
      }
      const float nm = -m_run;
      // O^T += V^T P^T over 16-key steps (kb, jj).  B operand: lane registers
      // 8*jj .. 8*jj+7 of S^T block kb, i.e. k index 8*hh + e <-> key
      // 32*kb + 16*jj + 8*(e/4) + 4*hh + e%4.  A operand (V^T, rows = channels
      // 32*db + lane%32): two transposing loads, keys 32*kb + 16*jj + 4*hh +
      // 0..3 and the same + 8.
      const uint16_t *vp = &Vs[buf][v_lane];
  #pragma unroll
      for (int kb = 0; kb < 2; ++kb)
  #pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          bf16x8 pb;
  #pragma unroll
          for (int e = 0; e < 8; ++e)
            pb[e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(kb ? s1[8 * jj + e] : s0[8 * jj + e], sc, nm));
          const uint4 w = __builtin_bit_cast(uint4, pb);
          l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.x), ones2, l_part, false);
          l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.y), ones2, l_part, false);
          l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.z), ones2, l_part, false);
          l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.w), ones2, l_part, false);
  #pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const bf16x4 lo = lds_read_tr16(vp + (32 * kb + 16 * jj) * VP + 32 * db);
            const bf16x4 hi = lds_read_tr16(vp + (32 * kb + 16 * jj + 8) * VP + 32 * db);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7),
                                                            pb, o[db], 0, 0, 0);
          }
        }
    };

    // Pipeline: at iteration i every wave multiplies tile i, rebuilds tile
    // i+1 from the data loaded during iteration i-1 and issues the loads of
    // tile i+2 (ids of tile i+3); one barrier per tile.
    __syncthreads();  // previous segment's tiles no longer read
    uint32_t id_next;   // id word of the item's key in tile+2
    load_data(0, load_id_word(0));
  #pragma unroll
    for (int c = 0; c < RB_STEPS; ++c) rebuild_step(c, 0);
    finish_item(0);
    load_data(1, load_id_word(1));
    id_next = load_id_word(2);
    __syncthreads();

    // Where the rebuild is not spread between the products, half of the
    // waves multiply before they rebuild and half after (the split flips
    // between waves w and w+4 and between waves 2k and 2k+1, whichever way
    // waves sit on SIMDs).
    const bool mfma_first = ((wave >> 2) ^ wave) & 1;
    for (int tile = 0; tile < n_tiles; ++tile) {
      if (RB_SPREAD || mfma_first) compute_tile(tile);
      if constexpr (!RB_SPREAD) {
  #pragma unroll
        for (int c = 0; c < RB_STEPS; ++c) rebuild_step(c, (tile & 1) ^ 1);
        finish_item((tile & 1) ^ 1);
      }
      load_data(tile + 2, id_next);
      id_next = load_id_word(tile + 3);
      if (!RB_SPREAD && !mfma_first) compute_tile(tile);
      __syncthreads();
    }

    const float l = pair_sum(l_part);
    if (q < a.n_q) {
      const bool empty = !(l > 0.0f);
      const float inv_l = empty ? 0.0f : 1.0f / l;
      const float lse = empty ? -INFINITY : (m_run + log2f(l)) * 0.6931471805599453f;
      // lane holds channels 32*db + 8*j + 4*hh + 0..3 in o[db][4j .. 4j+3]
      if (slot < 0) {
  #pragma unroll
        for (int db = 0; db < NDB; ++db)
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint64_t off = (uint64_t(h) * a.n_q + q) * D + 32 * db + 8 * j + 4 * hh;
            const float v0 = o[db][4 * j] * inv_l, v1 = o[db][4 * j + 1] * inv_l;
            const float v2 = o[db][4 * j + 2] * inv_l, v3 = o[db][4 * j + 3] * inv_l;
            if (a.out_bf16)
              *(uint2 *)((uint16_t *)a.out + off) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
            else
              *(float4 *)((float *)a.out + off) = make_float4(v0, v1, v2, v3);
          }
        if (a.lse && hh == 0) a.lse[uint64_t(h) * a.n_q + q] = lse;
      } else {
  #pragma unroll
        for (int db = 0; db < NDB; ++db)
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint64_t off = ((uint64_t(slot) * L.H + h) * a.n_q + q) * D + 32 * db + 8 * j + 4 * hh;
            *(float4 *)(a.part_o + off) = make_float4(o[db][4 * j] * inv_l, o[db][4 * j + 1] * inv_l,
                                                      o[db][4 * j + 2] * inv_l, o[db][4 * j + 3] * inv_l);
          }
        if (hh == 0) a.part_lse[(uint64_t(slot) * L.H + h) * a.n_q + q] = lse;
      }
    }
  }
}

// Merge the partials of query blocks shared by several blocks:
// O = sum_s w_s O_s / sum_s w_s with w_s = exp(lse_s - max).  One thread per
// (query, 4 channels); blockIdx.y = head.  Query blocks covered by one block
// were written directly and are skipped.
__global__ __launch_bounds__(256) void k_attend_merge(AttnArgs a) {
  const int D = a.L.D, D4 = D / 4;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(a.n_q) * D4) return;
  const int q = int(idx / D4), d4 = int(idx % D4), h = blockIdx.y;
  const int64_t T = a.n_ktiles, U = a.units_per_block;
  int nseg;
  if (a.head_blocks) {
    // the main segment, then the runs meeting the query block's tail
    const int64_t TL = T - a.main_tiles, qb = q / AT_BQ;
    nseg = TL == 0 ? 1 : 1 + int(((qb + 1) * TL - 1) / U - (qb * TL) / U) + 1;
  } else {
    const int64_t first = (int64_t(h) * a.n_qblocks + q / AT_BQ) * T;
    nseg = int((first + T - 1) / U - first / U) + 1;
  }
  if (nseg == 1) return;
  float ls[kMaxSplits];
  float mx = -INFINITY;
  for (int s = 0; s < nseg; ++s) {
    ls[s] = a.part_lse[(uint64_t(s) * a.L.H + h) * a.n_q + q];
    mx = fmaxf(mx, ls[s]);
  }
  float wsum = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < nseg; ++s) {
    if (ls[s] == -INFINITY) continue;
    const float w = expf(ls[s] - mx);
    wsum += w;
    const float4 v = *(const float4 *)(a.part_o + ((uint64_t(s) * a.L.H + h) * a.n_q + q) * D + 4 * d4);
    acc.x = fmaf(w, v.x, acc.x); acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z); acc.w = fmaf(w, v.w, acc.w);
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  const uint64_t off = (uint64_t(h) * a.n_q + q) * D + 4 * d4;
  if (a.out_bf16) {
    *(uint2 *)((uint16_t *)a.out + off) = make_uint2(
        uint32_t(f32_to_bf16_bits(acc.x * inv)) | (uint32_t(f32_to_bf16_bits(acc.y * inv)) << 16),
        uint32_t(f32_to_bf16_bits(acc.z * inv)) | (uint32_t(f32_to_bf16_bits(acc.w * inv)) << 16));
  } else {
    *(float4 *)((float *)a.out + off) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
  if (a.lse && d4 == 0) a.lse[uint64_t(h) * a.n_q + q] = wsum > 0.0f ? mx + logf(wsum) : -INFINITY;
}

// Two complete results over disjoint key sets (the packed cache and the fresh
// chunk) combined by their log-sum-exps: O = (w1 O1 + w2 O2) / (w1 + w2),
// w_i = exp(lse_i - max), LSE = max + log(w1 + w2); an empty side has
// lse = -inf and weight 0.  One thread per (query, 4 channels); blockIdx.y =
// head.
__global__ __launch_bounds__(256) void k_attend_merge2(MergeArgs m) {
  const int D4 = m.D / 4;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(m.n_q) * D4) return;
  const int q = int(idx / D4), d4 = int(idx % D4), h = blockIdx.y;
  const uint64_t r = uint64_t(h) * m.n_q + q;
  const float l1 = m.lse1[r], l2 = m.lse2[r];
  const float mx = fmaxf(l1, l2);
  const float w1 = l1 == -INFINITY ? 0.0f : expf(l1 - mx);
  const float w2 = l2 == -INFINITY ? 0.0f : expf(l2 - mx);
  const float ws = w1 + w2;
  const float inv = ws > 0.0f ? 1.0f / ws : 0.0f;
  const float4 a = *(const float4 *)(m.o1 + r * m.D + 4 * d4);
  const float4 b = *(const float4 *)(m.o2 + r * m.D + 4 * d4);
  const float4 o = make_float4(fmaf(w1, a.x, w2 * b.x) * inv, fmaf(w1, a.y, w2 * b.y) * inv,
                               fmaf(w1, a.z, w2 * b.z) * inv, fmaf(w1, a.w, w2 * b.w) * inv);
  const uint64_t off = r * m.D + 4 * d4;
  if (m.out_bf16)
    *(uint2 *)((uint16_t *)m.out + off) = make_uint2(pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w));
  else
    *(float4 *)((float *)m.out + off) = o;
  if (m.lse && d4 == 0) m.lse[r] = ws > 0.0f ? mx + logf(ws) : -INFINITY;
}

// ---------------------------------------------------------------- launchers

// blocks of a launch: one per run of units (per-head split: head_blocks per
// head), rounded up to a multiple of 8 when blocks are numbered XCD by XCD
// (blocks past the last run find no work)
static unsigned attend_grid(const AttnArgs &a) {
  const int64_t total = int64_t(a.n_ktiles) * a.n_qblocks * a.L.H;
  const unsigned g = a.head_blocks ? unsigned(a.head_blocks * a.L.H) : cdiv(total, a.units_per_block);
  return a.xcd_remap ? (g + 7) / 8 * 8 : g;
}

template <int D, int G, int BITS, bool BF, int S, bool OUTL>
static void launch_attend_s(const AttnArgs &a, const dim3 &grid, hipStream_t st) {
  QKV_LAUNCH((k_attend3<D, G, BITS, BF, S, false, OUTL>), grid, dim3(512), 0, st, a);
}

template <int D, int G, int BITS, bool BF>
static void launch_attend_t(const AttnArgs &a, hipStream_t st) {
  const dim3 grid(attend_grid(a));
  if (a.L.mask_off) {
    switch (a.L.S) {
      case 1: launch_attend_s<D, G, BITS, BF, 1, true>(a, grid, st); break;
      case 2: launch_attend_s<D, G, BITS, BF, 2, true>(a, grid, st); break;
      case 3: launch_attend_s<D, G, BITS, BF, 3, true>(a, grid, st); break;
      default: launch_attend_s<D, G, BITS, BF, 4, true>(a, grid, st); break;
    }
    return;
  }
  switch (a.L.S) {
    case 1: launch_attend_s<D, G, BITS, BF, 1, false>(a, grid, st); break;
    case 2: launch_attend_s<D, G, BITS, BF, 2, false>(a, grid, st); break;
    case 3: launch_attend_s<D, G, BITS, BF, 3, false>(a, grid, st); break;
    default: launch_attend_s<D, G, BITS, BF, 4, false>(a, grid, st); break;
  }
}

void launch_attend_fresh(const AttnArgs &a, hipStream_t st) {
  const dim3 grid(attend_grid(a));
  if (a.L.D == 64)
    QKV_LAUNCH((k_attend3<64, 32, 2, true, 1, true>), grid, dim3(512), 0, st, a);
  else
    QKV_LAUNCH((k_attend3<128, 32, 2, true, 1, true>), grid, dim3(512), 0, st, a);
  if (a.max_segments > 1)
    QKV_LAUNCH(k_attend_merge, dim3(cdiv(int64_t(a.n_q) * (a.L.D / 4), 256), a.L.H), dim3(256), 0, st, a);
}
void launch_attend_merge2(const MergeArgs &m, hipStream_t st) {
  QKV_LAUNCH(k_attend_merge2, dim3(cdiv(int64_t(m.n_q) * (m.D / 4), 256), m.H), dim3(256), 0, st, m);
}
// Split partials of qkv_attend_noalloc: a fixed device array instead of the
// arena's scratch region.  Every GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` only names the symbol: its
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

int noalloc_scratch_address(void **ptr) {
  return hipGetSymbolAddress(ptr, HIP_SYMBOL(scratch)) == hipSuccess ? 0 : -1;
}

void launch_attend(const AttnArgs &a, hipStream_t st) {
  QKV_DISPATCH_CODEC(a.L, launch_attend_t, a, st);
  if (a.max_segments > 1)
    QKV_LAUNCH(k_attend_merge, dim3(cdiv(int64_t(a.n_q) * (a.L.D / 4), 256), a.L.H), dim3(256), 0, st, a);
}
}  // namespace qkv
