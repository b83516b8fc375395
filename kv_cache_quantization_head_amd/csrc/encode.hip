// Encode kernels of the qkv library: chunk table, k-means (initial codebook,
// nearest-centroid assignment, centroid update), outlier channel flags, and
// the quantize/pack kernel (centroid or prediction subtraction + PRQ stages).
#include "common.h"

namespace qkv {

// ---------------------------------------------------------- encode kernels

// blockIdx.x = stream of the call (2*layer_rel + kv)
__global__ void k_header(EncodeArgs a) {
  if (threadIdx.x != 0) return;
  const int z = blockIdx.x;
  uint8_t *st = stream_ptr(a.arena, a.L, a.layer0 + (z >> 1), z & 1);
  StreamHeader *hdr = (StreamHeader *)(st + a.L.header_off);
  hdr->start[a.slot] = a.t0;
  hdr->start[a.slot + 1] = a.t0 + a.n;
  hdr->n_chunks = a.slot + 1;
  hdr->n_tokens = a.t0 + a.n;
}

// One wave per codebook row: blockIdx.x = group of 4 rows, y = head,
// z = stream of the call.  Row k is the previous call's snapshot row
// (centroid caching) or token floor(k*n/C) (strided start); the norm
// ||c_k||^2 (used only by the screening and its error bound) is summed over
// the wave in fp64.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void k_init(EncodeArgs a) {
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int CPL = D / 64;               // channels per lane
  const DevLayout &L = a.L;
  const int lane = threadIdx.x & 63;
  const int k = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int h = blockIdx.y, z = blockIdx.z, lrel = z >> 1, kv = z & 1;
  if (k >= L.C) return;
  uint8_t *st = stream_ptr(a.arena, L, a.layer0 + lrel, kv);
  uint8_t *cb = st + L.cb_off + uint64_t(a.slot) * L.cb_chunk + uint64_t(h) * L.cb_head;
  float *cn = (float *)(st + L.cn_off + uint64_t(a.slot) * L.cn_chunk + uint64_t(h) * L.cn_head);
  const uint8_t *src;
  if (a.prev_slot >= 0) {
    src = st + L.cb_off + uint64_t(a.prev_slot) * L.cb_chunk + uint64_t(h) * L.cb_head + uint64_t(k) * D * EB;
  } else {
    const int64_t row = (int64_t(k) * a.n) / L.C;
    src = (kv ? a.v_in : a.k_in) + (uint64_t(lrel) * L.H + h) * uint64_t(a.n) * D * EB + uint64_t(row) * D * EB;
  }
  uint8_t *dst = cb + uint64_t(k) * D * EB;
  double acc = 0.0;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int j = lane * CPL + c;
    float v;
    if constexpr (BF16) {
      const uint16_t b = ((const uint16_t *)src)[j];
      ((uint16_t *)dst)[j] = b;
      v = bf16_to_f32(b);
    } else {
      v = ((const float *)src)[j];
      ((float *)dst)[j] = v;
    }
    acc = acc + double(v) * double(v);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) cn[k] = float(acc);
}

// One thread per token.  blockIdx.x = token tile of 256, y = head, z = stream.
//
// Screening: s_k = ||c_k||^2 - 2 x.c_k in fp32 (FMA chain over D channels).
// Its error is below (D+4) 2^-24 (||x||^2 + ||c_k||^2) (dot-product bound
// gamma_D sum|x_j c_j| <= gamma_D (||x||^2+||c||^2)/2, doubled, plus the
// rounding of ||c||^2 and of the subtraction).  E below doubles that again.
// If the two best scores differ by more than 2E, the best one is the exact
// minimiser of the distance with a gap of more than E, far above fp64
// rounding; otherwise the whole wave recomputes D(t, k) for every k in fp64,
// channel by channel, and takes the lowest index among equal minima.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void k_assign(EncodeArgs a) {
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int TK = 64;
  __shared__ float cs[TK][D];
  __shared__ float cns[TK];
  const DevLayout &L = a.L;
  const int h = blockIdx.y, z = blockIdx.z, lrel = z >> 1, kv = z & 1;
  uint8_t *st = stream_ptr(a.arena, L, a.layer0 + lrel, kv);
  const uint8_t *x = (kv ? a.v_in : a.k_in) + (uint64_t(lrel) * L.H + h) * uint64_t(a.n) * D * EB;
  const uint8_t *cb = st + L.cb_off + uint64_t(a.slot) * L.cb_chunk + uint64_t(h) * L.cb_head;
  const float *cn = (const float *)(st + L.cn_off + uint64_t(a.slot) * L.cn_chunk + uint64_t(h) * L.cn_head);
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const bool valid = t < a.n;

  float xr[D];
  float xn = 0.0f;
#pragma unroll
  for (int j = 0; j < D; ++j) {
    xr[j] = valid ? load_elem<BF16>(x + uint64_t(t) * D * EB, j) : 0.0f;
    xn = fmaf(xr[j], xr[j], xn);
  }
  float s1 = INFINITY, s2 = INFINITY, cmax = 0.0f;
  int k1 = 0;
  for (int k0 = 0; k0 < L.C; k0 += TK) {
    __syncthreads();
    for (int i = threadIdx.x; i < TK * D; i += blockDim.x) {
      const int kk = i / D, j = i % D, k = k0 + kk;
      cs[kk][j] = k < L.C ? load_elem<BF16>(cb + uint64_t(k) * D * EB, j) : 0.0f;
    }
    if (threadIdx.x < TK) cns[threadIdx.x] = k0 + int(threadIdx.x) < L.C ? cn[k0 + threadIdx.x] : 0.0f;
    __syncthreads();
    const int kmax = min(TK, L.C - k0);
    for (int kk = 0; kk < kmax; ++kk) {
      float dot = 0.0f;
#pragma unroll
      for (int j = 0; j < D; ++j) dot = fmaf(xr[j], cs[kk][j], dot);
      const float s = cns[kk] - 2.0f * dot;
      cmax = fmaxf(cmax, cns[kk]);
      if (s < s1) {
        s2 = s1; s1 = s; k1 = k0 + kk;
      } else if (s < s2) {
        s2 = s;
      }
    }
  }
  const float E = float(D + 8) * 0x1p-23f * (xn + cmax);
  const bool flag = valid && !(s2 - s1 > 2.0f * E);

  const int lane = threadIdx.x & 63;
  uint64_t fm = __ballot(flag);
  while (fm) {
    const int src = __ffsll((unsigned long long)fm) - 1;
    fm &= fm - 1;
    const int tf = blockIdx.x * blockDim.x + (threadIdx.x & ~63) + src;
    const uint8_t *xrow = x + uint64_t(tf) * D * EB;
    double best = INFINITY;
    int bk = 0x7fffffff;
    for (int k = lane; k < L.C; k += 64) {
      const uint8_t *crow = cb + uint64_t(k) * D * EB;
      double dd = 0.0;
      for (int j = 0; j < D; ++j) {
        const double diff = double(load_elem<BF16>(xrow, j)) - double(load_elem<BF16>(crow, j));
        dd = dd + diff * diff;
      }
      if (dd < best) { best = dd; bk = k; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ob = __shfl_xor(best, off);
      const int ok = __shfl_xor(bk, off);
      if (ob < best || (ob == best && ok < bk)) { best = ob; bk = ok; }
    }
    if (lane == src) k1 = bk;
  }
  if (valid) {
    uint8_t *ids = st + L.ids_off + uint64_t(h) * L.ids_head;
    const int64_t tt = int64_t(a.t0) + t;
    if (L.id_bytes == 1) ids[tt] = uint8_t(k1);
    else ((uint16_t *)ids)[tt] = uint16_t(k1);
  }
}

// MFMA screening for bf16 caches with C <= 512.  The (stream, head, 256-token
// tile) space is flattened; block b takes tiles_per_block consecutive tiles
// (restaging the codebook when the (stream, head) changes); 8 waves, each
// owning 32 tokens of a tile (two 16-token MFMA column blocks).
//
// The head's codebook (bf16, rows padded to the 16-row MFMA block) and
// -||c||^2/2 are staged in LDS once per block.  For a 16-cluster block the
// accumulator starts at -(||c||^2 + ||x||^2)/2 and v_mfma_f32_16x16x32_bf16
// adds x.c, so acc = -D/2 (D the squared distance).  Each lane owns one token
// column and four cluster rows; the fp32 bits of acc with the low 9 bits
// replaced by the cluster index form a key whose unsigned order is the order
// of D (acc <= 0 up to rounding), ties to the lowest index, and the three
// smallest keys are kept with one v_min and two v_med3 per key.  The screening
// error (MFMA accumulation over D+1 terms, rounding of the start value, the
// 9 dropped bits) is below E; a token whose two best keys are within 2E (the
// third clear) joins the block's pair list, decided exactly in fp64 (two lanes
// per token) when the block moves to another head or ends; one whose best
// three are within 2E is rescored exactly against every centroid at once.
constexpr int kPairCap = 512;               // pair list entries per block
constexpr uint32_t kNoToken = 0xffffffffu;  // empty pair list slot
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void k_assign_mfma(EncodeArgs a, int tiles_per_block, int streams) {
  constexpr int KP = D + 8;                 // LDS row pitch (bf16 elements)
  constexpr int STEPS = D / 32;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const DevLayout &L = a.L;
  const int C16 = (L.C + 15) & ~15;
  uint16_t *cbs = (uint16_t *)smem;                          // [C16][KP]
  float *cnh = (float *)(smem + size_t(C16) * KP * 2);       // [C16]
  __shared__ uint32_t cmax_bits;
  // the block's list of pair tokens (within-call token index, two candidates)
  __shared__ uint32_t pq_tok[kPairCap], pq_cand[kPairCap];
  __shared__ int pq_n;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int n_tiles = (a.n + 255) / 256;
  const int64_t total = int64_t(n_tiles) * L.H * streams;
  int cur = -1;                             // (stream, head) whose codebook is in LDS
  const uint16_t *x = nullptr;
  uint8_t *ids = nullptr;
  float cmax = 0.0f;
  // Exact decision for n pair tokens held in registers, entry j at lane j:
  // token (etok, kNoToken for a skipped entry) and its two best candidates
  // (ecand, low and high 16 bits).  Entry j is scored by lanes 2j (first
  // candidate) and 2j+1 (second), the token row read in one go; the winner is
  // written to ids.
  auto decide_pairs = [&](uint32_t etok, uint32_t ecand, int n) {
    const int j = lane >> 1;
    const uint32_t tok = __shfl(etok, j), cc = __shfl(ecand, j);
    const int cand = int((lane & 1) ? (cc >> 16) : (cc & 0xffffu));
    const bool live = j < n && tok != kNoToken;
    double dd = INFINITY;
    if (live) {
      const uint16_t *xrow = x + uint64_t(tok) * D;
      const uint16_t *crow = cbs + cand * KP;
      dd = 0.0;
      uint4 xr[D / 8];
#pragma unroll
      for (int j8 = 0; j8 < D / 8; ++j8) xr[j8] = *(const uint4 *)(xrow + j8 * 8);
#pragma unroll
      for (int j8 = 0; j8 < D / 8; ++j8) {
        const uint4 xv = xr[j8];
        const uint4 cv = *(const uint4 *)(crow + j8 * 8);
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, cw[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t xb = (xw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
          const uint32_t cbb = (cw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
          const double diff = double(bf16_to_f32(xb)) - double(bf16_to_f32(cbb));
          dd = dd + diff * diff;
        }
      }
    }
    const double od = __shfl_xor(dd, 1);
    const int oc = __shfl_xor(cand, 1);
    const int win = (dd < od || (dd == od && cand < oc)) ? cand : oc;
    if (live && !(lane & 1)) {
      const int64_t tt = int64_t(a.t0) + tok;
      if (L.id_bytes == 1) ids[tt] = uint8_t(win);
      else ((uint16_t *)ids)[tt] = uint16_t(win);
    }
  };
  // Block-wide drain of the pair list (every thread calls it): wave w takes
  // entries 32w, 32w + 256, ...; the list is empty afterwards.
  auto drain_pairs = [&]() {
    __syncthreads();
    const int n = min(pq_n, kPairCap);
    for (int e0 = wave * 32; e0 < n; e0 += 8 * 32) {
      const int e = e0 + (lane & 31);
      const uint32_t etok = e < n ? pq_tok[e] : kNoToken, ecand = e < n ? pq_cand[e] : 0u;
      decide_pairs(etok, ecand, min(32, n - e0));
    }
  };
  for (int64_t f = int64_t(blockIdx.x) * tiles_per_block;
       f < min(total, int64_t(blockIdx.x + 1) * tiles_per_block); ++f) {
    const int tile = int(f % n_tiles);
    const int zh = int(f / n_tiles);
    if (zh != cur) {
      // decide the listed pairs of the previous (stream, head), then stage
      // the codebook of (stream, head) zh
      if (cur >= 0) drain_pairs();
      cur = zh;
      const int h = zh % L.H, z = zh / L.H, lrel = z >> 1, kv = z & 1;
      uint8_t *st = stream_ptr(a.arena, L, a.layer0 + lrel, kv);
      x = (const uint16_t *)((kv ? a.v_in : a.k_in)) + (uint64_t(lrel) * L.H + h) * uint64_t(a.n) * D;
      const uint16_t *cb = (const uint16_t *)(st + L.cb_off + uint64_t(a.slot) * L.cb_chunk + uint64_t(h) * L.cb_head);
      const float *cn = (const float *)(st + L.cn_off + uint64_t(a.slot) * L.cn_chunk + uint64_t(h) * L.cn_head);
      ids = st + L.ids_off + uint64_t(h) * L.ids_head;
      __syncthreads();  // previous codebook and pair list no longer read
      if (threadIdx.x == 0) {
        cmax_bits = 0;
        pq_n = 0;
      }
      __syncthreads();
      for (int i = threadIdx.x; i < C16 * (D / 8); i += blockDim.x) {
        const int k = i / (D / 8), c8 = i % (D / 8);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (k < L.C) v = *(const uint4 *)(cb + uint64_t(k) * D + c8 * 8);
        *(uint4 *)(cbs + k * KP + c8 * 8) = v;
      }
      for (int k = threadIdx.x; k < C16; k += blockDim.x) {
        const float c = k < L.C ? cn[k] : 0.0f;
        cnh[k] = k < L.C ? -0.5f * c : -INFINITY;
        if (k < L.C) atomicMax(&cmax_bits, __float_as_uint(c));
      }
      __syncthreads();
      cmax = __uint_as_float(cmax_bits);
    }
    const int tb = tile * 256 + wave * 32;
    bf16x8 xf[2][STEPS];
    float xnh[2], xn[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int t = tb + nt * 16 + c16;
      float ss = 0.0f;
#pragma unroll
      for (int step = 0; step < STEPS; ++step) {
        bf16x8 v;
        if (t < a.n) {
          v = *(const bf16x8 *)(x + uint64_t(t) * D + step * 32 + g4 * 8);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (__bf16)0.0f;
        }
        xf[nt][step] = v;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = (float)v[e];
          ss = fmaf(f, f, ss);
        }
      }
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      xn[nt] = ss;
      xnh[nt] = -0.5f * ss;
    }
    uint32_t m1[2], m2[2], m3[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) m1[nt] = m2[nt] = m3[nt] = 0xffffffffu;
    // The scores of a 16-cluster block are ranked while the products of the
    // next block run: each wave mixes the ranking's vector work between its
    // own products (measured on the device, a wave's back-to-back products
    // and the vector work of other waves on its SIMD overlap little).
    // Scheduling barriers keep the order.
    auto rank4 = [&](const floatx4 *acc, int k0, int r) {
      // with m1 <= m2 <= m3: new third = med3(m2, m3, key), new second =
      // med3(m1, m2, key), new first = min(m1, key)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const uint32_t key = (__float_as_uint(acc[nt][r]) & ~0x1ffu) | uint32_t(k0 + g4 * 4 + r);
        const uint32_t n3 = umed3(m2[nt], m3[nt], key);
        const uint32_t n2 = umed3(m1[nt], m2[nt], key);
        m1[nt] = min(m1[nt], key);
        m2[nt] = n2;
        m3[nt] = n3;
      }
    };
    // products of block k0 into acc; between its k-steps, ranking steps
    // [0, 4) of the previous block's scores (prev; none for the first block)
    auto block = [&](int k0, floatx4 *acc, const floatx4 *prev) {
      bf16x8 ca[STEPS];
#pragma unroll
      for (int step = 0; step < STEPS; ++step)
        ca[step] = *(const bf16x8 *)(cbs + (k0 + c16) * KP + step * 32 + g4 * 8);
      const float4 ch = *(const float4 *)(cnh + k0 + g4 * 4);
      if (prev) rank4(prev, k0 - 16, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        acc[nt] = floatx4{ch.x + xnh[nt], ch.y + xnh[nt], ch.z + xnh[nt], ch.w + xnh[nt]};
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ca[0], xf[nt][0], acc[nt], 0, 0, 0);
      }
#pragma unroll
      for (int step = 1; step < STEPS; ++step) {
        if (prev && step < 4) rank4(prev, k0 - 16, step);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ca[step], xf[nt][step], acc[nt], 0, 0, 0);
      }
      if (prev)
#pragma unroll
        for (int r = STEPS; r < 4; ++r) rank4(prev, k0 - 16, r);
    };
    floatx4 accp[2];
    block(0, accp, nullptr);
    for (int k0 = 16; k0 < C16; k0 += 16) {
      floatx4 accn[2];
      block(k0, accn, accp);
      accp[0] = accn[0];
      accp[1] = accn[1];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) rank4(accp, C16 - 16, r);
    // merge the sorted triples of the four lanes that share a token column
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int off = 16; off <= 32; off <<= 1) {
        const uint32_t b1 = __shfl_xor(m1[nt], off), b2 = __shfl_xor(m2[nt], off), b3 = __shfl_xor(m3[nt], off);
        const uint32_t r3 = min(min(m3[nt], b3), min(max(m2[nt], b1), max(m1[nt], b2)));
        const uint32_t r2 = min(max(m1[nt], b1), min(m2[nt], b2));
        m1[nt] = min(m1[nt], b1);
        m2[nt] = r2;
        m3[nt] = r3;
      }
    }
    auto decode = [](uint32_t m) {
      return m == 0xffffffffu ? INFINITY : -2.0f * __uint_as_float(m & ~0x1ffu);
    };
    // per token (lanes with g4 == 0 own the 16 tokens of each column block)
    bool pair[2], full[2];
    int k1v[2], k2v[2], kbest[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int t = tb + nt * 16 + c16;
      const bool valid = t < a.n && g4 == 0;
      const float d1 = decode(m1[nt]), d2 = decode(m2[nt]), d3 = decode(m3[nt]);
      const float E = float(D + 16) * 0x1p-22f * (xn[nt] + cmax) +
                      0x1p-12f * fmaxf(fabsf(d1), fmaxf(d2 == INFINITY ? 0.0f : fabsf(d2),
                                                        d3 == INFINITY ? 0.0f : fabsf(d3)));
      k1v[nt] = int(m1[nt] & 0x1ffu);
      k2v[nt] = int(m2[nt] & 0x1ffu);
      // decided by the screen / exact check of the two best / exact check of all
      pair[nt] = valid && !(d2 - d1 > 2.0f * E) && (d3 - d1 > 2.0f * E);
      full[nt] = valid && !(d2 - d1 > 2.0f * E) && !(d3 - d1 > 2.0f * E);
      kbest[nt] = k1v[nt];
    }
    // Pair tokens join the block's list (column block 0 first, then 1; each
    // in lane order): the j-th new one of the wave goes to slot base + j.  A
    // wave whose tokens do not all fit marks its slots below the capacity
    // empty and sends its pair tokens to the full rescoring.
    const uint64_t pm0 = __ballot(pair[0]), pm1 = __ballot(pair[1]);
    if (pm0 | pm1) {
      const int np0 = __popcll(pm0), np = np0 + __popcll(pm1);
      int base = 0;
      if (lane == 0) base = atomicAdd(&pq_n, np);
      base = __shfl(base, 0);
      const int j = lane;
      const bool take = j < np;
      const int jn = j < np0 ? 0 : 1;                         // column block of new token j
      // lane of new token j: the (j - np0*jn)-th set bit of its block's mask
      uint64_t m = jn ? pm1 : pm0;
      int rank = take ? j - np0 * jn : 0, src = 0;
#pragma unroll
      for (int w = 32; w >= 1; w >>= 1) {
        const int c = __popcll((m >> src) & ((uint64_t(1) << w) - 1));
        if (rank >= c) { rank -= c; src += w; }
      }
      // all four shuffles run on every lane (a shuffle under a divergent
      // select would read the select taken by the source lane)
      const int a1 = __shfl(k1v[0], src), a2 = __shfl(k2v[0], src);
      const int b1 = __shfl(k1v[1], src), b2 = __shfl(k2v[1], src);
      const uint32_t etok = uint32_t(tb + jn * 16 + src);
      const uint32_t ecand = jn ? (uint32_t(b1) | (uint32_t(b2) << 16)) : (uint32_t(a1) | (uint32_t(a2) << 16));
      if (base + np <= kPairCap) {
        if (take) {
          pq_tok[base + j] = etok;
          pq_cand[base + j] = ecand;
        }
      } else {
        // rescored against every centroid below
        if (take && base + j < kPairCap) pq_tok[base + j] = kNoToken;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          full[nt] = full[nt] || pair[nt];
          pair[nt] = false;
        }
      }
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int t = tb + nt * 16 + c16;
      const bool valid = t < a.n && g4 == 0;
      uint64_t fm = __ballot(full[nt]);
      while (fm) {
        const int src = __ffsll((unsigned long long)fm) - 1;
        fm &= fm - 1;
        const int tf = tb + nt * 16 + (src & 15);
        const uint16_t *xrow = x + uint64_t(tf) * D;
        double best = INFINITY;
        int bk = 0x7fffffff;
        for (int k = lane; k < L.C; k += 64) {
          const uint16_t *crow = cbs + k * KP;      // codebook row in LDS
          double dd = 0.0;
          for (int j8 = 0; j8 < D / 8; ++j8) {
            const uint4 xv = *(const uint4 *)(xrow + j8 * 8);
            const uint4 cv = *(const uint4 *)(crow + j8 * 8);
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, cw[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint32_t xb = (xw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
              const uint32_t cbb = (cw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
              const double diff = double(bf16_to_f32(xb)) - double(bf16_to_f32(cbb));
              dd = dd + diff * diff;
            }
          }
          if (dd < best) { best = dd; bk = k; }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          const double ob = __shfl_xor(best, off);
          const int ok = __shfl_xor(bk, off);
          if (ob < best || (ob == best && ok < bk)) { best = ob; bk = ok; }
        }
        if (lane == src) kbest[nt] = bk;
      }
      if (valid && !pair[nt]) {
        const int64_t tt = int64_t(a.t0) + t;
        if (L.id_bytes == 1) ids[tt] = uint8_t(kbest[nt]);
        else ((uint16_t *)ids)[tt] = uint16_t(kbest[nt]);
      }
    }
  }
  if (cur >= 0) drain_pairs();
}

// One wave per 4 clusters; blockIdx.x = group of 16 clusters, y = head, z = stream.
// Each wave scans the call's ids in token order and adds the member rows in
// fp64 (lane = D/64 channels), so every centroid sum is the sequential sum in
// token order.  Empty clusters keep their centroid.
template <int D, bool BF16>
__device__ __forceinline__ void finalize_centroid(uint8_t *cb, float *cn, int k, int C, int cnt,
                                                  const double *acc, int lane) {
  constexpr int CPL = D / 64;
  if (k >= C || cnt == 0) return;
  double nrm = 0.0;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const double mean = acc[c] / double(cnt);
    const int j = lane * CPL + c;
    float v;
    if constexpr (BF16) {
      const uint16_t b = f64_to_bf16_bits(mean);
      ((uint16_t *)cb)[uint64_t(k) * D + j] = b;
      v = bf16_to_f32(b);
    } else {
      v = float(mean);
      ((float *)cb)[uint64_t(k) * D + j] = v;
    }
    nrm = nrm + double(v) * double(v);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) nrm += __shfl_xor(nrm, off);
  if (lane == 0) cn[k] = float(nrm);
}

// Block = 16 waves, one cluster each (blockIdx.x = group of 16 clusters,
// y = head, z = stream).  The block stages a segment of the call's ids in LDS;
// each wave scans it in token order, appending its cluster's member token
// indices to a list in LDS; a full list (or the end of the ids) is drained by
// summing the listed rows in list order with UPD_UNROLL (bf16 rows of 128
// channels: UPD_UNROLL_BF, kept packed) row loads in flight, so every
// centroid sum is the sequential fp64 sum in token order.
// Raw (unformatted, stride 0) buffer resource over `bytes` bytes at p; the
// fourth word is the gfx9 data-format field for 32-bit raw access.  Loads past
// the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, int(bytes), 0x00020000);
}

constexpr int UPD_SEG = 16384;      // ids staged per pass
constexpr int UPD_CAP = 512;        // list entries per cluster
constexpr int UPD_UNROLL = 32;
constexpr int UPD_UNROLL_BF = 64;    // bf16 rows kept packed (one register per row and lane)

template <int D, bool BF16>
__device__ __forceinline__ void drain_list(const uint8_t *x, const int32_t *list, int count, double *acc,
                                           int lane, __amdgpu_buffer_rsrc_t xr) {
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int CPL = D / 64;
  if constexpr (BF16 && CPL == 2) {
    static_assert(UPD_UNROLL_BF == 64, "one list entry per lane");
    for (int i = 0; i < count; i += UPD_UNROLL_BF) {
      // lane e holds the e-th row index of the batch (tail: the last row,
      // reloaded but not added); each row address is formed in scalar
      // registers from the wave-uniform index
      const int mine = list[min(i + lane, count - 1)];
      uint32_t v[UPD_UNROLL_BF];
#pragma unroll
      for (int e = 0; e < UPD_UNROLL_BF; ++e) {
        const int row = __builtin_amdgcn_readlane(mine, e);
        v[e] = __builtin_amdgcn_raw_buffer_load_b32(xr, 4 * lane, row * (D * EB), 0);
      }
#pragma unroll
      for (int e = 0; e < UPD_UNROLL_BF; ++e) {
        if (i + e < count) {
          acc[0] = acc[0] + double(__uint_as_float(v[e] << 16));
          acc[1] = acc[1] + double(__uint_as_float(v[e] & 0xffff0000u));
        }
      }
    }
  } else {
    for (int i = 0; i < count; i += UPD_UNROLL) {
      float v[UPD_UNROLL][CPL];
#pragma unroll
      for (int e = 0; e < UPD_UNROLL; ++e) {
        const int row = list[min(i + e, count - 1)];   // tail: reload the last row, not added
        const uint8_t *rp = x + uint64_t(row) * D * EB;
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[e][c] = load_elem<BF16>(rp, lane * CPL + c);
      }
#pragma unroll
      for (int e = 0; e < UPD_UNROLL; ++e) {
        if (i + e < count) {
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[c] = acc[c] + double(v[e][c]);
        }
      }
    }
  }
}

template <int D, bool BF16>
__global__ __launch_bounds__(1024) void k_update(EncodeArgs a) {
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int CPL = D / 64;
  __shared__ __attribute__((aligned(16))) uint8_t sid_raw[UPD_SEG * 2];
  __shared__ int32_t lists[16][UPD_CAP];
  const DevLayout &L = a.L;
  const int h = blockIdx.y, z = blockIdx.z, lrel = z >> 1, kv = z & 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int k = blockIdx.x * 16 + wave;
  uint8_t *st = stream_ptr(a.arena, L, a.layer0 + lrel, kv);
  const uint8_t *x = (kv ? a.v_in : a.k_in) + (uint64_t(lrel) * L.H + h) * uint64_t(a.n) * D * EB;
  const __amdgpu_buffer_rsrc_t xr = raw_rsrc(x, uint32_t(a.n) * D * EB);
  const uint8_t *ids = st + L.ids_off + uint64_t(h) * L.ids_head + uint64_t(a.t0) * L.id_bytes;
  uint8_t *cb = st + L.cb_off + uint64_t(a.slot) * L.cb_chunk + uint64_t(h) * L.cb_head;
  float *cn = (float *)(st + L.cn_off + uint64_t(a.slot) * L.cn_chunk + uint64_t(h) * L.cn_head);

  double acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.0;
  int cnt = 0, fill = 0;              // wave-uniform
  int32_t *list = &lists[wave][0];
  const uint64_t below = (uint64_t(1) << lane) - 1;

  for (int seg0 = 0; seg0 < a.n; seg0 += UPD_SEG) {
    const int segn = min(UPD_SEG, a.n - seg0);
    __syncthreads();
    // stage the segment's ids (bytes; ids start on any byte, so copy bytewise
    // when unaligned, else 16 bytes at a time)
    const int nbytes = segn * L.id_bytes;
    const uint8_t *src = ids + uint64_t(seg0) * L.id_bytes;
    if ((reinterpret_cast<uintptr_t>(src) & 15) == 0) {
      for (int i = threadIdx.x; i < nbytes / 16; i += blockDim.x)
        *(uint4 *)(sid_raw + 16 * i) = *(const uint4 *)(src + 16 * i);
      for (int i = (nbytes / 16) * 16 + threadIdx.x; i < nbytes; i += blockDim.x) sid_raw[i] = src[i];
    } else {
      for (int i = threadIdx.x; i < nbytes; i += blockDim.x) sid_raw[i] = src[i];
    }
    __syncthreads();
    if (k < L.C) {
      for (int w0 = 0; w0 < segn; w0 += 64) {
        const int t = w0 + lane;
        int myid = -1;
        if (t < segn) myid = L.id_bytes == 1 ? int(sid_raw[t]) : int(((const uint16_t *)sid_raw)[t]);
        const uint64_t m = __ballot(myid == k);
        if (m == 0) continue;
        const int nm = __popcll(m);
        if (fill + nm > UPD_CAP) {
          drain_list<D, BF16>(x, list, fill, acc, lane, xr);
          fill = 0;
        }
        if ((m >> lane) & 1) list[fill + __popcll(m & below)] = seg0 + t;
        fill += nm;
        cnt += nm;
      }
    }
  }
  if (k >= L.C) return;
  if (fill) drain_list<D, BF16>(x, list, fill, acc, lane, xr);
  finalize_centroid<D, BF16>(cb, cn, k, L.C, cnt, acc, lane);
}

// Stable sort of one 256-token tile of a call's ids (blockIdx.x = tile,
// y = head, z = stream): keys (id << 8 | offset) are bitonic-sorted in LDS;
// the tile's permutation (offsets in (id, token) order) and, for every
// cluster k in [0, C], the position of its first member are written out.
__global__ __launch_bounds__(256) void k_tile_sort(EncodeArgs a) {
  __shared__ uint32_t keys[256];
  const DevLayout &L = a.L;
  const int tile = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
  const uint8_t *st = stream_ptr(a.arena, L, a.layer0 + (z >> 1), z & 1);
  const uint8_t *ids = st + L.ids_off + uint64_t(h) * L.ids_head + uint64_t(a.t0) * L.id_bytes;
  const int i = threadIdx.x;
  const int t = tile * 256 + i;
  keys[i] = t < a.n ? (uint32_t(load_id(ids, L.id_bytes, t)) << 8) | uint32_t(i) : 0xffffffffu;
  __syncthreads();
  for (int size = 2; size <= 256; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int j = i ^ stride;
      if (j > i) {
        const uint32_t u = keys[i], v = keys[j];
        const bool up = (i & size) == 0;
        if ((u > v) == up) { keys[i] = v; keys[j] = u; }
      }
      __syncthreads();
    }
  }
  const uint64_t unit = (uint64_t(z) * L.H + h) * uint64_t(a.sort_tiles) + tile;
  a.sort_perm[unit * 256 + i] = uint8_t(keys[i] & 0xffu);
  uint16_t *off = a.sort_off + unit * uint64_t(L.C + 1);
  for (int k = i; k <= L.C; k += blockDim.x) {
    const uint32_t target = uint32_t(k) << 8;
    int lo = 0, hi = 256;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (keys[mid] < target) lo = mid + 1; else hi = mid;
    }
    off[k] = uint16_t(lo);
  }
}

// The same outputs as k_tile_sort for C <= CMAX (256 or 1024), by a stable
// counting sort: a token's rank among the equal ids of its wave comes from
// ballots over the id's bits and a past-the-end flag; per-wave counts and a
// scan over the ids give each cluster's start and each wave's offset in it.
template <int CMAX>
__global__ __launch_bounds__(256) void k_tile_sort_count(EncodeArgs a) {
  constexpr int NB = CMAX == 256 ? 9 : 11;     // id bits + the past-the-end flag (id == CMAX)
  constexpr int PER = CMAX / 256;              // clusters per thread in the scan
  __shared__ uint32_t cnt[4][CMAX];
  __shared__ uint32_t wsum[4];
  const DevLayout &L = a.L;
  const int tile = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
  const uint8_t *st = stream_ptr(a.arena, L, a.layer0 + (z >> 1), z & 1);
  const uint8_t *ids = st + L.ids_off + uint64_t(h) * L.ids_head + uint64_t(a.t0) * L.id_bytes;
  const int i = threadIdx.x, wave = i >> 6, lane = i & 63;
  const int t = tile * 256 + i;
  const bool valid = t < a.n;
  const int id = valid ? load_id(ids, L.id_bytes, t) : CMAX;
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int p = 0; p < PER; ++p) cnt[w][p * 256 + i] = 0;
  uint64_t eq = ~uint64_t(0);                 // lanes of the wave with this lane's id
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint64_t m = __ballot((id >> b) & 1);
    eq &= ((id >> b) & 1) ? m : ~m;
  }
  const int rank = __popcll(eq & ((uint64_t(1) << lane) - 1));
  __syncthreads();
  if (valid && rank == 0) cnt[wave][id] = uint32_t(__popcll(eq));
  __syncthreads();
  // thread i now stands for clusters PER*i .. PER*i + PER-1
  uint32_t c[PER][4], tot[PER], sum = 0;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int kk = PER * i + p;
    tot[p] = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      c[p][w] = cnt[w][kk];
      tot[p] += c[p][w];
    }
    sum += tot[p];
  }
  uint32_t incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t start = incl - sum;
  for (int w = 0; w < wave; ++w) start += wsum[w];
  const uint64_t unit = (uint64_t(z) * L.H + h) * uint64_t(a.sort_tiles) + tile;
  uint16_t *off = a.sort_off + unit * uint64_t(L.C + 1);
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int kk = PER * i + p;
    uint32_t o = start;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      cnt[w][kk] = o;
      o += c[p][w];
    }
    if (kk <= L.C) off[kk] = uint16_t(start);
    start += tot[p];
  }
  if (i == 0 && L.C == CMAX) off[CMAX] = uint16_t(min(256, a.n - tile * 256));
  __syncthreads();
  // past-the-end tokens keep their place after the valid ones
  const int pos = valid ? int(cnt[wave][id]) + rank : i;
  a.sort_perm[unit * 256 + pos] = uint8_t(i);
}

// k-means update from the tile sort: one wave per cluster (blockIdx.x = group
// of 4 clusters, y = head, z = stream).  Lanes read the cluster's member range
// of 64 tiles at a time; a wave prefix sum lays the members out in token order
// (tiles ascending, offsets ascending inside a tile) in an LDS list, drained
// with UPD_UNROLL row loads in flight: the sum is the sequential fp64 sum in
// token order.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void k_update_sorted(EncodeArgs a) {
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int CPL = D / 64;
  __shared__ int32_t lists[4][UPD_CAP];
  const DevLayout &L = a.L;
  const int h = blockIdx.y, z = blockIdx.z, lrel = z >> 1, kv = z & 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int k = blockIdx.x * 4 + wave;
  if (k >= L.C) return;  // whole wave; no block barrier below
  uint8_t *st = stream_ptr(a.arena, L, a.layer0 + lrel, kv);
  const uint8_t *x = (kv ? a.v_in : a.k_in) + (uint64_t(lrel) * L.H + h) * uint64_t(a.n) * D * EB;
  const __amdgpu_buffer_rsrc_t xr = raw_rsrc(x, uint32_t(a.n) * D * EB);
  uint8_t *cb = st + L.cb_off + uint64_t(a.slot) * L.cb_chunk + uint64_t(h) * L.cb_head;
  float *cn = (float *)(st + L.cn_off + uint64_t(a.slot) * L.cn_chunk + uint64_t(h) * L.cn_head);
  const uint64_t unit0 = (uint64_t(z) * L.H + h) * uint64_t(a.sort_tiles);
  const uint8_t *perm = a.sort_perm + unit0 * 256;
  const uint16_t *off = a.sort_off + unit0 * uint64_t(L.C + 1);
  int32_t *list = &lists[wave][0];

  double acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.0;
  int cnt = 0, fill = 0;  // wave-uniform
  const int n_tiles = (a.n + 255) / 256;
  for (int tc = 0; tc < n_tiles; tc += 64) {
    const int tile = tc + lane;
    int beg = 0, num = 0;
    if (tile < n_tiles) {
      const uint16_t *o = off + uint64_t(tile) * (L.C + 1);
      beg = o[k];
      num = int(o[k + 1]) - beg;
    }
    int incl = num;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    const int total = __shfl(incl, 63);
    const int excl = incl - num;
    int done = 0;
    while (done < total) {
      if (fill == UPD_CAP) {
        drain_list<D, BF16>(x, list, fill, acc, lane, xr);
        fill = 0;
      }
      const int take = min(UPD_CAP - fill, total - done);
      const int e0 = max(0, done - excl), e1 = min(num, done + take - excl);
      // four member offsets read per round trip
      const uint8_t *pt = perm + uint64_t(tile) * 256 + beg;
      for (int e = e0; e < e1; e += 4) {
        int pv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) pv[u] = e + u < e1 ? int(pt[e + u]) : 0;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (e + u < e1) list[fill + excl + e + u - done] = tile * 256 + pv[u];
      }
      fill += take;
      done += take;
      cnt += take;
    }
  }
  if (fill) drain_list<D, BF16>(x, list, fill, acc, lane, xr);
  finalize_centroid<D, BF16>(cb, cn, k, L.C, cnt, acc, lane);
}

// Outlier channels, step 1: per (stream, head, token range p) the sums over
// the range's tokens of r^2 for every channel, r = fl32(x - c_id) the
// residual the stages will code, squared and summed in fp64.  Block = 4
// waves; a lane holds 8 consecutive channels of one token per step (16-byte
// loads; a wave covers 64 * 8 / D tokens per step), the waves' and slots'
// sums are added in a fixed order, so the result does not depend on timing.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void k_chan_stats(EncodeArgs a) {
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int LPT = D / 8;            // lanes per token
  constexpr int TPW = 64 / LPT;         // tokens per wave step
  __shared__ double part[4 * TPW][D];
  const DevLayout &L = a.L;
  const int p = blockIdx.x, h = blockIdx.y, z = blockIdx.z, lrel = z >> 1, kv = z & 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ts = lane / LPT, c0 = (lane % LPT) * 8;
  const int tb = int(int64_t(a.n) * p / kChanParts), te = int(int64_t(a.n) * (p + 1) / kChanParts);
  const uint8_t *st = stream_ptr(a.arena, L, a.layer0 + lrel, kv);
  const uint8_t *xb = (kv ? a.v_in : a.k_in) + (uint64_t(lrel) * L.H + h) * uint64_t(a.n) * (D * EB) + c0 * EB;
  const uint8_t *ids = st + L.ids_off + uint64_t(h) * L.ids_head;
  const uint8_t *cb = st + L.cb_off + uint64_t(a.slot) * L.cb_chunk + uint64_t(h) * L.cb_head + c0 * EB;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  for (int t = tb + wave * TPW + ts; t < te; t += 4 * TPW) {
    const int id = load_id(ids, L.id_bytes, int64_t(a.t0) + t);
    const uint8_t *xr = xb + uint64_t(t) * (D * EB);
    const uint8_t *cr = cb + uint64_t(id) * (D * EB);
    float xv[8], cv[8];
    if constexpr (BF16) {
      const uint4 u = *(const uint4 *)xr, c = *(const uint4 *)cr;
      const uint32_t uw[4] = {u.x, u.y, u.z, u.w}, cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xv[2 * i] = __uint_as_float(uw[i] << 16); xv[2 * i + 1] = __uint_as_float(uw[i] & 0xffff0000u);
        cv[2 * i] = __uint_as_float(cw[i] << 16); cv[2 * i + 1] = __uint_as_float(cw[i] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float4 u = ((const float4 *)xr)[i], c = ((const float4 *)cr)[i];
        xv[4 * i] = u.x; xv[4 * i + 1] = u.y; xv[4 * i + 2] = u.z; xv[4 * i + 3] = u.w;
        cv[4 * i] = c.x; cv[4 * i + 1] = c.y; cv[4 * i + 2] = c.z; cv[4 * i + 3] = c.w;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double r = double(xv[e] - cv[e]);
      acc[e] = fma(r, r, acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[wave * TPW + ts][c0 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    double sum = 0.0;
    for (int i = 0; i < 4 * TPW; ++i) sum += part[i][threadIdx.x];
    a.chan_part[((uint64_t(z) * L.H + h) * kChanParts + p) * D + threadIdx.x] = sum;
  }
}

// Outlier channels, step 2: one block of 128 threads per (head, stream);
// thread j owns channel j.  n_j = sqrt(sum of the ranges' sums, in range
// order); med and MAD are the means of the two middle values of the sorted
// norms and of the sorted |n_j - med| (rank sort in LDS, ties by channel).
// Channel j is flagged when 0.6745 (n_j - med) > 3.5 MAD and n_j > 2 med; the
// flags are stored as the d-bit mask of this call's slot.
template <int D>
__global__ __launch_bounds__(128) void k_chan_flags(EncodeArgs a) {
  __shared__ double vals[D], sorted[D];
  __shared__ double stat_s;
  const DevLayout &L = a.L;
  const int j = threadIdx.x, h = blockIdx.x, z = blockIdx.y, lrel = z >> 1, kv = z & 1;
  const bool own = j < D;
  double nj = 0.0;
  if (own) {
    const double *pp = a.chan_part + (uint64_t(z) * L.H + h) * kChanParts * D + j;
    double sum = 0.0;
    for (int p = 0; p < kChanParts; ++p) sum += pp[p * D];
    nj = sqrt(sum);
    vals[j] = nj;
  }
  __syncthreads();
  auto rank_store = [&](double v) {
    int rank = 0;
    for (int i = 0; i < D; ++i) {
      const double o = vals[i];
      rank += (o < v) || (o == v && i < j);
    }
    sorted[rank] = v;
  };
  if (own) rank_store(nj);
  __syncthreads();
  if (j == 0) stat_s = (sorted[D / 2 - 1] + sorted[D / 2]) * 0.5;
  __syncthreads();
  const double med = stat_s;
  const double dev = fabs(nj - med);
  if (own) vals[j] = dev;
  __syncthreads();
  if (own) rank_store(dev);
  __syncthreads();
  if (j == 0) stat_s = (sorted[D / 2 - 1] + sorted[D / 2]) * 0.5;
  __syncthreads();
  const double mad = stat_s;
  const bool flag = own && (0.6745 * (nj - med) > 3.5 * mad) && (nj > 2.0 * med);
  const uint64_t bits = __ballot(flag);
  if (own && (j & 63) == 0) {
    uint8_t *st = stream_ptr(a.arena, L, a.layer0 + lrel, kv);
    uint32_t *mw = (uint32_t *)(st + L.mask_off + uint64_t(a.slot) * L.mask_chunk + uint64_t(h) * L.mask_head) +
                   (j >> 5);
    mw[0] = uint32_t(bits);
    mw[1] = uint32_t(bits >> 32);
  }
}

// One thread per (token, group).  blockIdx.x = tile of 256 (token, group)
// items, y = head, z = stream.  Base = centroid of the token's cluster, or the
// cross-layer prediction when a.pred is set (then the reconstruction is also
// written to a.chain in bf16).
// CHAIN: also accumulate the reconstruction and write it to a.chain in bf16.
// OUTL: the call's flagged channels (mask of its slot) form one more group
// per token and stage, spread over the token's D/G threads (min and max
// combined across them); meta entry D/G holds its (sigma, z).
template <int D, int G, int BITS, bool BF16, bool CHAIN, bool OUTL = false>
__global__ __launch_bounds__(256) void k_quantize(EncodeArgs a) {
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int NG = D / G;
  constexpr int WORDS = G * BITS / 32;
  constexpr float LEVELS = float((1 << BITS) - 1);
  const DevLayout &L = a.L;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int t = idx / NG, g = idx % NG;
  if (t >= a.n) return;
  const int h = blockIdx.y, z = blockIdx.z, lrel = z >> 1, kv = z & 1;
  uint8_t *st = stream_ptr(a.arena, L, a.layer0 + lrel, kv);
  const uint8_t *xrow =
      (kv ? a.v_in : a.k_in) + ((uint64_t(lrel) * L.H + h) * uint64_t(a.n) + t) * D * EB;
  const int64_t tt = int64_t(a.t0) + t;

  float r[G], xh[G];
  if (a.pred) {
    const float *p = a.pred + ((uint64_t(kv) * L.H + h) * uint64_t(a.n) + t) * D + g * G;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      xh[j] = p[j];
      r[j] = load_elem<BF16>(xrow, g * G + j) - p[j];
    }
  } else {
    const uint8_t *ids = st + L.ids_off + uint64_t(h) * L.ids_head;
    const int id = load_id(ids, L.id_bytes, tt);
    const uint8_t *crow = st + L.cb_off + uint64_t(a.slot) * L.cb_chunk + uint64_t(h) * L.cb_head +
                          uint64_t(id) * D * EB;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float c = load_elem<BF16>(crow, g * G + j);
      xh[j] = c;
      r[j] = load_elem<BF16>(xrow, g * G + j) - c;
    }
  }
  constexpr int FW = (G + 31) / 32;
  uint32_t fm[FW];
  if constexpr (OUTL) {
    const uint32_t *mw = (const uint32_t *)(st + L.mask_off + uint64_t(a.slot) * L.mask_chunk +
                                            uint64_t(h) * L.mask_head);
#pragma unroll
    for (int i = 0; i < FW; ++i) fm[i] = mw[g * FW + i];
  }
  for (int s = 0; s < L.S; ++s) {
    if constexpr (OUTL) {
      // an empty asm statement makes the flag words opaque at every stage, so
      // the per-channel flags are extracted where used (a bit test each)
      // rather than held in registers across the stage loop
#pragma unroll
      for (int i = 0; i < FW; ++i) asm volatile("" : "+v"(fm[i]));
      float mn = INFINITY, mx = -INFINITY, omn = INFINITY, omx = -INFINITY;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const bool f = (fm[j >> 5] >> (j & 31)) & 1u;
        mn = fminf(mn, f ? INFINITY : r[j]);
        mx = fmaxf(mx, f ? -INFINITY : r[j]);
        omn = fminf(omn, f ? r[j] : INFINITY);
        omx = fmaxf(omx, f ? r[j] : -INFINITY);
      }
      // the token's threads are NG consecutive lanes
#pragma unroll
      for (int m = 1; m < NG; m <<= 1) {
        omn = fminf(omn, __shfl_xor(omn, m));
        omx = fmaxf(omx, __shfl_xor(omx, m));
      }
      // a group without channels stores (0, 0)
      const bool hn = mn <= mx, ho = omn <= omx;
      const uint16_t zb = hn ? f32_to_f16_bits(mn) : uint16_t(0);
      const float zf = f16_bits_to_f32(zb);
      const uint16_t sb = hn ? f32_to_f16_bits((mx - zf) / LEVELS) : uint16_t(0);
      const float sf = f16_bits_to_f32(sb);
      const uint16_t zbo = ho ? f32_to_f16_bits(omn) : uint16_t(0);
      const float zfo = f16_bits_to_f32(zbo);
      const uint16_t sbo = ho ? f32_to_f16_bits((omx - zfo) / LEVELS) : uint16_t(0);
      const float sfo = f16_bits_to_f32(sbo);
      // reciprocals of the two sigmas (0 for a degenerate group, which makes
      // every code 0 with r^ = z); opaque, so that the per-channel select
      // below is not turned into a division per channel
      float inv = sf != 0.0f ? 1.0f / sf : 0.0f, invo = sfo != 0.0f ? 1.0f / sfo : 0.0f;
      asm volatile("" : "+v"(inv), "+v"(invo));
      constexpr int PER_BYTE = 8 / BITS;
      uint32_t w[WORDS];
#pragma unroll
      for (int i = 0; i < WORDS; ++i) w[i] = 0;
#pragma unroll
      for (int j0 = 0; j0 < G; j0 += PER_BYTE) {
        float q[PER_BYTE];
#pragma unroll
        for (int e = 0; e < PER_BYTE; ++e) {
          const int j = j0 + e;
          const bool f = (fm[j >> 5] >> (j & 31)) & 1u;
          const float zj = f ? zfo : zf, sj = f ? sfo : sf, ij = f ? invo : inv;
          q[e] = fminf(fmaxf(rintf((r[j] - zj) * ij), 0.0f), LEVELS);
          const float rh = fmaf(q[e], sj, zj);
          r[j] = r[j] - rh;
          if constexpr (CHAIN) xh[j] = xh[j] + rh;
        }
        float byte = q[PER_BYTE - 1];
#pragma unroll
        for (int e = PER_BYTE - 2; e >= 0; --e) byte = fmaf(byte, float(1 << BITS), q[e]);
        const int bi = j0 / PER_BYTE;
        w[bi / 4] = __builtin_amdgcn_cvt_pk_u8_f32(byte, bi % 4, w[bi / 4]);
      }
      uint8_t *cp = st + L.codes_off + uint64_t(s) * L.codes_stage + uint64_t(h) * L.codes_head +
                    uint64_t(tt) * L.codes_token + uint64_t(g) * (G * BITS / 8);
      if constexpr (WORDS == 2) {
        *(uint2 *)cp = make_uint2(w[0], w[1]);
      } else {
#pragma unroll
        for (int i = 0; i < WORDS; i += 4) *(uint4 *)(cp + 4 * i) = make_uint4(w[i], w[i + 1], w[i + 2], w[i + 3]);
      }
      uint32_t *mp = (uint32_t *)(st + L.meta_off + uint64_t(s) * L.meta_stage + uint64_t(h) * L.meta_head +
                                  uint64_t(tt) * L.meta_token);
      mp[g] = uint32_t(sb) | (uint32_t(zb) << 16);
      if (g == 0) mp[NG] = uint32_t(sbo) | (uint32_t(zbo) << 16);
      continue;
    }
    float mn = r[0], mx = r[0];
#pragma unroll
    for (int j = 1; j < G; ++j) {
      mn = fminf(mn, r[j]);
      mx = fmaxf(mx, r[j]);
    }
    const uint16_t zb = f32_to_f16_bits(mn);
    const float zf = f16_bits_to_f32(zb);
    const uint16_t sb = f32_to_f16_bits((mx - zf) / LEVELS);
    const float sf = f16_bits_to_f32(sb);
    uint32_t w[WORDS];
    if (sf != 0.0f) {
      const float inv = 1.0f / sf;
      // codes packed a byte at a time: the byte's codes combined as an exact
      // small integer in fp32, then converted into its byte of the word
      // (v_cvt_pk_u8_f32)
      constexpr int PER_BYTE = 8 / BITS;
#pragma unroll
      for (int i = 0; i < WORDS; ++i) w[i] = 0;
#pragma unroll
      for (int j0 = 0; j0 < G; j0 += PER_BYTE) {
        float q[PER_BYTE];
#pragma unroll
        for (int e = 0; e < PER_BYTE; ++e) {
          const int j = j0 + e;
          q[e] = fminf(fmaxf(rintf((r[j] - zf) * inv), 0.0f), LEVELS);
          const float rh = fmaf(q[e], sf, zf);
          r[j] = r[j] - rh;
          if constexpr (CHAIN) xh[j] = xh[j] + rh;
        }
        float byte = q[PER_BYTE - 1];
#pragma unroll
        for (int e = PER_BYTE - 2; e >= 0; --e) byte = fmaf(byte, float(1 << BITS), q[e]);
        const int bi = j0 / PER_BYTE;   // byte index inside the group
        w[bi / 4] = __builtin_amdgcn_cvt_pk_u8_f32(byte, bi % 4, w[bi / 4]);
      }
    } else {
      // degenerate group: every code 0, r^ = z
      const float rh = fmaf(0.0f, sf, zf);
#pragma unroll
      for (int i = 0; i < WORDS; ++i) w[i] = 0;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        r[j] = r[j] - rh;
        if constexpr (CHAIN) xh[j] = xh[j] + rh;
      }
    }
    uint8_t *cp = st + L.codes_off + uint64_t(s) * L.codes_stage + uint64_t(h) * L.codes_head +
                  uint64_t(tt) * L.codes_token + uint64_t(g) * (G * BITS / 8);
    if constexpr (WORDS == 2) {
      *(uint2 *)cp = make_uint2(w[0], w[1]);
    } else {
#pragma unroll
      for (int i = 0; i < WORDS; i += 4) *(uint4 *)(cp + 4 * i) = make_uint4(w[i], w[i + 1], w[i + 2], w[i + 3]);
    }
    uint32_t *mp = (uint32_t *)(st + L.meta_off + uint64_t(s) * L.meta_stage + uint64_t(h) * L.meta_head +
                                uint64_t(tt) * L.meta_token) + g;
    *mp = uint32_t(sb) | (uint32_t(zb) << 16);
  }
  if constexpr (CHAIN) {
    uint16_t *cp = a.chain + ((uint64_t(kv) * L.H + h) * uint64_t(a.n) + t) * D + g * G;
#pragma unroll
    for (int j = 0; j < G; ++j) cp[j] = f32_to_bf16_bits(xh[j]);
  }
}

__global__ void k_set_header(uint8_t *arena, DevLayout L, int layer0, int n_chunks, int n_tokens) {
  if (threadIdx.x != 0) return;
  const int z = blockIdx.x;
  StreamHeader *hdr = (StreamHeader *)(stream_ptr(arena, L, layer0 + (z >> 1), z & 1) + L.header_off);
  hdr->n_chunks = n_chunks;
  hdr->n_tokens = n_tokens;
}

// ---------------------------------------------------------------- launchers

template <int D, bool BF>
static void launch_init_t(const EncodeArgs &a, int streams, hipStream_t st) {
  QKV_LAUNCH((k_init<D, BF>), dim3(cdiv(a.L.C, 4), a.L.H, streams), dim3(256), 0, st, a);
}
template <int D, bool BF>
static void launch_assign_t(const EncodeArgs &a, int streams, hipStream_t st) {
  if (BF && a.L.C <= 512) {
    // MFMA screening; about four 256-token tiles per block so that the
    // codebook is staged in LDS once per 1024 tokens
    // about 512 blocks (two per compute unit of a 256-CU device, each
    // holding its codebook in LDS), each taking an equal run of tiles
    const int64_t total = cdiv(a.n, 256) * int64_t(a.L.H) * streams;
    const int per_block = int(std::max<int64_t>(1, cdiv(total, 512)));
    const int C16 = (a.L.C + 15) & ~15;
    const size_t lds = size_t(C16) * (D + 8) * 2 + size_t(C16) * 4;
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_assign_mfma<D>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    QKV_LAUNCH((k_assign_mfma<D>), dim3(unsigned(cdiv(total, per_block))), dim3(512), lds, st,
                       a, per_block, streams);
    return;
  }
  QKV_LAUNCH((k_assign<D, BF>), dim3(cdiv(a.n, 256), a.L.H, streams), dim3(256), 0, st, a);
}
template <int D, bool BF>
static void launch_update_t(const EncodeArgs &a, int streams, hipStream_t st) {
  if (a.L.C <= kSortMaxClusters) {
    const dim3 grid(cdiv(a.n, 256), a.L.H, streams);
    if (a.L.C <= 256)
      QKV_LAUNCH(k_tile_sort_count<256>, grid, dim3(256), 0, st, a);
    else if (a.L.C <= 1024)
      QKV_LAUNCH(k_tile_sort_count<1024>, grid, dim3(256), 0, st, a);
    else
      QKV_LAUNCH(k_tile_sort, grid, dim3(256), 0, st, a);
    QKV_LAUNCH((k_update_sorted<D, BF>), dim3(cdiv(a.L.C, 4), a.L.H, streams), dim3(256), 0, st, a);
    return;
  }
  QKV_LAUNCH((k_update<D, BF>), dim3(cdiv(a.L.C, 16), a.L.H, streams), dim3(1024), 0, st, a);
}

template <int D, bool BF>
static void launch_chan_flags_t(const EncodeArgs &a, int streams, hipStream_t st) {
  QKV_LAUNCH((k_chan_stats<D, BF>), dim3(kChanParts, a.L.H, streams), dim3(256), 0, st, a);
  QKV_LAUNCH((k_chan_flags<D>), dim3(a.L.H, streams), dim3(128), 0, st, a);
}

template <int D, int G, int BITS, bool BF>
static void launch_quantize_t(const EncodeArgs &a, int streams, hipStream_t st) {
  const int64_t items = int64_t(a.n) * (D / G);
  const dim3 grid(cdiv(items, 256), a.L.H, streams);
  if (a.L.mask_off)
    QKV_LAUNCH((k_quantize<D, G, BITS, BF, false, true>), grid, dim3(256), 0, st, a);
  else if (a.chain)
    QKV_LAUNCH((k_quantize<D, G, BITS, BF, true>), grid, dim3(256), 0, st, a);
  else
    QKV_LAUNCH((k_quantize<D, G, BITS, BF, false>), grid, dim3(256), 0, st, a);
}

void launch_header(const EncodeArgs &a, int streams, hipStream_t st) {
  QKV_LAUNCH(k_header, dim3(streams), dim3(64), 0, st, a);
}
void launch_init(const EncodeArgs &a, int streams, hipStream_t st) {
  QKV_DISPATCH_D_BF16(a.L.D, a.L.kv_bf16, launch_init_t, a, streams, st);
}
void launch_assign(const EncodeArgs &a, int streams, hipStream_t st) {
  QKV_DISPATCH_D_BF16(a.L.D, a.L.kv_bf16, launch_assign_t, a, streams, st);
}
void launch_update(const EncodeArgs &a, int streams, hipStream_t st) {
  QKV_DISPATCH_D_BF16(a.L.D, a.L.kv_bf16, launch_update_t, a, streams, st);
}
void launch_chan_flags(const EncodeArgs &a, int streams, hipStream_t st) {
  QKV_DISPATCH_D_BF16(a.L.D, a.L.kv_bf16, launch_chan_flags_t, a, streams, st);
}
void launch_quantize(const EncodeArgs &a, int streams, hipStream_t st) {
  QKV_DISPATCH_CODEC(a.L, launch_quantize_t, a, streams, st);
}
void launch_set_header(uint8_t *arena, const DevLayout &L, int layer0, int n_layers, int n_chunks,
                       int n_tokens, hipStream_t st) {
  QKV_LAUNCH(k_set_header, dim3(2 * n_layers), dim3(64), 0, st, arena, L, layer0, n_chunks, n_tokens);
}

}  // namespace qkv
