// HIP kernels of the qkv library for gfx950 (CDNA4, wave64).
//
//   k_header      chunk table of every stream touched by an encode call
//   k_init        initial codebook of a call: previous snapshot (centroid
//                 caching) or strided tokens
//   k_assign_mfma nearest centroid per token for bf16 caches with C <= 512:
//                 bf16 MFMA scores screen the candidates under a proven error
//                 bound; close calls are decided by the exact fp64 distance,
//                 channels summed in order
//   k_assign      the same decision with fp32 VALU screening (fp32 caches,
//                 C > 512)
//   k_tile_sort(_count), k_update_sorted
//                 k-means update: stable per-tile sort of the ids, then fp64
//                 member sums in token order -> mean -> one rounding
//   k_update      the same update through in-LDS member lists (C > 4096)
//   k_quantize    centroid (or prediction) subtraction + S PRQ stages + packing
//   k_reconstruct unpack + dequantize + add base, fp32 or bf16 out
//   k_attend3     split-KV attention reading the packed cache: tiles are
//                 rebuilt in bf16 in LDS and fed to bf16 MFMA (32x32x16)
//   k_attend_merge  LSE merge of the split partials
//   k_xl_project, k_xl_predict  cross-layer block-diagonal + low-rank
//                 prediction in fp64 with a fixed summation order
//
// Every elementwise codec operation is IEEE fp32 with no contraction (the
// library is compiled with -ffp-contract=off; fused multiply-adds are
// written as fmaf where the definition has one).
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <stdint.h>

#include <type_traits>

#include "device.h"
#include "launch.h"

namespace qkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;  // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// median of three unsigned values (v_med3_u32)
__device__ __forceinline__ uint32_t umed3(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// two floats -> packed nearest-even bf16 pair (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// Round an fp64 value once to bf16 (nearest even): scale the significand to
// 8 bits by a power of two, round to an integer, scale back; all exact in fp64.
__device__ __forceinline__ uint16_t f64_to_bf16_bits(double v) {
  if (v == 0.0) return signbit(v) ? 0x8000u : 0u;
  int e = ilogb(v);
  e = e < -126 ? -126 : e;
  const double r = ldexp(rint(ldexp(v, 7 - e)), e - 7);
  const float f = (float)r;  // exact, or overflow to infinity
  return (uint16_t)(__float_as_uint(f) >> 16);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
// The 2-bit codes in the low and high nibble of byte B of w (each nibble
// 00qq): the conversion reads a nibble as an E2M1 value, which is q/2 for
// these patterns, and scales by 2 (a power of two, applied exactly), giving
// float(q) for two codes in one v_cvt_scalef32_pk_f32_fp4.
template <int B>
__device__ __forceinline__ f32x2 nibble_codes(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 2.0f, B);
}
// The 4-bit codes in bytes 2*HI and 2*HI+1 of w (each byte 0000qqqq): an
// E4M3 byte below 16 has the value byte * 2^-9, so the conversion scaled by
// 2^9 gives float(q) for two codes in one v_cvt_scalef32_pk_f32_fp8.
template <bool HI>
__device__ __forceinline__ f32x2 byte_codes(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 512.0f, HI);
}

// The 16 2-bit codes of word w (channel c at bits 2c, 2c+1) as floats.
__device__ __forceinline__ void widen_codes2(uint32_t w, float *q) {
  const uint32_t m0 = w & 0x33333333u, m1 = (w >> 2) & 0x33333333u;
  const f32x2 e0 = nibble_codes<0>(m0), e1 = nibble_codes<1>(m0), e2 = nibble_codes<2>(m0), e3 = nibble_codes<3>(m0);
  const f32x2 o0 = nibble_codes<0>(m1), o1 = nibble_codes<1>(m1), o2 = nibble_codes<2>(m1), o3 = nibble_codes<3>(m1);
  q[0] = e0[0]; q[1] = o0[0]; q[2] = e0[1]; q[3] = o0[1];
  q[4] = e1[0]; q[5] = o1[0]; q[6] = e1[1]; q[7] = o1[1];
  q[8] = e2[0]; q[9] = o2[0]; q[10] = e2[1]; q[11] = o2[1];
  q[12] = e3[0]; q[13] = o3[0]; q[14] = e3[1]; q[15] = o3[1];
}
// The 8 4-bit codes of word w (channel c at bits 4c .. 4c+3) as floats.
__device__ __forceinline__ void widen_codes4(uint32_t w, float *q) {
  const uint32_t m0 = w & 0x0f0f0f0fu, m1 = (w >> 4) & 0x0f0f0f0fu;
  const f32x2 e0 = byte_codes<false>(m0), e1 = byte_codes<true>(m0);
  const f32x2 o0 = byte_codes<false>(m1), o1 = byte_codes<true>(m1);
  q[0] = e0[0]; q[1] = o0[0]; q[2] = e0[1]; q[3] = o0[1];
  q[4] = e1[0]; q[5] = o1[0]; q[6] = e1[1]; q[7] = o1[1];
}

template <bool BF16>
__device__ __forceinline__ float load_elem(const uint8_t *base, uint64_t idx) {
  if constexpr (BF16) return bf16_to_f32(((const uint16_t *)base)[idx]);
  else return ((const float *)base)[idx];
}

__device__ __forceinline__ uint8_t *stream_ptr(uint8_t *arena, const DevLayout &L, int layer, int kv) {
  return arena + (uint64_t(layer) * 2 + uint64_t(kv)) * L.stream_bytes;
}
__device__ __forceinline__ const uint8_t *stream_ptr(const uint8_t *arena, const DevLayout &L,
                                                     int layer, int kv) {
  return arena + (uint64_t(layer) * 2 + uint64_t(kv)) * L.stream_bytes;
}

__device__ __forceinline__ int load_id(const uint8_t *ids, int id_bytes, int64_t t) {
  return id_bytes == 1 ? int(ids[t]) : int(((const uint16_t *)ids)[t]);
}

// Chunk (snapshot slot) of token t: the last chunk whose first token is <= t.
__device__ __forceinline__ int chunk_of(const StreamHeader *hdr, int t) {
  int lo = 0, hi = hdr->n_chunks - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (hdr->start[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

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
    for (int k0 = 0; k0 < C16; k0 += 16) {
      bf16x8 ca[STEPS];
#pragma unroll
      for (int step = 0; step < STEPS; ++step)
        ca[step] = *(const bf16x8 *)(cbs + (k0 + c16) * KP + step * 32 + g4 * 8);
      const float4 ch = *(const float4 *)(cnh + k0 + g4 * 4);
      uint32_t kidx[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) kidx[r] = uint32_t(k0 + g4 * 4 + r);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        floatx4 acc = {ch.x + xnh[nt], ch.y + xnh[nt], ch.z + xnh[nt], ch.w + xnh[nt]};
#pragma unroll
        for (int step = 0; step < STEPS; ++step)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ca[step], xf[nt][step], acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // with m1 <= m2 <= m3: new third = med3(m2, m3, key), new second =
          // med3(m1, m2, key), new first = min(m1, key)
          const uint32_t key = (__float_as_uint(acc[r]) & ~0x1ffu) | kidx[r];
          const uint32_t n3 = umed3(m2[nt], m3[nt], key);
          const uint32_t n2 = umed3(m1[nt], m2[nt], key);
          m1[nt] = min(m1[nt], key);
          m2[nt] = n2;
          m3[nt] = n3;
        }
      }
    }
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
      const float inv = 1.0f / sf, invo = 1.0f / sfo;
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
          // sigma 0 (degenerate group): code 0, r^ = z
          const float qq = fminf(fmaxf(rintf((r[j] - zj) * ij), 0.0f), LEVELS);
          q[e] = sj != 0.0f ? qq : 0.0f;
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

// ----------------------------------------------------------------- decode

// Rebuild one group (G channels) of token tt of head h in fp32:
// xhat = fl32(...fl32(base + rhat_1)... + rhat_S).  xh holds the base on entry.
template <int D, int G, int BITS>
__device__ __forceinline__ void add_stages(const uint8_t *st, const DevLayout &L, int h, int64_t tt,
                                           int g, float *xh) {
  constexpr int WORDS = G * BITS / 32;
  for (int s = 0; s < L.S; ++s) {
    const uint8_t *cp = st + L.codes_off + uint64_t(s) * L.codes_stage + uint64_t(h) * L.codes_head +
                        uint64_t(tt) * L.codes_token + uint64_t(g) * (G * BITS / 8);
    uint32_t w[WORDS];
    if constexpr (WORDS == 2) {
      const uint2 v = *(const uint2 *)cp;
      w[0] = v.x; w[1] = v.y;
    } else {
#pragma unroll
      for (int i = 0; i < WORDS; i += 4) {
        const uint4 v = *(const uint4 *)(cp + 4 * i);
        w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z; w[i + 3] = v.w;
      }
    }
    const uint32_t m = *((const uint32_t *)(st + L.meta_off + uint64_t(s) * L.meta_stage +
                                            uint64_t(h) * L.meta_head + uint64_t(tt) * L.meta_token) + g);
    const float sf = f16_bits_to_f32(uint16_t(m & 0xffffu));
    const float zf = f16_bits_to_f32(uint16_t(m >> 16));
    float q[G];
#pragma unroll
    for (int i = 0; i < WORDS; ++i) {
      if constexpr (BITS == 2) widen_codes2(w[i], q + 16 * i);
      else widen_codes4(w[i], q + 8 * i);
    }
#pragma unroll
    for (int j = 0; j < G; ++j) xh[j] = xh[j] + fmaf(q[j], sf, zf);
  }
}

// add_stages with the outlier group: channel j of the group is dequantized
// with meta entry D/G when bit j of fm (the token's chunk's mask words for
// the group's channels) is set.
template <int D, int G, int BITS>
__device__ __forceinline__ void add_stages_outl(const uint8_t *st, const DevLayout &L, int h, int64_t tt,
                                                int g, float *xh, const uint32_t *fm) {
  constexpr int NG = D / G;
  constexpr int WORDS = G * BITS / 32;
  for (int s = 0; s < L.S; ++s) {
    const uint8_t *cp = st + L.codes_off + uint64_t(s) * L.codes_stage + uint64_t(h) * L.codes_head +
                        uint64_t(tt) * L.codes_token + uint64_t(g) * (G * BITS / 8);
    uint32_t w[WORDS];
    if constexpr (WORDS == 2) {
      const uint2 v = *(const uint2 *)cp;
      w[0] = v.x; w[1] = v.y;
    } else {
#pragma unroll
      for (int i = 0; i < WORDS; i += 4) {
        const uint4 v = *(const uint4 *)(cp + 4 * i);
        w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z; w[i + 3] = v.w;
      }
    }
    const uint32_t *mrow = (const uint32_t *)(st + L.meta_off + uint64_t(s) * L.meta_stage +
                                              uint64_t(h) * L.meta_head + uint64_t(tt) * L.meta_token);
    const uint32_t m = mrow[g], mo = mrow[NG];
    const float sf = f16_bits_to_f32(uint16_t(m & 0xffffu)), zf = f16_bits_to_f32(uint16_t(m >> 16));
    const float sfo = f16_bits_to_f32(uint16_t(mo & 0xffffu)), zfo = f16_bits_to_f32(uint16_t(mo >> 16));
    float q[G];
#pragma unroll
    for (int i = 0; i < WORDS; ++i) {
      if constexpr (BITS == 2) widen_codes2(w[i], q + 16 * i);
      else widen_codes4(w[i], q + 8 * i);
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const bool f = (fm[j >> 5] >> (j & 31)) & 1u;
      xh[j] = xh[j] + fmaf(q[j], f ? sfo : sf, f ? zfo : zf);
    }
  }
}

// Centroid base of token tt (snapshot of its chunk).
template <int D, int G, bool CB_BF16>
__device__ __forceinline__ void centroid_base(const uint8_t *st, const DevLayout &L, int h, int tt, int g,
                                              float *xh) {
  constexpr int EB = CB_BF16 ? 2 : 4;
  const StreamHeader *hdr = (const StreamHeader *)(st + L.header_off);
  const int slot = chunk_of(hdr, tt);
  const int id = load_id(st + L.ids_off + uint64_t(h) * L.ids_head, L.id_bytes, tt);
  const uint8_t *crow = st + L.cb_off + uint64_t(slot) * L.cb_chunk + uint64_t(h) * L.cb_head +
                        uint64_t(id) * D * EB + uint64_t(g) * G * EB;
#pragma unroll
  for (int j = 0; j < G; ++j) xh[j] = load_elem<CB_BF16>(crow, j);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Store the 16-byte pieces `v` of this thread's contiguous output run
// (thread i of the wave owns bytes [i*P*16, (i+1)*P*16) of the wave's
// region starting at `dst`) so that each store instruction writes one
// contiguous 1 KiB span: the pieces are exchanged through the wave's LDS
// slice `buf` (P*1 KiB).  Stores in which a lane's 16 B sit a whole run
// apart from its neighbour's reach about half the HBM write bandwidth.
template <int P>
__device__ __forceinline__ void store_wave_contiguous(uint4 *dst, uint4 *buf, const uint4 *v, int lane,
                                                      int valid_lanes) {
#pragma unroll
  for (int j = 0; j < P; ++j) buf[lane * P + j] = v[j];
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int piece = j * 64 + lane;              // piece index inside the wave's region
    if (piece < valid_lanes * P) {
      // streaming output: non-temporal store (the data is not read back soon)
      const uint4 v = buf[piece];
      __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, (u32x4 *)&dst[piece]);
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// One thread per (token, group).  blockIdx.x = item tile, y = head, z = layer.
// The output of a wave (64 consecutive (token, group) items) is one
// contiguous run of memory; it is stored through LDS in lane-contiguous
// pieces.
template <int D, int G, int BITS, bool CB_BF16, bool OUTL = false>
__global__ __launch_bounds__(256) void k_reconstruct(ReconArgs a, int64_t out_tokens, int32_t out_t_off) {
  constexpr int NG = D / G;
  constexpr int PB = G * 2 / 16;             // 16-byte pieces of a group in bf16
  constexpr int PF = G * 4 / 16;             // ... in fp32
  // per-wave exchange slices of 64 x PS pieces (PS = PF for fp32 output,
  // else PB), sized at launch; a wave's stores of the output and of the
  // chain both use its own slice
  extern __shared__ uint4 xbuf_dyn[];
  const int PS = (a.out && !a.out_bf16) ? PF : PB;
  const DevLayout &L = a.L;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = idx / NG, g = idx % NG;
  const int h = blockIdx.y, lrel = blockIdx.z;
  const bool valid = t < a.n;
  // items of this wave that exist (the run ends at the last token)
  const int wave_item0 = idx - lane;
  const int valid_lanes = int(min<int64_t>(64, int64_t(a.n) * NG - wave_item0));
  if (valid_lanes <= 0) return;             // whole wave past the end
  const uint8_t *st = stream_ptr(a.arena, L, a.layer0 + lrel, a.kv);
  const int tt = a.t0 + min(t, a.n - 1);
  float xh[G];
  if (a.pred) {
    const float *p = a.pred + (uint64_t(h) * a.n + min(t, a.n - 1)) * D + g * G;
#pragma unroll
    for (int j = 0; j < G; ++j) xh[j] = p[j];
  } else {
    centroid_base<D, G, CB_BF16>(st, L, h, tt, g, xh);
  }
  if constexpr (OUTL) {
    constexpr int FW = (G + 31) / 32;
    const int slot = chunk_of((const StreamHeader *)(st + L.header_off), tt);
    const uint32_t *mw = (const uint32_t *)(st + L.mask_off + uint64_t(slot) * L.mask_chunk +
                                            uint64_t(h) * L.mask_head);
    uint32_t fm[FW];
#pragma unroll
    for (int i = 0; i < FW; ++i) fm[i] = mw[g * FW + i];
    add_stages_outl<D, G, BITS>(st, L, h, tt, g, xh, fm);
  } else {
    add_stages<D, G, BITS>(st, L, h, tt, g, xh);
  }
  // first item of the wave: token t_w = wave_item0 / NG, group 0 (runs of a
  // wave start at a token boundary because 64 % NG == 0)
  const int t_w = wave_item0 / NG;
  if (a.out) {
    const uint64_t o = ((uint64_t(lrel) * L.H + h) * uint64_t(out_tokens) + out_t_off + t_w) * D;
    if (a.out_bf16) {
      uint4 v[PB];
#pragma unroll
      for (int j = 0; j < PB; ++j)
        v[j] = make_uint4(pack_bf16x2(xh[8 * j], xh[8 * j + 1]), pack_bf16x2(xh[8 * j + 2], xh[8 * j + 3]),
                          pack_bf16x2(xh[8 * j + 4], xh[8 * j + 5]), pack_bf16x2(xh[8 * j + 6], xh[8 * j + 7]));
      store_wave_contiguous<PB>((uint4 *)((uint16_t *)a.out + o), xbuf_dyn + wave * 64 * PS, v, lane, valid_lanes);
    } else {
      uint4 v[PF];
#pragma unroll
      for (int j = 0; j < PF; ++j)
        v[j] = make_uint4(__float_as_uint(xh[4 * j]), __float_as_uint(xh[4 * j + 1]),
                          __float_as_uint(xh[4 * j + 2]), __float_as_uint(xh[4 * j + 3]));
      store_wave_contiguous<PF>((uint4 *)((float *)a.out + o), xbuf_dyn + wave * 64 * PS, v, lane, valid_lanes);
    }
  }
  if (a.chain) {
    uint4 v[PB];
#pragma unroll
    for (int j = 0; j < PB; ++j)
      v[j] = make_uint4(pack_bf16x2(xh[8 * j], xh[8 * j + 1]), pack_bf16x2(xh[8 * j + 2], xh[8 * j + 3]),
                        pack_bf16x2(xh[8 * j + 4], xh[8 * j + 5]), pack_bf16x2(xh[8 * j + 6], xh[8 * j + 7]));
    store_wave_contiguous<PB>((uint4 *)(a.chain + (uint64_t(h) * a.n + t_w) * D), xbuf_dyn + wave * 64 * PS, v, lane,
                              valid_lanes);
  }
  (void)valid;
}

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
//    2-bit codes are widened four at a time from one masked code word
//    (byte-to-float conversions).  Keys past the end rebuild to zero from
//    zeroed registers.
//  * Loads are software-pipelined: ids of tile i+2 and the packed data
//    (codes, scale/zero, centroid rows) of tile i+1 are in flight while tile
//    i is rebuilt and multiplied; half of the waves multiply before they
//    rebuild and half after, so that the MFMA work of one wave of a SIMD
//    overlaps the VALU work of the other.  The chunk table is cached in LDS.
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

__device__ __forceinline__ int chunk_of_lds(const int32_t *starts, int n_chunks, int t) {
  int lo = 0, hi = n_chunks - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (starts[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

constexpr float AT3_TAU = 8.0f;

// w[i] for a run-time i < N (selects, no indexed register access)
template <int N>
__device__ __forceinline__ uint32_t pick_word(const uint32_t *w, int i) {
  if constexpr (N == 2) return i ? w[1] : w[0];
  else return (i & 2) ? ((i & 1) ? w[3] : w[2]) : ((i & 1) ? w[1] : w[0]);
}

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
  constexpr int KP = D + 8;                // bf16 elements per K row in LDS
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
  const bool has_item = it_rem < 64 * NI;
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
  const int lb = a.xcd_remap ? (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8 : blockIdx.x;
  const int64_t T = a.n_ktiles, U = a.units_per_block;
  const int64_t total = T * a.n_qblocks * L.H;
  int64_t u = int64_t(lb) * U;
  const int64_t u_end = min(total, u + U);
  __syncthreads();  // chunk table in LDS
  while (u < u_end) {
    const int64_t seg = u / T;
    const int h = int(seg / a.n_qblocks), qblk = int(seg % a.n_qblocks);
    const int t0 = int(u % T);
    const int t1 = int(min(T, t0 + (u_end - u)));
    const int slot = (t0 == 0 && t1 == T) ? -1 : int(lb - (seg * T) / U);
    u += t1 - t0;
    const uint8_t *idp = FRESH ? nullptr : st + L.ids_off + uint64_t(h) * L.ids_head;
    const int ks = t0 * AT_BK;
    const int ke = min(a.n_keys, t1 * AT_BK);
    const int n_tiles = ke > ks ? (ke - ks + AT_BK - 1) / AT_BK : 0;

    if constexpr (OUTL) {
      // written after the previous segment's last tile barrier, read after
      // the barrier before this segment's first rebuild
      constexpr int MW = D / 32;
      const int per = nch_s * MW;
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

    // id of the item's key in a tile (-1: no key)
    auto load_ids = [&](int tile) -> int {
      if (!has_item || tile >= n_tiles) return -1;
      const int t = ks + tile * AT_BK + it_key;
      if (t >= ke) return -1;
      if constexpr (FRESH) return 0;
      return L.id_bytes == 1 ? int(idp[t]) : int(((const uint16_t *)idp)[t]);
    };
    struct Regs {
      uint32_t codes[SMAX][KW];
      uint32_t meta[SMAX];
      uint4 cent[KC];
    } R;
    // per-item pointers of the segment (key t = ks + AT_BK * tile + it_key)
    const int t_first = ks + it_key;
    const uint8_t *code_p = FRESH ? nullptr : st + L.codes_off + uint64_t(h) * L.codes_head +
                                              uint64_t(t_first) * L.codes_token + it_ch * BITS / 8;
    const uint8_t *meta_p = FRESH ? nullptr : st + L.meta_off + uint64_t(h) * L.meta_head +
                                              uint64_t(t_first) * L.meta_token + 4 * it_g;
    const uint8_t *cb_p = FRESH ? nullptr : st + L.cb_off + uint64_t(h) * L.cb_head + uint64_t(it_ch) * EB;
    // fresh rows: channels it_ch .. it_ch+31 of key t_first of head h
    const uint16_t *fresh_p = FRESH ? (it_kv ? a.v_new : a.k_new) + (uint64_t(h) * a.n_keys + t_first) * D + it_ch
                                    : nullptr;
    const uint64_t tile_codes = uint64_t(AT_BK) * L.codes_token, tile_meta = uint64_t(AT_BK) * L.meta_token;
    // packed data of the item's key: centroid slice, codes, (sigma, z); all
    // zero when there is no key, which rebuilds to zero
    auto load_data = [&](int tile, int id) {
      if (id < 0) {
  #pragma unroll
        for (int i = 0; i < KC; ++i) R.cent[i] = make_uint4(0u, 0u, 0u, 0u);
  #pragma unroll
        for (int s2 = 0; s2 < SMAX; ++s2) {
          R.meta[s2] = 0u;
  #pragma unroll
          for (int w = 0; w < KW; ++w) R.codes[s2][w] = 0u;
        }
        return;
      }
      if constexpr (FRESH) {
        const uint16_t *row = fresh_p + uint64_t(tile) * AT_BK * D;
  #pragma unroll
        for (int i = 0; i < KC; ++i) R.cent[i] = *(const uint4 *)(row + 8 * i);
        return;
      }
      const int cslot = nch_s > 1 ? chunk_of_lds(starts_s, nch_s, ks + tile * AT_BK + it_key) : 0;
      const uint8_t *crow = cb_p + uint64_t(cslot) * L.cb_chunk + uint64_t(id) * (D * EB);
  #pragma unroll
      for (int i = 0; i < KC; ++i) R.cent[i] = *(const uint4 *)(crow + 16 * i);
      const uint8_t *cp = code_p + uint64_t(tile) * tile_codes;
      const uint8_t *mp = meta_p + uint64_t(tile) * tile_meta;
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
    // centroid channel e of the item for a run-time e (a select tree over the
    // item's registers)
    auto cent_pick = [&](int e) -> float {
      if constexpr (CB_BF16) {
        const int wi = e >> 1;
        const uint4 a = (wi & 8) ? ((wi & 4) ? R.cent[3] : R.cent[2]) : ((wi & 4) ? R.cent[1] : R.cent[0]);
        const uint32_t w = (wi & 2) ? ((wi & 1) ? a.w : a.z) : ((wi & 1) ? a.y : a.x);
        return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
      } else {
        const int vi = e >> 2;
        const uint4 a0 = (vi & 2) ? ((vi & 1) ? R.cent[3] : R.cent[2]) : ((vi & 1) ? R.cent[1] : R.cent[0]);
        const uint4 a1 = (vi & 2) ? ((vi & 1) ? R.cent[7] : R.cent[6]) : ((vi & 1) ? R.cent[5] : R.cent[4]);
        const uint4 a = (vi & 4) ? a1 : a0;
        return __uint_as_float((e & 2) ? ((e & 1) ? a.w : a.z) : ((e & 1) ? a.y : a.x));
      }
    };
    // Rebuild the item for the products: xh = fmaf(q_S, sigma_S, ... fmaf(q_1,
    // sigma_1, c + (z_1 + ... + z_S))), then nearest-even bf16.  This differs
    // from the stage-by-stage reconstruction (c + rhat_1) + rhat_2 ... by a few
    // fp32 ulps, which changes the bf16 operand only for values within those
    // ulps of a bf16 rounding boundary.
    auto dequant_store = [&](int buf, int tile) {
      if (!has_item) return;
      if constexpr (FRESH) {
        uint16_t *dst = it_kv ? &Vs[buf][it_key * VP + it_ch] : &Ks[buf][it_key * KP + it_ch];
  #pragma unroll
        for (int i = 0; i < KC; ++i) *(uint4 *)(dst + 8 * i) = R.cent[i];
        return;
      }
      float xh[IC];
      float zs = 0.0f;
  #pragma unroll
      for (int s2 = 0; s2 < SMAX; ++s2) zs += f16_bits_to_f32(uint16_t(R.meta[s2] >> 16));
  #pragma unroll
      for (int e = 0; e < IC; ++e) xh[e] = cent_f32(e) + zs;
  #pragma unroll
      for (int s2 = 0; s2 < SMAX; ++s2) {
        const float sf = f16_bits_to_f32(uint16_t(R.meta[s2] & 0xffffu));
  #pragma unroll
        for (int b16 = 0; b16 < IC / 16; ++b16) stage16(&R.codes[s2][b16 * (BITS / 2)], sf, &xh[16 * b16]);
      }
      uint16_t *dst = it_kv ? &Vs[buf][it_key * VP + it_ch] : &Ks[buf][it_key * KP + it_ch];
  #pragma unroll
      for (int j = 0; j < IC; j += 8)
        *(uint4 *)(dst + j) = make_uint4(pack_bf16x2(xh[j], xh[j + 1]), pack_bf16x2(xh[j + 2], xh[j + 3]),
                                         pack_bf16x2(xh[j + 4], xh[j + 5]), pack_bf16x2(xh[j + 6], xh[j + 7]));
      if constexpr (OUTL) {
        // channels of the item flagged in the mask of the key's chunk (mask
        // words in LDS): rebuilt again with the outlier group's (sigma, z) and
        // the item's registers, stored over the first result; read only
        // here, so that nothing of it is held during the rebuild
        uint32_t fm = 0u;
        uint32_t mo[SMAX];
        const int t = ks + tile * AT_BK + it_key;
        if (t < ke) {
          const int cslot = nch_s > 1 ? chunk_of_lds(starts_s, nch_s, t) : 0;
          fm = masks_s[it_kv][cslot * (D / 32) + (it_ch >> 5)];
          if (fm) {
            const uint8_t *mop = meta_p + uint64_t(tile) * tile_meta + 4 * (D / G - it_g);
  #pragma unroll
            for (int s2 = 0; s2 < SMAX; ++s2) mo[s2] = *(const uint32_t *)(mop + uint64_t(s2) * L.meta_stage);
          }
        }
        if (fm) {
          float so[SMAX];
          float zso = 0.0f;
  #pragma unroll
          for (int s2 = 0; s2 < SMAX; ++s2) {
            so[s2] = f16_bits_to_f32(uint16_t(mo[s2] & 0xffffu));
            zso += f16_bits_to_f32(uint16_t(mo[s2] >> 16));
          }
          while (fm) {
            const int e = __builtin_ctz(fm);
            fm &= fm - 1u;
            float v = cent_pick(e) + zso;
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

    auto compute_tile = [&](int tile) {
      const int buf = tile & 1;
      const int kt0 = ks + tile * AT_BK;
      // S^T for keys 32*kb + (8*(r/4) + 4*hh + r%4) of the tile, query c32
      floatx16 s0, s1;
  #pragma unroll
      for (int r = 0; r < 16; ++r) { s0[r] = 0.0f; s1[r] = 0.0f; }
      const uint16_t *kp = &Ks[buf][c32 * KP + 8 * hh];
  #pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 k0 = *(const bf16x8 *)(kp + 16 * s);
        const bf16x8 k1 = *(const bf16x8 *)(kp + 32 * KP + 16 * s);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[s], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[s], s1, 0, 0, 0);
      }
      if (kt0 + AT_BK > ke) {
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt0 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key >= ke) s0[r] = -INFINITY;
          if (key + 32 >= ke) s1[r] = -INFINITY;
        }
      }
      float tmax = -INFINITY;
  #pragma unroll
      for (int r = 0; r < 16; ++r)
        tmax = __builtin_elementwise_maximum(tmax, __builtin_elementwise_maximum(s0[r], s1[r]));
      tmax = pair_max(tmax);
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

    // Pipeline: at iteration i every wave rebuilds tile i+1 from data loaded
    // during iteration i-1 and issues the loads of tile i+2 (ids of tile i+3);
    // one barrier per tile.  Two waves share each SIMD; half of the waves
    // multiply tile i before rebuilding and half after, so one wave's MFMA work
    // overlaps its partner's VALU work.  The split flips between waves w and
    // w+4 and between waves 2k and 2k+1, whichever way waves sit on SIMDs.
    const bool mfma_first = ((wave >> 2) ^ wave) & 1;
    __syncthreads();  // previous segment's tiles no longer read
    int id_next;   // id of the item's key in tile+2
    load_data(0, load_ids(0));
    dequant_store(0, 0);
    load_data(1, load_ids(1));
    id_next = load_ids(2);
    __syncthreads();

    for (int tile = 0; tile < n_tiles; ++tile) {
      const int buf = tile & 1;
      if (mfma_first) compute_tile(tile);
      if (tile + 1 < n_tiles) dequant_store(buf ^ 1, tile + 1);   // data of tile+1 already in R
      load_data(tile + 2, id_next);
      id_next = load_ids(tile + 3);
      if (!mfma_first) compute_tile(tile);
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
  const int64_t first = (int64_t(h) * a.n_qblocks + q / AT_BQ) * T;
  const int nseg = int((first + T - 1) / U - first / U) + 1;
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

// ------------------------------------------------------------ cross layer

// Cross-layer prediction (r <= 64), in fp64 with a fixed summation order per
// output: the projection sums over m = 0 .. H*D-1, the prediction over j, then
// over k.  Every product is of two bf16 values, hence exact in fp64, so
// fma(p, q, acc) equals acc + p*q rounded once: each output is exactly that
// sequence of fp64 additions, however the work is tiled.

// proj[t][k] = bf16(sum over m = 0 .. H*D-1 of y[t][m] V[m][k]).  Block = 256
// threads = (token groups of 4) x (output groups of 8: 4 groups for r <= 32,
// else 8), i.e. 256 or 128 tokens; the m axis is staged through LDS 32 at a
// time (transposed, fp32; outputs past r read zero columns).
constexpr int XL_MC = 32;
__host__ __device__ constexpr int xl_project_groups(int r) { return r <= 32 ? 4 : 8; }
__global__ __launch_bounds__(256) void k_xl_project(XlArgs a, int kv0) {
  __shared__ float ys[XL_MC][256 + 4];    // [m][token]
  __shared__ float vs[XL_MC][64 + 4];     // [m][k]
  const int KG = xl_project_groups(a.r), KP = 8 * KG, TG = 256 / KG, TT = 4 * TG;
  const int tid = threadIdx.x, kv = kv0 + blockIdx.y;
  const int kg = tid % KG, tg = tid / KG;
  const int t0 = blockIdx.x * TT;
  const uint64_t HD = uint64_t(a.H) * a.D;
  const uint16_t *Vw = a.weights + uint64_t(kv) * a.kv_weight_stride + HD * a.D + HD * a.r;
  const uint16_t *y = a.chain + uint64_t(kv) * HD * a.n;
  double acc[4][8];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[u][c] = 0.0;
  for (uint64_t m0 = 0; m0 < HD; m0 += XL_MC) {
    const int hh = int(m0 / a.D), j0 = int(m0 % a.D);   // a chunk lies inside one head (D % 32 == 0)
    __syncthreads();                                    // previous chunk consumed
    for (int e = tid; e < TT * XL_MC; e += 256) {
      const int tt = e / XL_MC, jj = e % XL_MC, t = min(t0 + tt, a.n - 1);
      ys[jj][tt] = bf16_to_f32(y[(uint64_t(hh) * a.n + t) * a.D + j0 + jj]);
    }
    for (int e = tid; e < XL_MC * KP; e += 256) {
      const int jj = e / KP, kk = e % KP;
      vs[jj][kk] = kk < a.r ? bf16_to_f32(Vw[(m0 + jj) * a.r + kk]) : 0.0f;
    }
    __syncthreads();
#pragma unroll 4
    for (int jj = 0; jj < XL_MC; ++jj) {
      const float4 yv = *(const float4 *)&ys[jj][4 * tg];
      const float4 v0 = *(const float4 *)&vs[jj][8 * kg], v1 = *(const float4 *)&vs[jj][8 * kg + 4];
      const double yd[4] = {double(yv.x), double(yv.y), double(yv.z), double(yv.w)};
      const double vd[8] = {double(v0.x), double(v0.y), double(v0.z), double(v0.w),
                            double(v1.x), double(v1.y), double(v1.z), double(v1.w)};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[u][c] = fma(yd[u], vd[c], acc[u][c]);
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int t = t0 + 4 * tg + u;
    if (t >= a.n) continue;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int kk = 8 * kg + c;
      if (kk < a.r) a.proj[(uint64_t(kv) * a.n + t) * a.r + kk] = bf16_to_f32(f64_to_bf16_bits(acc[u][c]));
    }
  }
}

// pred[h][t][i] = sum_j B_h[i][j] y[t][j] (order j), then + sum_k U[h*D+i][k]
// w[t][k] (order k), fp64, rounded once to fp32.  Block = 256 threads =
// (token groups of 4) x (output groups of 8) over token tiles of 4*256/(D/8)
// tokens; B_h and U_h are staged once per block (transposed, as bf16: two
// blocks fit a CU) and the block walks every gridDim.x-th token tile.
__global__ __launch_bounds__(256) void k_xl_predict(XlArgs a, int kv0) {
  extern __shared__ uint16_t xs16[];
  const int D = a.D, RP = (a.r + 7) & ~7;
  const int IG = D / 8, TG = 256 / IG, TT = 4 * TG;
  uint16_t *bsT = xs16;                       // [D j][D i] bf16
  uint16_t *usT = bsT + D * D;                // [RP k][D i]
  uint16_t *ysT = usT + RP * D;               // [D j][TT]
  uint16_t *wsT = ysT + D * TT;               // [RP k][TT]
  const int tid = threadIdx.x, h = blockIdx.y, kv = kv0 + blockIdx.z;
  const int ig = tid % IG, tg = tid / IG;
  const uint64_t HD = uint64_t(a.H) * D;
  const uint16_t *W = a.weights + uint64_t(kv) * a.kv_weight_stride;
  const uint16_t *B = a.b_weights ? a.b_weights + (uint64_t(kv) * a.H + h) * D * D : W + uint64_t(h) * D * D;
  const uint16_t *U = W + HD * D + uint64_t(h) * D * a.r;
  const uint16_t *y = a.chain + uint64_t(kv) * HD * a.n + uint64_t(h) * a.n * D;
  const float *w = a.proj + uint64_t(kv) * a.n * a.r;
  for (int e = tid; e < D * D; e += 256) {
    const int i = e / D, j = e % D;
    bsT[j * D + i] = B[e];
  }
  for (int e = tid; e < D * RP; e += 256) {
    const int i = e / RP, kk = e % RP;
    usT[kk * D + i] = kk < a.r ? U[uint64_t(i) * a.r + kk] : uint16_t(0);
  }
  const int n_tiles = (a.n + TT - 1) / TT;
  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int t0 = tile * TT;
    __syncthreads();                          // weights staged / previous tile consumed
    for (int e = tid; e < TT * D; e += 256) {
      const int tt = e / D, j = e % D, t = min(t0 + tt, a.n - 1);
      ysT[j * TT + tt] = y[uint64_t(t) * D + j];
    }
    for (int e = tid; e < TT * RP; e += 256) {
      const int tt = e / RP, kk = e % RP, t = min(t0 + tt, a.n - 1);
      // w holds bf16 values (rounded in the projection): exact in bf16
      wsT[kk * TT + tt] = kk < a.r ? f32_to_bf16_bits(w[uint64_t(t) * a.r + kk]) : uint16_t(0);
    }
    __syncthreads();
    double acc[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[u][c] = 0.0;
    auto step = [&](const uint16_t *ycol, const uint16_t *bcol) {
      const uint2 yv = *(const uint2 *)(ycol + 4 * tg);
      const uint4 bv = *(const uint4 *)(bcol + 8 * ig);
      const double yd[4] = {double(__uint_as_float(yv.x << 16)), double(__uint_as_float(yv.x & 0xffff0000u)),
                            double(__uint_as_float(yv.y << 16)), double(__uint_as_float(yv.y & 0xffff0000u))};
      const double bd[8] = {double(__uint_as_float(bv.x << 16)), double(__uint_as_float(bv.x & 0xffff0000u)),
                            double(__uint_as_float(bv.y << 16)), double(__uint_as_float(bv.y & 0xffff0000u)),
                            double(__uint_as_float(bv.z << 16)), double(__uint_as_float(bv.z & 0xffff0000u)),
                            double(__uint_as_float(bv.w << 16)), double(__uint_as_float(bv.w & 0xffff0000u))};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[u][c] = fma(bd[c], yd[u], acc[u][c]);
    };
    if (!a.lowrank_only) {
#pragma unroll 4
      for (int j = 0; j < D; ++j) step(ysT + j * TT, bsT + j * D);
    }
    for (int kk = 0; kk < a.r; ++kk) step(wsT + kk * TT, usT + kk * D);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + 4 * tg + u;
      if (t >= a.n) continue;
      float *pp = a.pred + (uint64_t(kv) * HD * a.n) + (uint64_t(h) * a.n + t) * D + 8 * ig;
      *(float4 *)pp = make_float4(float(acc[u][0]), float(acc[u][1]), float(acc[u][2]), float(acc[u][3]));
      *(float4 *)(pp + 4) = make_float4(float(acc[u][4]), float(acc[u][5]), float(acc[u][6]), float(acc[u][7]));
    }
  }
}

// Adapted predictor, step 1: per (token range p, head, kv, matrix) the fp64
// sums over the range's tokens of y y^T (matrix 0) and y (x - U w)^T
// (matrix 1), in token order.  Block = 16 x 16 threads, thread (ti, tj)
// owns entries [8 ti .. 8 ti + 7][8 tj .. 8 tj + 7]; tokens are staged
// through LDS 32 at a time (y as fp32, the second factor as fp64).
constexpr int RF_TC = 32;
__global__ __launch_bounds__(256) void k_xl_gram(RefitArgs a) {
  __shared__ float ys[RF_TC][128];
  __shared__ double zs[RF_TC][128];
  const int D = a.D, part = blockIdx.x, h = blockIdx.y, kv = blockIdx.z >> 1, mat = blockIdx.z & 1;
  const int tid = threadIdx.x, ti = tid / 16, tj = tid % 16;
  const int64_t t_beg = int64_t(a.n) * part / kRefitParts, t_end = int64_t(a.n) * (part + 1) / kRefitParts;
  const uint16_t *y = a.chain + (uint64_t(kv) * a.H + h) * uint64_t(a.n) * D;
  const uint16_t *x = (const uint16_t *)(kv ? a.v_in : a.k_in) + uint64_t(h) * a.n * D;
  const float *lr = a.low_rank + (uint64_t(kv) * a.H + h) * uint64_t(a.n) * D;
  const bool active = 8 * ti < D && 8 * tj < D;
  double acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;
  for (int64_t c0 = t_beg; c0 < t_end; c0 += RF_TC) {
    const int nc = int(min<int64_t>(RF_TC, t_end - c0));
    // eight channels per thread and step, every load of the chunk issued
    // before any is used (past the range: zeros)
    constexpr int NU = RF_TC * 128 / 8 / 256;
    uint4 yv[NU], xv[NU];
    float4 lv[NU][2];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int e8 = tid + 256 * u, tt = e8 / (D / 8), j = 8 * (e8 % (D / 8));
      yv[u] = xv[u] = make_uint4(0, 0, 0, 0);
      lv[u][0] = lv[u][1] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (tt < nc && e8 < RF_TC * D / 8) {
        const uint64_t off = uint64_t(c0 + tt) * D + j;
        yv[u] = *(const uint4 *)(y + off);
        if (mat) {
          xv[u] = *(const uint4 *)(x + off);
          lv[u][0] = *(const float4 *)(lr + off);
          lv[u][1] = *(const float4 *)(lr + off + 4);
        }
      }
    }
    __syncthreads();                          // previous chunk consumed
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int e8 = tid + 256 * u, tt = e8 / (D / 8), j = 8 * (e8 % (D / 8));
      if (e8 >= RF_TC * D / 8) continue;
      const uint32_t yw[4] = {yv[u].x, yv[u].y, yv[u].z, yv[u].w}, xw[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
      const float lf[8] = {lv[u][0].x, lv[u][0].y, lv[u][0].z, lv[u][0].w,
                           lv[u][1].x, lv[u][1].y, lv[u][1].z, lv[u][1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float yf = __uint_as_float((e & 1) ? (yw[e >> 1] & 0xffff0000u) : (yw[e >> 1] << 16));
        const float xf = __uint_as_float((e & 1) ? (xw[e >> 1] & 0xffff0000u) : (xw[e >> 1] << 16));
        ys[tt][j + e] = yf;
        zs[tt][j + e] = mat == 0 ? double(yf) : double(xf) - double(lf[e]);
      }
    }
    __syncthreads();
    if (active) {
      for (int tt = 0; tt < nc; ++tt) {
        double yi[8], zj[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) yi[i] = double(ys[tt][8 * ti + i]);
#pragma unroll
        for (int j = 0; j < 8; ++j) zj[j] = zs[tt][8 * tj + j];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = fma(yi[i], zj[j], acc[i][j]);
      }
    }
  }
  if (active) {
    double *g = a.gram + (((uint64_t(part) * 2 + kv) * 2 + mat) * a.H + h) * uint64_t(D) * D;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) g[uint64_t(8 * ti + i) * D + 8 * tj + j] = acc[i][j];
  }
}

// Adapted predictor, step 2: one block per (head, kv).  A = sum of the parts
// of y y^T (in part order) + lam I, lam = 2^-20 trace(A) / D; Cholesky
// factor L (left-looking, in LDS); then, 16 right-hand sides at a time, the
// columns c of R = sum of the parts of y (x - U w)^T are solved through
// L z' = r and L^T z = z', and row c of the block is z, rounded to bf16.
__global__ __launch_bounds__(256) void k_xl_solve(RefitArgs a) {
  extern __shared__ double lds64[];
  const int D = a.D, h = blockIdx.x, kv = blockIdx.y, tid = threadIdx.x;
  double *Lm = lds64;                 // [D][D]
  double *Z = lds64 + D * D;          // [16][D]
  __shared__ double lam_s;
  const uint64_t DD = uint64_t(D) * D;
  auto part_ptr = [&](int p, int mat) {
    return a.gram + (((uint64_t(p) * 2 + kv) * 2 + mat) * a.H + h) * DD;
  };
  for (int e = tid; e < D * D; e += 256) {
    double v = 0.0;
    for (int p = 0; p < kRefitParts; ++p) v += part_ptr(p, 0)[e];
    Lm[e] = v;
  }
  __syncthreads();
  if (tid == 0) {
    double tr = 0.0;
    for (int i = 0; i < D; ++i) tr += Lm[i * D + i];
    lam_s = 0x1p-20 * tr / D;
  }
  __syncthreads();
  if (tid < D) Lm[tid * D + tid] += lam_s;
  __syncthreads();
  // left-looking Cholesky: column j from the columns before it
  for (int j = 0; j < D; ++j) {
    if (tid == 0) {
      double s = Lm[j * D + j];
      for (int k = 0; k < j; ++k) s -= Lm[j * D + k] * Lm[j * D + k];
      Lm[j * D + j] = sqrt(s > 0.0 ? s : 0x1p-1000);
    }
    __syncthreads();
    const int i = j + 1 + tid;
    if (i < D) {
      double s = Lm[i * D + j];
      for (int k = 0; k < j; ++k) s -= Lm[i * D + k] * Lm[j * D + k];
      Lm[i * D + j] = s / Lm[j * D + j];
    }
    __syncthreads();
  }
  // 16 right-hand sides at a time: thread (cc, q) = column c0 + cc, terms k = q mod 16
  const int cc = tid / 16, q = tid % 16;
  for (int c0 = 0; c0 < D; c0 += 16) {
    for (int e = tid; e < 16 * D; e += 256) {
      const int col = e / D, row = e % D;
      double v = 0.0;
      for (int p = 0; p < kRefitParts; ++p) v += part_ptr(p, 1)[uint64_t(row) * D + c0 + col];
      Z[col * D + row] = v;
    }
    __syncthreads();
    for (int i = 0; i < D; ++i) {              // forward: L z' = r
      double s = 0.0;
      for (int k = q; k < i; k += 16) s += Lm[i * D + k] * Z[cc * D + k];
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) s += __shfl_xor(s, off, 16);
      if (q == 0) Z[cc * D + i] = (Z[cc * D + i] - s) / Lm[i * D + i];
      __syncthreads();
    }
    for (int i = D - 1; i >= 0; --i) {         // backward: L^T z = z'
      double s = 0.0;
      for (int k = i + 1 + q; k < D; k += 16) s += Lm[k * D + i] * Z[cc * D + k];
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) s += __shfl_xor(s, off, 16);
      if (q == 0) Z[cc * D + i] = (Z[cc * D + i] - s) / Lm[i * D + i];
      __syncthreads();
    }
    uint16_t *bo = a.b_out + (uint64_t(kv) * a.H + h) * DD;
    for (int e = tid; e < 16 * D; e += 256) {
      const int col = e / D, j = e % D;
      bo[uint64_t(c0 + col) * D + j] = f64_to_bf16_bits(Z[col * D + j]);
    }
    __syncthreads();
  }
}

// chunk table after a rewind: blockIdx.x = stream of the range
__global__ void k_set_header(uint8_t *arena, DevLayout L, int layer0, int n_chunks, int n_tokens) {
  if (threadIdx.x != 0) return;
  const int z = blockIdx.x;
  StreamHeader *hdr = (StreamHeader *)(stream_ptr(arena, L, layer0 + (z >> 1), z & 1) + L.header_off);
  hdr->n_chunks = n_chunks;
  hdr->n_tokens = n_tokens;
}

// ---------------------------------------------------------------- launchers

static inline unsigned cdiv(int64_t a, int64_t b) { return unsigned((a + b - 1) / b); }

#define QKV_DISPATCH_D_BF16(D_, BF_, FN, ...)                           \
  do {                                                                  \
    if (D_ == 64 && BF_) FN<64, true>(__VA_ARGS__);                     \
    else if (D_ == 64) FN<64, false>(__VA_ARGS__);                      \
    else if (BF_) FN<128, true>(__VA_ARGS__);                           \
    else FN<128, false>(__VA_ARGS__);                                   \
  } while (0)

template <int D, bool BF>
static void launch_init_t(const EncodeArgs &a, int streams, hipStream_t st) {
  hipLaunchKernelGGL((k_init<D, BF>), dim3(cdiv(a.L.C, 4), a.L.H, streams), dim3(256), 0, st, a);
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
    hipLaunchKernelGGL((k_assign_mfma<D>), dim3(unsigned(cdiv(total, per_block))), dim3(512), lds, st,
                       a, per_block, streams);
    return;
  }
  hipLaunchKernelGGL((k_assign<D, BF>), dim3(cdiv(a.n, 256), a.L.H, streams), dim3(256), 0, st, a);
}
template <int D, bool BF>
static void launch_update_t(const EncodeArgs &a, int streams, hipStream_t st) {
  if (a.L.C <= kSortMaxClusters) {
    const dim3 grid(cdiv(a.n, 256), a.L.H, streams);
    if (a.L.C <= 256)
      hipLaunchKernelGGL(k_tile_sort_count<256>, grid, dim3(256), 0, st, a);
    else if (a.L.C <= 1024)
      hipLaunchKernelGGL(k_tile_sort_count<1024>, grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(k_tile_sort, grid, dim3(256), 0, st, a);
    hipLaunchKernelGGL((k_update_sorted<D, BF>), dim3(cdiv(a.L.C, 4), a.L.H, streams), dim3(256), 0, st, a);
    return;
  }
  hipLaunchKernelGGL((k_update<D, BF>), dim3(cdiv(a.L.C, 16), a.L.H, streams), dim3(1024), 0, st, a);
}

template <int D, bool BF>
static void launch_chan_flags_t(const EncodeArgs &a, int streams, hipStream_t st) {
  hipLaunchKernelGGL((k_chan_stats<D, BF>), dim3(kChanParts, a.L.H, streams), dim3(256), 0, st, a);
  hipLaunchKernelGGL((k_chan_flags<D>), dim3(a.L.H, streams), dim3(128), 0, st, a);
}

template <int D, int G, int BITS, bool BF>
static void launch_quantize_t(const EncodeArgs &a, int streams, hipStream_t st) {
  const int64_t items = int64_t(a.n) * (D / G);
  const dim3 grid(cdiv(items, 256), a.L.H, streams);
  if (a.L.mask_off)
    hipLaunchKernelGGL((k_quantize<D, G, BITS, BF, false, true>), grid, dim3(256), 0, st, a);
  else if (a.chain)
    hipLaunchKernelGGL((k_quantize<D, G, BITS, BF, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_quantize<D, G, BITS, BF, false>), grid, dim3(256), 0, st, a);
}

template <int D, int G, int BITS, bool BF>
static void launch_recon_t(const ReconArgs &a, int n_layers, int64_t out_tokens, int out_t_off,
                           hipStream_t st) {
  const int64_t items = int64_t(a.n) * (D / G);
  // LDS: 4 waves x 64 lanes x one group of the output type
  const size_t lds = size_t(4) * 64 * G * (a.out && !a.out_bf16 ? 4 : 2);
  if (a.L.mask_off)
    hipLaunchKernelGGL((k_reconstruct<D, G, BITS, BF, true>), dim3(cdiv(items, 256), a.L.H, n_layers), dim3(256),
                       lds, st, a, out_tokens, out_t_off);
  else
    hipLaunchKernelGGL((k_reconstruct<D, G, BITS, BF>), dim3(cdiv(items, 256), a.L.H, n_layers), dim3(256),
                       lds, st, a, out_tokens, out_t_off);
}

template <int D, int G, int BITS, bool BF>
static void launch_attend_t(const AttnArgs &a, hipStream_t st) {
  const int64_t total = int64_t(a.n_ktiles) * a.n_qblocks * a.L.H;
  const dim3 grid(unsigned(cdiv(total, a.units_per_block)));
  if (a.L.mask_off) {
    switch (a.L.S) {
      case 1: hipLaunchKernelGGL((k_attend3<D, G, BITS, BF, 1, false, true>), grid, dim3(512), 0, st, a); break;
      case 2: hipLaunchKernelGGL((k_attend3<D, G, BITS, BF, 2, false, true>), grid, dim3(512), 0, st, a); break;
      case 3: hipLaunchKernelGGL((k_attend3<D, G, BITS, BF, 3, false, true>), grid, dim3(512), 0, st, a); break;
      default: hipLaunchKernelGGL((k_attend3<D, G, BITS, BF, 4, false, true>), grid, dim3(512), 0, st, a); break;
    }
    return;
  }
  switch (a.L.S) {
    case 1: hipLaunchKernelGGL((k_attend3<D, G, BITS, BF, 1>), grid, dim3(512), 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_attend3<D, G, BITS, BF, 2>), grid, dim3(512), 0, st, a); break;
    case 3: hipLaunchKernelGGL((k_attend3<D, G, BITS, BF, 3>), grid, dim3(512), 0, st, a); break;
    default: hipLaunchKernelGGL((k_attend3<D, G, BITS, BF, 4>), grid, dim3(512), 0, st, a); break;
  }
}

// (D, G, BITS, BF) dispatch for the codec-shaped kernels
#define QKV_DISPATCH_CODEC(L_, FN, ...)                                                   \
  do {                                                                                    \
    const int D_ = (L_).D, G_ = (L_).G, B_ = (L_).bits;                                   \
    const bool BF_ = (L_).kv_bf16 != 0;                                                   \
    if (D_ == 64 && G_ == 32 && B_ == 2) { if (BF_) FN<64, 32, 2, true>(__VA_ARGS__); else FN<64, 32, 2, false>(__VA_ARGS__); } \
    else if (D_ == 64 && G_ == 32) { if (BF_) FN<64, 32, 4, true>(__VA_ARGS__); else FN<64, 32, 4, false>(__VA_ARGS__); }      \
    else if (D_ == 64 && B_ == 2) { if (BF_) FN<64, 64, 2, true>(__VA_ARGS__); else FN<64, 64, 2, false>(__VA_ARGS__); }       \
    else if (D_ == 64) { if (BF_) FN<64, 64, 4, true>(__VA_ARGS__); else FN<64, 64, 4, false>(__VA_ARGS__); }                  \
    else if (G_ == 32 && B_ == 2) { if (BF_) FN<128, 32, 2, true>(__VA_ARGS__); else FN<128, 32, 2, false>(__VA_ARGS__); }     \
    else if (G_ == 32) { if (BF_) FN<128, 32, 4, true>(__VA_ARGS__); else FN<128, 32, 4, false>(__VA_ARGS__); }                \
    else if (B_ == 2) { if (BF_) FN<128, 64, 2, true>(__VA_ARGS__); else FN<128, 64, 2, false>(__VA_ARGS__); }                 \
    else { if (BF_) FN<128, 64, 4, true>(__VA_ARGS__); else FN<128, 64, 4, false>(__VA_ARGS__); }                              \
  } while (0)

void launch_header(const EncodeArgs &a, int streams, hipStream_t st) {
  hipLaunchKernelGGL(k_header, dim3(streams), dim3(64), 0, st, a);
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
void launch_reconstruct(const ReconArgs &a, int n_layers, int64_t out_tokens, int out_t_off, hipStream_t st) {
  QKV_DISPATCH_CODEC(a.L, launch_recon_t, a, n_layers, out_tokens, out_t_off, st);
}
void launch_attend_fresh(const AttnArgs &a, hipStream_t st) {
  const int64_t total = int64_t(a.n_ktiles) * a.n_qblocks * a.L.H;
  const dim3 grid(unsigned(cdiv(total, a.units_per_block)));
  if (a.L.D == 64)
    hipLaunchKernelGGL((k_attend3<64, 32, 2, true, 1, true>), grid, dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((k_attend3<128, 32, 2, true, 1, true>), grid, dim3(512), 0, st, a);
  if (a.max_segments > 1)
    hipLaunchKernelGGL(k_attend_merge, dim3(cdiv(int64_t(a.n_q) * (a.L.D / 4), 256), a.L.H), dim3(256), 0, st, a);
}
void launch_attend_merge2(const MergeArgs &m, hipStream_t st) {
  hipLaunchKernelGGL(k_attend_merge2, dim3(cdiv(int64_t(m.n_q) * (m.D / 4), 256), m.H), dim3(256), 0, st, m);
}
void launch_attend(const AttnArgs &a, hipStream_t st) {
  QKV_DISPATCH_CODEC(a.L, launch_attend_t, a, st);
  if (a.max_segments > 1)
    hipLaunchKernelGGL(k_attend_merge, dim3(cdiv(int64_t(a.n_q) * (a.L.D / 4), 256), a.L.H), dim3(256), 0, st, a);
}
void launch_xl_refit(const RefitArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(k_xl_gram, dim3(kRefitParts, a.H, 4), dim3(256), 0, st, a);
  const size_t lds = (size_t(a.D) * a.D + 16 * size_t(a.D)) * sizeof(double);
  (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_xl_solve),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  hipLaunchKernelGGL(k_xl_solve, dim3(a.H, 2), dim3(256), lds, st, a);
}
void launch_xl_predict(const XlArgs &a, int kv0, int n_kv, hipStream_t st) {
  // tiled kernels (fp32 LDS staging of the bf16 operands)
  const int TT = 4 * (256 / xl_project_groups(a.r));
  if (!a.skip_project) hipLaunchKernelGGL(k_xl_project, dim3(cdiv(a.n, TT), n_kv), dim3(256), 0, st, a, kv0);
  const int RP = (a.r + 7) & ~7;
  const int IG = a.D / 8, TTp = 4 * (256 / IG);
  const size_t lds = size_t(a.D * a.D + RP * a.D + a.D * TTp + RP * TTp) * 2;
  (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_xl_predict),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  // two blocks per CU fit (the staged weights); about 512 blocks in all,
  // each walking every gx-th token tile of its (head, kv)
  const int64_t n_tiles = cdiv(a.n, TTp);
  const int64_t hk = int64_t(a.H) * n_kv;
  const unsigned gx = unsigned(std::max<int64_t>(1, std::min<int64_t>(n_tiles, (512 + hk - 1) / hk)));
  hipLaunchKernelGGL(k_xl_predict, dim3(gx, a.H, n_kv), dim3(256), lds, st, a, kv0);
}
void launch_set_header(uint8_t *arena, const DevLayout &L, int layer0, int n_layers, int n_chunks,
                       int n_tokens, hipStream_t st) {
  hipLaunchKernelGGL(k_set_header, dim3(2 * n_layers), dim3(64), 0, st, arena, L, layer0, n_chunks, n_tokens);
}

}  // namespace qkv
