// Device helpers shared by the qkv kernel sources (gfx950, CDNA4, wave64):
// bf16/fp16 conversions, code widening, stream addressing, the chunk table
// lookup, and the template dispatch used by the launchers.
//
// Every elementwise codec operation is IEEE fp32 with no contraction (the
// library is compiled with -ffp-contract=off; fused multiply-adds are
// written as fmaf where the definition has one).
#pragma once
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
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
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

// chunk_of over a copy of the chunk table's first tokens in LDS
__device__ __forceinline__ int chunk_of_lds(const int32_t *starts, int n_chunks, int t) {
  int lo = 0, hi = n_chunks - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (starts[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------- launch helpers

static inline unsigned cdiv(int64_t a, int64_t b) { return unsigned((a + b - 1) / b); }

#define QKV_DISPATCH_D_BF16(D_, BF_, FN, ...)                           \
  do {                                                                  \
    if (D_ == 64 && BF_) FN<64, true>(__VA_ARGS__);                     \
    else if (D_ == 64) FN<64, false>(__VA_ARGS__);                      \
    else if (BF_) FN<128, true>(__VA_ARGS__);                           \
    else FN<128, false>(__VA_ARGS__);                                   \
  } while (0)

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

}  // namespace qkv
