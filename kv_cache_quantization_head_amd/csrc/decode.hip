// Reconstruction kernel of the qkv library: unpack, dequantize, add the base.
#include "common.h"

namespace qkv {

// ----------------------------------------------------------------- decode

// Codes and (sigma, z) of the stages of one group (G channels) of token tt
// of head h, all loaded before any is used so that their loads are in
// flight together (stages past L.S are left unset).
constexpr int kStagesMax = 4;
template <int G, int BITS>
struct GroupStages {
  static constexpr int WORDS = G * BITS / 32;
  uint32_t w[kStagesMax][WORDS];
  uint32_t m[kStagesMax];
};
template <int D, int G, int BITS>
__device__ __forceinline__ void load_stages(const uint8_t *st, const DevLayout &L, int h, int64_t tt, int g,
                                            GroupStages<G, BITS> &gs) {
  constexpr int WORDS = G * BITS / 32;
#pragma unroll
  for (int s = 0; s < kStagesMax; ++s) {
    if (s >= L.S) break;
    const uint8_t *cp = st + L.codes_off + uint64_t(s) * L.codes_stage + uint64_t(h) * L.codes_head +
                        uint64_t(tt) * L.codes_token + uint64_t(g) * (G * BITS / 8);
    if constexpr (WORDS == 2) {
      const uint2 v = *(const uint2 *)cp;
      gs.w[s][0] = v.x; gs.w[s][1] = v.y;
    } else {
#pragma unroll
      for (int i = 0; i < WORDS; i += 4) {
        const uint4 v = *(const uint4 *)(cp + 4 * i);
        gs.w[s][i] = v.x; gs.w[s][i + 1] = v.y; gs.w[s][i + 2] = v.z; gs.w[s][i + 3] = v.w;
      }
    }
    gs.m[s] = *((const uint32_t *)(st + L.meta_off + uint64_t(s) * L.meta_stage + uint64_t(h) * L.meta_head +
                                   uint64_t(tt) * L.meta_token) + g);
  }
}

// Rebuild one group in fp32: xhat = fl32(...fl32(base + rhat_1)... + rhat_S).
// xh holds the base on entry.
template <int G, int BITS>
__device__ __forceinline__ void add_stages(const GroupStages<G, BITS> &gs, int S, float *xh) {
  constexpr int WORDS = G * BITS / 32;
#pragma unroll
  for (int s = 0; s < kStagesMax; ++s) {
    if (s >= S) break;
    const float sf = f16_bits_to_f32(uint16_t(gs.m[s] & 0xffffu));
    const float zf = f16_bits_to_f32(uint16_t(gs.m[s] >> 16));
    float q[G];
#pragma unroll
    for (int i = 0; i < WORDS; ++i) {
      if constexpr (BITS == 2) widen_codes2(gs.w[s][i], q + 16 * i);
      else widen_codes4(gs.w[s][i], q + 8 * i);
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
                                              int slot, float *xh) {
  constexpr int EB = CB_BF16 ? 2 : 4;
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
  const uint8_t *st = stream_ptr(a.arena, L, a.layer0 + lrel, a.kv);
  // the chunk table (first token of each chunk) staged in LDS once per block
  __shared__ int32_t starts_s[kMaxChunks + 1];
  const StreamHeader *hdr = (const StreamHeader *)(st + L.header_off);
  const int nch = hdr->n_chunks;
  if (nch > 1 && (!a.pred || OUTL)) {
    for (int i = threadIdx.x; i < nch; i += blockDim.x) starts_s[i] = hdr->start[i];
    __syncthreads();
  }
  if (valid_lanes <= 0) return;             // whole wave past the end
  const int tt = a.t0 + min(t, a.n - 1);
  const int slot = nch > 1 && (!a.pred || OUTL) ? chunk_of_lds(starts_s, nch, tt) : 0;
  GroupStages<G, BITS> gs;
  if constexpr (!OUTL) load_stages<D, G, BITS>(st, L, h, tt, g, gs);
  float xh[G];
  if (a.pred) {
    const float *p = a.pred + (uint64_t(h) * a.n + min(t, a.n - 1)) * D + g * G;
#pragma unroll
    for (int j = 0; j < G; ++j) xh[j] = p[j];
  } else {
    centroid_base<D, G, CB_BF16>(st, L, h, tt, g, slot, xh);
  }
  if constexpr (OUTL) {
    constexpr int FW = (G + 31) / 32;
    const uint32_t *mw = (const uint32_t *)(st + L.mask_off + uint64_t(slot) * L.mask_chunk +
                                            uint64_t(h) * L.mask_head);
    uint32_t fm[FW];
#pragma unroll
    for (int i = 0; i < FW; ++i) fm[i] = mw[g * FW + i];
    add_stages_outl<D, G, BITS>(st, L, h, tt, g, xh, fm);
  } else {
    add_stages<G, BITS>(gs, L.S, xh);
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

// ---------------------------------------------------------------- launchers

template <int D, int G, int BITS, bool BF>
static void launch_recon_t(const ReconArgs &a, int n_layers, int64_t out_tokens, int out_t_off,
                           hipStream_t st) {
  const int64_t items = int64_t(a.n) * (D / G);
  // LDS: 4 waves x 64 lanes x one group of the output type
  const size_t lds = size_t(4) * 64 * G * (a.out && !a.out_bf16 ? 4 : 2);
  if (a.L.mask_off)
    QKV_LAUNCH((k_reconstruct<D, G, BITS, BF, true>), dim3(cdiv(items, 256), a.L.H, n_layers), dim3(256),
                       lds, st, a, out_tokens, out_t_off);
  else
    QKV_LAUNCH((k_reconstruct<D, G, BITS, BF>), dim3(cdiv(items, 256), a.L.H, n_layers), dim3(256),
                       lds, st, a, out_tokens, out_t_off);
}

void launch_reconstruct(const ReconArgs &a, int n_layers, int64_t out_tokens, int out_t_off, hipStream_t st) {
  QKV_DISPATCH_CODEC(a.L, launch_recon_t, a, n_layers, out_tokens, out_t_off, st);
}
}  // namespace qkv
