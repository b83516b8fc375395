// Cross-layer kernels of the qkv library: block-diagonal + low-rank
// prediction in fp64 with a fixed summation order, and the adapted-mode
// re-fit (Gram sums + Cholesky solve).
#include "common.h"

namespace qkv {

// ------------------------------------------------------------ cross layer

// Cross-layer prediction (r <= 64), in fp64 with a fixed summation order per
// output: the projection sums over m = 0 .. H*D-1, the prediction over j, then
// over k.  Every product is of two bf16 values, hence exact in fp64, so
// fma(p, q, acc) equals acc + p*q rounded once: each output is exactly that
// sequence of fp64 additions, however the work is tiled.

constexpr int XP_TT = 64;                    // tokens per tile
__device__ __forceinline__ int xp_perm(int k) { return (k & ~15) | ((k & 3) << 2) | ((k >> 2) & 3); }
__device__ __forceinline__ double xp_bf16(uint2 v, int s) {
  const uint32_t w = (s & 2) ? v.y : v.x;
  return double(__uint_as_float((s & 1) ? (w & 0xffff0000u) : (w << 16)));
}
typedef double xp_double4 __attribute__((ext_vector_type(4)));

// proj[t][k] = bf16(sum over m = 0 .. H*D-1 of y[t][m] V[m][k]) on the fp64
// matrix instruction, m ascending (see the prediction below for its order
// and operand layouts; here m = token, n = output k, k-index = input m).
// Block = 4 waves over 64 tokens (16 per wave, all r outputs: r/16
// accumulator tiles); the m axis is staged through LDS 64 at a time (a chunk
// lies inside one head), the next chunk's y and V loaded into registers
// while the current one is multiplied.
constexpr int XJ_MC = 64;                    // inputs m per chunk
constexpr int XJ_TT = 64;                    // tokens per block
template <int NT>   // accumulator tiles: outputs k < 16 NT (r <= 16 NT)
__global__ __launch_bounds__(256, 2) void k_xl_project(XlArgs a, int kv0) {
  constexpr int SP = XJ_MC + 4;              // LDS row stride (bf16)
  constexpr int RP = 16 * NT;
  __shared__ __attribute__((aligned(16))) uint16_t ys[XJ_TT * SP];  // [token][m'] (m permuted in runs of 16)
  __shared__ __attribute__((aligned(16))) uint16_t vs[64 * SP];     // [k][m']
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, kv = kv0 + blockIdx.y;
  const int ln = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * XJ_TT;
  const int D = a.D;
  const uint64_t HD = uint64_t(a.H) * D;
  const uint16_t *Vw = a.weights + uint64_t(kv) * a.kv_weight_stride + HD * D + HD * a.r;
  const uint16_t *y = a.chain + uint64_t(kv) * HD * a.n;
  constexpr int YPT = XJ_TT * XJ_MC / 8 / 256;   // 16-byte y pieces per thread
  constexpr int VPT = XJ_MC * RP / 256;          // V values per thread
  uint4 ypre[YPT];
  uint16_t vpre[VPT];
  auto fetch = [&](uint64_t m0) {
    const int hh = int(m0 / D), j0 = int(m0 % D);
#pragma unroll
    for (int i = 0; i < YPT; ++i) {
      const int e8 = tid + 256 * i, tt = e8 / (XJ_MC / 8), j8 = 8 * (e8 % (XJ_MC / 8));
      const int t = min(t0 + tt, a.n - 1);
      ypre[i] = *(const uint4 *)(y + (uint64_t(hh) * a.n + t) * D + j0 + j8);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int e = tid + 256 * i, jj = e / RP, k = e % RP;
      vpre[i] = k < a.r ? Vw[(m0 + jj) * a.r + k] : uint16_t(0);
    }
  };
  xp_double4 acc[NT];
#pragma unroll
  for (int it = 0; it < NT; ++it) acc[it] = xp_double4{0.0, 0.0, 0.0, 0.0};
  fetch(0);
  for (uint64_t m0 = 0; m0 < HD; m0 += XJ_MC) {
    __syncthreads();                         // previous chunk consumed
#pragma unroll
    for (int i = 0; i < YPT; ++i) {
      const int e8 = tid + 256 * i, tt = e8 / (XJ_MC / 8), j8 = 8 * (e8 % (XJ_MC / 8));
      const uint32_t v4[4] = {ypre[i].x, ypre[i].y, ypre[i].z, ypre[i].w};
#pragma unroll
      for (int q = 0; q < 8; ++q) ys[tt * SP + xp_perm(j8 + q)] = uint16_t(v4[q >> 1] >> (16 * (q & 1)));
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int e = tid + 256 * i, jj = e / RP, k = e % RP;
      vs[k * SP + xp_perm(jj)] = vpre[i];
    }
    __syncthreads();
    if (m0 + XJ_MC < HD) fetch(m0 + XJ_MC);
    const uint16_t *arow = ys + (16 * wave + ln) * SP + 4 * g;
    const uint16_t *brow = vs + ln * SP + 4 * g;
#pragma unroll 1
    for (int q = 0; q < XJ_MC / 16; ++q) {
      const uint2 av = *(const uint2 *)(arow + 16 * q);
      uint2 bv[NT];
#pragma unroll
      for (int it = 0; it < NT; ++it) bv[it] = *(const uint2 *)(brow + (16 * it) * SP + 16 * q);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const double ad = xp_bf16(av, s);
#pragma unroll
        for (int it = 0; it < NT; ++it)
          acc[it] = __builtin_amdgcn_mfma_f64_16x16x4f64(ad, xp_bf16(bv[it], s), acc[it], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 16 * wave + 4 * i + g;
    if (t >= a.n) continue;
#pragma unroll
    for (int it = 0; it < NT; ++it) {
      const int k = 16 * it + ln;
      if (k < a.r) a.proj[(uint64_t(kv) * a.n + t) * a.r + k] = bf16_to_f32(f64_to_bf16_bits(acc[it][i]));
    }
  }
}

// pred[h][t][i] = sum_j B_h[i][j] y[t][j] (order j), then + sum_k U[h*D+i][k]
// w[t][k] (order k), fp64, rounded once to fp32, on the fp64 matrix
// instruction v_mfma_f64_16x16x4_f64.  That instruction adds its four
// products to the accumulator one after another in k order, each sum
// rounded to fp64 (checked on the device against a sequential fp64
// reference: identical bits for 1M outputs whose operands span +-2^44, where
// the reverse, pairwise and single-rounding orders each differ in about 3.5 %
// of them), so a chain of them over ascending k is the same sequence of fp64
// additions as the definition.  Operand layouts of the 16x16x4 shape: A[m][k]
// in lane m + 16 k, B[k][n] in lane n + 16 k, D[m][n] in lane n + 16 (m % 4),
// register m / 4.  Here m = token, n = output channel, k = input channel j
// (then rank k).  Block = 4 waves over a tile of 64 tokens, wave w taking
// tokens 16 w .. 16 w + 15 and all D outputs (D/16 accumulator tiles); a
// block walks a consecutive range of (tensor, head, token tile) units.  In LDS every operand row keeps its k index permuted inside
// each run of 16 (k = 16 q + 4 s + g stored at 16 q + 4 g + s), so that the
// lane of k-group g reads the values of four consecutive k-steps s in one
// 8-byte load.
template <int D, int NT>   // NT: runs of 16 ranks (r <= 16 NT)
__global__ __launch_bounds__(256, 2) void k_xl_predict(XlArgs a, int kv0, int n_kv) {
  constexpr int NI = D / 16, BP = D + 4;     // accumulator tiles; B / y row stride (bf16)
  constexpr int RP = 16 * NT, UP = RP + 4;   // padded rank; U / w row stride (bf16)
  extern __shared__ uint16_t xs16[];
  uint16_t *Bs = xs16;                       // [D i][BP]: B_h[i][j] at xp_perm(j)
  uint16_t *Us = Bs + D * BP;                // [D i][UP]: U[h*D+i][k] at xp_perm(k), 0 past r
  uint16_t *Ys = Us + D * UP;                // [XP_TT t][BP]: y[t][j] at xp_perm(j)
  uint16_t *Ws = Ys + XP_TT * BP;            // [XP_TT t][UP]: w[t][k] at xp_perm(k), 0 past r
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const uint64_t HD = uint64_t(a.H) * D;
  // The (head, tensor, token tile) units, tensor-major then head, are split
  // into equal consecutive ranges, one per block; B_h and U_h are staged
  // again where a block's range moves to another head.
  const int n_tiles = (a.n + XP_TT - 1) / XP_TT;
  const int64_t n_units = int64_t(n_tiles) * a.H * n_kv;
  const int64_t u0 = n_units * blockIdx.x / gridDim.x, u1 = n_units * (blockIdx.x + 1) / gridDim.x;
  auto chain_of = [&](int hk) {              // hk = kv_rel * H + h
    return a.chain + uint64_t(kv0 + hk / a.H) * HD * a.n + uint64_t(hk % a.H) * a.n * D;
  };
  auto proj_of = [&](int hk) { return a.proj + uint64_t(kv0 + hk / a.H) * a.n * a.r; };
  // the next unit's y rows and w values are loaded into registers while the
  // current one is multiplied (16-byte pieces of y; w as bf16 bits)
  constexpr int YPT = XP_TT * D / 8 / 256;   // y pieces per thread
  constexpr int WPT = XP_TT * RP / 256;      // w values per thread
  uint4 ypre[YPT];
  uint16_t wpre[WPT];
  auto fetch = [&](int64_t u) {
    const int hk = int(u / n_tiles), t0 = int(u % n_tiles) * XP_TT;
    const uint16_t *y = chain_of(hk);
    const float *w = proj_of(hk);
#pragma unroll
    for (int i = 0; i < YPT; ++i) {
      const int e8 = tid + 256 * i, tt = e8 / (D / 8), j8 = 8 * (e8 % (D / 8)), t = min(t0 + tt, a.n - 1);
      ypre[i] = *(const uint4 *)(y + uint64_t(t) * D + j8);
    }
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int e = tid + 256 * i, tt = e / RP, k = e % RP, t = min(t0 + tt, a.n - 1);
      // w holds bf16 values (rounded in the projection): exact in bf16
      wpre[i] = k < a.r ? f32_to_bf16_bits(w[uint64_t(t) * a.r + k]) : uint16_t(0);
    }
  };
  int staged = -1;                           // head whose B_h and U_h are in LDS
  if (u0 < u1) fetch(u0);
  for (int64_t u = u0; u < u1; ++u) {
    const int hk = int(u / n_tiles), t0 = int(u % n_tiles) * XP_TT;
    __syncthreads();                         // previous unit consumed
    if (hk != staged) {                      // block-uniform
      const int kv = kv0 + hk / a.H, h = hk % a.H;
      const uint16_t *W = a.weights + uint64_t(kv) * a.kv_weight_stride;
      const uint16_t *B = a.b_weights ? a.b_weights + (uint64_t(kv) * a.H + h) * D * D : W + uint64_t(h) * D * D;
      const uint16_t *U = W + HD * D + uint64_t(h) * D * a.r;
      for (int e = tid; e < D * D; e += 256) Bs[(e / D) * BP + xp_perm(e % D)] = B[e];
      for (int e = tid; e < D * RP; e += 256) {
        const int i = e / RP, k = e % RP;
        Us[i * UP + xp_perm(k)] = k < a.r ? U[uint64_t(i) * a.r + k] : uint16_t(0);
      }
      staged = hk;
    }
#pragma unroll
    for (int i = 0; i < YPT; ++i) {
      const int e8 = tid + 256 * i, tt = e8 / (D / 8), j8 = 8 * (e8 % (D / 8));
      const uint32_t v4[4] = {ypre[i].x, ypre[i].y, ypre[i].z, ypre[i].w};
#pragma unroll
      for (int q = 0; q < 8; ++q) Ys[tt * BP + xp_perm(j8 + q)] = uint16_t(v4[q >> 1] >> (16 * (q & 1)));
    }
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int e = tid + 256 * i, tt = e / RP, k = e % RP;
      Ws[tt * UP + xp_perm(k)] = wpre[i];
    }
    __syncthreads();
    if (u + 1 < u1) fetch(u + 1);
    float *pred = a.pred + uint64_t(kv0 + hk / a.H) * HD * a.n + uint64_t(hk % a.H) * a.n * D;
    xp_double4 acc[NI];
#pragma unroll
    for (int it = 0; it < NI; ++it) acc[it] = xp_double4{0.0, 0.0, 0.0, 0.0};
    // 16 k values (four k-steps) per round: A from the token rows, B from the
    // weight rows of every accumulator tile
    auto rounds = [&](const uint16_t *arow, const uint16_t *brows, int stride, int nq) {
      for (int q = 0; q < nq; ++q) {
        const uint2 av = *(const uint2 *)(arow + 16 * q);
        uint2 bv[NI];
#pragma unroll
        for (int it = 0; it < NI; ++it) bv[it] = *(const uint2 *)(brows + (16 * it) * stride + 16 * q);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const double ad = xp_bf16(av, s);
#pragma unroll
          for (int it = 0; it < NI; ++it)
            acc[it] = __builtin_amdgcn_mfma_f64_16x16x4f64(ad, xp_bf16(bv[it], s), acc[it], 0, 0, 0);
        }
      }
    };
    if (!a.lowrank_only) rounds(Ys + (16 * wave + m) * BP + 4 * g, Bs + m * BP + 4 * g, BP, D / 16);
    rounds(Ws + (16 * wave + m) * UP + 4 * g, Us + m * UP + 4 * g, UP, RP / 16);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 16 * wave + 4 * r + g;
      if (t >= a.n) continue;
#pragma unroll
      for (int it = 0; it < NI; ++it) pred[uint64_t(t) * D + 16 * it + m] = float(acc[it][r]);
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
// ---------------------------------------------------------------- launchers

void launch_xl_refit(const RefitArgs &a, hipStream_t st) {
  QKV_LAUNCH(k_xl_gram, dim3(kRefitParts, a.H, 4), dim3(256), 0, st, a);
  const size_t lds = (size_t(a.D) * a.D + 16 * size_t(a.D)) * sizeof(double);
  (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_xl_solve),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  QKV_LAUNCH(k_xl_solve, dim3(a.H, 2), dim3(256), lds, st, a);
}
template <int D, int NT>
static void xl_predict_launch(const XlArgs &a, int kv0, int n_kv, const dim3 &grid, size_t lds, hipStream_t st) {
  (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_xl_predict<D, NT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  QKV_LAUNCH((k_xl_predict<D, NT>), grid, dim3(256), lds, st, a, kv0, n_kv);
}
void launch_xl_predict(const XlArgs &a, int kv0, int n_kv, hipStream_t st) {
  if (!a.skip_project) {
    const dim3 grid(cdiv(a.n, XJ_TT), n_kv);
    if (a.r <= 16) QKV_LAUNCH(k_xl_project<1>, grid, dim3(256), 0, st, a, kv0);
    else if (a.r <= 32) QKV_LAUNCH(k_xl_project<2>, grid, dim3(256), 0, st, a, kv0);
    else if (a.r <= 48) QKV_LAUNCH(k_xl_project<3>, grid, dim3(256), 0, st, a, kv0);
    else QKV_LAUNCH(k_xl_project<4>, grid, dim3(256), 0, st, a, kv0);
  }
  const int RP = (a.r + 15) & ~15;
  const size_t lds = size_t((a.D + XP_TT) * (a.D + 4) + (a.D + XP_TT) * (RP + 4)) * 2;
  // two blocks per CU (staged weights + one token tile); at most 512 blocks
  // in all, so that they run in one round, each walking every gx-th token
  // tile of its (head, kv)
  // two blocks per CU (staged weights + one token tile), at most 512 in all
  // so that they run in one round
  const int64_t n_units = cdiv(a.n, XP_TT) * int64_t(a.H) * n_kv;
  const dim3 grid(unsigned(std::min<int64_t>(n_units, 512)));
  if (a.D == 64) {
    switch (RP / 16) {
      case 1: xl_predict_launch<64, 1>(a, kv0, n_kv, grid, lds, st); break;
      case 2: xl_predict_launch<64, 2>(a, kv0, n_kv, grid, lds, st); break;
      case 3: xl_predict_launch<64, 3>(a, kv0, n_kv, grid, lds, st); break;
      default: xl_predict_launch<64, 4>(a, kv0, n_kv, grid, lds, st); break;
    }
  } else {
    switch (RP / 16) {
      case 1: xl_predict_launch<128, 1>(a, kv0, n_kv, grid, lds, st); break;
      case 2: xl_predict_launch<128, 2>(a, kv0, n_kv, grid, lds, st); break;
      case 3: xl_predict_launch<128, 3>(a, kv0, n_kv, grid, lds, st); break;
      default: xl_predict_launch<128, 4>(a, kv0, n_kv, grid, lds, st); break;
    }
  }
}
}  // namespace qkv
