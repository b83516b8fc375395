// Self-check of the property the cross-layer kernels rely on: the fp64
// matrix instruction v_mfma_f64_16x16x4_f64 adds its four products to the
// accumulator one after another in k order, rounding each sum to fp64, so
// that a chain of them equals the sequential fp64 sum of the definition.
//
// Each of N tests multiplies a 16x4 by a 4x16 matrix of bf16 values (their
// products are exact in fp64) onto a 16x16 fp64 accumulator, with exponents
// spread wide enough that the order of the additions shows in the result,
// and compares every output bit for bit with the sequential sum
// ((((c + p0) + p1) + p2) + p3).  The reverse order is counted too, to show
// that the test can tell orders apart.  Exit status 0 when no output
// differs from the sequential sum.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

typedef double f64x4 __attribute__((ext_vector_type(4)));

// Operand layouts of the 16x16x4 shape: A[m][k] in lane m + 16 k, B[k][n] in
// lane n + 16 k, D[m][n] in lane n + 16 (m % 4), register m / 4.
__global__ void k_check(const double *A, const double *B, const double *C, double *D) {
  const int t = blockIdx.x, l = threadIdx.x, m = l & 15, k = l >> 4;
  const double a = A[t * 64 + m * 4 + k];       // A row-major [16][4]
  const double b = B[t * 64 + k * 16 + m];      // B row-major [4][16]
  f64x4 c;
  for (int r = 0; r < 4; ++r) c[r] = C[t * 256 + (k + 4 * r) * 16 + m];
  const f64x4 d = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
  for (int r = 0; r < 4; ++r) D[t * 256 + (k + 4 * r) * 16 + m] = d[r];
}

// SplitMix64 (Steele, Lea, Flood 2014) as the seeded generator
static uint64_t next_u64(uint64_t &s) {
  uint64_t z = (s += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
// a random bf16 value (8 significant bits) with exponent in [-span, span]
static double bf16_value(uint64_t &s, int span) {
  const uint64_t r = next_u64(s);
  const int e = int(r % uint64_t(2 * span + 1)) - span;
  const double mant = 1.0 + double((r >> 20) & 127) / 128.0;
  return ((r >> 40) & 1 ? -1.0 : 1.0) * std::ldexp(mant, e);
}

int main() {
  const int N = 2048;
  uint64_t seed = 20260601;
  std::vector<double> A(N * 64), B(N * 64), C(N * 256), D(N * 256);
  for (int t = 0; t < N; ++t) {
    const int span = 4 + t % 40;
    for (int i = 0; i < 64; ++i) {
      A[t * 64 + i] = bf16_value(seed, span);
      B[t * 64 + i] = bf16_value(seed, span);
    }
    for (int i = 0; i < 256; ++i) C[t * 256 + i] = bf16_value(seed, 2 * span) * (1.0 + (i % 7) / 1024.0);
  }
  double *dA = nullptr, *dB = nullptr, *dC = nullptr, *dD = nullptr;
  if (hipMalloc(&dA, A.size() * 8) != hipSuccess || hipMalloc(&dB, B.size() * 8) != hipSuccess ||
      hipMalloc(&dC, C.size() * 8) != hipSuccess || hipMalloc(&dD, D.size() * 8) != hipSuccess) {
    std::printf("device allocation failed\n");
    return 2;
  }
  hipMemcpy(dA, A.data(), A.size() * 8, hipMemcpyHostToDevice);
  hipMemcpy(dB, B.data(), B.size() * 8, hipMemcpyHostToDevice);
  hipMemcpy(dC, C.data(), C.size() * 8, hipMemcpyHostToDevice);
  hipLaunchKernelGGL(k_check, dim3(N), dim3(64), 0, 0, dA, dB, dC, dD);
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(D.data(), dD, D.size() * 8, hipMemcpyDeviceToHost) != hipSuccess) {
    std::printf("kernel failed\n");
    return 2;
  }
  long seq_diff = 0, rev_diff = 0;
  for (int t = 0; t < N; ++t)
    for (int i = 0; i < 16; ++i)
      for (int j = 0; j < 16; ++j) {
        double p[4];
        for (int k = 0; k < 4; ++k) p[k] = A[t * 64 + i * 4 + k] * B[t * 64 + k * 16 + j];  // exact
        double seq = C[t * 256 + i * 16 + j], rev = seq;
        for (int k = 0; k < 4; ++k) seq = seq + p[k];
        for (int k = 3; k >= 0; --k) rev = rev + p[k];
        const double got = D[t * 256 + i * 16 + j];
        seq_diff += std::memcmp(&got, &seq, 8) != 0;
        rev_diff += std::memcmp(&got, &rev, 8) != 0;
      }
  std::printf("outputs %d differ_from_sequential %ld differ_from_reverse %ld\n", N * 256, seq_diff, rev_diff);
  hipFree(dA); hipFree(dB); hipFree(dC); hipFree(dD);
  return seq_diff == 0 ? 0 : 1;
}
