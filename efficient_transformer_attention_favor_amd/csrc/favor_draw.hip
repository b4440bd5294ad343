// Random feature matrices drawn on the device from a seed (the favor_draw_features entry point).
//
// "Rethinking Attention with Performers" (review page), section "제안 방법": the softmax
// kernel is estimated with random features whose rows are made orthogonal (orthogonal random
// features) to lower the variance of the estimate.  Redrawing W, e.g. between training steps,
// then needs no host work and no transfer: one workgroup per (head, block of d rows)
//   1. fills a d x d block with Gaussians: Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
//      "Parallel random numbers: as easy as 1, 2, 3", SC 2011) on counter (p mod 2^32,
//      p div 2^32, 0, 0), key (seed mod 2^32, seed div 2^32), for Gaussian pair p; the two
//      64-bit halves of the output, shifted right by 11, give u1 = (a + 1) 2^-53 and
//      u2 = b 2^-53, and Box-Muller gives the even number radius cos(2 pi u2), the odd one
//      radius sin(2 pi u2), radius = sqrt(-2 ln u1).  Gaussian e of head h, block b, row i,
//      column j is e = ((h nblocks + b) d + i) d + j.
//   2. (orthogonal) runs modified Gram-Schmidt on the block's rows in row order in LDS,
//      float64, and scales each orthonormal row by the length of the same Gaussian row;
//   3. writes the rows below m as float32.
// The work is tiny (m d^2 flops per head) and runs at launch latency; float64 keeps the
// orthogonality error far below float32 rounding.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "../../include/favor.h"

namespace favor {
namespace {

constexpr int kDrawThreads = 256;
constexpr int kDrawMaxD = 128;

struct Ctr {
  unsigned c0, c1, c2, c3;
};

__device__ __forceinline__ Ctr philox4x32_10(Ctr c, unsigned k0, unsigned k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const unsigned long long p0 = 0xD2511F53ull * c.c0, p1 = 0xCD9E8D57ull * c.c2;
    c = Ctr{(unsigned)(p1 >> 32) ^ c.c1 ^ k0, (unsigned)p1, (unsigned)(p0 >> 32) ^ c.c3 ^ k1, (unsigned)p0};
  }
  return c;
}

__device__ double gaussian(unsigned long long seed, unsigned long long e) {
  const unsigned long long p = e >> 1;
  const Ctr r = philox4x32_10(Ctr{(unsigned)p, (unsigned)(p >> 32), 0u, 0u}, (unsigned)seed, (unsigned)(seed >> 32));
  const unsigned long long a = (((unsigned long long)r.c1 << 32) | r.c0) >> 11;
  const unsigned long long b = (((unsigned long long)r.c3 << 32) | r.c2) >> 11;
  const double u1 = ((double)a + 1.0) * 0x1p-53, u2 = (double)b * 0x1p-53;
  const double radius = sqrt(-2.0 * log(u1)), angle = 2.0 * M_PI * u2;
  return (e & 1) ? radius * sin(angle) : radius * cos(angle);
}

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x += __shfl_xor(x, s);
  return x;
}

__global__ void __launch_bounds__(kDrawThreads)
    draw_kernel(int m, int d, int nblk, unsigned long long seed, int orthogonal, float* __restrict__ W) {
  __shared__ double g[kDrawMaxD][kDrawMaxD + 1];
  __shared__ double len[kDrawMaxD];
  const int hb = blockIdx.x, h = hb / nblk, b = hb % nblk;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  constexpr int waves = kDrawThreads / 64;
  const unsigned long long base = (unsigned long long)hb * d * d;
  const int rows = min(d, m - b * d);  // rows of this block below m
  float* Wb = W + ((size_t)h * m + (size_t)b * d) * d;
  if (!orthogonal) {
    for (int e = t; e < rows * d; e += kDrawThreads) Wb[e] = (float)gaussian(seed, base + e);
    return;
  }
  for (int e = t; e < d * d; e += kDrawThreads) g[e / d][e % d] = gaussian(seed, base + e);
  __syncthreads();
  for (int i = wave; i < rows; i += waves) {
    double s = 0.0;
    for (int j = lane; j < d; j += 64) s += g[i][j] * g[i][j];
    s = wave_sum(s);
    if (lane == 0) len[i] = sqrt(s);
  }
  for (int i = 0; i < rows; ++i) {
    // row i has lost the directions of rows 0..i-1: normalise it
    if (wave == 0) {
      double s = 0.0;
      for (int j = lane; j < d; j += 64) s += g[i][j] * g[i][j];
      const double nrm = sqrt(wave_sum(s));
      for (int j = lane; j < d; j += 64) g[i][j] = g[i][j] / nrm;
    }
    __syncthreads();
    // remove its direction from the later rows, one wave per row
    for (int r = i + 1 + wave; r < rows; r += waves) {
      double s = 0.0;
      for (int j = lane; j < d; j += 64) s += g[r][j] * g[i][j];
      const double dot = wave_sum(s);
      for (int j = lane; j < d; j += 64) g[r][j] = g[r][j] - dot * g[i][j];
    }
    __syncthreads();
  }
  for (int e = t; e < rows * d; e += kDrawThreads) {
    const int i = e / d, j = e - i * d;
    Wb[e] = (float)(g[i][j] * len[i]);
  }
}

}  // namespace
}  // namespace favor

extern "C" favor_status favor_draw_features(int32_t heads_w, int32_t num_features, int32_t head_dim, uint64_t seed,
                                            int32_t orthogonal, float* W, void* stream) {
  if (heads_w < 1 || heads_w > 65536 || num_features < 1 || num_features > 65536 || head_dim < 1 ||
      (orthogonal != 0 && orthogonal != 1) || W == nullptr)
    return FAVOR_ERR_INVALID_ARG;
  if (head_dim > favor::kDrawMaxD) return FAVOR_ERR_UNSUPPORTED;
  const int nblk = (num_features + head_dim - 1) / head_dim;
  if ((long long)heads_w * nblk > 0x7fffffffLL) return FAVOR_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(favor::draw_kernel, dim3((unsigned)(heads_w * nblk)), dim3(favor::kDrawThreads), 0,
                     static_cast<hipStream_t>(stream), num_features, head_dim, nblk, (unsigned long long)seed,
                     orthogonal, W);
  return hipGetLastError() == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}
