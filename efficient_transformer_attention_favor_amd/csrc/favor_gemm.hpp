// Float32 building blocks shared by the materialised-feature paths (gradients, generalised
// feature maps): a batched GEMM with causal-mask and accumulate epilogues, split
// contractions, padded-row helpers, the [V, 1] row kernel and the chunk prefix scan.
// Everything sits in an anonymous namespace: each translation unit gets its own copy.
#pragma once

#include <hip/hip_runtime.h>

#include "favor_device.hpp"
#include "favor_plan.hpp"

namespace favor {
namespace {

// ---- batched float32 GEMM: C = op(A) op(B), 64 x 64 tiles, 16-deep k steps ----------
// op(A) is M x K: A stored [M][K] (TA false) or [K][M] (TA true), leading dimension lda;
// op(B) is K x N: B stored [K][N] (TB false) or [N][K] (TB true).  Batch entry z uses
// A + mapA(z) sA, B + mapB(z) sB, C + z sC.  256 threads, 4 x 4 outputs each; the grid is
// one dimension (batch entries x row tiles x column tiles), so any batch count fits.
// flags: kAccum adds to C instead of overwriting it; kTril zeroes the outputs with column >
// row (the causal mask of a 64 x 64 chunk product).
// With ksplit > 1 (long contractions with few output tiles) the batch index enumerates
// (split, batch entry); split s covers contraction indices [s kc, (s+1) kc) and writes its
// partial to C + (s batch + z) sC, summed afterwards in split order by sum_splits.
constexpr int GT = 64, GK = 16, GLD = GT + 4;
constexpr int kAccum = 1, kTril = 2;

// Operand block read by batch entry z: ((z / div) % mod) * mul + z % inner.
struct BMap {
  int div, mod, mul, inner;
};
constexpr BMap kIdent{1, 0x7fffffff, 1, 1};
constexpr BMap modulo(int n) { return BMap{1, n, 1, 1}; }
__device__ __forceinline__ long long block_of(const BMap& b, int z) {
  return (long long)((z / b.div) % b.mod) * b.mul + z % b.inner;
}

template <bool TA, bool TB>
__global__ void __launch_bounds__(256)
    gemm_f32(const float* __restrict__ A, const float* __restrict__ B, float* __restrict__ C, int M, int N, int K,
             int lda, int ldb, int ldc, long long sA, long long sB, long long sC, BMap mapA, BMap mapB, int batch,
             int kc, int flags) {
  __shared__ __attribute__((aligned(16))) float As[GK][GLD];
  __shared__ __attribute__((aligned(16))) float Bs[GK][GLD];
  const int tn = (N + GT - 1) / GT, tm = (M + GT - 1) / GT;
  const int bx = blockIdx.x % tn, by = (blockIdx.x / tn) % tm, zs = blockIdx.x / (tn * tm);
  const int z = zs % batch, split = zs / batch;
  A += block_of(mapA, z) * sA;
  B += block_of(mapB, z) * sB;
  C += (long long)zs * sC;
  const int kbeg = split * kc, kend = min(K, kbeg + kc);
  const int m0 = by * GT, n0 = bx * GT;
  const int t = threadIdx.x, tx = t % 16, ty = t / 16;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = kbeg; k0 < kend; k0 += GK) {
#pragma unroll
    for (int e = t; e < GT * GK; e += 256) {
      // consecutive threads walk the operand's contiguous dimension
      const int mm = TA ? e % GT : e / GK, kk = TA ? e / GT : e % GK;
      const int gm = m0 + mm, gk = k0 + kk;
      float x = 0.f;
      if (gm < M && gk < kend) x = TA ? A[(long long)gk * lda + gm] : A[(long long)gm * lda + gk];
      As[kk][mm] = x;
    }
#pragma unroll
    for (int e = t; e < GT * GK; e += 256) {
      const int nn = TB ? e / GK : e % GT, kk = TB ? e % GK : e / GT;
      const int gn = n0 + nn, gk = k0 + kk;
      float x = 0.f;
      if (gn < N && gk < kend) x = TB ? B[(long long)gn * ldb + gk] : B[(long long)gk * ldb + gn];
      Bs[kk][nn] = x;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < GK; ++kk) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&As[kk][ty * 4]);
      const f32x4 b = *reinterpret_cast<const f32x4*>(&Bs[kk][tx * 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + ty * 4 + i;
    if (gm >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tx * 4 + j;
      if (gn >= N) continue;
      float x = (flags & kTril) && gn > gm ? 0.f : acc[i][j];
      if (flags & kAccum) x += C[(long long)gm * ldc + gn];
      C[(long long)gm * ldc + gn] = x;
    }
  }
}

inline unsigned gemm_blocks(int M, int N, long long entries) {
  return (unsigned)(((N + GT - 1) / GT) * (long long)((M + GT - 1) / GT) * entries);
}

template <bool TA, bool TB>
favor_status gemm(const float* A, const float* B, float* C, int M, int N, int K, int lda, int ldb, int ldc,
                  long long sA, long long sB, long long sC, BMap mapA, BMap mapB, int batch, hipStream_t st,
                  int flags = 0) {
  hipLaunchKernelGGL((gemm_f32<TA, TB>), dim3(gemm_blocks(M, N, batch)), dim3(256), 0, st, A, B, C, M, N, K, lda,
                     ldb, ldc, sA, sB, sC, mapA, mapB, batch, K, flags);
  return hipGetLastError() == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}

// C[z] = sum over s of P[s][z] (in split order), each [M][N] dense.
__global__ void __launch_bounds__(256) sum_splits(const float* __restrict__ P, float* __restrict__ C, long long n,
                                                  int splits) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int k = 0; k < splits; ++k) s += P[(long long)k * n + i];
  C[i] = s;
}

// Splits of a long contraction so that the launch has about 4096 workgroups, each split at
// least 256 deep (a multiple of the 16-deep step).
inline int ksplit_for(int M, int N, int K, int batch) {
  const long long tiles = (long long)((N + GT - 1) / GT) * ((M + GT - 1) / GT) * batch;
  long long s = (4096 + tiles - 1) / tiles;
  const long long smax = (K + 255) / 256;
  if (s > smax) s = smax;
  return s < 1 ? 1 : (int)s;
}

// C (dense [M][N] per batch entry) = op(A) op(B) with a split contraction; P holds
// splits * batch * M * N floats of partials.
template <bool TA, bool TB>
favor_status gemm_split(const float* A, const float* B, float* C, float* P, int M, int N, int K, int lda, int ldb,
                        long long sA, long long sB, BMap mapA, BMap mapB, int batch, int splits, hipStream_t st) {
  const int kc = ((K + splits - 1) / splits + GK - 1) / GK * GK;
  hipLaunchKernelGGL((gemm_f32<TA, TB>), dim3(gemm_blocks(M, N, (long long)batch * splits)), dim3(256), 0, st, A,
                     B, P, M, N, K, lda, ldb, N, sA, sB, (long long)M * N, mapA, mapB, batch, kc, 0);
  if (hipGetLastError() != hipSuccess) return FAVOR_ERR_HIP;
  const long long n = (long long)batch * M * N;
  hipLaunchKernelGGL(sum_splits, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, P, C, n, splits);
  return hipGetLastError() == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}

// ---- row kernels: one wave per row, 4 rows per workgroup -----------------------------
// Float32 intermediates may hold Lp >= L rows per head (zero padding up to a whole number
// of chunks); the user's tensors hold L.  Row r of a padded matrix is position r % Lp of
// head r / Lp.

__device__ __forceinline__ long long unpadded_row(long long r, int L, int Lp, bool* real) {
  const long long h = r / Lp, pos = r - h * Lp;
  *real = pos < L;
  return h * L + pos;
}
__device__ __forceinline__ long long padded_row(long long r, int L, int Lp) {
  const long long h = r / L;
  return h * Lp + (r - h * L);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x += __shfl_xor(x, s);
  return x;
}

// V1 = [V, 1] as float32 [rows][D+1] (rows padded; padding rows all zero).
template <class T, int D>
__global__ void __launch_bounds__(256)
    ones_column(const T* __restrict__ V, float* __restrict__ V1, long long rows, int L, int Lp) {
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int l = threadIdx.x & 63;
  bool real;
  const long long u = unpadded_row(r, L, Lp, &real);
  for (int c = l; c <= D; c += 64) V1[r * (D + 1) + c] = !real ? 0.f : c < D ? (float)V[u * D + c] : 1.f;
}

// ---- chunk scans (causal) --------------------------------------------------------------
// One thread per summary element e (n = m (D+1) per chunk), one head per grid row.

// S[h][c] <- sum over c' < c of S[h][c'], in place, in chunk order.
__global__ void __launch_bounds__(256) chunk_prefix(float* __restrict__ S, int NC, int n) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  float* p = S + (size_t)blockIdx.y * NC * n + e;
  float run = 0.f;
  int c = 0;
  for (; c + 4 <= NC; c += 4) {
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = p[(size_t)(c + u) * n];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      p[(size_t)(c + u) * n] = run;
      run += x[u];
    }
  }
  for (; c < NC; ++c) {
    const float x = p[(size_t)c * n];
    p[(size_t)c * n] = run;
    run += x;
  }
}

inline size_t a256(size_t x) { return (x + 255) & ~size_t(255); }

inline int row_blocks(long long rows) { return (int)((rows + 3) / 4); }

}  // namespace
}  // namespace favor
