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

// ---- batched float32 GEMM on the matrix cores: C = op(A) op(B) ---------------------------
// op(A) is M x K: A stored [M][K] (TA false) or [K][M] (TA true), leading dimension lda;
// op(B) is K x N: B stored [K][N] (TB false) or [N][K] (TB true).  Batch entry z uses
// A + mapA(z) sA, B + mapB(z) sB, C + z sC.  The grid is one dimension (batch entries x row
// tiles x column tiles), so any batch count fits.
// Workgroup: a 64 x 64 tile of C, 4 waves in a 2 x 2 grid of 32 x 32 tiles, each
// accumulated with v_mfma_f32_32x32x2_f32 (float32 in, float32 accumulate).  Contraction
// slabs of 32 are staged through LDS as [row][k] (k contiguous), the next slab's global
// loads in flight while the current one is multiplied.  Within a slab, lane group g
// (lanes 32 g .. 32 g + 31) supplies k = 8 h + 4 g + j to MFMA (h, j), so one 16-byte LDS
// read feeds four MFMAs.  Waves whose 32 x 32 tile lies wholly outside C skip the products.
// flags: kAccum adds to C instead of overwriting it; kTril zeroes the outputs with column >
// row (the causal mask of a 64 x 64 chunk product); kMulAux multiplies the result
// elementwise by epi.aux (indexed like C); kRowSum also writes the row sums of the result
// over each 32-column tile to epi.rowp[z][row][col / 32] (z stride epi.srp, row stride
// epi.ldrp), to be added up in column order by the reader (deterministic).
// With ksplit > 1 (long contractions with few output tiles) the batch index enumerates
// (split, batch entry); split s covers contraction indices [s kc, (s+1) kc) and writes its
// partial to C + (s batch + z) sC, summed afterwards in split order by sum_splits.
constexpr int GT = 64, GK = 32, GLD = GK + 4;
constexpr int kAccum = 1, kTril = 2, kMulAux = 4, kRowSum = 8;

struct Epi {
  const float* aux = nullptr;
  float* rowp = nullptr;
  int ldrp = 0;
  long long srp = 0;
};

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
             int kc, int flags, Epi epi) {
  constexpr int PER = GT * GK / 256;  // operand elements per thread and slab
  __shared__ __attribute__((aligned(16))) float As[GT][GLD];
  __shared__ __attribute__((aligned(16))) float Bs[GT][GLD];
  const int tn = (N + GT - 1) / GT, tm = (M + GT - 1) / GT;
  const int bx = blockIdx.x % tn, by = (blockIdx.x / tn) % tm, zs = blockIdx.x / (tn * tm);
  const int z = zs % batch, split = zs / batch;
  A += block_of(mapA, z) * sA;
  B += block_of(mapB, z) * sB;
  C += (long long)zs * sC;
  const int kbeg = split * kc, kend = min(K, kbeg + kc);
  const int m0 = by * GT, n0 = bx * GT;
  const int t = threadIdx.x, wave = t >> 6, l = t & 63, c32 = l & 31, g = l >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const bool active = m0 + 32 * wm < M && n0 + 32 * wn < N;

  // element e of a slab: consecutive threads walk the operand's contiguous dimension
  auto a_rc = [&](int e, int& row, int& k) {
    row = TA ? e % GT : e / GK;
    k = TA ? e / GT : e % GK;
  };
  auto b_rc = [&](int e, int& col, int& k) {
    col = TB ? e / GK : e % GT;
    k = TB ? e % GK : e / GT;
  };
  float ra[PER], rb[PER];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      int row, k, col, kb;
      a_rc(t + 256 * u, row, k);
      const int gm = m0 + row, gk = k0 + k;
      ra[u] = gm < M && gk < kend ? (TA ? A[(long long)gk * lda + gm] : A[(long long)gm * lda + gk]) : 0.f;
      b_rc(t + 256 * u, col, kb);
      const int gn = n0 + col, gkb = k0 + kb;
      rb[u] = gn < N && gkb < kend ? (TB ? B[(long long)gn * ldb + gkb] : B[(long long)gkb * ldb + gn]) : 0.f;
    }
  };

  f32x16 acc = zero16();
  if (kbeg < kend) fetch(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += GK) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      int row, k, col, kb;
      a_rc(t + 256 * u, row, k);
      As[row][k] = ra[u];
      b_rc(t + 256 * u, col, kb);
      Bs[col][kb] = rb[u];
    }
    __syncthreads();
    if (k0 + GK < kend) fetch(k0 + GK);
    if (active) {
#pragma unroll
      for (int h = 0; h < GK / 8; ++h) {
        if (k0 + 8 * h >= kend) break;  // a ragged last slab (e.g. K = d + 1) skips its empty groups
        const f32x4 a = *reinterpret_cast<const f32x4*>(&As[32 * wm + c32][8 * h + 4 * g]);
        const f32x4 b = *reinterpret_cast<const f32x4*>(&Bs[32 * wn + c32][8 * h + 4 * g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mma(a[j], b[j], acc);
      }
    }
    __syncthreads();
  }
  if (!active) return;
  // accumulator r of lane (c32, g): row 8 (r / 4) + 4 g + r % 4, column c32 of the wave's tile
  const int gn = n0 + 32 * wn + c32;
  const float* aux = epi.aux + (long long)zs * sC;
  const int mrow = m0 + 32 * wm + 4 * g;  // + 8 (r / 4) + r % 4
  auto ok = [&](int r) { return mrow + 8 * (r >> 2) + (r & 3) < M && gn < N; };
  auto at = [&](int r) { return (long long)(mrow + 8 * (r >> 2) + (r & 3)) * ldc + gn; };
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = (flags & kTril) && gn > mrow + 8 * (r >> 2) + (r & 3) ? 0.f : acc[r];
  // all loads of the epilogue are issued before any store
  if (flags & kAccum) {
    float cv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) cv[r] = ok(r) ? C[at(r)] : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] += cv[r];
  }
  if (flags & kMulAux) {
    float av[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) av[r] = ok(r) ? aux[at(r)] : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] *= av[r];
  }
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (ok(r)) C[at(r)] = x[r];
  if (flags & kRowSum) {  // wave-uniform: sums over the 32 columns of each lane group
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float y = ok(r) ? x[r] : 0.f;
#pragma unroll
      for (int s = 1; s < 32; s <<= 1) y += __shfl_xor(y, s);
      const int gm = mrow + 8 * (r >> 2) + (r & 3);
      if (c32 == (r & 31) && gm < M) epi.rowp[(long long)zs * epi.srp + (long long)gm * epi.ldrp + (n0 >> 5) + wn] = y;
    }
  }
}

inline unsigned gemm_blocks(int M, int N, long long entries) {
  return (unsigned)(((N + GT - 1) / GT) * (long long)((M + GT - 1) / GT) * entries);
}

template <bool TA, bool TB>
favor_status gemm(const float* A, const float* B, float* C, int M, int N, int K, int lda, int ldb, int ldc,
                  long long sA, long long sB, long long sC, BMap mapA, BMap mapB, int batch, hipStream_t st,
                  int flags = 0, Epi epi = Epi{}) {
  hipLaunchKernelGGL((gemm_f32<TA, TB>), dim3(gemm_blocks(M, N, batch)), dim3(256), 0, st, A, B, C, M, N, K, lda,
                     ldb, ldc, sA, sB, sC, mapA, mapB, batch, K, flags, epi);
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
// least 256 deep (a multiple of the contraction slab).
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
                     B, P, M, N, K, lda, ldb, N, sA, sB, (long long)M * N, mapA, mapB, batch, kc, 0, Epi{});
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
