// The positive random feature map on its own (the favor_features entry point).
//
// "Rethinking Attention with Performers" (review page), section "제안 방법": the softmax
// kernel is estimated with positive random features,
//   phi(x) = exp(W x - |x|^2/2 - c) / sqrt(m),
// where any constant c cancels in the attention output and only keeps the exponentials in
// range.  This file materialises phi for every row of Q or K as a float32 [rows][m]
// tensor, with c the row maximum of the exponent (queries) or its maximum over a whole
// (batch, kv head) (keys), and reports c in natural-log units.  The attention kernels keep
// phi on chip; this entry point exists to inspect it.
//
// Per wave: 32 rows, one 32-feature tile at a time, C = W_ft X^T on the MFMA (lane = row,
// accumulator register = feature), exponents in log2 units (W scaled by log2 e, the norm
// term subtracted on the VALU).  Queries: one pass for the row maximum, a second that
// recomputes the tile and writes phi.  Keys: a pass that folds the head maximum into an
// order-preserving unsigned encoding with atomicMax (exact, so the result does not depend
// on the order), then the writing pass, then a decode into c_out.  Internal callers may ask
// for Lo >= L output rows per head: rows L..Lo-1 of each head are then written as zeros.
#include <hip/hip_runtime.h>

#include <math.h>

#include <type_traits>

#include "favor_device.hpp"
#include "favor_ops.hpp"
#include "favor_plan.hpp"

namespace favor {
namespace {

constexpr int kFeatWaves = 4;
// bf16 problems with m <= kFeatLdsM: the workgroup (8 waves, 256 rows) first stages the
// fp16 W log2e rows of its head in LDS, so W is read and converted once per workgroup
// instead of once per wave and feature tile.
constexpr int kFeatLdsM = 256, kFeatLdsWaves = 8;

// Monotone map float -> uint32 (larger float, larger code) and its inverse.
__device__ __forceinline__ unsigned enc_order(float x) {
  const unsigned u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float dec_order(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// MODE 0: queries (row stabiliser, two passes in the kernel); 1: keys, head-maximum pass;
// 2: keys, writing pass with the head maximum from pass 1.
template <class T, int D, int MODE, bool LW>
__global__ void __launch_bounds__(64 * (LW ? kFeatLdsWaves : kFeatWaves))
    features_kernel(const T* __restrict__ X, const float* __restrict__ W, int L, int Lo, int H, int G, int Hw,
                    int m, float* __restrict__ phi, float* __restrict__ c_out) {
  using P = Prec<T>;
  using wfrag = typename P::wfrag;
  constexpr int NKC = D / P::KS;
  constexpr int NWV = LW ? kFeatLdsWaves : kFeatWaves;
  constexpr int LDW = D + 8;  // fp16 W row stride in LDS (16-byte aligned rows)
  __shared__ __attribute__((aligned(16))) f16 Wl[LW ? kFeatLdsM * LDW : 8];
  const int bh = blockIdx.y, h = bh % H;
  const int hkv = h / G;  // G = query heads per kv head (1 on the key side)
  const int wave = threadIdx.x >> 6, l = lane_id(), col = l & 31, g = l >> 5;
  const int row = (blockIdx.x * NWV + wave) * 32 + col;
  const bool valid = row < L, out_row = row < Lo;
  const size_t grow = (size_t)bh * L + row, orow = (size_t)bh * Lo + row;
  const float* Wh = W + (size_t)(Hw == 1 ? 0 : hkv) * m * D;
  if constexpr (LW) {
    for (int e = threadIdx.x; e < m * (D / 8); e += 64 * NWV) {
      const int f = e / (D / 8), c8 = (e - f * (D / 8)) * 8;
      const f32x4 a = *reinterpret_cast<const f32x4*>(Wh + (size_t)f * D + c8);
      const f32x4 b = *reinterpret_cast<const f32x4*>(Wh + (size_t)f * D + c8 + 4);
      f16x8 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = (f16)(a[j] * kLog2e);
        v[j + 4] = (f16)(b[j] * kLog2e);
      }
      *reinterpret_cast<f16x8*>(Wl + f * LDW + c8) = v;
    }
    __syncthreads();
  }

  wfrag xf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc)
    xf[kc] = valid ? to_wfrag(load_frag_k(X + grow * D, kc, g)) : zero_frag(wfrag{});
  float nrm = sumsq(xf);
  nrm += partner32(nrm);
  const float half_norm = 0.5f * kLog2e * nrm;

  // Exponent tile ft: e[r] = log2e (w_f . x - |x|^2/2), f = 32 ft + 8(r/4) + 4g + r%4.
  auto tile = [&](int ft) {
    f32x16 c = zero16();
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      wfrag wp;
      if constexpr (LW)
        wp = *reinterpret_cast<const f16x8*>(Wl + (32 * ft + col) * LDW + 16 * kc + 8 * g);
      else
        load_w_frag(Wh + (size_t)(32 * ft + col) * D, kc, g, wp);
      c = mma(wp, xf[kc], c);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) c[r] -= half_norm;
    return c;
  };
  const float inv_sqrt_m = 1.0f / sqrtf((float)m);
  auto write = [&](float cst) {
    for (int ft = 0; ft < m / 32; ++ft) {
      const f32x16 e = tile(ft);
      if (!out_row) continue;
      float* dst = phi + orow * m + 32 * ft + 4 * g;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = valid ? fast_exp2(e[4 * r4 + i] - cst) * inv_sqrt_m : 0.f;
        }
        *reinterpret_cast<f32x4*>(dst + 8 * r4) = v;
      }
    }
  };

  if constexpr (MODE == 2) {
    write(dec_order(reinterpret_cast<const unsigned*>(c_out)[bh]));
    return;
  }
  float mx = -INFINITY;
  for (int ft = 0; ft < m / 32; ++ft) {
    const f32x16 e = tile(ft);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, e[r]);
  }
  mx = fmaxf(mx, partner32(mx));  // the other half of this row's features
  if constexpr (MODE == 0) {
    write(mx);
    if (valid && g == 0) c_out[orow] = mx / kLog2e;
  } else {
    if (!valid) mx = -INFINITY;
#pragma unroll
    for (int s = 16; s >= 1; s >>= 1) mx = fmaxf(mx, __shfl_xor(mx, s));
    if (l == 0) atomicMax(reinterpret_cast<unsigned*>(c_out) + bh, enc_order(mx));
  }
}

__global__ void head_max_init(unsigned* c, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) c[i] = enc_order(-INFINITY);
}

__global__ void head_max_decode(float* c, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) c[i] = dec_order(reinterpret_cast<const unsigned*>(c)[i]) / kLog2e;
}

// One launch of features_kernel in mode MODE over rows of H heads (G query heads per W head).
template <class T, int D, int MODE>
bool launch_mode(const Plan& s, const T* X, const float* W, int Lo, int H, int G, float* phi, float* c,
                 hipStream_t st) {
  const int nh = s.B * H;
  if constexpr (std::is_same<T, bf16>::value) {
    if (s.m <= kFeatLdsM) {
      constexpr int R = 32 * kFeatLdsWaves;
      hipLaunchKernelGGL((features_kernel<T, D, MODE, true>), dim3((Lo + R - 1) / R, nh), dim3(64 * kFeatLdsWaves),
                         0, st, X, W, s.L, Lo, H, G, s.Hw, s.m, phi, c);
      return hipGetLastError() == hipSuccess;
    }
  }
  {
    constexpr int R = 32 * kFeatWaves;
    hipLaunchKernelGGL((features_kernel<T, D, MODE, false>), dim3((Lo + R - 1) / R, nh), dim3(64 * kFeatWaves), 0,
                       st, X, W, s.L, Lo, H, G, s.Hw, s.m, phi, c);
  }
  return hipGetLastError() == hipSuccess;
}

template <class T, int D>
favor_status run_features(const Plan& s, int side, const void* Xv, const float* W, float* phi, float* c, int Lo,
                          hipStream_t st) {
  const T* X = static_cast<const T*>(Xv);
  if (side == 0)
    return launch_mode<T, D, 0>(s, X, W, Lo, s.Hq, s.G, phi, c, st) ? FAVOR_OK : FAVOR_ERR_HIP;
  const int nh = s.B * s.Hkv;
  const int ib = (nh + 255) / 256;
  hipLaunchKernelGGL(head_max_init, dim3(ib), dim3(256), 0, st, reinterpret_cast<unsigned*>(c), nh);
  if (hipGetLastError() != hipSuccess) return FAVOR_ERR_HIP;
  if (!launch_mode<T, D, 1>(s, X, W, Lo, s.Hkv, 1, phi, c, st)) return FAVOR_ERR_HIP;
  if (!launch_mode<T, D, 2>(s, X, W, Lo, s.Hkv, 1, phi, c, st)) return FAVOR_ERR_HIP;
  hipLaunchKernelGGL(head_max_decode, dim3(ib), dim3(256), 0, st, c, nh);
  return hipGetLastError() == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}

}  // namespace

favor_status launch_features(const Plan& s, int side, const void* X, const float* W, float* phi, float* c,
                             hipStream_t st, int Lo) {
  if (Lo < s.L) Lo = s.L;
  if (s.dtype == FAVOR_BF16)
    return s.d == 64 ? run_features<bf16, 64>(s, side, X, W, phi, c, Lo, st)
                     : run_features<bf16, 128>(s, side, X, W, phi, c, Lo, st);
  return s.d == 64 ? run_features<float, 64>(s, side, X, W, phi, c, Lo, st)
                   : run_features<float, 128>(s, side, X, W, phi, c, Lo, st);
}

}  // namespace favor

extern "C" favor_status favor_features(const favor_problem* p, int32_t side, const void* X, const float* W,
                                       float* phi_out, float* c_out, void* stream) {
  favor::Plan s;
  const favor_status st = favor::make_plan(p, &s);
  if (st != FAVOR_OK) return st;
  if (side != 0 && side != 1) return FAVOR_ERR_INVALID_ARG;
  if (X == nullptr || W == nullptr || phi_out == nullptr || c_out == nullptr) return FAVOR_ERR_INVALID_ARG;
  return favor::launch_features(s, side, X, W, phi_out, c_out, static_cast<hipStream_t>(stream));
}
