// Bidirectional FAVOR+ for float32 problems on gfx950: the key side and the readout with
// the work spread over many short waves, for problems whose few heads would otherwise
// leave most of the chip idle behind long float32-MFMA chains.
//
// Method: "Rethinking Attention with Performers" (review page), "제안 방법": positive random
// features phi(x) = exp(W x - |x|^2 / 2) / sqrt(m) (the 1/sqrt(m) cancels in the ratio),
// attention in linear order out = phi(Q) S_v / phi(Q) S_1 with S = phi(K)^T [V, 1].
// Exponents are in log2 units (W scaled by log2 e); every contraction runs on
// v_mfma_f32_32x32x2_f32 (float32 operands, float32 accumulation).
//
// Key side (small_kv_f32_kernel): one workgroup per (kv head, position range, 32-feature
// tile); its four waves take the range's 32-position blocks in turn.  Per block a wave forms
// E = K W^T - |k|^2/2 (C[key][feature], lane = feature), keeps a running maximum c_f per
// feature (moved lazily by kTau, the partial rescaled), and adds phi^T [V, 1] with the
// accumulator registers as the A operand and V read straight from global memory.  The four
// partials meet in LDS at the range's largest c_f.  Output per (head, range, tile):
//   ps[D + 1][32] (value rows in natural order, row D the ones column), pc[32] = c_f.
//
// Readout (small_readout_f32_kernel): one workgroup per (kv head, 32-row tile of the G
// query heads' rows); wave w owns feature tiles w, w + NW, ... (NW = 4)  It merges the ranges'
// partials of its tiles into MFMA operands (S_f rescaled to the largest c_f), then
//   C[feature][query] = W Q^T + c_f,  M_w = the row maxima over its features,
//   phi = 2^(C - M_w),  num_w = S_v^T phi,  den_w = S_1 . phi,
// and the waves' partials meet in LDS: out = sum_w 2^(M_w - M) num_w / sum_w 2^(M_w - M) den_w.
#include <hip/hip_runtime.h>

#include <math.h>

#include "favor_device.hpp"
#include "favor_ops.hpp"
#include "favor_plan.hpp"

namespace favor {

// ======================================================================================
// key side
// ======================================================================================
template <int D>
__global__ void __launch_bounds__(256) small_kv_f32_kernel(const float* __restrict__ K, const float* __restrict__ V,
                                                           const float* __restrict__ W, int L, int Hkv, int Hw,
                                                           int m, int R, int T_ranges, float* __restrict__ ps,
                                                           float* __restrict__ pc) {
  constexpr int NW = 4, NDT = D / 32, LDK = D + 1, NS = D / 2;
  __shared__ float Kl[NW][32 * LDK];           // the wave's block of keys
  __shared__ float Nr[NW][32];                 // -|k|^2/2 log2 e of those keys (-inf past the range)
  __shared__ float Cs[NW][32];                 // the waves' stabilisers, then the merged ones
  __shared__ float Red[NW - 1][NDT * 16 * 64 + 64];  // partials of waves 1..3
  const int NFT = m / 32;
  int id = blockIdx.x;
  const int ft = id % NFT;
  id /= NFT;
  const int t = id % T_ranges, bh = id / T_ranges, hkv = bh % Hkv;
  const int wave = threadIdx.x >> 6, l = lane_id(), col = l & 31, g = l >> 5;
  const float* Kh = K + (size_t)bh * L * D;
  const float* Vh = V + (size_t)bh * L * D;
  const float* Wr = W + ((size_t)(Hw == 1 ? 0 : hkv) * m + 32 * ft + col) * D;

  // W operand (B, lane = feature): step s carries contraction index 2 s + g
  float wreg[NS];
#pragma unroll
  for (int c = 0; c < D / 4; ++c) {
    const f32x4 w4 = *reinterpret_cast<const f32x4*>(Wr + 4 * c);
    wreg[2 * c] = (g == 0 ? w4[0] : w4[1]) * kLog2e;
    wreg[2 * c + 1] = (g == 0 ? w4[2] : w4[3]) * kLog2e;
  }

  const int pb = t * R, pe = min(pb + R, L);
  f32x16 S[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) S[dt] = zero16();
  float s1 = 0.f, crun = -INFINITY;  // this lane's feature 32 ft + col (both lane halves)
  float* kl = Kl[wave];
  for (int p0 = pb + 32 * wave; p0 < pe; p0 += 32 * NW) {
    // V operands of the block (B, lane = value): step r contracts key 8 (r/4) + 4 g + r%4;
    // rows past the range are read clamped to its last row (their phi is 0)
    float vop[NDT][16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = min(p0 + 8 * (r >> 2) + 4 * g + (r & 3), pe - 1);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vop[dt][r] = Vh[(size_t)key * D + 32 * dt + col];
    }
    // keys of the block into the wave's LDS rows (rows past the range read as zero)
#pragma unroll
    for (int j = 0; j < D / 8; ++j) {
      const int c = l + 64 * j, row = c / (D / 4), c4 = (c % (D / 4)) * 4;
      const f32x4 v = p0 + row < pe ? *reinterpret_cast<const f32x4*>(Kh + (size_t)(p0 + row) * D + c4)
                                     : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) kl[row * LDK + c4 + i] = v[i];
    }
    asm volatile("" ::: "memory");  // the wave's LDS writes above before its reads below
    {
      // |k|^2 of key col: each lane half sums half of the row
      float n = 0.f;
#pragma unroll 16
      for (int k = 0; k < D / 2; ++k) {
        const float x = kl[col * LDK + g * (D / 2) + k];
        n = __builtin_fmaf(x, x, n);
      }
      n = pair_sum(n);
      if (g == 0) Nr[wave][col] = p0 + col < pe ? -0.5f * kLog2e * n : -INFINITY;
    }
    asm volatile("" ::: "memory");
    // E = K W^T as two independent chains (even and odd steps)
    f32x16 e0 = zero16(), e1 = zero16();
#pragma unroll
    for (int s = 0; s < NS; s += 2) {
      e0 = mma(kl[col * LDK + 2 * s + g], wreg[s], e0);
      e1 = mma(kl[col * LDK + 2 * s + 2 + g], wreg[s + 1], e1);
    }
    // row bias -|k|^2/2 of key 8 (r/4) + 4 g + r%4, block maximum per feature
    float mx = -INFINITY;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 nb = *reinterpret_cast<const f32x4*>(&Nr[wave][8 * r4 + 4 * g]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        e0[4 * r4 + q] += e1[4 * r4 + q] + nb[q];
        mx = fmaxf(mx, e0[4 * r4 + q]);
      }
    }
    mx = pair_max(mx);
    // c_f: set by the first block, moved when a block passes it by more than kTau
    if (crun == -INFINITY || mx > crun + kTau) {
      const float fct = crun == -INFINITY ? 0.f : fast_exp2(crun - mx);
      crun = mx;
      s1 *= fct;
      if (g == 0) Cs[wave][col] = fct;
    } else if (g == 0) {
      Cs[wave][col] = 1.f;
    }
    asm volatile("" ::: "memory");
    // S[feature][value] is C[feature][value]: lane = value, register r = feature 8 (r/4) + 4 g + r%4
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 f = *reinterpret_cast<const f32x4*>(&Cs[wave][8 * r4 + 4 * g]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) S[dt][4 * r4 + q] *= f[q];
    }
    float bs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      e0[r] = fast_exp2(e0[r] - crun);
      bs += e0[r];
    }
    s1 += pair_sum(bs);
    // S += phi^T [V]
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) S[dt] = mma(e0[r], vop[dt][r], S[dt]);
    asm volatile("" ::: "memory");  // this block's LDS reads before the next block's writes
  }

  // ---- the four partials meet at the range's largest c_f ------------------------------
  if (g == 0) Cs[wave][col] = crun;
  __syncthreads();
  float cm = Cs[0][col];
#pragma unroll
  for (int w = 1; w < NW; ++w) cm = fmaxf(cm, Cs[w][col]);
  s1 *= crun == -INFINITY ? 0.f : fast_exp2(crun - cm);
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    f32x4 own = *reinterpret_cast<const f32x4*>(&Cs[wave][8 * r4 + 4 * g]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float c = Cs[0][8 * r4 + 4 * g + q];
#pragma unroll
      for (int w = 1; w < NW; ++w) c = fmaxf(c, Cs[w][8 * r4 + 4 * g + q]);
      const float f = own[q] == -INFINITY ? 0.f : fast_exp2(own[q] - c);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) S[dt][4 * r4 + q] *= f;
    }
  }
  if (wave > 0) {
    float* dst = Red[wave - 1];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<f32x4*>(dst + ((dt * 4 + r4) * 64 + l) * 4) =
            f32x4{S[dt][4 * r4], S[dt][4 * r4 + 1], S[dt][4 * r4 + 2], S[dt][4 * r4 + 3]};
    dst[NDT * 16 * 64 + l] = s1;
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < NW; ++w) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(&Red[w - 1][((dt * 4 + r4) * 64 + l) * 4]);
#pragma unroll
        for (int q = 0; q < 4; ++q) S[dt][4 * r4 + q] += v[q];
      }
    s1 += Red[w - 1][NDT * 16 * 64 + l];
  }
  const size_t unit = ((size_t)bh * T_ranges + t) * NFT + ft;
  float* out_s = ps + unit * (size_t)(D + 1) * 32;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *reinterpret_cast<f32x4*>(out_s + (size_t)(32 * dt + col) * 32 + 8 * r4 + 4 * g) =
          f32x4{S[dt][4 * r4], S[dt][4 * r4 + 1], S[dt][4 * r4 + 2], S[dt][4 * r4 + 3]};
  if (g == 0) {
    out_s[(size_t)D * 32 + col] = s1;
    pc[((size_t)bh * T_ranges + t) * m + 32 * ft + col] = cm;
  }
}

// ======================================================================================
// readout
// ======================================================================================
template <int D> struct SmallRo {
  // waves at most (feature tiles beyond go round); four waves leave each one the whole
  // register file of its SIMD, which the merged partials and two accumulator chains need
  static constexpr int NW = 4;
  static constexpr int NDT = D / 32;
  static constexpr int LDQ = D + 1;
};

template <int D>
__global__ void __launch_bounds__(64 * SmallRo<D>::NW) small_readout_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ W, const float* __restrict__ ps,
    const float* __restrict__ pc, float* __restrict__ out, int L, int Hq, int Hkv, int Hw, int m, int T_ranges,
    int tiles_per_head) {
  using Cfg = SmallRo<D>;
  constexpr int NWM = Cfg::NW, NDT = Cfg::NDT, LDQ = Cfg::LDQ, NS = D / 2, NU = NDT * 4;
  __shared__ float Ql[32 * LDQ];
  __shared__ float Red[NWM][NDT * 16 * 64];
  __shared__ float2 Dm[NWM][32];
  const int NFT = m / 32;
  const int nw = blockDim.x >> 6;  // waves: min(NFT, NWM)
  const int bh = blockIdx.x / tiles_per_head, tile0 = blockIdx.x % tiles_per_head;
  const int b = bh / Hkv, hkv = bh % Hkv, G = Hq / Hkv;
  const int wave = threadIdx.x >> 6, l = lane_id(), col = l & 31, g = l >> 5;
  const size_t rows = (size_t)G * L;
  const float* Qb = Q + ((size_t)b * Hq + (size_t)hkv * G) * L * D;
  float* Ob = out + ((size_t)b * Hq + (size_t)hkv * G) * L * D;
  const float* Wh = W + (size_t)(Hw == 1 ? 0 : hkv) * m * D;

  // ---- per feature tile: the W operand and the ranges' partials merged at the largest c_f
  // (A operand: step s carries contraction index 2 s + g; register r of this lane group is
  // feature 8 (r/4) + 4 g + r%4 of the tile).  The loads of TG ranges and RB register groups
  // go out together (past the last range the last one is re-read with weight 0).
  float wv[NS], cf[16], sv[NDT][16], s1[16];
  auto prep = [&](int ft) {
    const float* wr = Wh + (size_t)(32 * ft + col) * D;
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      const f32x4 w4 = *reinterpret_cast<const f32x4*>(wr + 4 * c);
      wv[2 * c] = g == 0 ? w4[0] : w4[1];
      wv[2 * c + 1] = g == 0 ? w4[2] : w4[3];
    }
    constexpr int TG = 4, RB = D == 64 ? 4 : 1;
    const float* pch = pc + (size_t)bh * T_ranges * m + 32 * ft;
#pragma unroll
    for (int r = 0; r < 16; ++r) cf[r] = -INFINITY;
    for (int t0 = 0; t0 < T_ranges; t0 += TG) {
      f32x4 cv[TG][4];
#pragma unroll
      for (int u = 0; u < TG; ++u)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          cv[u][r4] = *reinterpret_cast<const f32x4*>(pch + (size_t)min(t0 + u, T_ranges - 1) * m + 8 * r4 + 4 * g);
#pragma unroll
      for (int u = 0; u < TG; ++u)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
          for (int q = 0; q < 4; ++q) cf[4 * r4 + q] = fmaxf(cf[4 * r4 + q], cv[u][r4][q]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s1[r] = 0.f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) sv[dt][r] = 0.f;
    }
    for (int t0 = 0; t0 < T_ranges; t0 += TG) {
#pragma unroll
      for (int rb = 0; rb < 4; rb += RB) {
        f32x4 cv[RB][TG], ov[RB][TG], vv[RB][TG][NDT];
#pragma unroll
        for (int j = 0; j < RB; ++j)
#pragma unroll
          for (int u = 0; u < TG; ++u) {
            const int r4 = rb + j, t = min(t0 + u, T_ranges - 1);
            const float* src = ps + (((size_t)bh * T_ranges + t) * NFT + ft) * (size_t)(D + 1) * 32;
            cv[j][u] = *reinterpret_cast<const f32x4*>(pch + (size_t)t * m + 8 * r4 + 4 * g);
            ov[j][u] = *reinterpret_cast<const f32x4*>(src + (size_t)D * 32 + 8 * r4 + 4 * g);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
              vv[j][u][dt] = *reinterpret_cast<const f32x4*>(src + (size_t)(32 * dt + col) * 32 + 8 * r4 + 4 * g);
          }
#pragma unroll
        for (int j = 0; j < RB; ++j)
#pragma unroll
          for (int u = 0; u < TG; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int r = 4 * (rb + j) + q;
              const float f = t0 + u < T_ranges ? fast_exp2(cv[j][u][q] - cf[r]) : 0.f;
              s1[r] = __builtin_fmaf(f, ov[j][u][q], s1[r]);
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt) sv[dt][r] = __builtin_fmaf(f, vv[j][u][dt][q], sv[dt][r]);
            }
      }
    }
  };
  // one feature tile per wave: prepared once for all row tiles of the workgroup
  const bool once = NFT <= nw;
  if (once) prep(wave);

  for (size_t tile = tile0; tile * 32 < rows; tile += tiles_per_head) {
    const size_t row0 = tile * 32;
    __syncthreads();  // the previous tile's readers of Ql, Red, Dm are done
    // the tile's queries (rows past the end read as zero)
    for (int c = threadIdx.x; c < 32 * (D / 4); c += blockDim.x) {
      const int row = c / (D / 4), c4 = (c % (D / 4)) * 4;
      const f32x4 v = row0 + row < rows ? *reinterpret_cast<const f32x4*>(Qb + (row0 + row) * D + c4)
                                         : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) Ql[row * LDQ + c4 + i] = v[i];
    }
    __syncthreads();

    f32x16 num[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) num[dt] = zero16();
    float den = 0.f, Mw = -INFINITY;
    for (int ft = wave; ft < NFT; ft += nw) {
      if (!once) prep(ft);
      // ---- C[feature][query] = W Q^T + c_f (lane = query) ---------------------------------
      f32x16 e0 = zero16(), e1 = zero16();
#pragma unroll
      for (int s2 = 0; s2 < NS; s2 += 2) {
        e0 = mma(wv[s2] * kLog2e, Ql[col * LDQ + 2 * s2 + g], e0);
        e1 = mma(wv[s2 + 1] * kLog2e, Ql[col * LDQ + 2 * s2 + 2 + g], e1);
      }
      float mt = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        e0[r] += e1[r] + cf[r];
        mt = fmaxf(mt, e0[r]);
      }
      mt = pair_max(mt);
      // the wave's row maxima over its tiles so far; earlier tiles' terms rescale
      const float mn = fmaxf(Mw, mt);
      const float fo = Mw == -INFINITY ? 0.f : fast_exp2(Mw - mn);
      Mw = mn;
      den *= fo;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) num[dt][r] *= fo;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        e0[r] = fast_exp2(e0[r] - Mw);
        den = __builtin_fmaf(e0[r], s1[r], den);
      }
      // num[value][query] += S_v^T phi: step r contracts feature 8 (r/4) + 4 g + r%4
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) num[dt] = mma(sv[dt][r], e0[r], num[dt]);
    }
    den = pair_sum(den);
    // ---- the waves' partials meet -------------------------------------------------------
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<f32x4*>(&Red[wave][((dt * 4 + r4) * 64 + l) * 4]) =
            f32x4{num[dt][4 * r4], num[dt][4 * r4 + 1], num[dt][4 * r4 + 2], num[dt][4 * r4 + 3]};
    if (g == 0) Dm[wave][col] = float2{den, Mw};
    __syncthreads();
    float M = -INFINITY;
    for (int w = 0; w < nw; ++w) M = fmaxf(M, Dm[w][col].y);
    float dd = 0.f;
    for (int w = 0; w < nw; ++w) {
      const float2 dm = Dm[w][col];
      dd = __builtin_fmaf(dm.y == -INFINITY ? 0.f : fast_exp2(dm.y - M), dm.x, dd);
    }
    const float inv = 1.f / dd;
    const size_t row = row0 + col;
    if (row < rows) {
      // group u: value tile u / 4, registers 4 (u % 4) .. = values 32 (u / 4) + 8 (u % 4) + 4 g ..
      for (int u = wave; u < NU; u += nw) {
        const int dt = u >> 2, r4 = u & 3;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < nw; ++w) {
          const float2 dm = Dm[w][col];
          const float sc = dm.y == -INFINITY ? 0.f : fast_exp2(dm.y - M);
          const f32x4 v = *reinterpret_cast<const f32x4*>(&Red[w][((dt * 4 + r4) * 64 + l) * 4]);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(sc, v[q], acc[q]);
        }
        *reinterpret_cast<f32x4*>(Ob + row * D + 32 * dt + 8 * r4 + 4 * g) =
            f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
      }
    }
  }
}

// ======================================================================================
// launchers
// ======================================================================================
bool small_f32_path(const Plan& s) { return s.dtype == FAVOR_F32 && s.mode == FAVOR_BIDIRECTIONAL; }

favor_status launch_small_f32(const Plan& s, const float* Q, const float* K, const float* V, const float* W,
                              float* out, char* ws, hipStream_t st, const Marks& mk) {
  float* ps = reinterpret_cast<float*>(ws + s.off_gs);
  float* pc = reinterpret_cast<float*>(ws + s.off_gc);
  const int NFT = s.m / 32;
  if (!mk.mark(0, st)) return FAVOR_ERR_HIP;
  const unsigned kv_wg = (unsigned)(s.BH * s.T * NFT);
  if (s.d == 64)
    hipLaunchKernelGGL(small_kv_f32_kernel<64>, dim3(kv_wg), dim3(256), 0, st, K, V, W, s.L, s.Hkv, s.Hw, s.m, s.R,
                       s.T, ps, pc);
  else
    hipLaunchKernelGGL(small_kv_f32_kernel<128>, dim3(kv_wg), dim3(256), 0, st, K, V, W, s.L, s.Hkv, s.Hw, s.m,
                       s.R, s.T, ps, pc);
  if (hipGetLastError() != hipSuccess || !mk.mark(1, st) || !mk.mark(2, st)) return FAVOR_ERR_HIP;
  // about kReadoutTarget workgroups, one 32-row tile each at most
  const long long tiles = ((long long)s.G * s.L + 31) / 32;
  long long per_head = (2LL * kReadoutTarget + s.BH - 1) / s.BH;
  if (per_head > tiles) per_head = tiles;
  const int nwm = s.d == 64 ? SmallRo<64>::NW : SmallRo<128>::NW;
  const int nw = NFT < nwm ? NFT : nwm;
  const dim3 grid((unsigned)(s.BH * per_head)), block(64 * nw);
  if (s.d == 64)
    hipLaunchKernelGGL(small_readout_f32_kernel<64>, grid, block, 0, st, Q, W, ps, pc, out, s.L, s.Hq, s.Hkv, s.Hw,
                       s.m, s.T, (int)per_head);
  else
    hipLaunchKernelGGL(small_readout_f32_kernel<128>, grid, block, 0, st, Q, W, ps, pc, out, s.L, s.Hq, s.Hkv, s.Hw,
                       s.m, s.T, (int)per_head);
  if (hipGetLastError() != hipSuccess || !mk.mark(3, st)) return FAVOR_ERR_HIP;
  return FAVOR_OK;
}

}  // namespace favor
