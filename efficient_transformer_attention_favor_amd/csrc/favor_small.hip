// Bidirectional FAVOR+ for float32 problems on gfx950: the key side and the readout with
// the work spread over many short waves, for problems whose few heads would otherwise
// leave most of the chip idle behind long float32-MFMA chains.
//
// Method: "Rethinking Attention with Performers" (review page), "제안 방법": positive random
// features phi(x) = exp(W x - |x|^2 / 2) / sqrt(m) (the 1/sqrt(m) cancels in the ratio),
// attention in linear order out = phi(Q) S_v / phi(Q) S_1 with S = phi(K)^T [V, 1].
// Exponents are in log2 units (W scaled by log2 e); every contraction runs on
// v_mfma_f32_32x32x2_f32 (float32 operands, float32 accumulation).  The contraction index
// of the exponent products is split by lane half (lane group g supplies indices
// (d/2) g + s), so a lane holds one contiguous half of a key, query or W row and loads it
// straight into operand registers.
//
// Key side (small_kv_unit): per (kv head, position range, 32-feature tile), four waves
// taking the range's 32-position blocks in turn (the next block's rows in flight for
// d = 64).  Per block a wave forms E = K W^T - |k|^2/2 (C[key][feature], lane = feature),
// keeps a running maximum c_f per feature (moved lazily by kTau, the partial rescaled), and
// adds phi^T [V, 1] with the accumulator registers as the A operand and V read straight
// from global memory.  The four partials meet in LDS at the range's largest c_f.  Output
// per (head, range, tile): ps[D + 1][32] (value rows in natural order, row D the ones
// column), pc[32] = c_f.
//
// Readout (small_readout_body): per (kv head, 32-row tile of the G query heads' rows); wave
// w owns feature tiles w, w + NW, ... (NW = 4).  It merges the ranges' partials of its tile
// online (running maximum per feature, earlier sums rescaled), then
//   C[feature][query] = W Q^T + c_f,  M_w = the row maxima over its features,
//   phi = 2^(C - M_w),  num_w = S_v^T phi,  den_w = S_1 . phi,
// and the waves' partials meet in LDS: out = sum_w 2^(M_w - M) num_w / sum_w 2^(M_w - M) den_w.
//
// Launches: small_fused_f32_kernel runs both in one launch (workgroup b: key-side unit b,
// a grid barrier, then row tile b) when every unit and tile has a workgroup of its own on
// the device's compute units; otherwise small_kv_f32_kernel then small_readout_f32_kernel.
#include <hip/hip_runtime.h>

#include <math.h>

#include <stdlib.h>

#include <atomic>
#include <type_traits>

#include "favor_device.hpp"
#include "favor_ops.hpp"
#include "favor_plan.hpp"

namespace favor {

// ======================================================================================
// key side
// ======================================================================================
template <int D> struct SmallKv {
  static constexpr int NW = 4, NDT = D / 32;
  // LDS in floats: the waves' key row norms, their stabilisers, and the partials of waves
  // 1..3 for the merge
  static constexpr int NR = NW * 32, CS = NW * 32, RED = (NW - 1) * (NDT * 16 * 64 + 64);
  static constexpr size_t LDS = sizeof(float) * (NR + CS + RED);
};

// One key-side unit (kv head, range, 32-feature tile) on the workgroup's four waves; sm is
// SmallKv<D>::LDS bytes of LDS.  Every thread of the workgroup takes part (workgroup barriers).
template <int D>
__device__ __forceinline__ void small_kv_unit(float* sm, int id, const float* __restrict__ K,
                                              const float* __restrict__ V, const float* __restrict__ W, int L,
                                              int Hkv, int Hw, int m, int R, int T_ranges, float* __restrict__ ps,
                                              float* __restrict__ pc) {
  using Cfg = SmallKv<D>;
  constexpr int NW = Cfg::NW, NDT = Cfg::NDT, NS = D / 2;
  float(*Nr)[32] = reinterpret_cast<float(*)[32]>(sm);                       // -|k|^2/2 log2 e (-inf past the range)
  float(*Cs)[32] = reinterpret_cast<float(*)[32]>(sm + Cfg::NR);             // stabilisers, then the merged ones
  float(*Red)[NDT * 16 * 64 + 64] =
      reinterpret_cast<float(*)[NDT * 16 * 64 + 64]>(sm + Cfg::NR + Cfg::CS);  // partials of waves 1..3
  const int NFT = m / 32;
  const int ft = id % NFT;
  id /= NFT;
  const int t = id % T_ranges, bh = id / T_ranges, hkv = bh % Hkv;
  const int wave = threadIdx.x >> 6, l = lane_id(), col = l & 31, g = l >> 5;
  const float* Kh = K + (size_t)bh * L * D;
  const float* Vh = V + (size_t)bh * L * D;
  const float* Wr = W + ((size_t)(Hw == 1 ? 0 : hkv) * m + 32 * ft + col) * D;

  // W operand (B, lane = feature): step s carries contraction index (D/2) g + s, so each
  // lane holds one contiguous half of its feature's row (and of each key's row below)
  float wreg[NS];
#pragma unroll
  for (int c = 0; c < NS / 4; ++c) {
    const f32x4 w4 = *reinterpret_cast<const f32x4*>(Wr + (D / 2) * g + 4 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) wreg[4 * c + i] = w4[i] * kLog2e;
  }

  const int pb = t * R, pe = min(pb + R, L);
  f32x16 S[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) S[dt] = zero16();
  float s1 = 0.f, crun = -INFINITY;  // this lane's feature 32 ft + col (both lane halves)

  // One 32-key block in registers: the A operand (key col, half g of its row) and the V
  // operands (B, lane = value): step r contracts key 8 (r/4) + 4 g + r%4.  Rows past the
  // range are read clamped to its last row; their row bias is -inf, so their phi is 0.
  struct Blk {
    f32x4 k[NS / 4];
    float v[NDT][16];
  };
  auto fetch = [&](int p0, Blk& b) {
    const float* kr = Kh + (size_t)min(p0 + col, pe - 1) * D + (D / 2) * g;
#pragma unroll
    for (int c = 0; c < NS / 4; ++c) b.k[c] = *reinterpret_cast<const f32x4*>(kr + 4 * c);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = min(p0 + 8 * (r >> 2) + 4 * g + (r & 3), pe - 1);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) b.v[dt][r] = Vh[(size_t)key * D + 32 * dt + col];
    }
  };
  auto block = [&](int p0, const Blk& b) {
    {
      // |k|^2 of key col: each lane half sums its half of the row
      float n = 0.f;
#pragma unroll
      for (int c = 0; c < NS / 4; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) n = __builtin_fmaf(b.k[c][i], b.k[c][i], n);
      n = pair_sum(n);
      if (g == 0) Nr[wave][col] = p0 + col < pe ? -0.5f * kLog2e * n : -INFINITY;
    }
    asm volatile("" ::: "memory");
    // E = K W^T as two independent chains (even and odd steps)
    f32x16 e0 = zero16(), e1 = zero16();
#pragma unroll
    for (int c = 0; c < NS / 4; ++c) {
      e0 = mma(b.k[c][0], wreg[4 * c], e0);
      e1 = mma(b.k[c][1], wreg[4 * c + 1], e1);
      e0 = mma(b.k[c][2], wreg[4 * c + 2], e0);
      e1 = mma(b.k[c][3], wreg[4 * c + 3], e1);
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
      for (int r = 0; r < 16; ++r) S[dt] = mma(e0[r], b.v[dt][r], S[dt]);
    asm volatile("" ::: "memory");  // this block's LDS reads before the next block's writes
  };

  // the wave's blocks p0 = pb + 32 (wave + NW i); for d = 64 the next block's rows are in
  // flight while one is computed (d = 128 leaves no registers for a second block)
  int p0 = pb + 32 * wave;
  if constexpr (D == 64) {
    Blk cur, nxt;
    if (p0 < pe) fetch(p0, cur);
    for (; p0 < pe; p0 += 32 * NW) {
      if (p0 + 32 * NW < pe) fetch(p0 + 32 * NW, nxt);
      block(p0, cur);
      cur = nxt;
    }
  } else {
    for (; p0 < pe; p0 += 32 * NW) {
      Blk cur;
      fetch(p0, cur);
      block(p0, cur);
    }
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
  if (wave == 0) {
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
}

template <int D>
__global__ void __launch_bounds__(256) small_kv_f32_kernel(const float* __restrict__ K, const float* __restrict__ V,
                                                           const float* __restrict__ W, int L, int Hkv, int Hw,
                                                           int m, int R, int T_ranges, float* __restrict__ ps,
                                                           float* __restrict__ pc) {
  __shared__ __attribute__((aligned(16))) float sm[SmallKv<D>::LDS / sizeof(float)];
  small_kv_unit<D>(sm, blockIdx.x, K, V, W, L, Hkv, Hw, m, R, T_ranges, ps, pc);
}

// ======================================================================================
// readout
// ======================================================================================
template <int D> struct SmallRo {
  // waves at most (feature tiles beyond go round); four waves leave each one the whole
  // register file of its SIMD, which the merged partials and two accumulator chains need
  static constexpr int NW = 4;
  static constexpr int NDT = D / 32;
  // LDS: the waves' numerator partials, their (den, max) pairs
  static constexpr int RED = NW * NDT * 16 * 64;
  static constexpr size_t LDS_RED = sizeof(float) * RED + sizeof(float2) * NW * 32;
  // d = 64: the ranges' partials of a wave's feature tile staged in LDS by DMA before the
  // merge (up to kSmallRanges ranges: S rows, then the stabilisers), aliased with the above
  static constexpr bool STAGE = D == 64;
  static constexpr int SW = kSmallRanges * ((D + 1) * 32 + 32);  // floats per wave
  static constexpr size_t LDS_STAGE = STAGE ? sizeof(float) * NW * SW : 0;
  static constexpr size_t LDS = LDS_RED > LDS_STAGE ? LDS_RED : LDS_STAGE;
};

typedef __attribute__((address_space(3))) void lds_void_t;

// The readout of workgroup blk's 32-row tiles; nw waves (min(m / 32, 4)) own the feature
// tiles, further waves of the workgroup only join its barriers.  sm is SmallRo<D>::LDS
// bytes of LDS.  poison multiplies the reciprocal denominators (1, or NaN to mark the rows
// of a launch whose key-side partials are not known to be complete).
template <int D>
__device__ __forceinline__ void small_readout_body(float* sm, int blk, int nw, const float* __restrict__ Q,
                                                   const float* __restrict__ W, const float* __restrict__ ps,
                                                   const float* __restrict__ pc, float* __restrict__ out, int L,
                                                   int Hq, int Hkv, int Hw, int m, int T_ranges, int tiles_per_head,
                                                   float poison) {
  using Cfg = SmallRo<D>;
  constexpr int NWM = Cfg::NW, NDT = Cfg::NDT, NS = D / 2, NU = NDT * 4;
  float(*Red)[NDT * 16 * 64] = reinterpret_cast<float(*)[NDT * 16 * 64]>(sm);
  float2(*Dm)[32] = reinterpret_cast<float2(*)[32]>(sm + Cfg::RED);
  const int NFT = m / 32;
  const int bh = blk / tiles_per_head, tile0 = blk % tiles_per_head;
  const int b = bh / Hkv, hkv = bh % Hkv, G = Hq / Hkv;
  const int wave = threadIdx.x >> 6, l = lane_id(), col = l & 31, g = l >> 5;
  const size_t rows = (size_t)G * L;
  const float* Qb = Q + ((size_t)b * Hq + (size_t)hkv * G) * L * D;
  float* Ob = out + ((size_t)b * Hq + (size_t)hkv * G) * L * D;
  const float* Wh = W + (size_t)(Hw == 1 ? 0 : hkv) * m * D;

  // ---- per feature tile: the W operand and the ranges' partials merged at the largest c_f
  // (A operand: step s carries contraction index (D/2) g + s; register r of this lane group is
  // feature 8 (r/4) + 4 g + r%4 of the tile).
  float wv[NS], cf[16], sv[NDT][16], s1[16];
  // The ranges' partials of tile ft (S rows, then the stabilisers) into the wave's LDS
  // staging rows by DMA, 1 KB per instruction (the 128-byte tails by lanes 0..7).
  float* stg = sm + (size_t)wave * Cfg::SW;
  auto stage = [&](int ft) {
    constexpr int UB = (D + 1) * 32 * 4, NB = UB / 1024, TAIL = (UB - NB * 1024) / 16;
    const float* pcs = pc + (size_t)bh * T_ranges * m + 32 * ft;
    for (int t = 0; t < T_ranges; ++t) {
      const float* src = ps + (((size_t)bh * T_ranges + t) * NFT + ft) * (size_t)(D + 1) * 32;
      float* dst = stg + (size_t)t * (D + 1) * 32;
#pragma unroll
      for (int k = 0; k < NB; ++k)
        __builtin_amdgcn_global_load_lds((const void*)(src + 256 * k + 4 * l), (lds_void_t*)(dst + 256 * k), 16, 0, 0);
      if (l < TAIL)
        __builtin_amdgcn_global_load_lds((const void*)(src + 256 * NB + 4 * l), (lds_void_t*)(dst + 256 * NB), 16, 0, 0);
      if (l < 8)
        __builtin_amdgcn_global_load_lds((const void*)(pcs + (size_t)t * m + 4 * l),
                                         (lds_void_t*)(stg + kSmallRanges * (D + 1) * 32 + 32 * t), 16, 0, 0);
    }
  };
  auto load_w = [&](int ft) {
    const float* wr = Wh + (size_t)(32 * ft + col) * D + (D / 2) * g;
#pragma unroll
    for (int c = 0; c < NS / 4; ++c) {
      const f32x4 w4 = *reinterpret_cast<const f32x4*>(wr + 4 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[4 * c + i] = w4[i] * kLog2e;
    }
  };
  // the W operand of tile ft and the merge of its ranges' partials
  auto prep = [&](int ft, auto staged_tag) {
    constexpr bool STG = decltype(staged_tag)::value;
    load_w(ft);
    // Online merge over the ranges (running maximum per feature, earlier sums rescaled when
    // it rises), so the loads of TG ranges -- stabilisers and partials alike -- go out
    // together in one round (past the last range the last one is re-read with weight 0).
    constexpr int TG = D == 64 ? 4 : 2;
    const float* pch = pc + (size_t)bh * T_ranges * m + 32 * ft;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      cf[r] = -INFINITY;
      s1[r] = 0.f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) sv[dt][r] = 0.f;
    }
    for (int t0 = 0; t0 < T_ranges; t0 += TG) {
      f32x4 cv[TG][4], ov[TG][4], vv[TG][4][NDT];
#pragma unroll
      for (int u = 0; u < TG; ++u) {
        const int t = min(t0 + u, T_ranges - 1);
        const float* src = STG ? stg + (size_t)t * (D + 1) * 32
                               : ps + (((size_t)bh * T_ranges + t) * NFT + ft) * (size_t)(D + 1) * 32;
        const float* csrc = STG ? stg + kSmallRanges * (D + 1) * 32 + 32 * t : pch + (size_t)t * m;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          cv[u][r4] = *reinterpret_cast<const f32x4*>(csrc + 8 * r4 + 4 * g);
          ov[u][r4] = *reinterpret_cast<const f32x4*>(src + (size_t)D * 32 + 8 * r4 + 4 * g);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            vv[u][r4][dt] = *reinterpret_cast<const f32x4*>(src + (size_t)(32 * dt + col) * 32 + 8 * r4 + 4 * g);
        }
      }
#pragma unroll
      for (int u = 0; u < TG; ++u) {
        if (t0 + u >= T_ranges) break;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 4 * r4 + q;
            const float c = cv[u][r4][q], nm = fmaxf(cf[r], c);
            const float a = cf[r] == -INFINITY ? 0.f : fast_exp2(cf[r] - nm);
            const float b = fast_exp2(c - nm);
            cf[r] = nm;
            s1[r] = __builtin_fmaf(b, ov[u][r4][q], s1[r] * a);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) sv[dt][r] = __builtin_fmaf(b, vv[u][r4][dt][q], sv[dt][r] * a);
          }
      }
    }
  };
  // B operand of the exponents: query row0 + col, half g of its row (rows past the end are
  // read clamped to the last row and never stored); the first tile's rows are in flight
  // while the partials are merged
  f32x4 qv[NS / 4];
  auto load_q = [&](size_t row0) {
    const float* qr = Qb + min(row0 + col, rows - 1) * D + (D / 2) * g;
#pragma unroll
    for (int c = 0; c < NS / 4; ++c) qv[c] = *reinterpret_cast<const f32x4*>(qr + 4 * c);
  };
  if ((size_t)tile0 * 32 < rows) load_q((size_t)tile0 * 32);
  // one feature tile per wave: prepared once for all row tiles of the workgroup (for
  // d = 64 from the LDS-staged partials: every range's loads in one DMA round, no registers
  // held while they are in flight)
  const bool once = NFT <= nw;
  if (Cfg::STAGE && once && T_ranges <= kSmallRanges) {
    if (wave < NFT) stage(wave);
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));  // vmcnt(0): the DMA has landed
    __syncthreads();
    if (wave < NFT) prep(wave, std::true_type{});
  } else if (once && wave < NFT) {
    prep(wave, std::false_type{});
  }

  for (size_t tile = tile0; tile * 32 < rows; tile += tiles_per_head) {
    const size_t row0 = tile * 32;
    if (tile != (size_t)tile0) load_q(row0);
    __syncthreads();  // the previous tile's readers of Red, Dm are done

    f32x16 num[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) num[dt] = zero16();
    float den = 0.f, Mw = -INFINITY;
    for (int ft = wave; ft < NFT; ft += nw) {
      if (!once) prep(ft, std::false_type{});
      // ---- C[feature][query] = W Q^T + c_f (lane = query) ---------------------------------
      f32x16 e0 = zero16(), e1 = zero16();
#pragma unroll
      for (int c = 0; c < NS / 4; ++c) {
        e0 = mma(wv[4 * c], qv[c][0], e0);
        e1 = mma(wv[4 * c + 1], qv[c][1], e1);
        e0 = mma(wv[4 * c + 2], qv[c][2], e0);
        e1 = mma(wv[4 * c + 3], qv[c][3], e1);
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
    const float inv = poison / dd;
    const size_t row = row0 + col;
    if (row < rows && wave < nw) {
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

template <int D>
__global__ void __launch_bounds__(64 * SmallRo<D>::NW) small_readout_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ W, const float* __restrict__ ps,
    const float* __restrict__ pc, float* __restrict__ out, int L, int Hq, int Hkv, int Hw, int m, int T_ranges,
    int tiles_per_head) {
  __shared__ __attribute__((aligned(16))) float sm[SmallRo<D>::LDS / sizeof(float)];
  small_readout_body<D>(sm, blockIdx.x, blockDim.x >> 6, Q, W, ps, pc, out, L, Hq, Hkv, Hw, m, T_ranges,
                        tiles_per_head, 1.f);
}


// ======================================================================================
// one launch for small problems: the key-side units, a grid-wide barrier, the readout
// ======================================================================================
// Polls before a workgroup gives up waiting at the barrier (about a second); a launch whose
// workgroups are all resident passes it in microseconds.  The environment variable
// FAVOR_BARRIER_POLLS_FOR_TESTS lowers the limit, so a test can make the wait give up (the
// kernel still finishes; the rows of the workgroups that gave up are NaN).
constexpr int kBarrierPolls = 1 << 20;

// Grid-wide barrier for a launch of n <= 256 workgroups that are all resident at once.
// bar[0] is an epoch the workgroups read as e at the start of the launch (before any of
// them can pass the barrier); bar[1 + b] is workgroup b's arrival flag.  Workgroup b
// arrives by storing (e + 1) ^ tag in its flag and waits until every flag holds that value;
// workgroup 0 then moves the epoch to e + 1.  Flags left by an earlier launch hold another
// value (a replayed launch with the same tag has moved on by one epoch; a fresh workspace
// matches only by accident of 2^-64), so nothing needs clearing between calls.  No
// read-modify-write: each workgroup writes its own word.  Ordering: every wave waits for
// its stores, one agent-scope release (the XCD's L2 written back) precedes the flag, and
// the polling wave takes one agent-scope acquire after the last flag.  The wait is bounded:
// returns false if the flags did not all arrive within max_polls polls.
__device__ __forceinline__ unsigned long long barrier_epoch(const unsigned long long* bar) {
  return __hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool grid_barrier(unsigned long long* bar, unsigned long long epoch, unsigned tag,
                                             unsigned n, int max_polls) {
  __shared__ int ok_s;
  const unsigned long long want = (epoch + 1) ^ tag;
  // vmcnt(0): the wave's stores have reached the L2 before the release writes it back
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
  __syncthreads();
  if (threadIdx.x < 64) {
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_store(bar + 1 + blockIdx.x, want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // lane i watches flags i, i + 64, ...
    bool mine = true;
    for (unsigned j = threadIdx.x; j < n; j += 64) {
      int i = 0;
      bool seen = __hip_atomic_load(bar + 1 + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == want;
      while (!seen && i < max_polls) {
        __builtin_amdgcn_s_sleep(1);
        seen = __hip_atomic_load(bar + 1 + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == want;
        ++i;
      }
      mine = mine && seen;
    }
    const bool ok = !wave_any(!mine);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (threadIdx.x == 0) {
      ok_s = ok ? 1 : 0;
      if (blockIdx.x == 0 && ok) __hip_atomic_store(bar, epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  return ok_s != 0;
}

// Workgroup b runs key-side unit b (b < n_kv), waits for every unit, then reads out its
// 32-row tile (one tile per workgroup: tiles_per_head = all tiles of a head).  Rows of a
// launch whose barrier gave up are written as NaN.
template <int D>
__global__ void __launch_bounds__(256) small_fused_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ W, float* __restrict__ ps, float* __restrict__ pc, float* __restrict__ out,
    unsigned long long* __restrict__ bar, unsigned tag, int max_polls, int L, int Hq, int Hkv, int Hw, int m, int R,
    int T_ranges, int n_kv, int tiles_per_head, int n_ro) {
  constexpr size_t LDS = SmallKv<D>::LDS > SmallRo<D>::LDS ? SmallKv<D>::LDS : SmallRo<D>::LDS;
  __shared__ __attribute__((aligned(16))) float sm[LDS / sizeof(float)];
  const unsigned long long epoch = barrier_epoch(bar);
  for (int u = blockIdx.x; u < n_kv; u += gridDim.x) {
    small_kv_unit<D>(sm, u, K, V, W, L, Hkv, Hw, m, R, T_ranges, ps, pc);
    __syncthreads();  // LDS free for the next unit
  }
  const bool ok = grid_barrier(bar, epoch, tag, gridDim.x, max_polls);
  const int NFT = m / 32;
  const int nw = NFT < SmallRo<D>::NW ? NFT : SmallRo<D>::NW;
  for (int u = blockIdx.x; u < n_ro; u += gridDim.x) {
    small_readout_body<D>(sm, u, nw, Q, W, ps, pc, out, L, Hq, Hkv, Hw, m, T_ranges, tiles_per_head,
                          ok ? 1.f : __builtin_nanf(""));
    __syncthreads();
  }
}

// ======================================================================================
// launchers
// ======================================================================================
namespace {

// Compute units of the current device (0 if the query fails), cached per device.
int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// A fresh 32-bit tag per launch of the one-launch path (odd, mixed so that it is unlikely
// to match stale workspace contents).
unsigned next_barrier_tag() {
  static std::atomic<unsigned> counter{0};
  unsigned x = counter.fetch_add(1, std::memory_order_relaxed) * 0x9E3779B9u + 0x7F4A7C15u;
  x ^= x >> 16;
  x *= 0x85EBCA6Bu;
  x ^= x >> 13;
  return x | 1u;
}

}  // namespace

bool small_f32_path(const Plan& s) { return s.dtype == FAVOR_F32 && s.mode == FAVOR_BIDIRECTIONAL; }

// One launch when every key-side unit and every 32-row tile has a workgroup of its own and
// all of them can be resident at once on the current device (one per CU).
bool small_f32_fused(const Plan& s) {
  if (!small_f32_path(s)) return false;
  const long long kv_wg = (long long)s.BH * s.T * (s.m / 32);
  const long long n_ro = (long long)s.BH * (((long long)s.G * s.L + 31) / 32);
  const int cus = device_cu_count();
  const long long lim = cus < kCUs ? cus : kCUs;  // the workspace holds kCUs arrival flags
  return lim > 0 && kv_wg <= lim && n_ro <= lim;
}

favor_status launch_small_f32(const Plan& s, const float* Q, const float* K, const float* V, const float* W,
                              float* out, char* ws, hipStream_t st, const Marks& mk) {
  float* ps = reinterpret_cast<float*>(ws + s.off_gs);
  float* pc = reinterpret_cast<float*>(ws + s.off_gc);
  const int NFT = s.m / 32;
  if (!mk.mark(0, st)) return FAVOR_ERR_HIP;
  const unsigned kv_wg = (unsigned)(s.BH * s.T * NFT);
  const long long tiles = ((long long)s.G * s.L + 31) / 32;
  const long long n_ro = (long long)s.BH * tiles;
  if (small_f32_fused(s)) {
    const unsigned grid = (unsigned)(n_ro > (long long)kv_wg ? n_ro : (long long)kv_wg);
    unsigned long long* bar = reinterpret_cast<unsigned long long*>(ws + s.off_bar);
    const unsigned tag = next_barrier_tag();
    int polls = kBarrierPolls;
    if (const char* e = getenv("FAVOR_BARRIER_POLLS_FOR_TESTS")) {
      const long v = strtol(e, nullptr, 10);
      polls = v < 0 ? 0 : (v < kBarrierPolls ? (int)v : kBarrierPolls);
    }
    if (s.d == 64)
      hipLaunchKernelGGL(small_fused_f32_kernel<64>, dim3(grid), dim3(256), 0, st, Q, K, V, W, ps, pc, out, bar, tag,
                         polls, s.L, s.Hq, s.Hkv, s.Hw, s.m, s.R, s.T, (int)kv_wg, (int)tiles, (int)n_ro);
    else
      hipLaunchKernelGGL(small_fused_f32_kernel<128>, dim3(grid), dim3(256), 0, st, Q, K, V, W, ps, pc, out, bar,
                         tag, polls, s.L, s.Hq, s.Hkv, s.Hw, s.m, s.R, s.T, (int)kv_wg, (int)tiles, (int)n_ro);
    // one kernel: the key-side slot holds it, the readout slot is empty
    if (hipGetLastError() != hipSuccess || !mk.mark(1, st) || !mk.mark(2, st) || !mk.mark(3, st))
      return FAVOR_ERR_HIP;
    return FAVOR_OK;
  }
  if (s.d == 64)
    hipLaunchKernelGGL(small_kv_f32_kernel<64>, dim3(kv_wg), dim3(256), 0, st, K, V, W, s.L, s.Hkv, s.Hw, s.m, s.R,
                       s.T, ps, pc);
  else
    hipLaunchKernelGGL(small_kv_f32_kernel<128>, dim3(kv_wg), dim3(256), 0, st, K, V, W, s.L, s.Hkv, s.Hw, s.m,
                       s.R, s.T, ps, pc);
  if (hipGetLastError() != hipSuccess || !mk.mark(1, st) || !mk.mark(2, st)) return FAVOR_ERR_HIP;
  // about kReadoutTarget workgroups, one 32-row tile each at most
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
