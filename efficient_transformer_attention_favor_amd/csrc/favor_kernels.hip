// FAVOR+ attention forward for MI355X (gfx950): HIP kernels and the C ABI entry points.
//
// Method: "Rethinking Attention with Performers" (review page), sections "요약" and
// "제안 방법": softmax attention is replaced by positive random features,
//   phi(x) = exp(W x - |x|^2/2 - c) / sqrt(m),
// evaluated in linear order, out_i = phi(q_i) S_v / phi(q_i) S_1 with S = phi(K)^T [V, 1]
// (bidirectional) or S restricted to positions j <= i (causal).  Constants c and 1/sqrt(m)
// cancel between numerator and denominator and are chosen for range only.
//
// Kernels (exponents are kept in log2 units: W is scaled by log2(e) on load):
//   kv_summary   keys/values of one kv head, one position range per workgroup: per wave a
//                slice of 64 features; phi(K_blk) = exp2(K_blk W^T - |k|^2 log2e / 2 - c_f)
//                on the MFMA (the bias enters as one extra MFMA), then S += phi^T [V, 1].
//                c_f is a per-feature running maximum, moved lazily (kTau).
//   kv_combine   bidirectional: S = sum_t 2^(c_t,f - c_f) S_t over the position ranges.
//   readout      bidirectional: per query tile, phi(Q) W-contraction on the MFMA with a
//                running row maximum, then out^T = S^T phi(Q)^T and the division.
//   causal_scan  causal: exclusive prefix of the per-segment summaries, all rescaled to a
//                global per-head stabiliser.
//   causal_chunk causal: per segment, 32-position blocks in order with the carried summary
//                in registers (features split over the waves), the intra-block triangle on
//                the MFMA, and a cross-wave sum of the per-wave partial outputs.
#include <hip/hip_runtime.h>

#include <math.h>

#include "favor_device.hpp"
#include "favor_plan.hpp"

namespace favor {

template <class T> struct Ld;
template <> struct Ld<bf16> {
  template <int D> static constexpr int K = D + 8;     // natural-operand rows (b128 reads)
  template <int D> static constexpr int V = D + 16;    // transposed-operand rows (tr reads)
};
template <> struct Ld<float> {
  template <int D> static constexpr int K = D + 1;
  template <int D> static constexpr int V = D + 4;
};

// Stage rows [p0, p0+32) of a [L][D] tensor into LDS (zero rows past L).  Value tiles get
// the column permutation vperm_inv within every 32-column tile.
template <class T, int D, bool PERMUTE>
__device__ __forceinline__ void stage_rows(T* dst, int ld, const T* src, int p0, int L) {
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = D / EPC;         // chunks per row
  for (int c = threadIdx.x; c < 32 * CPR; c += blockDim.x) {
    const int row = c / CPR, c0 = (c % CPR) * EPC;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (p0 + row < L) v = *reinterpret_cast<const f32x4*>(src + (size_t)(p0 + row) * D + c0);
    T* drow = dst + row * ld;
    if (!PERMUTE) {
      if (sizeof(T) == 2) {  // bf16 row strides keep 8-byte alignment
        *reinterpret_cast<float2*>(drow + c0) = float2{v[0], v[1]};
        *reinterpret_cast<float2*>(drow + c0 + EPC / 2) = float2{v[2], v[3]};
      } else {
        float* d = reinterpret_cast<float*>(drow + c0);
        d[0] = v[0];
        d[1] = v[1];
        d[2] = v[2];
        d[3] = v[3];
      }
    } else {
      const int tile = c0 & ~31;
      // EPC/2 consecutive columns stay consecutive under vperm_inv (blocks of 4)
      if (sizeof(T) == 2) {
        *reinterpret_cast<float2*>(drow + tile + vperm_inv(c0 & 31)) = float2{v[0], v[1]};
        *reinterpret_cast<float2*>(drow + tile + vperm_inv((c0 & 31) + 4)) = float2{v[2], v[3]};
      } else {
        float* d = reinterpret_cast<float*>(drow + tile + vperm_inv(c0 & 31));
        d[0] = v[0];
        d[1] = v[1];
        d[2] = v[2];
        d[3] = v[3];
      }
    }
  }
}

// ======================================================================================
// kv_summary: per (position range t, kv head bh) the partial summary
//   S_t[f][c] = sum_{p in range} 2^(E_pf - c_f) [V, 1][p][c],
//   E_pf = log2e (w_f . k_p - |k_p|^2 / 2),
// stored fragment-native: tile (ft, ct) of 32 features x 32 value columns as
// [16 registers][64 lanes] floats; register r / lane l holds feature 32 ft + 8(r/4) +
// 4(l/32) + r%4 and value column 32 ct + vperm(l%32) (the ones column is ct = d/32, lane 0).
// ======================================================================================
template <class T, int D>
__global__ void __launch_bounds__(256) kv_summary_kernel(const T* __restrict__ K,
                                                         const T* __restrict__ V,
                                                         const float* __restrict__ W, int L,
                                                         int Hkv, int Hw, int m, int R, int T_ranges,
                                                         float* __restrict__ part_s,
                                                         float* __restrict__ part_c) {
  using P = Prec<T>;
  using frag = typename P::frag;
  constexpr int NKC = D / P::KS;
  constexpr int NDT = D / 32 + 1;
  constexpr int LDK = Ld<T>::template K<D>;
  constexpr int LDV = Ld<T>::template V<D>;
  __shared__ __attribute__((aligned(16))) T Kl[32 * LDK];
  __shared__ __attribute__((aligned(16))) T Vl[32 * LDV];

  const int t = blockIdx.x, bh = blockIdx.y, hkv = bh % Hkv;
  const int wave = threadIdx.x >> 6, l = lane_id(), col = l & 31, g = l >> 5;
  // Up to 4 waves (256 features) per workgroup.  A wave past num_features (m not a
  // multiple of 256) mirrors the first slice so the workgroup barriers stay uniform, and
  // stores nothing.
  const bool active = (int)(blockIdx.z * 4 + wave) * 64 < m;
  const int f0 = active ? (blockIdx.z * 4 + wave) * 64 : 0;
  const float* Wh = W + (size_t)(Hw == 1 ? 0 : hkv) * m * D;
  const T* Kh = K + (size_t)bh * L * D;
  const T* Vh = V + (size_t)bh * L * D;

  // W^T as the B operand: column = feature f0 + 32 nt + col.
  frag wf[2][P::NSPLIT][NKC];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      frag tmp[P::NSPLIT];
      load_w_frag(Wh + (size_t)(f0 + 32 * nt + col) * D, kc, g, tmp);
#pragma unroll
      for (int s = 0; s < P::NSPLIT; ++s) wf[nt][s][kc] = tmp[s];
    }

  float cst[2] = {0.f, 0.f};  // stabiliser of this lane's feature (log2 units)
  frag biasB[2] = {bias_cols(0.f, g, frag{}), bias_cols(0.f, g, frag{})};
  f32x16 S[2][NDT];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) S[nt][dt] = zero16();

  frag ones = zero_frag(frag{});
  if (col == 0) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int j = 0; j < 8; ++j) ones[j] = (bf16)1.f;
    } else {
      ones = 1.f;
    }
  }

  const int p_begin = t * R;
  const int p_end = min(p_begin + R, L);
  bool first = true;
  for (int p0 = p_begin; p0 < p_end; p0 += 32) {
    __syncthreads();
    stage_rows<T, D, false>(Kl, LDK, Kh, p0, L);
    stage_rows<T, D, true>(Vl, LDV, Vh, p0, L);
    __syncthreads();

    // K block as the A operand (row = key col), |k|^2 -> bias operand.
    frag kf[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) kf[kc] = load_frag_k(Kl + col * LDK, kc, g);
    float nrm = sumsq(kf);
    nrm += partner32(nrm);
    const frag biasA = bias_rows(0.5f * kLog2e * nrm, g, frag{});

    f32x16 c1[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      c1[nt] = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int s = 0; s < P::NSPLIT; ++s) c1[nt] = mma(kf[kc], wf[nt][s][kc], c1[nt]);
      c1[nt] = mma(biasA, biasB[nt], c1[nt]);
    }
    if (p0 + 32 > L) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (p0 + 8 * (r >> 2) + 4 * g + (r & 3) >= L) c1[nt][r] = -INFINITY;
    }

    // Running per-feature maximum, moved when a block exceeds it by more than kTau.
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mx = c1[nt][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, c1[nt][r]);
      mx = fmaxf(mx, partner32(mx));
      float shift = 0.f;
      if (mx != -INFINITY && (first || mx > kTau)) shift = mx;
      if (wave_any(shift != 0.f)) {
        cst[nt] += shift;
#pragma unroll
        for (int r = 0; r < 16; ++r) c1[nt][r] -= shift;
        biasB[nt] = bias_cols(cst[nt], g, frag{});
        if (!first) {
          const float fct = fast_exp2(-shift);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float fr = __shfl(fct, 8 * (r >> 2) + 4 * g + (r & 3));
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) S[nt][dt][r] *= fr;
          }
        }
      }
    }
    first = false;

    // phi^T as the A operand (row = feature, contraction = key), then S += phi^T [V, 1].
    frag pa[2][P::NF32];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x16 e;
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = fast_exp2(c1[nt][r]);
      acc_to_frags(e, pa[nt]);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int h = 0; h < P::NF32; ++h) {
        const frag vb = dt < NDT - 1 ? lds_frag_rows(Vl, LDV, 0, 32 * dt, h) : ones;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) S[nt][dt] = mma(pa[nt][h], vb, S[nt][dt]);
      }
  }

  if (!active) return;
  const size_t base = ((size_t)bh * T_ranges + t) * (size_t)m * (D + 32);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int ft = f0 / 32 + nt;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      float* dst = part_s + base + (size_t)(ft * NDT + dt) * 1024;
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[r * 64 + l] = S[nt][dt][r];
    }
    if (g == 0) part_c[((size_t)bh * T_ranges + t) * m + f0 + 32 * nt + col] = cst[nt];
  }
}

// ======================================================================================
// kv_combine (bidirectional): S[f] = sum_t 2^(c_t,f - c_f) S_t[f], c_f = max_t c_t,f.
// Grid (m/32 feature tiles, B*Hkv).  Fixed summation order t = 0, 1, ...
// ======================================================================================
__global__ void __launch_bounds__(256) kv_combine_kernel(const float* __restrict__ part_s,
                                                         const float* __restrict__ part_c, int T_ranges,
                                                         int m, int NDT, float* __restrict__ S_out,
                                                         float* __restrict__ c_out) {
  const int ft = blockIdx.x, bh = blockIdx.y;
  const size_t tile_elems = (size_t)m * NDT * 32;
  for (int e = threadIdx.x; e < NDT * 1024; e += blockDim.x) {
    const int r = (e & 1023) >> 6, l = e & 63;
    const int f = 32 * ft + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
    const float* pc = part_c + (size_t)bh * T_ranges * m + f;
    float cm = -INFINITY;
    for (int t = 0; t < T_ranges; ++t) cm = fmaxf(cm, pc[(size_t)t * m]);
    const size_t off = (size_t)ft * NDT * 1024 + e;
    const float* ps = part_s + (size_t)bh * T_ranges * tile_elems + off;
    float acc = 0.f;
    for (int t = 0; t < T_ranges; ++t) acc += fast_exp2(pc[(size_t)t * m] - cm) * ps[(size_t)t * tile_elems];
    S_out[(size_t)bh * tile_elems + off] = acc;
    if (e < 1024 && (l & 31) == 0) c_out[(size_t)bh * m + f] = cm;
  }
}

// ======================================================================================
// readout (bidirectional).  Grid (workgroups per kv head, B*Hkv), 4 waves; each wave owns
// 32 query rows per step.  The G query heads of a kv head are G*L contiguous rows.
// LDS holds W (hi/lo) and S^T (rows: value columns in vperm order, then the ones row;
// features of each 32-tile reordered so one lane's 8 operand values are contiguous) for
// a pass of MP features; more than one pass re-stages them per query tile.
// ======================================================================================
template <class T, int D> struct ReadoutCfg;
template <int D> struct ReadoutCfg<bf16, D> {
  static constexpr int MP = D == 64 ? 256 : 128;
  static constexpr int LDW = D + 8;
  static constexpr int LDS = MP + 8;
};
template <int D> struct ReadoutCfg<float, D> {
  static constexpr int MP = D == 64 ? 128 : 64;
  static constexpr int LDW = D + 1;
  static constexpr int LDS = MP + 1;
};

// position of feature fi (0..31 within a tile) in the S^T LDS row
template <class T> __device__ __forceinline__ int s_pos(int fi);
template <> __device__ __forceinline__ int s_pos<bf16>(int fi) {
  // lane group g, operand h, slot j hold feature 16h + 8(j/4) + 4g + j%4 at 16h + 8g + j
  const int h = fi >> 4, j4 = (fi >> 3) & 1, g = (fi >> 2) & 1, j = fi & 3;
  return 16 * h + 8 * g + 4 * j4 + j;
}
template <> __device__ __forceinline__ int s_pos<float>(int fi) { return fi; }

__device__ __forceinline__ bf16x8 s_frag(const bf16* Sl, int ld, int row, int ft, int h, int g) {
  return *reinterpret_cast<const bf16x8*>(Sl + row * ld + 32 * ft + 16 * h + 8 * g);
}
__device__ __forceinline__ float s_frag(const float* Sl, int ld, int row, int ft, int r, int g) {
  return Sl[row * ld + 32 * ft + 8 * (r >> 2) + 4 * g + (r & 3)];
}

template <class T, int D>
__global__ void __launch_bounds__(256) readout_kernel(const T* __restrict__ Q, const float* __restrict__ W,
                                                      const float* __restrict__ S_in,
                                                      const float* __restrict__ c_in, T* __restrict__ out,
                                                      int L, int Hq, int Hkv, int Hw, int m) {
  using P = Prec<T>;
  using frag = typename P::frag;
  using Cfg = ReadoutCfg<T, D>;
  constexpr int NKC = D / P::KS;
  constexpr int NDT = D / 32 + 1;
  constexpr int MP = Cfg::MP, LDW = Cfg::LDW, LDSS = Cfg::LDS;
  constexpr int SROWS = (NDT - 1) * 32 + 1;
  __shared__ __attribute__((aligned(16))) T Wl[P::NSPLIT][MP * LDW];
  __shared__ __attribute__((aligned(16))) T Sl[SROWS * LDSS];
  __shared__ float red[256];

  const int bh = blockIdx.y, b = bh / Hkv, hkv = bh % Hkv, G = Hq / Hkv;
  const int wave = threadIdx.x >> 6, l = lane_id(), col = l & 31, g = l >> 5;
  const size_t rows = (size_t)G * L;
  const T* Qb = Q + ((size_t)b * Hq + (size_t)hkv * G) * L * D;
  T* Ob = out + ((size_t)b * Hq + (size_t)hkv * G) * L * D;
  const float* Wh = W + (size_t)(Hw == 1 ? 0 : hkv) * m * D;
  const size_t tile_elems = (size_t)m * NDT * 32;
  const float* Sh = S_in + (size_t)bh * tile_elems;
  const float* ch = c_in + (size_t)bh * m;

  // Head-wide stabiliser c* = max_f c_f; S_f is rescaled by 2^(c_f - c*) when staged.
  float cm = -INFINITY;
  for (int f = threadIdx.x; f < m; f += blockDim.x) cm = fmaxf(cm, ch[f]);
  red[threadIdx.x] = cm;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  const float cstar = red[0];

  const int npass = (m + MP - 1) / MP;
  auto stage = [&](int pass) {
    const int fb = pass * MP, nf = min(MP, m - fb);
    for (int e = threadIdx.x; e < nf * D; e += blockDim.x) {
      const int fi = e / D, k = e % D;
      const float x = Wh[(size_t)(fb + fi) * D + k] * kLog2e;
      if constexpr (sizeof(T) == 2) {
        const bf16 hi = (bf16)x;
        Wl[0][fi * LDW + k] = hi;
        Wl[P::NSPLIT - 1][fi * LDW + k] = (bf16)(x - (float)hi);
      } else {
        Wl[0][fi * LDW + k] = x;
      }
    }
    for (int e = threadIdx.x; e < SROWS * nf; e += blockDim.x) {
      const int row = e / nf, fi = e % nf;
      const int f = fb + fi, ft = f >> 5, fr = f & 31;
      const int gg = (fr >> 2) & 1, r = 4 * (fr >> 3) + (fr & 3);
      const int dt = row >> 5, rho = row & 31;
      const float v = Sh[(size_t)(ft * NDT + dt) * 1024 + r * 64 + rho + 32 * gg] * fast_exp2(ch[f] - cstar);
      Sl[row * LDSS + (fi & ~31) + s_pos<T>(fi & 31)] = (T)v;
    }
  };
  if (npass == 1) {
    stage(0);
    __syncthreads();
  }

  const size_t ntiles = (rows + 127) / 128;
  for (size_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const size_t myrow = tile * 128 + wave * 32 + col;
    const bool valid = myrow < rows;
    frag qf[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
      qf[kc] = valid ? load_frag_k(Qb + myrow * D, kc, g) : zero_frag(frag{});

    f32x16 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = zero16();
    float M = -INFINITY;

    for (int pass = 0; pass < npass; ++pass) {
      if (npass > 1) {
        __syncthreads();
        stage(pass);
        __syncthreads();
      }
      const int nft = min(MP, m - pass * MP) / 32;
      for (int ft = 0; ft < nft; ++ft) {
        f32x16 c1 = zero16();
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
          for (int s = 0; s < P::NSPLIT; ++s) {
            const frag a = load_frag_k(&Wl[s][(32 * ft + col) * LDW], kc, g);
            c1 = mma(a, qf[kc], c1);
          }
        float mx = c1[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, c1[r]);
        mx = fmaxf(mx, partner32(mx));
        if (wave_any(mx > M + kTau)) {
          const float nm = mx > M + kTau ? mx : M;
          const float fct = fast_exp2(M - nm);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[dt][r] *= fct;
          M = nm;
        }
        f32x16 e;
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = fast_exp2(c1[r] - M);
        frag pf[P::NF32];
        acc_to_frags(e, pf);
#pragma unroll
        for (int h = 0; h < P::NF32; ++h) {
#pragma unroll
          for (int dt = 0; dt < NDT - 1; ++dt) acc[dt] = mma(s_frag(Sl, LDSS, 32 * dt + col, ft, h, g), pf[h], acc[dt]);
          const frag a1 = col == 0 ? s_frag(Sl, LDSS, 32 * (NDT - 1), ft, h, g) : zero_frag(frag{});
          acc[NDT - 1] = mma(a1, pf[h], acc[NDT - 1]);
        }
      }
    }

    float den = acc[NDT - 1][0];
    const float dp = partner32(den);
    den = g ? dp : den;
    const float inv = 1.f / den;
    if (valid) {
      T* orow = Ob + myrow * D;
#pragma unroll
      for (int dt = 0; dt < NDT - 1; ++dt) {
        if constexpr (sizeof(T) == 2) {
          bf16x8 o0, o1;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            o0[j] = (bf16)(acc[dt][j] * inv);
            o1[j] = (bf16)(acc[dt][8 + j] * inv);
          }
          *reinterpret_cast<bf16x8*>(orow + 32 * dt + 16 * g) = o0;
          *reinterpret_cast<bf16x8*>(orow + 32 * dt + 16 * g + 8) = o1;
        } else {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 o = {acc[dt][4 * q4] * inv, acc[dt][4 * q4 + 1] * inv, acc[dt][4 * q4 + 2] * inv,
                       acc[dt][4 * q4 + 3] * inv};
            *reinterpret_cast<f32x4*>(orow + 32 * dt + 16 * g + 4 * q4) = o;
          }
        }
      }
    }
  }
}


// ======================================================================================
// causal_scan: per kv head, c* = max over segments and features of the segment
// stabilisers, and the exclusive prefix P_t = sum_{t' < t} 2^(c_t',f - c*) S_t' of the
// segment summaries (fragment-native, same layout as kv_summary).  Grid (m/32 * (d/32+1)
// tiles, B*Hkv); fixed order t = 0, 1, ...
// ======================================================================================
__global__ void __launch_bounds__(256) causal_scan_kernel(const float* __restrict__ part_s,
                                                          const float* __restrict__ part_c, int T_ranges,
                                                          int m, int NDT, float* __restrict__ prefix,
                                                          float* __restrict__ cstar_out) {
  __shared__ float red[256];
  const int tile = blockIdx.x, bh = blockIdx.y;
  const size_t tile_elems = (size_t)m * NDT * 32;
  const float* pc = part_c + (size_t)bh * T_ranges * m;
  float cm = -INFINITY;
  for (int i = threadIdx.x; i < T_ranges * m; i += blockDim.x) cm = fmaxf(cm, pc[i]);
  red[threadIdx.x] = cm;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  const float cstar = red[0];
  if (tile == 0 && threadIdx.x == 0) cstar_out[bh] = cstar;
  const int ft = tile / NDT;
  for (int e = threadIdx.x; e < 1024; e += blockDim.x) {
    const int r = e >> 6, l = e & 63;
    const int f = 32 * ft + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
    const size_t off = (size_t)bh * T_ranges * tile_elems + (size_t)tile * 1024 + e;
    float acc = 0.f;
    for (int t = 0; t < T_ranges; ++t) {
      prefix[off + (size_t)t * tile_elems] = acc;
      acc += fast_exp2(pc[(size_t)t * m + f] - cstar) * part_s[off + (size_t)t * tile_elems];
    }
  }
}

// ======================================================================================
// causal_chunk: grid (segments, B*Hq), m/64 waves; wave w owns features [64w, 64w+64).
// Per 32-position block p0 of the segment, in order:
//   phi_Q,w  = 2^(W_w Q^T - M_w)             (M_w: this wave's row maximum)
//   phi_K,w  = 2^(K W_w^T - |k|^2 log2e/2 - c*) (c*: global per kv head, from the scan)
//   num_w^T  = carry_w^T phi_Q,w^T + [V,1]^T tril(phi_K,w phi_Q,w^T)
//   carry_w += phi_K,w^T [V, 1]
// then out = sum_w 2^(M_w - M) num_w / sum_w 2^(M_w - M) den_w across the waves (LDS).
// The carry of a segment starts at the scan's exclusive prefix.
// ======================================================================================
template <class T> struct CausalLd;
template <> struct CausalLd<bf16> { static constexpr int PK = 48; };  // phi_K rows: 32 keys + pad
template <> struct CausalLd<float> { static constexpr int PK = 33; };

template <class T, int D, int NWMAX>
__global__ void __launch_bounds__(64 * NWMAX) causal_chunk_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const float* __restrict__ W,
    const float* __restrict__ prefix, const float* __restrict__ cstar_in, T* __restrict__ out, int L, int Hq,
    int Hkv, int Hw, int m, int R, int T_ranges) {
  using P = Prec<T>;
  using frag = typename P::frag;
  constexpr int NKC = D / P::KS;
  constexpr int NDT = D / 32 + 1;
  constexpr int LDK = Ld<T>::template K<D>;
  constexpr int LDV = Ld<T>::template V<D>;
  constexpr int LDP = CausalLd<T>::PK;
  constexpr int LDR = D + 4;  // reduction rows: D partial values, den, row max
  // The cross-wave reduction handles 32 / QSPLIT query rows at a time so that the LDS
  // footprint stays within 160 KB for wide heads and many waves.
  constexpr int BASE_LDS = (2 * 32 * LDK + 32 * LDV + NWMAX * 64 * LDP) * (int)sizeof(T);
  constexpr int QSPLIT = BASE_LDS + NWMAX * 32 * LDR * 4 <= 160 * 1024       ? 1
                         : BASE_LDS + NWMAX * 16 * LDR * 4 <= 160 * 1024 ? 2
                                                                         : 4;
  constexpr int QR = 32 / QSPLIT;
  __shared__ __attribute__((aligned(16))) T Ql[32 * LDK];
  __shared__ __attribute__((aligned(16))) T Kl[32 * LDK];
  __shared__ __attribute__((aligned(16))) T Vl[32 * LDV];
  __shared__ __attribute__((aligned(16))) T Pk[NWMAX][64 * LDP];
  __shared__ __attribute__((aligned(16))) float Red[NWMAX][QR * LDR];

  const int seg = blockIdx.x, bhq = blockIdx.y;
  const int b = bhq / Hq, hq = bhq % Hq, hkv = hq / (Hq / Hkv), bh = b * Hkv + hkv;
  const int nw = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, l = lane_id(), col = l & 31, g = l >> 5;
  const int f0 = wave * 64;
  const float* Wh = W + (size_t)(Hw == 1 ? 0 : hkv) * m * D;
  const T* Qh = Q + (size_t)bhq * L * D;
  T* Oh = out + (size_t)bhq * L * D;
  const T* Kh = K + (size_t)bh * L * D;
  const T* Vh = V + (size_t)bh * L * D;

  frag wf[2][P::NSPLIT][NKC];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      frag tmp[P::NSPLIT];
      load_w_frag(Wh + (size_t)(f0 + 32 * nt + col) * D, kc, g, tmp);
#pragma unroll
      for (int s = 0; s < P::NSPLIT; ++s) wf[nt][s][kc] = tmp[s];
    }
  const float cstar = cstar_in[bh];
  const frag biasB = bias_cols(cstar, g, frag{});

  // carry of this wave's features, from the exclusive prefix of the segment
  f32x16 carry[2][NDT];
  {
    const size_t tile_elems = (size_t)m * NDT * 32;
    const float* pf = prefix + ((size_t)bh * T_ranges + seg) * tile_elems;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const float* src = pf + (size_t)((f0 / 32 + nt) * NDT + dt) * 1024;
#pragma unroll
        for (int r = 0; r < 16; ++r) carry[nt][dt][r] = src[r * 64 + l];
      }
  }
  frag ones = zero_frag(frag{});
  if (col == 0) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int j = 0; j < 8; ++j) ones[j] = (bf16)1.f;
    } else {
      ones = 1.f;
    }
  }
  T* pk = Pk[wave];
  float* red = Red[wave];

  const int p_begin = seg * R;
  const int p_end = min(p_begin + R, L);
  for (int p0 = p_begin; p0 < p_end; p0 += 32) {
    __syncthreads();
    stage_rows<T, D, false>(Ql, LDK, Qh, p0, L);
    stage_rows<T, D, false>(Kl, LDK, Kh, p0, L);
    stage_rows<T, D, true>(Vl, LDV, Vh, p0, L);
    __syncthreads();

    // phi_Q of this wave's features: C = W_w Q^T (features x queries), lane = query.
    frag qf[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) qf[kc] = load_frag_k(Ql + col * LDK, kc, g);
    f32x16 cq[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      cq[nt] = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int s = 0; s < P::NSPLIT; ++s) cq[nt] = mma(wf[nt][s][kc], qf[kc], cq[nt]);
    }
    float Mw = cq[0][0];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) Mw = fmaxf(Mw, cq[nt][r]);
    Mw = fmaxf(Mw, partner32(Mw));
    frag qb[2][P::NF32];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x16 e;
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = fast_exp2(cq[nt][r] - Mw);
      acc_to_frags(e, qb[nt]);
    }

    // phi_K of this wave's features: C = K W_w^T (keys x features), lane = feature.
    frag kf[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) kf[kc] = load_frag_k(Kl + col * LDK, kc, g);
    float nrm = sumsq(kf);
    nrm += partner32(nrm);
    const frag biasA = bias_rows(0.5f * kLog2e * nrm, g, frag{});
    frag ka[2][P::NF32];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x16 ck = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int s = 0; s < P::NSPLIT; ++s) ck = mma(kf[kc], wf[nt][s][kc], ck);
      ck = mma(biasA, biasB, ck);
      f32x16 e;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = p0 + 8 * (r >> 2) + 4 * g + (r & 3);
        e[r] = key < L ? fast_exp2(ck[r]) : 0.f;
      }
      acc_to_frags(e, ka[nt]);
      // phi_K to LDS as [feature][key] for the transposed read below
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        T* dst = pk + (32 * nt + col) * LDP + 8 * r4 + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = (T)e[4 * r4 + i];
      }
    }

    // num^T = carry^T phi_Q^T  (rows: value columns, lanes: queries)
    f32x16 num[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      num[dt] = zero16();
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        frag ca[P::NF32];
        acc_to_frags(carry[nt][dt], ca);
#pragma unroll
        for (int h = 0; h < P::NF32; ++h) num[dt] = mma(ca[h], qb[nt][h], num[dt]);
      }
    }
    // intra-block triangle: A^T = phi_K phi_Q^T (keys x queries), keep key <= query
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    f32x16 at = zero16();
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int h = 0; h < P::NF32; ++h) at = mma(lds_frag_rows(pk, LDP, 32 * nt, 0, h), qb[nt][h], at);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (8 * (r >> 2) + 4 * g + (r & 3) > col) at[r] = 0.f;
    frag ab[P::NF32];
    acc_to_frags(at, ab);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int h = 0; h < P::NF32; ++h) {
        const frag va = dt < NDT - 1 ? lds_frag_rows(Vl, LDV, 0, 32 * dt, h) : ones;
        num[dt] = mma(va, ab[h], num[dt]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) carry[nt][dt] = mma(ka[nt][h], va, carry[nt][dt]);
      }

    // this wave's partial to LDS (D values, den, row maximum per query), then the
    // cross-wave sum; one reduction item = (query, 8 value columns).
#pragma unroll
    for (int qh = 0; qh < QSPLIT; ++qh) {
      const int qrow = col - qh * QR;
      if (qrow >= 0 && qrow < QR) {
#pragma unroll
        for (int dt = 0; dt < NDT - 1; ++dt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 v = {num[dt][4 * q4], num[dt][4 * q4 + 1], num[dt][4 * q4 + 2], num[dt][4 * q4 + 3]};
            *reinterpret_cast<f32x4*>(red + qrow * LDR + 32 * dt + 16 * g + 4 * q4) = v;
          }
        if (g == 0) {
          red[qrow * LDR + D] = num[NDT - 1][0];
          red[qrow * LDR + D + 1] = Mw;
        }
      }
      __syncthreads();
      for (int it = threadIdx.x; it < QR * (D / 8); it += blockDim.x) {
        const int q = it / (D / 8), c0 = (it % (D / 8)) * 8;
        const int pos = p0 + qh * QR + q;
        if (pos >= L) continue;
        float M = -INFINITY;
        for (int w = 0; w < nw; ++w) M = fmaxf(M, Red[w][q * LDR + D + 1]);
        float den = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < nw; ++w) {
          const float* rw = Red[w] + q * LDR;
          const float sc = fast_exp2(rw[D + 1] - M);
          den += sc * rw[D];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += sc * rw[c0 + i];
        }
        const float inv = 1.f / den;
        T* orow = Oh + (size_t)pos * D + c0;
        if constexpr (sizeof(T) == 2) {
          bf16x8 o;
#pragma unroll
          for (int i = 0; i < 8; ++i) o[i] = (bf16)(acc[i] * inv);
          *reinterpret_cast<bf16x8*>(orow) = o;
        } else {
          f32x4 o0 = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
          f32x4 o1 = {acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
          *reinterpret_cast<f32x4*>(orow) = o0;
          *reinterpret_cast<f32x4*>(orow + 4) = o1;
        }
      }
      if (QSPLIT > 1) __syncthreads();
    }
  }
}

}  // namespace favor

// ======================================================================================
// Host side: dispatch and the C ABI.
// ======================================================================================
namespace favor {
namespace {

inline int ceil_div_i(long long a, long long b) { return (int)((a + b - 1) / b); }

// Records ev[i] (if given) before the i-th kernel of a call and after the last one.
struct Marks {
  hipEvent_t* ev;
  int n;
  bool mark(int i, hipStream_t st) const {
    return ev == nullptr || i >= n || hipEventRecord(ev[i], st) == hipSuccess;
  }
};

template <class T, int D>
favor_status run_bidirectional(const Plan& s, const T* Q, const T* K, const T* V, const float* W, T* out,
                               char* ws, hipStream_t st, const Marks& mk) {
  float* part_s = reinterpret_cast<float*>(ws + s.off_part_s);
  float* part_c = reinterpret_cast<float*>(ws + s.off_part_c);
  float* S = reinterpret_cast<float*>(ws + s.off_s);
  float* c = reinterpret_cast<float*>(ws + s.off_c);
  const int nw = s.m / kFeatPerWave;
  if (!mk.mark(0, st)) return FAVOR_ERR_HIP;
  hipLaunchKernelGGL((kv_summary_kernel<T, D>), dim3(s.T, s.BH, ceil_div_i(nw, 4)), dim3(kWave * (nw < 4 ? nw : 4)), 0, st, K, V, W, s.L,
                     s.Hkv, s.Hw, s.m, s.R, s.T, part_s, part_c);
  if (hipGetLastError() != hipSuccess || !mk.mark(1, st)) return FAVOR_ERR_HIP;
  hipLaunchKernelGGL(kv_combine_kernel, dim3(s.NFT, s.BH), dim3(256), 0, st, part_s, part_c, s.T, s.m, s.NDT,
                     S, c);
  if (hipGetLastError() != hipSuccess || !mk.mark(2, st)) return FAVOR_ERR_HIP;
  const long long rows = (long long)s.G * s.L;
  const int tiles = ceil_div_i(rows, 4 * kQueriesPerWave);
  int per_head = ceil_div_i(kRangeTarget, s.BH);
  if (per_head > tiles) per_head = tiles;
  if (per_head < 1) per_head = 1;
  hipLaunchKernelGGL((readout_kernel<T, D>), dim3(per_head, s.BH), dim3(256), 0, st, Q, W, S, c, out, s.L,
                     s.Hq, s.Hkv, s.Hw, s.m);
  if (hipGetLastError() != hipSuccess || !mk.mark(3, st)) return FAVOR_ERR_HIP;
  return FAVOR_OK;
}

template <class T, int D>
favor_status run_causal(const Plan& s, const T* Q, const T* K, const T* V, const float* W, T* out, char* ws,
                        hipStream_t st, const Marks& mk) {
  float* part_s = reinterpret_cast<float*>(ws + s.off_part_s);
  float* part_c = reinterpret_cast<float*>(ws + s.off_part_c);
  float* cstar = reinterpret_cast<float*>(ws + s.off_c);
  float* prefix = reinterpret_cast<float*>(ws + s.off_p);
  const int nw = s.m / kFeatPerWave;
  if (!mk.mark(0, st)) return FAVOR_ERR_HIP;
  hipLaunchKernelGGL((kv_summary_kernel<T, D>), dim3(s.T, s.BH, ceil_div_i(nw, 4)), dim3(kWave * (nw < 4 ? nw : 4)),
                     0, st, K, V, W, s.L, s.Hkv, s.Hw, s.m, s.R, s.T, part_s, part_c);
  if (hipGetLastError() != hipSuccess || !mk.mark(1, st)) return FAVOR_ERR_HIP;
  hipLaunchKernelGGL(causal_scan_kernel, dim3(s.NFT * s.NDT, s.BH), dim3(256), 0, st, part_s, part_c, s.T, s.m,
                     s.NDT, prefix, cstar);
  if (hipGetLastError() != hipSuccess || !mk.mark(2, st)) return FAVOR_ERR_HIP;
  if (nw <= 4)
    hipLaunchKernelGGL((causal_chunk_kernel<T, D, 4>), dim3(s.T, s.B * s.Hq), dim3(kWave * nw), 0, st, Q, K, V, W,
                       prefix, cstar, out, s.L, s.Hq, s.Hkv, s.Hw, s.m, s.R, s.T);
  else
    hipLaunchKernelGGL((causal_chunk_kernel<T, D, 8>), dim3(s.T, s.B * s.Hq), dim3(kWave * nw), 0, st, Q, K, V, W,
                       prefix, cstar, out, s.L, s.Hq, s.Hkv, s.Hw, s.m, s.R, s.T);
  if (hipGetLastError() != hipSuccess || !mk.mark(3, st)) return FAVOR_ERR_HIP;
  return FAVOR_OK;
}

template <class T>
favor_status run_typed(const Plan& s, const void* Q, const void* K, const void* V, const float* W, void* out,
                       char* ws, hipStream_t st, const Marks& mk) {
  const T* q = static_cast<const T*>(Q);
  const T* k = static_cast<const T*>(K);
  const T* v = static_cast<const T*>(V);
  T* o = static_cast<T*>(out);
  if (s.mode == FAVOR_BIDIRECTIONAL)
    return s.d == 64 ? run_bidirectional<T, 64>(s, q, k, v, W, o, ws, st, mk)
                     : run_bidirectional<T, 128>(s, q, k, v, W, o, ws, st, mk);
  return s.d == 64 ? run_causal<T, 64>(s, q, k, v, W, o, ws, st, mk)
                   : run_causal<T, 128>(s, q, k, v, W, o, ws, st, mk);
}

}  // namespace
}  // namespace favor

extern "C" {

size_t favor_workspace_bytes(const favor_problem* p) {
  favor::Plan s;
  return favor::make_plan(p, &s) == FAVOR_OK ? s.bytes : 0;
}

const char* favor_status_string(favor_status s) {
  switch (s) {
    case FAVOR_OK: return "ok";
    case FAVOR_ERR_INVALID_ARG: return "invalid argument";
    case FAVOR_ERR_UNSUPPORTED: return "unsupported problem (head_dim, num_features, dtype, mode or chunk)";
    case FAVOR_ERR_WORKSPACE: return "workspace missing or smaller than favor_workspace_bytes()";
    case FAVOR_ERR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

int32_t favor_abi_version(void) { return FAVOR_ABI_VERSION; }

static favor_status attn_fwd_impl(const favor_problem* p, const void* Q, const void* K, const void* V,
                                  const float* W, void* out, void* workspace, size_t workspace_bytes, void* stream,
                                  const favor::Marks& mk) {
  favor::Plan s;
  const favor_status st = favor::make_plan(p, &s);
  if (st != FAVOR_OK) return st;
  if (Q == nullptr || K == nullptr || V == nullptr || W == nullptr || out == nullptr) return FAVOR_ERR_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < s.bytes || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return FAVOR_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (s.dtype == FAVOR_BF16) return favor::run_typed<favor::bf16>(s, Q, K, V, W, out, ws, hs, mk);
  return favor::run_typed<float>(s, Q, K, V, W, out, ws, hs, mk);
}

favor_status favor_attn_fwd(const favor_problem* p, const void* Q, const void* K, const void* V, const float* W,
                            void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return attn_fwd_impl(p, Q, K, V, W, out, workspace, workspace_bytes, stream, favor::Marks{nullptr, 0});
}

favor_status favor_attn_fwd_timed(const favor_problem* p, const void* Q, const void* K, const void* V,
                                  const float* W, void* out, void* workspace, size_t workspace_bytes, void* stream,
                                  void* const* events, int32_t n_events) {
  if (events == nullptr || n_events < FAVOR_FWD_KERNELS + 1) return FAVOR_ERR_INVALID_ARG;
  for (int i = 0; i < FAVOR_FWD_KERNELS + 1; ++i)
    if (events[i] == nullptr) return FAVOR_ERR_INVALID_ARG;
  return attn_fwd_impl(p, Q, K, V, W, out, workspace, workspace_bytes, stream,
                       favor::Marks{reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)), n_events});
}

favor_status favor_features(const favor_problem* p, int32_t side, const void* X, const float* W, float* phi_out,
                            float* c_out, void* stream) {
  favor::Plan s;
  const favor_status st = favor::make_plan(p, &s);
  if (st != FAVOR_OK) return st;
  if (side != 0 && side != 1) return FAVOR_ERR_INVALID_ARG;
  if (X == nullptr || W == nullptr || phi_out == nullptr || c_out == nullptr) return FAVOR_ERR_INVALID_ARG;
  (void)stream;
  return FAVOR_ERR_UNSUPPORTED;
}

}  // extern "C"
