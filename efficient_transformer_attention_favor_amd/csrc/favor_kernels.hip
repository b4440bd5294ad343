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
//   (the readout sums the position-range partials while staging them)
//   readout      bidirectional: per query tile, phi(Q) W-contraction on the MFMA with a
//                running row maximum, then out^T = S^T phi(Q)^T and the division.
//   causal_scan  causal: exclusive prefix of the per-segment summaries, all rescaled to a
//                global per-head stabiliser.
//   causal_chunk causal: per segment, 32-position blocks in order with the carried summary
//                in registers (features split over the waves), the intra-block triangle on
//                the MFMA, and a cross-wave sum of the per-wave partial outputs.
#include <hip/hip_runtime.h>

#include <math.h>

#include <type_traits>

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
// kv_summary: per (kv head bh, position range t, 64-feature slice) the partial summary
//   S[f][c] = sum_{p in range} 2^(E_pf - c_f) [V, 1][p][c],   E_pf = log2e (w_f.k_p - |k_p|^2/2)
// KW waves split the slice's features into NTW-tile groups and the range into position
// groups; each wave streams 32-position blocks with its features' W in registers:
// E = K_blk W^T (+ one bias MFMA carrying -|k|^2 log2e/2 - c_f), phi = 2^E,
// S += phi^T [V, 1] (V transposed through wave-private LDS).  The wave partials of a
// feature group are merged in LDS after rescaling to the largest c_f.  Output (float32):
//   gs[bh][t][row][f], row = 32 ct + rho holds value column 32 ct + vperm(rho) (ct < d/32),
//   row d holds the ones column (S_1);  gc[bh][t][f] = c_f (log2 units).
// Workgroup ids are laid out so the feature slices of one (bh, t) share an XCD (and its L2
// copy of K and V): block b runs on XCD b % 8.
// ======================================================================================
template <class T, int D> struct KvCfg;
template <> struct KvCfg<bf16, 64> { static constexpr int KW = 8, NTW = 1; };   // 2 waves / SIMD
template <> struct KvCfg<bf16, 128> { static constexpr int KW = 4, NTW = 1; };
template <> struct KvCfg<float, 64> { static constexpr int KW = 4, NTW = 2; };
template <> struct KvCfg<float, 128> { static constexpr int KW = 4, NTW = 1; };

template <class T, int D>
__global__ void __launch_bounds__((64 * KvCfg<T, D>::KW)) kv_summary_kernel(
    const T* __restrict__ K, const T* __restrict__ V, const float* __restrict__ W, int L, int Hkv, int Hw, int m,
    int R, int T_ranges, int n_units, float* __restrict__ gs, float* __restrict__ gc) {
  using P = Prec<T>;
  using frag = typename P::frag;
  constexpr int KW = KvCfg<T, D>::KW, NTW = KvCfg<T, D>::NTW;
  constexpr int FG = 2 / NTW;   // feature groups per workgroup (64 features)
  constexpr int PG = KW / FG;   // position groups
  constexpr int NKC = D / P::KS;
  constexpr int NDT = D / 32 + 1;
  constexpr int LDV = Ld<T>::template V<D>;
  constexpr int ACC = NTW * NDT * 1024;  // floats of one wave's partial (fragment order)
  __shared__ __attribute__((aligned(16))) T Vl[KW][32 * LDV];
  __shared__ __attribute__((aligned(16))) float Red[(PG / 2) * FG][ACC];
  __shared__ float Cs[KW][32 * NTW];

  const int NFS = m / 64;
  const int xcd = blockIdx.x & 7, kq = blockIdx.x >> 3;
  const int slice = kq % NFS, unit = (kq / NFS) * 8 + xcd;
  if (unit >= n_units) return;
  const int bh = unit / T_ranges, t = unit % T_ranges, hkv = bh % Hkv;
  const int wave = threadIdx.x >> 6, l = lane_id(), col = l & 31, g = l >> 5;
  const int fgi = wave % FG, pgi = wave / FG;
  const int f0 = slice * 64 + fgi * 32 * NTW;
  const float* Wh = W + (size_t)(Hw == 1 ? 0 : hkv) * m * D;
  const T* Kh = K + (size_t)bh * L * D;
  const T* Vh = V + (size_t)bh * L * D;
  T* vl = Vl[wave];

  frag wf[NTW][P::NSPLIT][NKC];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      frag tmp[P::NSPLIT];
      load_w_frag(Wh + (size_t)(f0 + 32 * nt + col) * D, kc, g, tmp);
#pragma unroll
      for (int s = 0; s < P::NSPLIT; ++s) wf[nt][s][kc] = tmp[s];
    }

  float cst[NTW];  // stabiliser of this lane's feature (log2 units)
  frag biasB[NTW];
  f32x16 S[NTW][NDT];
  frag ones = zero_frag(frag{});
  if (col == 0) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int j = 0; j < 8; ++j) ones[j] = (bf16)1.f;
    } else {
      ones = 1.f;
    }
  }

  const int pb = t * R, pe = min(pb + R, L);
  const int Rw = ((R + 32 * PG - 1) / (32 * PG)) * 32;
  const int wb = pb + pgi * Rw, we = min(wb + Rw, pe);
  constexpr int EPC = 16 / sizeof(T);   // elements per 16-byte chunk
  constexpr int CPR = D / EPC;          // chunks per row
  constexpr int CPL = 32 * CPR / 64;    // chunks per lane per block
  // Block loads are software-pipelined: block p0 + 32 is fetched into registers while
  // block p0 is computed.  Loads are clamped into the range (rows past its end are real
  // data whose features get a +huge row bias, i.e. phi = 0).
  f32x4 vn[CPL];
  frag kn[NKC];
  auto fetch = [&](int q0) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = l + 64 * i, row = min(q0 + c / CPR, we - 1), c0 = (c % CPR) * EPC;
      vn[i] = *reinterpret_cast<const f32x4*>(Vh + (size_t)row * D + c0);
    }
    const int krow = min(q0 + col, we - 1);
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) kn[kc] = load_frag_k(Kh + (size_t)krow * D, kc, g);
  };

  // One 32-position block.  Stabiliser modes: 0 = first block of the fast pass (c_f :=
  // this block's maximum), 1 = fast pass (c_f fixed: no VALU work on the accumulators),
  // 2 = fallback pass (running maximum, moved lazily, accumulators rescaled).
  auto block = [&](int p0, auto mode_tag) {
    constexpr int MODE = decltype(mode_tag)::value;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = l + 64 * i, row = c / CPR, c0 = (c % CPR) * EPC;
      const f32x4 v = vn[i];
      T* drow = vl + row * LDV + (c0 & ~31);
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<float2*>(drow + vperm_inv(c0 & 31)) = float2{v[0], v[1]};
        *reinterpret_cast<float2*>(drow + vperm_inv((c0 & 31) + 4)) = float2{v[2], v[3]};
      } else {
        *reinterpret_cast<f32x4*>(drow + vperm_inv(c0 & 31)) = v;
      }
    }
    frag kf[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) kf[kc] = kn[kc];
    fetch(min(p0 + 32, we - 1));
    float nrm = sumsq(kf);
    nrm += partner32(nrm);
    const float rb = p0 + col < we ? 0.5f * kLog2e * nrm : 1e30f;
    const frag biasA = bias_rows(rb, g, frag{});

    f32x16 c1[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      c1[nt] = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int s = 0; s < P::NSPLIT; ++s) c1[nt] = mma(kf[kc], wf[nt][s][kc], c1[nt]);
      c1[nt] = mma(biasA, biasB[nt], c1[nt]);
    }

    if constexpr (MODE == 0) {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        float mx = c1[nt][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, c1[nt][r]);
        mx = fmaxf(mx, partner32(mx));
        cst[nt] = mx;
#pragma unroll
        for (int r = 0; r < 16; ++r) c1[nt][r] -= mx;
        biasB[nt] = bias_cols(mx, g, frag{});
      }
    } else if constexpr (MODE == 2) {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        float mx = c1[nt][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, c1[nt][r]);
        mx = fmaxf(mx, partner32(mx));
        const bool first = cst[nt] == -INFINITY;
        float shift = 0.f;
        if (first || mx > kTau) shift = mx;
        if (wave_any(shift != 0.f)) {
          const float base = first ? 0.f : cst[nt];
          cst[nt] = base + shift;
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
        } else if (first) {
          cst[nt] = 0.f;  // block maximum is exactly 0
        }
      }
    }

    frag pa[NTW][P::NF32];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      f32x16 e;
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = fast_exp2(c1[nt][r]);
      acc_to_frags(e, pa[nt]);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int h = 0; h < P::NF32; ++h) {
        const frag vb = dt < NDT - 1 ? lds_frag_rows(vl, LDV, 0, 32 * dt, h) : ones;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) S[nt][dt] = mma(pa[nt][h], vb, S[nt][dt]);
      }
    asm volatile("" ::: "memory");  // this block's LDS reads before the next block's writes
  };
  auto reset = [&]() {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      cst[nt] = -INFINITY;
      biasB[nt] = bias_cols(0.f, g, frag{});
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) S[nt][dt] = zero16();
    }
  };

  // Fast pass: stabiliser fixed at the first block's maximum.  Only an overflow (a later
  // block more than ~2^100 above the first) makes it non-finite; then the range is redone
  // with the running maximum.
  reset();
  if (wb < we) {
    fetch(wb);
    block(wb, std::integral_constant<int, 0>{});
    for (int p0 = wb + 32; p0 < we; p0 += 32) block(p0, std::integral_constant<int, 1>{});
  }
  float chk = 0.f;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) chk += S[nt][dt][r];
  if (wave_any(!(chk - chk == 0.f))) {
    reset();
    fetch(wb);
    for (int p0 = wb; p0 < we; p0 += 32) block(p0, std::integral_constant<int, 2>{});
  }

  // ---- merge the position-group partials of each feature group --------------------
  if (g == 0) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) Cs[wave][32 * nt + col] = cst[nt];
  }
  __syncthreads();
  float cmax[NTW];  // merged stabiliser of this lane's C1 feature (column col)
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    cmax[nt] = -INFINITY;
#pragma unroll
    for (int q = 0; q < PG; ++q) cmax[nt] = fmaxf(cmax[nt], Cs[q * FG + fgi][32 * nt + col]);
  }
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int fl = 32 * nt + 8 * (r >> 2) + 4 * g + (r & 3);
      float cm = -INFINITY;
#pragma unroll
      for (int q = 0; q < PG; ++q) cm = fmaxf(cm, Cs[q * FG + fgi][fl]);
      const float sc = cm == -INFINITY ? 0.f : fast_exp2(Cs[wave][fl] - cm);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) S[nt][dt][r] *= sc;
    }
  auto dump = [&](float* dst) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[((nt * NDT + dt) * 16 + r) * 64 + l] = S[nt][dt][r];
  };
  auto absorb = [&](const float* src) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) S[nt][dt][r] += src[((nt * NDT + dt) * 16 + r) * 64 + l];
  };
#pragma unroll
  for (int step = PG / 2; step >= 1; step >>= 1) {
    if (pgi >= step && pgi < 2 * step) dump(Red[(pgi - step) * FG + fgi]);
    __syncthreads();
    if (pgi < step) absorb(Red[pgi * FG + fgi]);
    __syncthreads();
  }
  if (pgi != 0) return;

  const size_t unit_off = (size_t)bh * T_ranges + t;
  float* out_s = gs + unit_off * (size_t)(D + 1) * m;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
    for (int dt = 0; dt < NDT - 1; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 v = {S[nt][dt][4 * r4], S[nt][dt][4 * r4 + 1], S[nt][dt][4 * r4 + 2], S[nt][dt][4 * r4 + 3]};
        *reinterpret_cast<f32x4*>(out_s + (size_t)(32 * dt + col) * m + f0 + 32 * nt + 8 * r4 + 4 * g) = v;
      }
    if (col == 0)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 v = {S[nt][NDT - 1][4 * r4], S[nt][NDT - 1][4 * r4 + 1], S[nt][NDT - 1][4 * r4 + 2],
                   S[nt][NDT - 1][4 * r4 + 3]};
        *reinterpret_cast<f32x4*>(out_s + (size_t)D * m + f0 + 32 * nt + 8 * r4 + 4 * g) = v;
      }
    if (g == 0) gc[unit_off * m + f0 + 32 * nt + col] = cmax[nt];
  }
}

// ======================================================================================
// readout (bidirectional).  Grid (workgroups per kv head, B*Hkv), NWAVE waves; each wave
// owns QN x 32 query rows per step (the G query heads of a kv head are G*L contiguous
// rows).  LDS holds W (hi/lo) and S^T for a pass of MP features: rows are value columns in
// vperm order then the ones row; within a 32-feature tile the features are reordered so
// one lane's 8 operand values are contiguous.  S is summed over the position ranges and
// rescaled to the head's largest stabiliser while staged; with more than one pass W and S
// are re-staged per query tile.
// ======================================================================================
template <class T, int D> struct ReadoutCfg;
template <int D> struct ReadoutCfg<bf16, D> {
  static constexpr int MP = D == 64 ? 256 : 128;
  static constexpr int LDW = D + 8;
  static constexpr int LDS = MP + 8;
  static constexpr int NWAVE = D == 64 ? 8 : 4;   // D = 64: 2 waves / SIMD
  static constexpr int QN = D == 64 ? 2 : 1;
};
template <int D> struct ReadoutCfg<float, D> {
  static constexpr int MP = D == 64 ? 128 : 64;
  static constexpr int LDW = D + 1;
  static constexpr int LDS = MP + 1;
  static constexpr int NWAVE = 4;
  static constexpr int QN = D == 64 ? 2 : 1;
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
__global__ void __launch_bounds__((64 * ReadoutCfg<T, D>::NWAVE))
    readout_kernel(const T* __restrict__ Q, const float* __restrict__ W, const float* __restrict__ gs,
                   const float* __restrict__ gc, T* __restrict__ out, int L, int Hq, int Hkv, int Hw, int m,
                   int T_ranges) {
  using P = Prec<T>;
  using frag = typename P::frag;
  using Cfg = ReadoutCfg<T, D>;
  constexpr int NKC = D / P::KS;
  constexpr int NDT = D / 32 + 1;
  constexpr int MP = Cfg::MP, LDW = Cfg::LDW, LDSS = Cfg::LDS, QN = Cfg::QN;
  constexpr int NT = 64 * Cfg::NWAVE;
  constexpr int SROWS = D + 1;
  constexpr int TILE = Cfg::NWAVE * QN * 32;
  __shared__ __attribute__((aligned(16))) T Wl[P::NSPLIT][MP * LDW];
  __shared__ __attribute__((aligned(16))) T Sl[SROWS * LDSS];
  __shared__ float red[NT];

  const int bh = blockIdx.y, b = bh / Hkv, hkv = bh % Hkv, G = Hq / Hkv;
  const int wave = threadIdx.x >> 6, l = lane_id(), col = l & 31, g = l >> 5;
  const size_t rows = (size_t)G * L;
  const T* Qb = Q + ((size_t)b * Hq + (size_t)hkv * G) * L * D;
  T* Ob = out + ((size_t)b * Hq + (size_t)hkv * G) * L * D;
  const float* Wh = W + (size_t)(Hw == 1 ? 0 : hkv) * m * D;
  const float* gsh = gs + (size_t)bh * T_ranges * (D + 1) * m;
  const float* gch = gc + (size_t)bh * T_ranges * m;

  // Head-wide stabiliser c* = max over ranges and features.
  float cm = -INFINITY;
  for (int i = threadIdx.x; i < T_ranges * m; i += NT) cm = fmaxf(cm, gch[i]);
  red[threadIdx.x] = cm;
  __syncthreads();
  for (int s = NT / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  const float cstar = red[0];

  const int npass = (m + MP - 1) / MP;
  auto stage = [&](int pass) {
    const int fb = pass * MP, nf = min(MP, m - fb);
    // W rows: 4 float4 loads in flight per thread per step
    constexpr int UW = 4;
    for (int e0 = threadIdx.x; e0 < nf * (D / 4); e0 += UW * NT) {
      f32x4 x[UW];
#pragma unroll
      for (int u = 0; u < UW; ++u) {
        const int e = e0 + u * NT;
        x[u] = e < nf * (D / 4) ? *reinterpret_cast<const f32x4*>(Wh + (size_t)(fb + e / (D / 4)) * D + (e % (D / 4)) * 4)
                                : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < UW; ++u) {
        const int e = e0 + u * NT;
        if (e >= nf * (D / 4)) continue;
        const int fi = e / (D / 4), k4 = (e % (D / 4)) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float xs = x[u][i] * kLog2e;
          if constexpr (sizeof(T) == 2) {
            const bf16 hi = (bf16)xs;
            Wl[0][fi * LDW + k4 + i] = hi;
            Wl[P::NSPLIT - 1][fi * LDW + k4 + i] = (bf16)(xs - (float)hi);
          } else {
            Wl[0][fi * LDW + k4 + i] = xs;
          }
        }
      }
    }
    // S rows: sum over the position ranges, rescaled to c*
    constexpr int US = 4;
    const int nsv = SROWS * (nf / 4);
    for (int e0 = threadIdx.x; e0 < nsv; e0 += US * NT) {
      f32x4 acc[US];
#pragma unroll
      for (int u = 0; u < US; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int t = 0; t < T_ranges; ++t) {
        f32x4 v[US], c[US];
#pragma unroll
        for (int u = 0; u < US; ++u) {
          const int e = min(e0 + u * NT, nsv - 1);
          const int row = e / (nf / 4), fi = (e % (nf / 4)) * 4;
          v[u] = *reinterpret_cast<const f32x4*>(gsh + ((size_t)t * (D + 1) + row) * m + fb + fi);
          c[u] = *reinterpret_cast<const f32x4*>(gch + (size_t)t * m + fb + fi);
        }
#pragma unroll
        for (int u = 0; u < US; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[u][i] += v[u][i] * fast_exp2(c[u][i] - cstar);
      }
#pragma unroll
      for (int u = 0; u < US; ++u) {
        const int e = e0 + u * NT;
        if (e >= nsv) continue;
        const int row = e / (nf / 4), fi = (e % (nf / 4)) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) Sl[row * LDSS + ((fi + i) & ~31) + s_pos<T>((fi + i) & 31)] = (T)acc[u][i];
      }
    }
  };
  if (npass == 1) {
    stage(0);
    __syncthreads();
  }

  const size_t ntiles = (rows + TILE - 1) / TILE;
  for (size_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    size_t myrow[QN];
    bool valid[QN];
    frag qf[QN][NKC];
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      myrow[q] = tile * TILE + (size_t)(wave * QN + q) * 32 + col;
      valid[q] = myrow[q] < rows;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
        qf[q][kc] = valid[q] ? load_frag_k(Qb + myrow[q] * D, kc, g) : zero_frag(frag{});
    }
    f32x16 acc[QN][NDT];
    float M[QN];
    // One 32-feature tile.  Modes: 0 = first tile (M := its row maximum), 1 = M fixed (no
    // VALU work on the accumulators), 2 = fallback (running maximum, moved lazily).
    // Feature exponents of tile ft: C = W_ft Q^T (features x queries), lane = query; with
    // BIAS the row stabiliser -M enters as one more MFMA.
    auto c1_tile = [&](int ft, f32x16 (&c1)[QN], auto bias_tag) {
#pragma unroll
      for (int q = 0; q < QN; ++q) c1[q] = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int s = 0; s < P::NSPLIT; ++s) {
          const frag a = load_frag_k(&Wl[s][(32 * ft + col) * LDW], kc, g);
#pragma unroll
          for (int q = 0; q < QN; ++q) c1[q] = mma(a, qf[q][kc], c1[q]);
        }
      if constexpr (decltype(bias_tag)::value) {
        const frag unitA = bias_unit_rows(g, frag{});
#pragma unroll
        for (int q = 0; q < QN; ++q) c1[q] = mma(unitA, bias_cols(M[q], g, frag{}), c1[q]);
      }
    };
    // phi = 2^(c1 [- M]) and acc += S_ft^T phi.
    auto readout_tile = [&](int ft, const f32x16 (&c1)[QN], auto sub_tag) {
      frag pf[QN][P::NF32];
#pragma unroll
      for (int q = 0; q < QN; ++q) {
        f32x16 e;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          e[r] = fast_exp2(decltype(sub_tag)::value ? c1[q][r] - M[q] : c1[q][r]);
        acc_to_frags(e, pf[q]);
      }
#pragma unroll
      for (int h = 0; h < P::NF32; ++h) {
#pragma unroll
        for (int dt = 0; dt < NDT - 1; ++dt) {
          const frag a = s_frag(Sl, LDSS, 32 * dt + col, ft, h, g);
#pragma unroll
          for (int q = 0; q < QN; ++q) acc[q][dt] = mma(a, pf[q][h], acc[q][dt]);
        }
        const frag a1 = col == 0 ? s_frag(Sl, LDSS, D, ft, h, g) : zero_frag(frag{});
#pragma unroll
        for (int q = 0; q < QN; ++q) acc[q][NDT - 1] = mma(a1, pf[q][h], acc[q][NDT - 1]);
      }
    };
    auto rowmax = [&](const f32x16& c) {
      float mx = c[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, c[r]);
      return fmaxf(mx, partner32(mx));
    };
    using Yes = std::integral_constant<bool, true>;
    using No = std::integral_constant<bool, false>;
    // Fast pass: the stabiliser is fixed at the first tile's row maximum and folded into
    // the W-contraction (bias MFMA), so the loop does exponentials only.  Fallback: plain
    // order with a lazily moved running maximum.
    auto run = [&](bool fast) {
#pragma unroll
      for (int q = 0; q < QN; ++q) {
        M[q] = -INFINITY;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[q][dt] = zero16();
      }
      for (int pass = 0; pass < npass; ++pass) {
        if (npass > 1) {
          __syncthreads();
          stage(pass);
          __syncthreads();
        }
        const int nft = min(MP, m - pass * MP) / 32;
        if (fast) {
          int ft = 0;
          if (pass == 0) {
            f32x16 c1[QN];
            c1_tile(0, c1, No{});
#pragma unroll
            for (int q = 0; q < QN; ++q) M[q] = rowmax(c1[q]);
            readout_tile(0, c1, Yes{});
            ft = 1;
          }
          for (; ft < nft; ++ft) {
            f32x16 c1[QN];
            c1_tile(ft, c1, Yes{});
            readout_tile(ft, c1, No{});
          }
        } else {
          for (int ft = 0; ft < nft; ++ft) {
            f32x16 c1[QN];
            c1_tile(ft, c1, No{});
#pragma unroll
            for (int q = 0; q < QN; ++q) {
              const float mx = rowmax(c1[q]);
              if (wave_any(mx > M[q] + kTau)) {
                const float nm = mx > M[q] + kTau ? mx : M[q];
                const float fct = fast_exp2(M[q] - nm);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                  for (int r = 0; r < 16; ++r) acc[q][dt][r] *= fct;
                M[q] = nm;
              }
            }
            readout_tile(ft, c1, Yes{});
          }
        }
      }
    };
    // Fast pass with the stabiliser fixed at the first feature tile's row maximum; a
    // non-finite denominator (an overflow) sends the whole tile to the fallback.
    run(true);
    bool bad = false;
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      const float dq = acc[q][NDT - 1][0];
      bad |= !(dq - dq == 0.f);
    }
    if (__syncthreads_or(bad)) run(false);

#pragma unroll
    for (int q = 0; q < QN; ++q) {
      float den = acc[q][NDT - 1][0];
      const float dp = partner32(den);
      den = g ? dp : den;
      const float inv = 1.f / den;
      if (!valid[q]) continue;
      T* orow = Ob + myrow[q] * D;
#pragma unroll
      for (int dt = 0; dt < NDT - 1; ++dt) {
        if constexpr (sizeof(T) == 2) {
          bf16x8 o0, o1;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            o0[j] = (bf16)(acc[q][dt][j] * inv);
            o1[j] = (bf16)(acc[q][dt][8 + j] * inv);
          }
          *reinterpret_cast<bf16x8*>(orow + 32 * dt + 16 * g) = o0;
          *reinterpret_cast<bf16x8*>(orow + 32 * dt + 16 * g + 8) = o1;
        } else {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 o = {acc[q][dt][4 * q4] * inv, acc[q][dt][4 * q4 + 1] * inv, acc[q][dt][4 * q4 + 2] * inv,
                       acc[q][dt][4 * q4 + 3] * inv};
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
// segment summaries (read in kv_summary's row layout, written fragment-native for the
// chunk kernel's carry registers: tile (ft, ct) of 32 features x 32 value columns as
// [16 registers][64 lanes], register r / lane l = feature 32 ft + 8(r/4) + 4(l/32) + r%4,
// value column 32 ct + vperm(l%32); ct = d/32 is the ones column at lane%32 == 0).
// Grid (m/32 * (d/32+1) tiles, B*Hkv); fixed order t = 0, 1, ...
// ======================================================================================
__global__ void __launch_bounds__(256) causal_scan_kernel(const float* __restrict__ gs,
                                                          const float* __restrict__ gc, int T_ranges, int m,
                                                          int D, float* __restrict__ prefix,
                                                          float* __restrict__ cstar_out) {
  __shared__ float red[256];
  const int NDT = D / 32 + 1;
  const int tile = blockIdx.x, bh = blockIdx.y;
  const size_t tile_elems = (size_t)m * NDT * 32;
  const float* pc = gc + (size_t)bh * T_ranges * m;
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
  const int ft = tile / NDT, dt = tile % NDT;
  for (int e = threadIdx.x; e < 1024; e += blockDim.x) {
    const int r = e >> 6, l = e & 63, rho = l & 31;
    const int f = 32 * ft + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
    const int row = dt < NDT - 1 ? 32 * dt + rho : (rho == 0 ? D : -1);
    float* dst = prefix + (size_t)bh * T_ranges * tile_elems + (size_t)tile * 1024 + e;
    float acc = 0.f;
    for (int t = 0; t < T_ranges; ++t) {
      dst[(size_t)t * tile_elems] = acc;
      if (row >= 0)
        acc += fast_exp2(pc[(size_t)t * m + f] - cstar) *
               gs[(((size_t)bh * T_ranges + t) * (D + 1) + row) * m + f];
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
favor_status launch_kv_summary(const Plan& s, const T* K, const T* V, const float* W, float* gs, float* gc,
                               hipStream_t st) {
  const int units = s.BH * s.T;
  const int nfs = s.m / kFeatPerWave;
  hipLaunchKernelGGL((kv_summary_kernel<T, D>), dim3(8 * ceil_div_i(units, 8) * nfs), dim3(64 * KvCfg<T, D>::KW), 0,
                     st, K, V, W,
                     s.L, s.Hkv, s.Hw, s.m, s.R, s.T, units, gs, gc);
  return hipGetLastError() == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}

template <class T, int D>
favor_status run_bidirectional(const Plan& s, const T* Q, const T* K, const T* V, const float* W, T* out,
                               char* ws, hipStream_t st, const Marks& mk) {
  float* gs = reinterpret_cast<float*>(ws + s.off_gs);
  float* gc = reinterpret_cast<float*>(ws + s.off_gc);
  if (!mk.mark(0, st)) return FAVOR_ERR_HIP;
  favor_status rc = launch_kv_summary<T, D>(s, K, V, W, gs, gc, st);
  if (rc != FAVOR_OK) return rc;
  if (!mk.mark(1, st) || !mk.mark(2, st)) return FAVOR_ERR_HIP;  // no middle kernel
  using Cfg = ReadoutCfg<T, D>;
  const long long rows = (long long)s.G * s.L;
  const int tiles = ceil_div_i(rows, Cfg::NWAVE * Cfg::QN * 32);
  int per_head = ceil_div_i(kReadoutTarget, s.BH);
  if (per_head > tiles) per_head = tiles;
  if (per_head < 1) per_head = 1;
  hipLaunchKernelGGL((readout_kernel<T, D>), dim3(per_head, s.BH), dim3(64 * Cfg::NWAVE), 0, st, Q, W, gs, gc, out,
                     s.L, s.Hq, s.Hkv, s.Hw, s.m, s.T);
  if (hipGetLastError() != hipSuccess || !mk.mark(3, st)) return FAVOR_ERR_HIP;
  return FAVOR_OK;
}

template <class T, int D>
favor_status run_causal(const Plan& s, const T* Q, const T* K, const T* V, const float* W, T* out, char* ws,
                        hipStream_t st, const Marks& mk) {
  float* gs = reinterpret_cast<float*>(ws + s.off_gs);
  float* gc = reinterpret_cast<float*>(ws + s.off_gc);
  float* prefix = reinterpret_cast<float*>(ws + s.off_p);
  float* cstar = reinterpret_cast<float*>(ws + s.off_cstar);
  const int nw = s.m / kFeatPerWave;
  if (!mk.mark(0, st)) return FAVOR_ERR_HIP;
  favor_status rc = launch_kv_summary<T, D>(s, K, V, W, gs, gc, st);
  if (rc != FAVOR_OK || !mk.mark(1, st)) return rc != FAVOR_OK ? rc : FAVOR_ERR_HIP;
  hipLaunchKernelGGL(causal_scan_kernel, dim3(s.NFT * s.NDT, s.BH), dim3(256), 0, st, gs, gc, s.T, s.m, s.d,
                     prefix, cstar);
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

}  // extern "C"
