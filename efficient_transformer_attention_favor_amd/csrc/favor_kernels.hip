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
//   kv_summary   keys/values of one kv head, one position range and 64 features per
//                workgroup: phi(K_blk) = exp2(K_blk W^T - |k|^2 log2e / 2 - c_f) on the MFMA
//                (the bias enters as one extra MFMA), then S += phi^T [V, 1].  c_f is the
//                per-feature maximum of the range's first block (running maximum only on
//                overflow).  With one range per head (bf16) it writes the readout's LDS
//                images directly: S_v / S_1 in bf16 and c_f + log2 S_1,f per feature.
//   readout      bidirectional: per 32-row query tile, the W contraction on the MFMA, the
//                key stabiliser c_f and the row stabiliser entering through one bias MFMA,
//                then out^T = S^T phi(Q)^T and the division.
//   causal_scan  causal: exclusive prefix of the per-segment summaries, all rescaled to a
//                global per-head stabiliser.
//   causal_chunk causal: per segment, 32-position blocks in order with the carried summary
//                in registers (features split over the waves), the intra-block triangle on
//                the MFMA, and a cross-wave sum of the per-wave partial outputs.
#include <hip/hip_runtime.h>

#include <math.h>

#include <mutex>
#include <type_traits>

#include "favor_device.hpp"
#include "favor_ops.hpp"
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
// groups; each wave streams 32-position blocks with its features' W in registers (bf16
// d = 64: the slice's W in LDS, shared by the workgroup's waves):
// E = K_blk W^T (+ one bias MFMA carrying -|k|^2 log2e/2 - c_f), phi = 2^E,
// S += phi^T [V, 1] (V transposed through wave-private LDS).  The wave partials of a
// feature group are merged in LDS after rescaling to the largest c_f.  Output (float32):
//   gs[bh][t][row][f], row = 32 ct + rho holds value column 32 ct + vperm(rho) (ct < d/32),
//   row d holds the ones column (S_1);  gc[bh][t][f] = c_f (log2 units).
// Workgroup ids are laid out so the feature slices of one (bh, t) share an XCD (and its L2
// copy of K and V): block b runs on XCD b % 8.
// ======================================================================================
// KW waves per workgroup, NTW 32-feature tiles per wave, MINB workgroups per CU the
// registers must allow.  OCC: the causal bf16 d = 64 key side as four-wave workgroups at
// three waves per SIMD, which sum S_1 by bf16 dot products instead of a ones-column MFMA
// tile to free that tile's registers (the compiler still spills a few); its default runs
// eight-wave workgroups at two waves per SIMD.
template <class T, int D, bool OCC = false> struct KvCfg;
template <> struct KvCfg<bf16, 64, false> { static constexpr int KW = 8, NTW = 2, MINB = 1; };
template <> struct KvCfg<bf16, 64, true> { static constexpr int KW = 4, NTW = 2, MINB = 3; };
template <bool O> struct KvCfg<bf16, 128, O> { static constexpr int KW = 4, NTW = 1, MINB = 1; };
template <bool O> struct KvCfg<float, 64, O> { static constexpr int KW = 4, NTW = 1, MINB = 1; };
template <bool O> struct KvCfg<float, 128, O> { static constexpr int KW = 4, NTW = 1, MINB = 1; };

// With one range per kv head and bf16 data (img_s != nullptr) the workgroup writes, instead
// of gs / gc, the readout's LDS images of its 64 features: S'^T rows in readout order, the
// bias operands of c_f, and (one head of each W) the fp16 W rows.
// SEG (causal segments): each wave owns one whole segment instead of a share of a range,
// so the position groups of a workgroup are PG consecutive segments and every wave writes
// its own partial with its own stabilisers (no merge, no workgroup barrier).
// RELU: the feature map ReLU(W k) in place of the exponential (no norm term, no
// stabiliser: c_f = 0 throughout, so the partials merge as plain sums).  W keeps its
// log2 e scale, which both sides share and the ratio cancels.
template <class T, int D, bool SEG, bool RELU = false, bool OCC = false>
__global__ void __launch_bounds__((64 * KvCfg<T, D, OCC>::KW), (KvCfg<T, D, OCC>::MINB)) kv_summary_kernel(
    const T* __restrict__ K, const T* __restrict__ V, const float* __restrict__ W, int L, int Hkv, int Hw, int m,
    int R, int T_ranges, int n_units, float* __restrict__ gs, float* __restrict__ gc, char* __restrict__ img_w,
    char* __restrict__ img_s, char* __restrict__ img_cb) {
  using P = Prec<T>;
  using frag = typename P::frag;
  using wfrag = typename P::wfrag;
  static_assert(SEG || !OCC, "the three-waves-per-SIMD form is the segment path's");
  constexpr int KW = KvCfg<T, D, OCC>::KW, NTW = KvCfg<T, D, OCC>::NTW;
  constexpr int FG = 2 / NTW;   // feature groups per workgroup (64 features)
  constexpr int PG = KW / FG;   // position groups
  constexpr int NKC = D / P::KS;
  // MFMA accumulator tiles: the value columns, then (except in the OCC form, which sums
  // S_1 by dot products to free the tile's registers) the ones column
  constexpr int NDV = D / 32;
  constexpr int NDT = NDV + (OCC ? 0 : 1);
  constexpr int LDV = Ld<T>::template V<D>;
  constexpr int ACC = NTW * NDT * 1024;  // floats of one wave's partial (fragment order)
  __shared__ __attribute__((aligned(16))) T Vl[KW][32 * LDV];
  __shared__ __attribute__((aligned(16))) float Red[(PG / 2) * FG][ACC];
  __shared__ __attribute__((aligned(16))) float Cs[KW][32 * NTW];
  // bf16, d = 64: the slice's fp16 W rows live in LDS (shared by the waves) and blocks are
  // loaded at their start, not one block ahead, which keeps a wave within 256 registers
  // (two waves per SIMD hide each other's latency)
  constexpr bool WLDS = sizeof(T) == 2 && D == 64;
  constexpr int LDWL = D + 8;
  __shared__ __attribute__((aligned(16))) typename P::welem Wl[WLDS ? 64 * LDWL : 1];

  const int NFS = m / 64;
  const int xcd = blockIdx.x & 7, kq = blockIdx.x >> 3;
  const int slice = kq % NFS, unit = (kq / NFS) * 8 + xcd;
  if (unit >= n_units) return;
  const int wave = threadIdx.x >> 6, l = lane_id(), col = l & 31, g = l >> 5;
  const int fgi = wave % FG, pgi = wave / FG;
  const int TG = SEG ? (T_ranges + PG - 1) / PG : T_ranges;  // units per kv head
  const int bh = unit / TG, hkv = bh % Hkv;
  const int t = SEG ? (unit % TG) * PG + pgi : unit % TG;
  const int f0 = slice * 64 + fgi * 32 * NTW;
  const float* Wh = W + (size_t)(Hw == 1 ? 0 : hkv) * m * D;
  const T* Kh = K + (size_t)bh * L * D;
  const T* Vh = V + (size_t)bh * L * D;
  T* vl = Vl[wave];

  wfrag wf[WLDS ? 1 : NTW][WLDS ? 1 : NKC];
  if constexpr (WLDS) {
    // rows slice*64 .. +63 scaled by log2 e, 8 elements per thread and step
    for (int c = threadIdx.x; c < 64 * D / 8; c += blockDim.x) {
      const int r = c / (D / 8), c0 = (c % (D / 8)) * 8;
      const float* src = Wh + (size_t)(slice * 64 + r) * D + c0;
      const f32x4 a = *reinterpret_cast<const f32x4*>(src), b = *reinterpret_cast<const f32x4*>(src + 4);
      wfrag v;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = (typename P::welem)(a[j] * kLog2e);
        v[j + 4] = (typename P::welem)(b[j] * kLog2e);
      }
      *reinterpret_cast<wfrag*>(&Wl[r * LDWL + c0]) = v;
    }
    __syncthreads();
  }
  if (SEG && t >= T_ranges) return;  // after the workgroup-wide W staging
  if constexpr (!WLDS) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) load_w_frag(Wh + (size_t)(f0 + 32 * nt + col) * D, kc, g, wf[nt][kc]);
  }
  // the W operand of feature tile nt, contraction slab kc
  auto wop = [&](int nt, int kc) -> wfrag {
    if constexpr (WLDS)
      return *reinterpret_cast<const wfrag*>(&Wl[(f0 - slice * 64 + 32 * nt + col) * LDWL + 16 * kc + 8 * g]);
    else
      return wf[nt][kc];
  };

  float cst[NTW];  // stabiliser of this lane's feature (log2 units)
  wfrag biasB[NTW];
  f32x16 S[NTW][NDT];
  // OCC: S_1 of feature 32 nt + col over this lane half's keys, summing the same rounded phi
  // values the S_v products take; the two lane halves are added at the end
  float s1[NTW];
  auto frag_sum = [](const frag& x, float acc) {
    if constexpr (sizeof(T) == 2) {
      bf16x2 one2;
      one2[0] = one2[1] = (bf16)1.f;
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        bf16x2 v2;
        v2[0] = x[j];
        v2[1] = x[j + 1];
        acc = __builtin_amdgcn_fdot2_f32_bf16(v2, one2, acc, false);
      }
      return acc;
    } else {
      return acc + x;
    }
  };
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
  const int Rw = SEG ? R : ((R + 32 * PG - 1) / (32 * PG)) * 32;
  const int wb = SEG ? pb : pb + pgi * Rw, we = min(wb + Rw, pe);
  constexpr int EPC = 16 / sizeof(T);   // elements per 16-byte chunk
  constexpr int CPR = D / EPC;          // chunks per row
  constexpr int CPL = 32 * CPR / 64;    // chunks per lane per block
  // Block loads are software-pipelined: block p0 + 32 is fetched into registers while
  // block p0 is computed.  Loads are clamped into the range (rows past its end are real
  // data whose features get the kMaskedRow bias, i.e. phi = 0).
  f32x4 vn[CPL];
  frag kn[NKC];
  // bf16: raw buffer loads range-checked against the head (rows past L read as zero; the
  // block offset is in the vector offset, which the check covers), so the per-lane offsets
  // are fixed and a block costs one add per tensor.
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, L * D * (int)sizeof(T), kBufWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, L * D * (int)sizeof(T), kBufWord3);
  auto fetch = [&](int q0) {
    if constexpr (sizeof(T) == 2) {
      const int vo = q0 * D * 2 + 16 * l, ko = (q0 + col) * D * 2 + 16 * g;
#pragma unroll
      for (int i = 0; i < CPL; ++i)
        vn[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, vo + 1024 * i, 0, 0));
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
        kn[kc] = __builtin_bit_cast(frag, __builtin_amdgcn_raw_buffer_load_b128(krs, ko + 32 * kc, 0, 0));
    } else {
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = l + 64 * i, row = min(q0 + c / CPR, we - 1), c0 = (c % CPR) * EPC;
        vn[i] = *reinterpret_cast<const f32x4*>(Vh + (size_t)row * D + c0);
      }
      const int krow = min(q0 + col, we - 1);
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) kn[kc] = load_frag_k(Kh + (size_t)krow * D, kc, g);
    }
  };

  // One 32-position block.  Stabiliser modes: 0 = first block of the fast pass (c_f :=
  // this block's maximum), 1 = fast pass (c_f fixed: no VALU work on the accumulators),
  // 2 = fallback pass (running maximum, moved lazily, accumulators rescaled).
  auto block = [&](int p0, auto mode_tag) {
    constexpr int MODE = decltype(mode_tag)::value;
    if constexpr (WLDS) fetch(p0);
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
    wfrag kf[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) kf[kc] = to_wfrag(kn[kc]);
    if constexpr (!WLDS) fetch(min(p0 + 32, we - 1));
    // the W contraction first: the norm and the bias operand are built while it runs
    f32x16 c1[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      c1[nt] = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) c1[nt] = mma(kf[kc], wop(nt, kc), c1[nt]);
    }
    float rb = kMaskedRow;  // keys past the range: features exactly 0
    if constexpr (RELU) {
      if (p0 + col < we) rb = 0.f;
    } else {
      float nrm = sumsq(kf);
      nrm += partner32(nrm);
      if (p0 + col < we) rb = 0.5f * kLog2e * nrm;
    }
    const wfrag biasA = bias_rows(rb, g, wfrag{});
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) c1[nt] = mma(biasA, biasB[nt], c1[nt]);

    if constexpr (RELU) {
      // no stabiliser
    } else if constexpr (MODE == 0) {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        float mx = c1[nt][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, c1[nt][r]);
        mx = fmaxf(mx, partner32(mx));
        cst[nt] = mx;
#pragma unroll
        for (int r = 0; r < 16; ++r) c1[nt][r] -= mx;
        biasB[nt] = bias_cols(mx, g, wfrag{});
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
          biasB[nt] = bias_cols(cst[nt], g, wfrag{});
          if (!first) {
            const float fct = fast_exp2(-shift);
            if constexpr (OCC) s1[nt] *= fct;
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
      for (int r = 0; r < 16; ++r) e[r] = RELU ? fmaxf(c1[nt][r], 0.f) : fast_exp2(c1[nt][r]);
      acc_to_frags(e, pa[nt]);
      if constexpr (OCC) {
        float sum = s1[nt];
#pragma unroll
        for (int h = 0; h < P::NF32; ++h) sum = frag_sum(pa[nt][h], sum);
        s1[nt] = sum;
      }
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int h = 0; h < P::NF32; ++h) {
        const frag vb = dt < NDV ? lds_frag_rows(vl, LDV, 0, 32 * dt, h) : ones;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) S[nt][dt] = mma(pa[nt][h], vb, S[nt][dt]);
      }
    asm volatile("" ::: "memory");  // this block's LDS reads before the next block's writes
  };
  auto reset = [&]() {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      cst[nt] = RELU ? 0.f : -INFINITY;
      biasB[nt] = bias_cols(0.f, g, wfrag{});
      s1[nt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) S[nt][dt] = zero16();
    }
  };

  // Fast pass: stabiliser fixed at the first block's maximum.  Only an overflow (a later
  // block more than ~2^100 above the first) makes it non-finite; then the range is redone
  // with the running maximum.
  reset();
  if (wb < we) {
    if constexpr (!WLDS) fetch(wb);
    block(wb, std::integral_constant<int, 0>{});
    for (int p0 = wb + 32; p0 < we; p0 += 32) block(p0, std::integral_constant<int, 1>{});
  }
  float chk = 0.f;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    if constexpr (OCC) chk += s1[nt];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) chk += S[nt][dt][r];
  }
  if (!RELU && wave_any(!(chk - chk == 0.f))) {
    reset();
    if constexpr (!WLDS) fetch(wb);
    for (int p0 = wb; p0 < we; p0 += 32) block(p0, std::integral_constant<int, 2>{});
  }

  // The partial of unit_off (float32 gs rows in vperm order, row D the ones column, and
  // gc) relative to the stabilisers cmx of this lane's C1 features; in the OCC form s1t holds
  // S_1 of feature 32 nt + col with both lane halves added.
  // causal segment summaries (SEG) are stored in the problem's summary type (bf16 for bf16
  // problems), range partials in float32
  auto store_partial = [&](size_t unit_off, const float (&cmx)[NTW], const float (&s1t)[NTW]) {
    using GST = std::conditional_t<SEG, typename SumOf<T>::type, float>;
    GST* out_s = reinterpret_cast<GST*>(gs) + unit_off * (size_t)(D + 1) * m;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
      for (int dt = 0; dt < NDV; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 v = {S[nt][dt][4 * r4], S[nt][dt][4 * r4 + 1], S[nt][dt][4 * r4 + 2], S[nt][dt][4 * r4 + 3]};
          store_sum4(out_s + (size_t)(32 * dt + col) * m + f0 + 32 * nt + 8 * r4 + 4 * g, v);
        }
      if constexpr (OCC) {
        if (g == 0) out_s[(size_t)D * m + f0 + 32 * nt + col] = (GST)s1t[nt];
      } else if (col == 0) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 v = {S[nt][NDV][4 * r4], S[nt][NDV][4 * r4 + 1], S[nt][NDV][4 * r4 + 2], S[nt][NDV][4 * r4 + 3]};
          store_sum4(out_s + (size_t)D * m + f0 + 32 * nt + 8 * r4 + 4 * g, v);
        }
      }
      if (g == 0) gc[unit_off * m + f0 + 32 * nt + col] = cmx[nt];
    }
  };
  if constexpr (SEG) {
    float s1t[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) s1t[nt] = OCC ? s1[nt] + partner32(s1[nt]) : 0.f;
    store_partial((size_t)bh * T_ranges + t, cst, s1t);
    return;
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
  // registers 4 r4 .. 4 r4 + 3 hold features 32 nt + 8 r4 + 4 g + (0..3): one 16-byte read
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int fb = 32 * nt + 8 * r4 + 4 * g;
      const f32x4 own = *reinterpret_cast<const f32x4*>(&Cs[wave][fb]);
      f32x4 cm = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int q = 0; q < PG; ++q) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(&Cs[q * FG + fgi][fb]);
#pragma unroll
        for (int i = 0; i < 4; ++i) cm[i] = fmaxf(cm[i], o[i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sc = cm[i] == -INFINITY ? 0.f : fast_exp2(own[i] - cm[i]);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) S[nt][dt][4 * r4 + i] *= sc;
      }
    }
  // partial exchange in 16-byte pieces: piece (nt, dt, r4) of lane l at ((nt NDT + dt) 4 + r4) 256 + 4 l
  auto dump = [&](float* dst) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *reinterpret_cast<f32x4*>(dst + ((nt * NDT + dt) * 4 + r4) * 256 + 4 * l) =
              f32x4{S[nt][dt][4 * r4], S[nt][dt][4 * r4 + 1], S[nt][dt][4 * r4 + 2], S[nt][dt][4 * r4 + 3]};
  };
  auto absorb = [&](const float* src) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(src + ((nt * NDT + dt) * 4 + r4) * 256 + 4 * l);
#pragma unroll
          for (int i = 0; i < 4; ++i) S[nt][dt][4 * r4 + i] += v[i];
        }
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
  if constexpr (sizeof(T) == 2 && !RELU) {
    if (img_s != nullptr) {
      // The image holds S_v / S_1 per feature (rows already in vperm order: V was staged
      // permuted, lane col is row 32 dt + col) and c'_f = c_f + log2 S_1,f, so the readout's
      // denominator is the plain sum of its features.  S_1 (ones column, lane col 0) is
      // spread to the other lanes by shuffles.
      constexpr int LDSS = kImgMP + 8, LDW = D + 8;
      bf16* is = reinterpret_cast<bf16*>(img_s + (size_t)bh * img_s_bytes(D));
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const int ftile = (f0 + 32 * nt) >> 5;
        // S_1 of this lane's register features (held by lane 32 g) and of feature col of the
        // tile (held by lane 32 ((col >> 2) & 1), register 4 (col >> 3) + col % 4)
        float rs1[16], s1col = 0.f;
        const int src = 32 * ((col >> 2) & 1), rcol = 4 * (col >> 3) + (col & 3);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          rs1[r] = __builtin_amdgcn_rcpf(__shfl(S[nt][NDT - 1][r], 32 * g));
          const float v = __shfl(S[nt][NDT - 1][r], src);
          if (r == rcol) s1col = v;
        }
#pragma unroll
        for (int dt = 0; dt < NDT - 1; ++dt) {
          const int row = 32 * dt + col;
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            bf16x4_t v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = (bf16)(S[nt][dt][4 * a + j] * rs1[4 * a + j]);
            *reinterpret_cast<bf16x4_t*>(is + (size_t)row * LDSS + 32 * ftile + 16 * (a >> 1) + 8 * g + 4 * (a & 1)) =
                v;
          }
        }
        const int f = f0 + 32 * nt + col;
        f16x8* icb = reinterpret_cast<f16x8*>(img_cb + (size_t)bh * img_cb_bytes(m));
        if (g == 0) {
          f16x8 cb = zero_frag(f16x8{});
          split3(cmax[nt] + __builtin_amdgcn_logf(s1col), cb, 0);
          cb[3] = cb[4] = cb[5] = (f16)1.f;
          icb[2 * f] = cb;
          icb[2 * f + 1] = zero_frag(f16x8{});
        }
        // one writer per W head: batch 0 (kv head 0 when W is shared)
        if (bh < Hkv && (Hw != 1 || bh == 0)) {
          f16* iw = reinterpret_cast<f16*>(img_w + (size_t)(Hw == 1 ? 0 : hkv) * img_w_bytes(D, m));
#pragma unroll
          for (int kc = 0; kc < NKC; ++kc) *reinterpret_cast<f16x8*>(iw + (size_t)f * LDW + 16 * kc + 8 * g) = wop(nt, kc);
        }
      }
      return;
    }
  }
  const float no_s1[NTW] = {};  // the range path keeps S_1 in its ones tile
  store_partial(unit_off, cmax, no_s1);
}

// ======================================================================================
// kv_summary_bf16: the bidirectional key side for bf16 problems.  Workgroup = (kv head bh,
// position range t, 64-feature slice), 4 waves (one per SIMD).  The waves split the range
// into contiguous position groups; each streams its 32-position blocks with the slice's two
// feature tiles of W (fp16, x log2 e) in registers:
//   E = K_blk W^T - |k|^2 log2e / 2 - c_f   (4 or 8 MFMAs per tile + one bias MFMA)
//   phi = 2^E (bf16),  S_v += phi^T V  (V transposed through wave-private LDS),
//   S_1 += sum over the block's keys of phi (VALU dot products of the same bf16 values).
// K and V rows of the next NPF blocks are in flight in registers while a block is computed
// (global-memory latency is several blocks' worth of work).  c_f is fixed at the first
// block's per-feature maximum; only an overflow makes the fast pass non-finite, and then the
// wave redoes its positions with a lazily moved running maximum.  The four waves' partials
// are merged in LDS after rescaling to the largest c_f; wave 0 writes either the readout's
// LDS images (one range per head) or float32 partials gs / gc in the layout of
// kv_summary_kernel.
// ======================================================================================
template <int D> struct KvBf16 {
  static constexpr int NW = 4;                    // waves per workgroup
  static constexpr int NPF = D == 64 ? 3 : 2;     // blocks in flight per wave
  static constexpr int NKC = D / 16;              // 16-deep contraction slabs over d
  static constexpr int NDV = D / 32;              // value-column tiles
  static constexpr int LDV = D + 16;              // V staging rows (transposed reads)
  static constexpr int CPL = 32 * (D / 8) / 64;   // 16-byte V chunks per lane and block
  static constexpr int PART = 2 * NDV * 16 + 2;   // floats of one lane's partial (S_v, S_1)
  static constexpr int VBYTES = NW * 32 * LDV * 2;
  static constexpr int MBYTES = (NW - 1) * 64 * PART * 4;
  static constexpr int LDSB = VBYTES > MBYTES ? VBYTES : MBYTES;
};

template <int D>
__global__ void __launch_bounds__(64 * KvBf16<D>::NW) kv_summary_bf16_kernel(
    const bf16* __restrict__ K, const bf16* __restrict__ V, const float* __restrict__ W, int L, int Hkv, int Hw,
    int m, int R, int T_ranges, int n_units, float* __restrict__ gs, float* __restrict__ gc, char* __restrict__ img_w,
    char* __restrict__ img_s, char* __restrict__ img_cb) {
  using Cfg = KvBf16<D>;
  constexpr int NW = Cfg::NW, NPF = Cfg::NPF, NKC = Cfg::NKC, NDV = Cfg::NDV, LDV = Cfg::LDV, CPL = Cfg::CPL;
  constexpr int PART = Cfg::PART;
  // V staging during the stream; the merge buffers of waves 1..NW-1 afterwards
  __shared__ __attribute__((aligned(16))) char Sh[Cfg::LDSB];
  __shared__ __attribute__((aligned(16))) float Cs[NW][64];

  const int NFS = m / 64;
  const int xcd = blockIdx.x & 7, kq = blockIdx.x >> 3;
  const int slice = kq % NFS, unit = (kq / NFS) * 8 + xcd;
  if (unit >= n_units) return;
  const int wave = threadIdx.x >> 6, l = lane_id(), col = l & 31, g = l >> 5;
  const int bh = unit / T_ranges, hkv = bh % Hkv, t = unit % T_ranges;
  const int f0 = slice * 64;
  const float* Wh = W + (size_t)(Hw == 1 ? 0 : hkv) * m * D;
  bf16* vl = reinterpret_cast<bf16*>(Sh) + wave * 32 * LDV;

  f16x8 wf[2][NKC];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) load_w_frag(Wh + (size_t)(f0 + 32 * nt + col) * D, kc, g, wf[nt][kc]);

  const int pb = t * R, pe = min(pb + R, L);
  const int Rw = ((R + 32 * NW - 1) / (32 * NW)) * 32;
  const int wb = pb + wave * Rw, we = min(wb + Rw, pe);
  const int nblk = wb < we ? (we - wb + 31) / 32 : 0;

  // Raw buffer loads range-checked against the head (rows past L read as zero); a block's
  // offset sits in the vector offset, which the check covers.
  const bf16* Kh = K + (size_t)bh * L * D;
  const bf16* Vh = V + (size_t)bh * L * D;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, L * D * 2, kBufWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, L * D * 2, kBufWord3);
  struct Blk {
    bf16x8 k[NKC];
    f32x4 v[CPL];
  };
  auto fetch = [&](int p0, Blk& b) {
    const int ko = (p0 + col) * D * 2 + 16 * g, vo = p0 * D * 2 + 16 * l;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
      b.k[kc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, ko + 32 * kc, 0, 0));
#pragma unroll
    for (int i = 0; i < CPL; ++i)
      b.v[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, vo + 1024 * i, 0, 0));
  };

  float cst[2];            // stabiliser of this lane's feature 32 nt + col (log2 units)
  f16x8 biasB[2];
  f32x16 S[2][NDV];
  float s1[2];             // this lane's half of the block keys' sum of phi, feature 32 nt + col
  auto reset = [&]() {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      cst[nt] = -INFINITY;
      biasB[nt] = bias_cols(0.f, g, f16x8{});
      s1[nt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < NDV; ++dt) S[nt][dt] = zero16();
    }
  };
  bf16x2 one2;
  one2[0] = one2[1] = (bf16)1.f;

  // One 32-position block.  MODE 0: first block (c_f := its per-feature maximum); 1: c_f
  // fixed; 2: fallback, running maximum moved lazily with the accumulators rescaled.
  auto block = [&](int p0, const Blk& b, auto mode_tag) {
    constexpr int MODE = decltype(mode_tag)::value;
    // V rows to LDS with the column permutation vperm_inv inside each 32-column tile
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = l + 64 * i, row = c / (D / 8), c0 = (c % (D / 8)) * 8;
      bf16* drow = vl + row * LDV + (c0 & ~31);
      *reinterpret_cast<float2*>(drow + vperm_inv(c0 & 31)) = float2{b.v[i][0], b.v[i][1]};
      *reinterpret_cast<float2*>(drow + vperm_inv((c0 & 31) + 4)) = float2{b.v[i][2], b.v[i][3]};
    }
    f16x8 kf[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) kf[kc] = to_wfrag(b.k[kc]);
    f32x16 c1[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      c1[nt] = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) c1[nt] = mma(kf[kc], wf[nt][kc], c1[nt]);
    }
    float nrm = sumsq(kf);
    nrm += partner32(nrm);
    const float rb = p0 + col < we ? 0.5f * kLog2e * nrm : kMaskedRow;
    const f16x8 biasA = bias_rows(rb, g, f16x8{});
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) c1[nt] = mma(biasA, biasB[nt], c1[nt]);

    if constexpr (MODE == 0) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float mx = c1[nt][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, c1[nt][r]);
        mx = fmaxf(mx, partner32(mx));
        cst[nt] = mx;
#pragma unroll
        for (int r = 0; r < 16; ++r) c1[nt][r] -= mx;
        biasB[nt] = bias_cols(mx, g, f16x8{});
      }
    } else if constexpr (MODE == 2) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
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
          biasB[nt] = bias_cols(cst[nt], g, f16x8{});
          if (!first) {
            const float fct = fast_exp2(-shift);
            s1[nt] *= fct;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float fr = __shfl(fct, 8 * (r >> 2) + 4 * g + (r & 3));
#pragma unroll
              for (int dt = 0; dt < NDV; ++dt) S[nt][dt][r] *= fr;
            }
          }
        } else if (first) {
          cst[nt] = 0.f;  // block maximum is exactly 0
        }
      }
    }

    bf16x8 pa[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x16 e;
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = fast_exp2(c1[nt][r]);
      acc_to_frags(e, pa[nt]);
      float sum = s1[nt];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          bf16x2 v2;
          v2[0] = pa[nt][h][j];
          v2[1] = pa[nt][h][j + 1];
          sum = __builtin_amdgcn_fdot2_f32_bf16(v2, one2, sum, false);
        }
      s1[nt] = sum;
    }
#pragma unroll
    for (int dt = 0; dt < NDV; ++dt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8 vb = lds_frag_rows(vl, LDV, 0, 32 * dt, h);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) S[nt][dt] = mma(pa[nt][h], vb, S[nt][dt]);
      }
    asm volatile("" ::: "memory");  // this block's LDS reads before the next block's writes
  };

  // Fast pass: NPF blocks in flight, the ring of registers unrolled so that it rotates
  // statically.  Every step issues its fetch (past the last block it re-reads the first),
  // so the number of loads in flight is the same on every path and the waits for a block
  // leave the later blocks' loads outstanding.
  reset();
  if (nblk > 0) {
    auto pos = [&](int bi) { return bi < nblk ? wb + 32 * bi : wb; };
    Blk ring[NPF];
#pragma unroll
    for (int j = 0; j < NPF; ++j) fetch(pos(j), ring[j]);
    // block 0 sets the stabilisers
    block(wb, ring[0], std::integral_constant<int, 0>{});
    fetch(pos(NPF), ring[0]);
    int bi = 1;
    for (; bi + NPF <= nblk; bi += NPF) {
#pragma unroll
      for (int j = 0; j < NPF; ++j) {
        const int slot = (1 + j) % NPF;  // block bi + j sits in slot (bi + j) % NPF, bi = 1 mod NPF
        block(wb + 32 * (bi + j), ring[slot], std::integral_constant<int, 1>{});
        fetch(pos(bi + j + NPF), ring[slot]);
      }
    }
#pragma unroll
    for (int j = 0; j < NPF; ++j)
      if (bi + j < nblk) block(wb + 32 * (bi + j), ring[(1 + j) % NPF], std::integral_constant<int, 1>{});
  }
  float chk = s1[0] + s1[1];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int dt = 0; dt < NDV; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) chk += S[nt][dt][r];
  if (wave_any(!(chk - chk == 0.f))) {
    reset();
    for (int bi = 0; bi < nblk; ++bi) {
      Blk bl;
      fetch(wb + 32 * bi, bl);
      block(wb + 32 * bi, bl, std::integral_constant<int, 2>{});
    }
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) s1[nt] += partner32(s1[nt]);

  // ---- merge the waves' partials (same features, different positions) ---------------
  if (g == 0) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) Cs[wave][32 * nt + col] = cst[nt];
  }
  __syncthreads();  // also: every wave's V staging reads are done
  float cmax[2];    // merged stabiliser of this lane's feature 32 nt + col
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    cmax[nt] = -INFINITY;
#pragma unroll
    for (int q = 0; q < NW; ++q) cmax[nt] = fmaxf(cmax[nt], Cs[q][32 * nt + col]);
    s1[nt] *= cmax[nt] == -INFINITY ? 0.f : fast_exp2(cst[nt] - cmax[nt]);
  }
  // registers 4 r4 .. 4 r4 + 3 hold features 32 nt + 8 r4 + 4 g + (0..3)
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int fb = 32 * nt + 8 * r4 + 4 * g;
      const f32x4 own = *reinterpret_cast<const f32x4*>(&Cs[wave][fb]);
      f32x4 cm = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(&Cs[q][fb]);
#pragma unroll
        for (int i = 0; i < 4; ++i) cm[i] = fmaxf(cm[i], o[i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sc = cm[i] == -INFINITY ? 0.f : fast_exp2(own[i] - cm[i]);
#pragma unroll
        for (int dt = 0; dt < NDV; ++dt) S[nt][dt][4 * r4 + i] *= sc;
      }
    }
  // partial exchange: piece (nt, dt, r4) of lane l at ((nt NDV + dt) 4 + r4) 256 + 4 l, then
  // s1 at 2 NDV 16 64 + 2 l
  float* mb = reinterpret_cast<float*>(Sh);
  if (wave > 0) {
    float* dst = mb + (size_t)(wave - 1) * 64 * PART;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int dt = 0; dt < NDV; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *reinterpret_cast<f32x4*>(dst + ((nt * NDV + dt) * 4 + r4) * 256 + 4 * l) =
              f32x4{S[nt][dt][4 * r4], S[nt][dt][4 * r4 + 1], S[nt][dt][4 * r4 + 2], S[nt][dt][4 * r4 + 3]};
    *reinterpret_cast<float2*>(dst + 2 * NDV * 16 * 64 + 2 * l) = float2{s1[0], s1[1]};
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int q = 1; q < NW; ++q) {
    const float* src = mb + (size_t)(q - 1) * 64 * PART;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int dt = 0; dt < NDV; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(src + ((nt * NDV + dt) * 4 + r4) * 256 + 4 * l);
#pragma unroll
          for (int i = 0; i < 4; ++i) S[nt][dt][4 * r4 + i] += v[i];
        }
    const float2 o = *reinterpret_cast<const float2*>(src + 2 * NDV * 16 * 64 + 2 * l);
    s1[0] += o.x;
    s1[1] += o.y;
  }

  const size_t unit_off = (size_t)bh * T_ranges + t;
  if (img_s != nullptr) {
    // The image holds S_v / S_1 per feature (rows already in vperm order: V was staged
    // permuted, lane col is row 32 dt + col) and c'_f = c_f + log2 S_1,f, so the readout's
    // denominator is the plain sum of its features.  S_1 of feature 32 nt + j sits in lane j.
    constexpr int LDSS = kImgMP + 8, LDW = D + 8;
    bf16* is = reinterpret_cast<bf16*>(img_s + (size_t)bh * img_s_bytes(D));
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int ftile = (f0 + 32 * nt) >> 5;
      float rs1[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) rs1[r] = __builtin_amdgcn_rcpf(__shfl(s1[nt], 8 * (r >> 2) + 4 * g + (r & 3)));
#pragma unroll
      for (int dt = 0; dt < NDV; ++dt) {
        const int row = 32 * dt + col;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          bf16x4_t v;
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = (bf16)(S[nt][dt][4 * a + j] * rs1[4 * a + j]);
          *reinterpret_cast<bf16x4_t*>(is + (size_t)row * LDSS + 32 * ftile + 16 * (a >> 1) + 8 * g + 4 * (a & 1)) = v;
        }
      }
      const int f = f0 + 32 * nt + col;
      f16x8* icb = reinterpret_cast<f16x8*>(img_cb + (size_t)bh * img_cb_bytes(m));
      if (g == 0) {
        f16x8 cb = zero_frag(f16x8{});
        split3(cmax[nt] + __builtin_amdgcn_logf(s1[nt]), cb, 0);
        cb[3] = cb[4] = cb[5] = (f16)1.f;
        icb[2 * f] = cb;
        icb[2 * f + 1] = zero_frag(f16x8{});
      }
      // one writer per W head: batch 0 (kv head 0 when W is shared)
      if (bh < Hkv && (Hw != 1 || bh == 0)) {
        f16* iw = reinterpret_cast<f16*>(img_w + (size_t)(Hw == 1 ? 0 : hkv) * img_w_bytes(D, m));
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) *reinterpret_cast<f16x8*>(iw + (size_t)f * LDW + 16 * kc + 8 * g) = wf[nt][kc];
      }
    }
    return;
  }
  // float32 partial: gs rows in vperm order (lane col is row 32 dt + col), row D the ones
  // column (S_1), gc the stabilisers
  float* out_s = gs + unit_off * (size_t)(D + 1) * m;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
    for (int dt = 0; dt < NDV; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 v = {S[nt][dt][4 * r4], S[nt][dt][4 * r4 + 1], S[nt][dt][4 * r4 + 2], S[nt][dt][4 * r4 + 3]};
        *reinterpret_cast<f32x4*>(out_s + (size_t)(32 * dt + col) * m + f0 + 32 * nt + 8 * r4 + 4 * g) = v;
      }
    if (g == 0) {
      out_s[(size_t)D * m + f0 + 32 * nt + col] = s1[nt];
      gc[unit_off * m + f0 + 32 * nt + col] = cmax[nt];
    }
  }
}

// s_waitcnt immediate (gfx9 encoding) that waits for vector memory only: vmcnt <= n.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

typedef __attribute__((address_space(3))) void lds_void_t;

// ======================================================================================
// readout (bidirectional).  Grid (workgroups per kv head, B*Hkv), NWAVE waves; each wave
// owns QN x 32 query rows per step (the G query heads of a kv head are G*L contiguous
// rows).  LDS holds W (fp16 for bf16 problems) and S^T for a pass of MP features: rows are value columns in
// vperm order then the ones row; within a 32-feature tile the features are reordered so
// one lane's 8 operand values are contiguous.  S is summed over the position ranges and
// rescaled to the head's largest stabiliser while staged; with more than one pass W and S
// are re-staged per query tile.
// ======================================================================================
template <class T, int D> struct ReadoutCfg;
template <int D> struct ReadoutCfg<bf16, D> {  // features beyond the fast readout's LDS
  static constexpr int MP = 128;
  static constexpr int LDW = D + 8;
  static constexpr int LDS = MP + 8;
  static constexpr int NWAVE = 8;
  static constexpr int QN = 1;
};
template <int D> struct ReadoutCfg<float, D> {
  static constexpr int MP = D == 64 ? 128 : 64;
  static constexpr int LDW = D + 1;
  static constexpr int LDS = MP + 1;
  static constexpr int NWAVE = 4;
  static constexpr int QN = 1;  // f32 MFMAs are slow: more waves, shorter chains
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

// RELU: the feature map ReLU(W q) with the key side's RELU partials (no stabilisers); a
// row whose denominator is 0 (no positive weight) is written as zeros.
template <class T, int D, bool RELU = false>
__global__ void __launch_bounds__((64 * ReadoutCfg<T, D>::NWAVE))
    readout_kernel(const T* __restrict__ Q, const float* __restrict__ W, const float* __restrict__ gs,
                   const float* __restrict__ gc, T* __restrict__ out, int L, int Hq, int Hkv, int Hw, int m,
                   int T_ranges) {
  using P = Prec<T>;
  using frag = typename P::frag;
  using wfrag = typename P::wfrag;
  using welem = typename P::welem;
  using Cfg = ReadoutCfg<T, D>;
  constexpr int NKC = D / P::KS;
  constexpr int NDT = D / 32 + 1;
  // RELU with bf16 data stages up to 256 features per pass (W and S^T in 140 KB of LDS at
  // d = 128): with m <= 256 they are staged once, not once per query tile
  constexpr int MP = RELU && sizeof(T) == 2 ? 256 : Cfg::MP;
  constexpr int LDW = Cfg::LDW, LDSS = RELU && sizeof(T) == 2 ? MP + 8 : Cfg::LDS, QN = Cfg::QN;
  constexpr int NT = 64 * Cfg::NWAVE;
  constexpr int SROWS = D + 1;
  constexpr int TILE = Cfg::NWAVE * QN * 32;
  __shared__ __attribute__((aligned(16))) welem Wl[MP * LDW];
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
        for (int i = 0; i < 4; ++i) Wl[fi * LDW + k4 + i] = (welem)(x[u][i] * kLog2e);
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
    wfrag qf[QN][NKC];
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      myrow[q] = tile * TILE + (size_t)(wave * QN + q) * 32 + col;
      valid[q] = myrow[q] < rows;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
        qf[q][kc] = valid[q] ? to_wfrag(load_frag_k(Qb + myrow[q] * D, kc, g)) : zero_frag(wfrag{});
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
      for (int kc = 0; kc < NKC; ++kc) {
        const wfrag a = load_frag_k(&Wl[(32 * ft + col) * LDW], kc, g);
#pragma unroll
        for (int q = 0; q < QN; ++q) c1[q] = mma(a, qf[q][kc], c1[q]);
      }
      if constexpr (decltype(bias_tag)::value) {
        const wfrag unitA = bias_unit_rows(g, wfrag{});
#pragma unroll
        for (int q = 0; q < QN; ++q) c1[q] = mma(unitA, bias_cols(M[q], g, wfrag{}), c1[q]);
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
          e[r] = RELU ? fmaxf(c1[q][r], 0.f) : fast_exp2(decltype(sub_tag)::value ? c1[q][r] - M[q] : c1[q][r]);
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
        if (RELU) {
          for (int ft = 0; ft < nft; ++ft) {
            f32x16 c1[QN];
            c1_tile(ft, c1, No{});
            readout_tile(ft, c1, No{});
          }
        } else if (fast) {
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
    if (!RELU && __syncthreads_or(bad)) run(false);

#pragma unroll
    for (int q = 0; q < QN; ++q) {
      float den = acc[q][NDT - 1][0];
      const float dp = partner32(den);
      den = g ? dp : den;
      const float inv = RELU ? (den > 0.f ? 1.f / den : 0.f) : 1.f / den;
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
// readout for bf16 problems (bidirectional).  1-D grid: workgroup b runs on XCD b % 8 and
// all workgroups of a kv head share one XCD (and its L2 copy of W and S).  NWAVE waves,
// each streaming its own chunks of 32 QN query rows (the G query heads of a kv head are G*L
// contiguous rows) with no workgroup barrier between chunks; the next chunk's Q is loaded
// while the current one is computed.
// LDS: W * log2e in fp16, S'^T in bf16 (rows: value columns in vperm order, the ones row,
// then a zero row; features reordered within 32-feature tiles so one lane's 8 operand
// values are contiguous) and per feature the bias operand carrying its key stabiliser c_f.
// The key side leaves S_f = 2^c_f S'_f per position range; here c_f = max over ranges and
// S'_f = sum_t 2^(c_tf - c_f) S'_tf.  Instead of rescaling S to one head-wide constant, c_f
// goes into the query exponent: phi_q,f = 2^(w_f.q log2e + c_f - M_q), M_q the row
// stabiliser, so the readout uses S' directly.
// Each wave handles QN 32-row query tiles per chunk, so every W and S' fragment read
// from LDS feeds QN MFMAs and the W contractions of the tiles form independent chains.
// ======================================================================================
template <int D> struct RoBf16 {
  static constexpr int MP = kImgMP;               // most features (m <= MP)
  static constexpr int LDW = D + 8;               // fp16 W rows
  static constexpr int LDSS = MP + 8;             // bf16 S'^T rows
  static constexpr int NWAVE = 8;                 // waves per workgroup
  static constexpr int QN = 1;  // 32-row query tiles per wave and chunk (more, shorter chunks)
};

// B operand of the query bias MFMA: picks up c_f (A slots 0-2) and adds -M (slots 3-5).
__device__ __forceinline__ f16x8 qbias_cols(float M, int g, bool with_m) {
  f16x8 f = zero_frag(f16x8{});
  if (g == 0) {
    f[0] = f[1] = f[2] = (f16)1.f;
    if (with_m) split3(-M, f, 3);
  }
  return f;
}


template <int D>
__global__ void __launch_bounds__(64 * RoBf16<D>::NWAVE)
    readout_bf16_kernel(const bf16* __restrict__ Q, const float* __restrict__ W, const float* __restrict__ gs,
                        const float* __restrict__ gc, const char* __restrict__ img_w,
                        const char* __restrict__ img_s, const char* __restrict__ img_cb, bf16* __restrict__ out, int L,
                        int Hq, int Hkv, int Hw, int m, int T_ranges, int BH, int per_head) {
  using Cfg = RoBf16<D>;
  constexpr int MP = Cfg::MP, LDW = Cfg::LDW, LDSS = Cfg::LDSS, NW = Cfg::NWAVE, QN = Cfg::QN;
  constexpr int NT = 64 * NW;
  constexpr int NKC = D / 16;
  constexpr int NDV = D / 32;  // value-column tiles
  static_assert(LDSS == kImgMP + 8 && MP == kImgMP, "image layout");
  __shared__ __attribute__((aligned(16))) f16 Wl[MP * LDW];
  __shared__ __attribute__((aligned(16))) bf16 Sl[img_s_bytes(D) / 2];  // rows of LDSS (D used)
  __shared__ __attribute__((aligned(16))) f16x8 Cb[2 * MP];  // [feature][lane group]
  __shared__ float Cf[MP], Rs[MP];

  const int xcd = blockIdx.x & 7, kq = blockIdx.x >> 3;
  const int bh = (kq / per_head) * 8 + xcd, sub = kq % per_head;
  if (bh >= BH) return;
  const int b = bh / Hkv, hkv = bh % Hkv, G = Hq / Hkv;
  const int wave = threadIdx.x >> 6, l = lane_id(), col = l & 31, g = l >> 5;
  const int rows = G * L;
  const bf16* Qb = Q + ((size_t)b * Hq + (size_t)hkv * G) * L * D;
  bf16* Ob = out + ((size_t)b * Hq + (size_t)hkv * G) * L * D;
  const float* Wh = W + (size_t)(Hw == 1 ? 0 : hkv) * m * D;
  const float* gsh = gs + (size_t)bh * T_ranges * (D + 1) * m;
  const float* gch = gc + (size_t)bh * T_ranges * m;

  const int nchunks = (rows + 32 * QN - 1) / (32 * QN);
  const int stride = per_head * NW;
  // Q of the wave's next chunk is loaded while the current one is computed (rows past
  // the end are clamped to the last row and never stored).
  bf16x8 qn[QN][NKC];
  auto fetch_q = [&](int ch) {
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      const int row = min((ch * QN + q) * 32 + col, rows - 1);
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) qn[q][kc] = load_frag_k(Qb + (size_t)row * D, kc, g);
    }
  };

  if (img_s != nullptr) {
    // One position range per head: W, S_v / S_1 and the bias rows (c_f + log2 S_1,f)
    // arrive as ready LDS images, copied by LDS DMA in 1 KB blocks spread over the waves.
    auto copy = [&](void* dst, const char* src, int nbytes) {
      for (int k = wave; k < nbytes / 1024; k += NW)
        __builtin_amdgcn_global_load_lds((const void*)(src + 1024 * k + 16 * l),
                                         (lds_void_t*)((char*)dst + 1024 * k), 16, 0, 0);
    };
    copy(Wl, img_w + (size_t)(Hw == 1 ? 0 : hkv) * img_w_bytes(D, m), (int)img_w_bytes(D, m));
    copy(Sl, img_s + (size_t)bh * img_s_bytes(D), (int)img_s_bytes(D));
    copy(Cb, img_cb + (size_t)bh * img_cb_bytes(m), (int)img_cb_bytes(m));
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    fetch_q(min(sub * NW + wave, nchunks - 1));
  } else {
    fetch_q(min(sub * NW + wave, nchunks - 1));
    // Stage W, S_v / S_1 and the bias rows of all m <= MP features from the position-range
    // partials: c_f = max_t c_tf, S_f = sum_t 2^(c_tf - c_f) S_tf (8 loads in flight per
    // thread for the large tables).
    constexpr int U = 8;
    for (int f = threadIdx.x; f < m; f += NT) {
      float c = -INFINITY;
      for (int t = 0; t < T_ranges; ++t) c = fmaxf(c, gch[(size_t)t * m + f]);
      float s1 = 0.f;
      for (int t = 0; t < T_ranges; ++t) s1 += fast_exp2(gch[(size_t)t * m + f] - c) * gsh[((size_t)t * (D + 1) + D) * m + f];
      f16x8 cb = zero_frag(f16x8{});
      split3(c + __builtin_amdgcn_logf(s1), cb, 0);
      cb[3] = cb[4] = cb[5] = (f16)1.f;
      Cb[2 * f] = cb;
      Cb[2 * f + 1] = zero_frag(f16x8{});
      Cf[f] = c;
      Rs[f] = 1.f / s1;
    }
    const int nw4 = m * (D / 4);
    for (int e0 = threadIdx.x; e0 < nw4; e0 += U * NT) {
      f32x4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = min(e0 + u * NT, nw4 - 1);
        x[u] = *reinterpret_cast<const f32x4*>(Wh + (size_t)(e / (D / 4)) * D + (e % (D / 4)) * 4);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + u * NT;
        if (e >= nw4) continue;
        const int fi = e / (D / 4), k4 = (e % (D / 4)) * 4;
        typedef f16 f16x4 __attribute__((ext_vector_type(4)));
        f16x4 h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = (f16)(x[u][i] * kLog2e);
        *reinterpret_cast<f16x4*>(&Wl[fi * LDW + k4]) = h;
      }
    }
    __syncthreads();  // Cf, Rs
    const int nsv = D * (m / 4);
    for (int e0 = threadIdx.x; e0 < nsv; e0 += U * NT) {
      f32x4 acc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int t = 0; t < T_ranges; ++t) {
        f32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int e = min(e0 + u * NT, nsv - 1);
          const int row = e / (m / 4), fi = (e % (m / 4)) * 4;
          v[u] = *reinterpret_cast<const f32x4*>(gsh + ((size_t)t * (D + 1) + row) * m + fi);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int e = min(e0 + u * NT, nsv - 1);
          const int fi = (e % (m / 4)) * 4;
          const f32x4 c = *reinterpret_cast<const f32x4*>(gch + (size_t)t * m + fi);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[u][i] += v[u][i] * fast_exp2(c[i] - Cf[fi + i]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + u * NT;
        if (e >= nsv) continue;
        const int row = e / (m / 4), fi = (e % (m / 4)) * 4;
        bf16x4_t h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = (bf16)(acc[u][i] * Rs[fi + i]);
        *reinterpret_cast<bf16x4_t*>(&Sl[row * LDSS + (fi & ~31) + s_pos<bf16>(fi & 31)]) = h;
      }
    }
  }
  __syncthreads();

  for (int r0 = sub * NW; r0 < nchunks; r0 += stride) {
    const int ch = r0 + wave;
    if (ch >= nchunks) break;  // nothing left for this wave
    int myrow[QN];
    bool valid[QN];
    f16x8 qf[QN][NKC];
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      myrow[q] = (ch * QN + q) * 32 + col;
      valid[q] = myrow[q] < rows;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) qf[q][kc] = to_wfrag(qn[q][kc]);
    }
    fetch_q(min(ch + stride, nchunks - 1));
    f32x16 acc[QN][NDV];
    float den[QN], M[QN];  // den: this lane's half of the features

    // Feature exponents of tile ft, features x queries, lane = query:
    // W_ft Q^T + c'_f [- M] (one accumulator chain; the other wave on the SIMD and the
    // readout products of the previous tile fill the MFMA pipe meanwhile).
    auto c1_tile = [&](int ft, f32x16 (&c1)[QN], bool with_m) {
#pragma unroll
      for (int q = 0; q < QN; ++q) c1[q] = zero16();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const f16x8 a = load_frag_k(&Wl[(32 * ft + col) * LDW], kc, g);
#pragma unroll
        for (int q = 0; q < QN; ++q) c1[q] = mma(a, qf[q][kc], c1[q]);
      }
      const f16x8 ba = Cb[2 * (32 * ft + col) + g];
#pragma unroll
      for (int q = 0; q < QN; ++q) c1[q] = mma(ba, qbias_cols(M[q], g, with_m), c1[q]);
    };
    // phi' = 2^(c1 - sub) rounded to bf16: den += sum of phi' (the same bf16 values the
    // numerator uses, summed in fp32 by dot2 against (1, 1)), acc += (S_v / S_1)_ft^T phi'.
    bf16x2 one2;
    one2[0] = one2[1] = (bf16)1.f;
    auto readout_tile = [&](int ft, const f32x16 (&c1)[QN], bool sub_m) {
      bf16x8 pf[QN][2];
#pragma unroll
      for (int q = 0; q < QN; ++q) {
        f32x16 e;
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = fast_exp2(sub_m ? c1[q][r] - M[q] : c1[q][r]);
        acc_to_frags(e, pf[q]);
        float sum = den[q];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            bf16x2 v;
            v[0] = pf[q][h][j];
            v[1] = pf[q][h][j + 1];
            sum = __builtin_amdgcn_fdot2_f32_bf16(v, one2, sum, false);
          }
        den[q] = sum;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int dt = 0; dt < NDV; ++dt) {
          const bf16x8 a = s_frag(Sl, LDSS, 32 * dt + col, ft, h, g);
#pragma unroll
          for (int q = 0; q < QN; ++q) acc[q][dt] = mma(a, pf[q][h], acc[q][dt]);
        }
    };
    auto rowmax = [&](const f32x16& c) {
      float mx = c[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, c[r]);
      return fmaxf(mx, partner32(mx));
    };
    const int nft = m / 32;
    auto run = [&](bool fast) {
#pragma unroll
      for (int q = 0; q < QN; ++q) {
        M[q] = -INFINITY;
        den[q] = 0.f;
#pragma unroll
        for (int dt = 0; dt < NDV; ++dt) acc[q][dt] = zero16();
      }
      if (fast) {
        // Stabiliser fixed at the first tile's row maximum, then folded into the bias.
        {
          f32x16 c1[QN];
          c1_tile(0, c1, false);
#pragma unroll
          for (int q = 0; q < QN; ++q) M[q] = rowmax(c1[q]);
          readout_tile(0, c1, true);
        }
        for (int ft = 1; ft < nft; ++ft) {
          f32x16 c1[QN];
          c1_tile(ft, c1, true);
          readout_tile(ft, c1, false);
        }
      } else {
        for (int ft = 0; ft < nft; ++ft) {
          f32x16 c1[QN];
          c1_tile(ft, c1, false);
#pragma unroll
          for (int q = 0; q < QN; ++q) {
            const float mx = rowmax(c1[q]);
            if (wave_any(mx > M[q] + kTau)) {
              const float nm = mx > M[q] + kTau ? mx : M[q];
              const float fct = fast_exp2(M[q] - nm);
              den[q] *= fct;
#pragma unroll
              for (int dt = 0; dt < NDV; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[q][dt][r] *= fct;
              M[q] = nm;
            }
          }
          readout_tile(ft, c1, true);
        }
      }
#pragma unroll
      for (int q = 0; q < QN; ++q) den[q] += partner32(den[q]);
    };
    // Only an overflow (a later feature tile ~2^100 above the first) makes the fast pass
    // non-finite; then this wave's rows are redone with the running maximum.
    run(true);
    bool bad = false;
#pragma unroll
    for (int q = 0; q < QN; ++q) bad |= valid[q] && !(den[q] - den[q] == 0.f && den[q] > 0.f);
    if (wave_any(bad)) run(false);

#pragma unroll
    for (int q = 0; q < QN; ++q) {
      const float inv = 1.f / den[q];
      if (!valid[q]) continue;
      bf16* orow = Ob + (size_t)myrow[q] * D;
#pragma unroll
      for (int dt = 0; dt < NDV; ++dt) {
        bf16x8 o0, o1;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          o0[j] = (bf16)(acc[q][dt][j] * inv);
          o1[j] = (bf16)(acc[q][dt][8 + j] * inv);
        }
        *reinterpret_cast<bf16x8*>(orow + 32 * dt + 16 * g) = o0;
        *reinterpret_cast<bf16x8*>(orow + 32 * dt + 16 * g + 8) = o1;
      }
    }
  }
}

// ======================================================================================
// causal_chunk (float32 problems, and bf16 with d = 128 and m > 256): grid (segments,
// B*Hq), m/(32 NTC) waves; wave w owns NTC 32-feature tiles.  Per 32-position block p0 of
// the segment, in order:
//   phi_K,w  = 2^(K W_w^T - |k|^2 log2e/2 - c_f)  (c_f per feature: the scan's prefix
//              maximum, raised with the carry rescaled when the block's keys pass it by kTau)
//   phi_Q,w  = 2^(W_w Q^T + c_f - M_w)            (M_w: this wave's row maximum)
//   num_w^T  = carry_w^T phi_Q,w^T + [V,1]^T tril(phi_K,w phi_Q,w^T)
//   carry_w += phi_K,w^T [V, 1]
// then out = sum_w 2^(M_w - M) num_w / sum_w 2^(M_w - M) den_w across the waves (LDS).
// The carry of a segment starts at the scan's exclusive prefix.  A block whose keys spread
// by more than kSpreadChunk for one feature (over the first keys of the sequence), or pass
// c_f by more than kSpreadChunk, is wide: the first pass records it per segment and the repair pass
// (REPAIR) redoes those segments, taking each wide block one position at a time.
// ======================================================================================
template <class T> struct CausalLd;
template <> struct CausalLd<bf16> { static constexpr int PK = 48; };  // phi_K rows: 32 keys + pad
template <> struct CausalLd<float> { static constexpr int PK = 33; };
constexpr float kSpreadChunk = 100.f;  // as kSpread of the bf16 causal kernels (log2 units)

// PART (wide heads, d = 128 with m > 256, whose two feature tiles per wave would spill):
// the features run as two launches over feature ranges starting at fbase.  PART = 1 writes
// each row's partial (numerators, denominator, row maximum) to part [rows][D+4]; PART = 2
// merges its own with that partial (max-rescaled sum) and writes out.  PART = 0: one launch.
// RELU: the feature map ReLU(W x) on both sides (no norm term, c_f = 0 with no raises, no
// row maxima, no wide blocks: the first pass is the whole pass); a row with a zero
// denominator is written as zeros.
template <class T, int D, int NTC, int NWMAX, int PART, bool REPAIR, bool RELU = false>
__global__ void __launch_bounds__(64 * NWMAX) causal_chunk_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const float* __restrict__ W,
    const typename SumOf<T>::type* __restrict__ prefix, const float* __restrict__ prefix_c, T* __restrict__ out,
    int L, int Hq,
    int Hkv, int Hw, int m, int R, int T_ranges, int fbase, float* __restrict__ part, int* __restrict__ wide,
    int n_units) {
  using P = Prec<T>;
  using frag = typename P::frag;
  using wfrag = typename P::wfrag;
  constexpr int NKC = D / P::KS;
  constexpr int NDT = D / 32 + 1;
  constexpr int LDK = Ld<T>::template K<D>;
  constexpr int LDV = Ld<T>::template V<D>;
  constexpr int LDP = CausalLd<T>::PK;
  constexpr int LDR = D + 4;  // reduction rows: D partial values, den, row max
  // The cross-wave reduction handles 32 / QSPLIT query rows at a time so that the LDS
  // footprint stays within 160 KB for wide heads and many waves.
  constexpr int FW = 32 * NTC;  // features per wave
  constexpr int BASE_LDS = (2 * 32 * LDK + 32 * LDV + NWMAX * FW * LDP) * (int)sizeof(T) + NWMAX * FW * 4 + 64;
  constexpr int QSPLIT = BASE_LDS + NWMAX * 32 * LDR * 4 <= 160 * 1024       ? 1
                         : BASE_LDS + NWMAX * 16 * LDR * 4 <= 160 * 1024 ? 2
                                                                         : 4;
  constexpr int QR = 32 / QSPLIT;
  // Q and K are staged already in the W-contraction type (fp16 for bf16 problems), once
  // per workgroup instead of once per wave.
  using WE = typename P::welem;
  __shared__ __attribute__((aligned(16))) WE Ql[32 * LDK];
  __shared__ __attribute__((aligned(16))) WE Kl[32 * LDK];
  __shared__ __attribute__((aligned(16))) T Vl[32 * LDV];
  __shared__ __attribute__((aligned(16))) T Pk[NWMAX][FW * LDP];
  __shared__ __attribute__((aligned(16))) float Red[NWMAX][QR * LDR];
  __shared__ __attribute__((aligned(16))) float CshL[NWMAX][FW];  // the block's c_f moves
  __shared__ int flagw[NWMAX];

  const int nw = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, l = lane_id(), col = l & 31, g = l >> 5;
  const int f0 = fbase + wave * FW;
  float* Csh = CshL[wave];
  T* pk = Pk[wave];
  float* red = Red[wave];

  auto run_segment = [&](const int seg, const int bhq) {
  const int b = bhq / Hq, hq = bhq % Hq, hkv = hq / (Hq / Hkv), bh = b * Hkv + hkv;
  const float* Wh = W + (size_t)(Hw == 1 ? 0 : hkv) * m * D;
  const T* Qh = Q + (size_t)bhq * L * D;
  T* Oh = out + (size_t)bhq * L * D;
  const T* Kh = K + (size_t)bh * L * D;
  const T* Vh = V + (size_t)bh * L * D;

  wfrag wf[NTC][NKC];
#pragma unroll
  for (int nt = 0; nt < NTC; ++nt)
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) load_w_frag(Wh + (size_t)(f0 + 32 * nt + col) * D, kc, g, wf[nt][kc]);
  // c_f of this lane's feature 32 nt + col (-inf while no key has set it); its bias
  // operands are built where they are used (keys: -c_f, 0 while unset; queries: +c_f)
  float cf[NTC];
  const float* pcs = prefix_c + ((size_t)bh * T_ranges + seg) * m;
#pragma unroll
  for (int nt = 0; nt < NTC; ++nt) cf[nt] = RELU ? 0.f : pcs[f0 + 32 * nt + col];

  // carry of this wave's features, from the exclusive prefix of the segment ([d+1][m]:
  // lane col takes row 32 dt + col, register r feature 8(r/4) + 4g + r%4 of the tile)
  f32x16 carry[NTC][NDT];
  {
    const typename SumOf<T>::type* pf = prefix + ((size_t)bh * T_ranges + seg) * (size_t)(D + 1) * m;
#pragma unroll
    for (int nt = 0; nt < NTC; ++nt)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int row = dt < NDT - 1 ? 32 * dt + col : D;
        const bool live = dt < NDT - 1 || col == 0;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 v = {0.f, 0.f, 0.f, 0.f};
          if (live) v = load_sum4(pf + (size_t)row * m + f0 + 32 * nt + 8 * r4 + 4 * g);
#pragma unroll
          for (int i = 0; i < 4; ++i) carry[nt][dt][4 * r4 + i] = v[i];
        }
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

  const int p_begin = seg * R;
  const int p_end = min(p_begin + R, L);
  constexpr int EPC = 16 / (int)sizeof(T), CPR = D / EPC, NCH = 32 * CPR;
  // bf16: range-checked buffer loads (a head is under 2^31 bytes, so its byte offsets fit
  // 32 bits): a chunk of a row past L gets the head's size as offset and reads as zero
  const unsigned head_bytes = (unsigned)L * (unsigned)D * (unsigned)sizeof(T);
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void*)Qh, (short)0, (int)head_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, (int)head_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, (int)head_bytes, kBufWord3);
  auto put = [&](WE* dst, int ld, const f32x4& v, int row, int c0) {
    WE* drow = dst + row * ld;
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<wfrag*>(drow + c0) = to_wfrag(__builtin_bit_cast(frag, v));
    } else {
      float* d = reinterpret_cast<float*>(drow + c0);
      d[0] = v[0];
      d[1] = v[1];
      d[2] = v[2];
      d[3] = v[3];
    }
  };
  auto put_v = [&](const f32x4& v, int row, int c0) {  // value columns permuted by vperm_inv
    const int tile = c0 & ~31;
    T* drow = Vl + row * LDV;
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
  };
  auto row_max = [&](const f32x16& c) {
    float mx = c[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, c[r]);
    return pair_max(mx);
  };
  // wide block: see the kernel's comment (masked keys sit near -kMaskedRow)
  auto is_wide = [&](const f32x16& ck, float mx, bool init) {
    if (!init) return mx > kSpreadChunk;
    float mn = INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mn = fminf(mn, ck[r] > -0.5f * kMaskedRow ? ck[r] : INFINITY);
    return mx - pair_min(mn) > kSpreadChunk;
  };
  auto key_exp = [&](const wfrag (&kf)[NKC], const wfrag& biasA, int nt) {
    f32x16 ck = zero16();
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) ck = mma(kf[kc], wf[nt][kc], ck);
    return mma(biasA, bias_cols(cf[nt] == -INFINITY ? 0.f : cf[nt], g, wfrag{}), ck);
  };
  bool wide_w = false;

  // The carry loads complete here: otherwise the compiler's wait for the carry registers,
  // merged over the loop back edge, also waits for every later load.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  for (int p0 = p_begin; p0 < p_end; p0 += 32) {
    __syncthreads();  // the previous block's readers of Ql / Kl / Vl are done
    for (int c = threadIdx.x; c < NCH; c += blockDim.x) {
      const int row = c / CPR, c0 = (c % CPR) * EPC;
      f32x4 q = {0.f, 0.f, 0.f, 0.f}, kk = {0.f, 0.f, 0.f, 0.f};
      if constexpr (sizeof(T) == 2) {
        const unsigned off = p0 + row < L ? ((unsigned)(p0 + row) * D + c0) * (unsigned)sizeof(T) : head_bytes;
        q = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, (int)off, 0, 0));
        kk = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, (int)off, 0, 0));
        put_v(__builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, (int)off, 0, 0)), row, c0);
      } else if (p0 + row < L) {
        q = *reinterpret_cast<const f32x4*>(Qh + (size_t)(p0 + row) * D + c0);
        kk = *reinterpret_cast<const f32x4*>(Kh + (size_t)(p0 + row) * D + c0);
      }
      put(Ql, LDK, q, row, c0);
      put(Kl, LDK, kk, row, c0);
    }
    if constexpr (sizeof(T) != 2) stage_rows<T, D, true>(Vl, LDV, Vh, p0, L);
    __syncthreads();
    const int pend = min(p0 + 32, L);

    // step(lo, hi, check): the positions [lo, hi) of the block (keys outside masked, rows
    // outside not stored).  The repair pass first tests the whole block (check) and returns
    // true, having changed nothing, when it is wide; the caller then takes the block one
    // position at a time.
    auto step = [&](const int lo, const int hi, const bool check) -> bool {
      if (REPAIR && !check) __syncthreads();  // the previous position's reduction is read
      wfrag kf[NKC];
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) kf[kc] = load_frag_k(Kl + col * LDK, kc, g);
      // keys outside the window (and past L: zero rows in LDS) get the masking row bias:
      // their features are exactly 0
      const bool kin = p0 + col >= lo && p0 + col < hi;
      float rb = kMaskedRow;
      if constexpr (RELU) {
        if (kin) rb = 0.f;
      } else {
        const float nrm = pair_sum(sumsq(kf));
        if (kin) rb = 0.5f * kLog2e * nrm;
      }
      const wfrag biasA = bias_rows(rb, g, wfrag{});
      if (REPAIR && check) {
        bool wd = false;
#pragma unroll
        for (int nt = 0; nt < NTC; ++nt) {
          const f32x16 ck = key_exp(kf, biasA, nt);
          wd = wd || is_wide(ck, row_max(ck), cf[nt] == -INFINITY);
        }
        const bool any = wave_any(wd);
        if (l == 0) flagw[wave] = any ? 1 : 0;
        __syncthreads();
        int a = 0;
        for (int w = 0; w < nw; ++w) a |= flagw[w];
        if (a != 0) return true;
      }

      // phi_K of this wave's features: C = K W_w^T (keys x features), lane = feature; c_f
      // raised first where the block's keys pass it
      frag ka[NTC][P::NF32];
      bool shifted = false;
#pragma unroll
      for (int nt = 0; nt < NTC; ++nt) {
        f32x16 ck = key_exp(kf, biasA, nt);
        f32x16 e;
        if constexpr (RELU) {
#pragma unroll
          for (int r = 0; r < 16; ++r) e[r] = fmaxf(ck[r], 0.f);
        } else {
          const float mx = row_max(ck);
          const bool init = cf[nt] == -INFINITY;
          if (!REPAIR && check) wide_w = wide_w || is_wide(ck, mx, init);
          const float shift = init || mx > kTau ? mx : 0.f;
          Csh[32 * nt + col] = init ? -INFINITY : -shift;  // both lane halves write the same value
          if (init || shift != 0.f) cf[nt] = (init ? 0.f : cf[nt]) + shift;
          shifted = shifted || shift != 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) e[r] = fast_exp2(ck[r] - shift);
        }
        acc_to_frags(e, ka[nt]);
        // phi_K to LDS as [feature][key] for the transposed read below (the operand values:
        // register r holds key 8(r/4) + 4g + r%4)
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              bf16x4_t v;
#pragma unroll
              for (int i = 0; i < 4; ++i) v[i] = ka[nt][h][4 * hh + i];
              *reinterpret_cast<bf16x4_t*>(pk + (32 * nt + col) * LDP + 8 * (2 * h + hh) + 4 * g) = v;
            }
        } else {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            T* dst = pk + (32 * nt + col) * LDP + 8 * r4 + 4 * g;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = e[4 * r4 + i];
          }
        }
      }
      asm volatile("" ::: "memory");  // the wave's LDS writes above before its reads below
      // the carry (ones column included) of a raised feature scales by 2^(old - new), 0
      // where it was unset
      if (!RELU && wave_any(shifted)) {
#pragma unroll
        for (int nt = 0; nt < NTC; ++nt)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 sh = *reinterpret_cast<const f32x4*>(Csh + 32 * nt + 8 * r4 + 4 * g);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float fct = fast_exp2(sh[q]);
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt) carry[nt][dt][4 * r4 + q] *= fct;
            }
          }
      }

      // phi_Q of this wave's features: C = W_w Q^T + c_f (features x queries), lane = query
      wfrag qf[NKC];
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) qf[kc] = load_frag_k(Ql + col * LDK, kc, g);
      f32x16 cq[NTC];
      float Mw = -INFINITY;
#pragma unroll
      for (int nt = 0; nt < NTC; ++nt) {
        cq[nt] = zero16();
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) cq[nt] = mma(wf[nt][kc], qf[kc], cq[nt]);
        if constexpr (!RELU) {
          // every c_f is set once the block's keys are in (each feature saw a key)
          cq[nt] = mma(bias_rows(-cf[nt], g, wfrag{}), bias_cols(0.f, g, wfrag{}), cq[nt]);
          Mw = fmaxf(Mw, row_max(cq[nt]));
        }
      }
      if constexpr (RELU) Mw = 0.f;
      frag qb[NTC][P::NF32];
#pragma unroll
      for (int nt = 0; nt < NTC; ++nt) {
        f32x16 e;
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = RELU ? fmaxf(cq[nt][r], 0.f) : fast_exp2(cq[nt][r] - Mw);
        acc_to_frags(e, qb[nt]);
      }

      // num^T = carry^T phi_Q^T  (rows: value columns, lanes: queries)
      f32x16 num[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        num[dt] = zero16();
#pragma unroll
        for (int nt = 0; nt < NTC; ++nt) {
          frag ca[P::NF32];
          acc_to_frags(carry[nt][dt], ca);
#pragma unroll
          for (int h = 0; h < P::NF32; ++h) num[dt] = mma(ca[h], qb[nt][h], num[dt]);
        }
      }
      // intra-block triangle: A^T = phi_K phi_Q^T (keys x queries), keep key <= query
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
      __builtin_amdgcn_wave_barrier();
      f32x16 at = zero16();
#pragma unroll
      for (int nt = 0; nt < NTC; ++nt)
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
          for (int nt = 0; nt < NTC; ++nt) carry[nt][dt] = mma(ka[nt][h], va, carry[nt][dt]);
        }

      // this wave's partial to LDS (D values, den, row maximum per query), then the
      // cross-wave sum; one reduction item = (query, 4 value columns), spread over all threads.
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
        for (int it = threadIdx.x; it < QR * (D / 4); it += blockDim.x) {
          const int q = it / (D / 4), c0 = (it % (D / 4)) * 4;
          const int pos = p0 + qh * QR + q;
          if (pos < lo || pos >= hi) continue;
          float M = -INFINITY;
          for (int w = 0; w < nw; ++w) M = fmaxf(M, Red[w][q * LDR + D + 1]);
          float den = 0.f;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          for (int w = 0; w < nw; ++w) {
            const float* rw = Red[w] + q * LDR;
            const float2 dm = *reinterpret_cast<const float2*>(rw + D);  // den, row maximum
            const f32x4 v = *reinterpret_cast<const f32x4*>(rw + c0);
            const float sc = fast_exp2(dm.y - M);
            den += sc * dm.x;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += sc * v[i];
          }
          if constexpr (PART != 0) {
            float* prow = part + ((size_t)bhq * L + pos) * (D + 4);  // 16-byte aligned rows
            if constexpr (PART == 1) {
              *reinterpret_cast<f32x4*>(prow + c0) = acc;
              if (c0 == 0) {
                prow[D] = den;
                prow[D + 1] = M;
              }
              continue;
            } else {
              const float den1 = prow[D], M1 = prow[D + 1];
              const f32x4 acc1 = *reinterpret_cast<const f32x4*>(prow + c0);
              const float Mn = fmaxf(M, M1), s0 = fast_exp2(M - Mn), s1 = fast_exp2(M1 - Mn);
              den = den * s0 + den1 * s1;
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[i] = acc[i] * s0 + acc1[i] * s1;
            }
          }
          const float inv = RELU ? (den > 0.f ? __builtin_amdgcn_rcpf(den) : 0.f) : __builtin_amdgcn_rcpf(den);
          T* orow = Oh + (size_t)pos * D + c0;
          if constexpr (sizeof(T) == 2) {
            bf16x4_t o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (bf16)(acc[i] * inv);
            *reinterpret_cast<bf16x4_t*>(orow) = o;
          } else {
            *reinterpret_cast<f32x4*>(orow) = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
          }
        }
        if (QSPLIT > 1) __syncthreads();
      }
      return false;
    };
    if constexpr (REPAIR) {
      // the whole block with the wide test, then (when wide) its positions one at a time
      for (int q = p0 - 1; q < pend; ++q) {
        const bool whole = q < p0;
        if (!step(whole ? p0 : q, whole ? pend : q + 1, whole) && whole) break;
      }
    } else {
      step(p0, pend, true);
    }
  }
  if (!REPAIR) {
    const bool any = wave_any(wide_w);
    __syncthreads();  // flagw is free
    if (l == 0) flagw[wave] = any ? 1 : 0;
    __syncthreads();
    if (threadIdx.x == 0) {
      int a = 0;
      for (int w = 0; w < nw; ++w) a |= flagw[w];
      wide[(size_t)bhq * T_ranges + seg] = a;
    }
  }
  };
  if constexpr (REPAIR) {
    for (int u = blockIdx.x; u < n_units; u += gridDim.x)
      if (wide[u] != 0) run_segment(u % T_ranges, u / T_ranges);
  } else {
    run_segment(blockIdx.x, blockIdx.y);
  }
}

}  // namespace favor

// ======================================================================================
// Host side: dispatch and the C ABI.
// ======================================================================================
namespace favor {
namespace {

inline int ceil_div_i(long long a, long long b) { return (int)((a + b - 1) / b); }

// The causal key side: one wave per segment and 64-feature slice.  The three-waves-per-SIMD
// form is taken where it holds all of them in fewer resident rounds than the default's two
// waves per SIMD (rounds counted on the kCUs model); elsewhere its spills cost more than
// the occupancy gains.  The choice rests on the problem alone, never the device, so a
// problem's result bits (S_1 is summed differently in the two forms) do not depend on it.
template <class T, int D, bool RELU>
favor_status launch_kv_segments(const Plan& s, const T* K, const T* V, const float* W, float* gs, float* gc,
                                hipStream_t st) {
  using A = KvCfg<T, D, false>;
  using B = KvCfg<T, D, true>;
  const int nfs = s.m / kFeatPerWave;
  if constexpr (A::KW != B::KW || A::MINB != B::MINB) {
    const long long waves = (long long)s.BH * s.T * nfs, slots = 4LL * kCUs;
    if (ceil_div_i(waves, 3 * slots) < ceil_div_i(waves, 2 * slots)) {
      constexpr int PG = B::KW * B::NTW / 2;  // segments per workgroup
      const int units = s.BH * ceil_div_i(s.T, PG);
      hipLaunchKernelGGL((kv_summary_kernel<T, D, true, RELU, true>), dim3(8 * ceil_div_i(units, 8) * nfs),
                         dim3(64 * B::KW), 0, st, K, V, W, s.L, s.Hkv, s.Hw, s.m, s.R, s.T, units, gs, gc, nullptr,
                         nullptr, nullptr);
      return hipGetLastError() == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
    }
  }
  constexpr int PG = A::KW * A::NTW / 2;
  const int units = s.BH * ceil_div_i(s.T, PG);
  hipLaunchKernelGGL((kv_summary_kernel<T, D, true, RELU, false>), dim3(8 * ceil_div_i(units, 8) * nfs),
                     dim3(64 * A::KW), 0, st, K, V, W, s.L, s.Hkv, s.Hw, s.m, s.R, s.T, units, gs, gc, nullptr,
                     nullptr, nullptr);
  return hipGetLastError() == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}

template <class T, int D>
favor_status launch_kv_summary(const Plan& s, const T* K, const T* V, const float* W, float* gs, float* gc,
                               char* ws, hipStream_t st) {
  const int nfs = s.m / kFeatPerWave;
  if (s.mode == FAVOR_CAUSAL) return launch_kv_segments<T, D, false>(s, K, V, W, gs, gc, st);
  const int units = s.BH * s.T;
  if constexpr (std::is_same<T, bf16>::value) {
    hipLaunchKernelGGL((kv_summary_bf16_kernel<D>), dim3(8 * ceil_div_i(units, 8) * nfs), dim3(64 * KvBf16<D>::NW), 0,
                       st, K, V, W, s.L, s.Hkv, s.Hw, s.m, s.R, s.T, units, gs, gc, s.img ? ws + s.off_img_w : nullptr,
                       s.img ? ws + s.off_img_s : nullptr, s.img ? ws + s.off_img_cb : nullptr);
    return hipGetLastError() == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
  } else {
    hipLaunchKernelGGL((kv_summary_kernel<T, D, false>), dim3(8 * ceil_div_i(units, 8) * nfs), dim3(64 * KvCfg<T, D>::KW),
                       0, st, K, V, W, s.L, s.Hkv, s.Hw, s.m, s.R, s.T, units, gs, gc, nullptr, nullptr, nullptr);
    return hipGetLastError() == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
  }
}

template <class T, int D>
favor_status run_bidirectional(const Plan& s, const T* Q, const T* K, const T* V, const float* W, T* out,
                               char* ws, hipStream_t st, const Marks& mk) {
  if constexpr (std::is_same<T, float>::value) {
    // float32: the key side and the readout spread over feature tiles
    return launch_small_f32(s, Q, K, V, W, out, ws, st, mk);
  }
  float* gs = reinterpret_cast<float*>(ws + s.off_gs);
  float* gc = reinterpret_cast<float*>(ws + s.off_gc);
  if (!mk.mark(0, st)) return FAVOR_ERR_HIP;
  favor_status rc = launch_kv_summary<T, D>(s, K, V, W, gs, gc, ws, st);
  if (rc != FAVOR_OK) return rc;
  if (!mk.mark(1, st) || !mk.mark(2, st)) return FAVOR_ERR_HIP;  // no middle kernel
  const long long rows = (long long)s.G * s.L;
  if constexpr (std::is_same<T, bf16>::value) {
    if (s.m <= RoBf16<D>::MP) {
    using Cfg = RoBf16<D>;
    const int rounds = ceil_div_i(rows, Cfg::NWAVE * Cfg::QN * 32);
    int per_head = ceil_div_i(kReadoutTarget, s.BH);
    if (per_head > rounds) per_head = rounds;
    if (per_head < 1) per_head = 1;
    hipLaunchKernelGGL((readout_bf16_kernel<D>), dim3(8 * per_head * ceil_div_i(s.BH, 8)), dim3(64 * Cfg::NWAVE),
                       0, st, Q, W, gs, gc, s.img ? ws + s.off_img_w : nullptr, s.img ? ws + s.off_img_s : nullptr,
                       s.img ? ws + s.off_img_cb : nullptr, out, s.L, s.Hq, s.Hkv, s.Hw, s.m, s.T, s.BH, per_head);
    } else {
      using Cfg = ReadoutCfg<T, D>;
      const int tiles = ceil_div_i(rows, Cfg::NWAVE * Cfg::QN * 32);
      int per_head = ceil_div_i(kReadoutTarget, s.BH);
      if (per_head > tiles) per_head = tiles;
      if (per_head < 1) per_head = 1;
      hipLaunchKernelGGL((readout_kernel<T, D>), dim3(per_head, s.BH), dim3(64 * Cfg::NWAVE), 0, st, Q, W, gs, gc,
                         out, s.L, s.Hq, s.Hkv, s.Hw, s.m, s.T);
    }
  } else {
    using Cfg = ReadoutCfg<T, D>;
    const int tiles = ceil_div_i(rows, Cfg::NWAVE * Cfg::QN * 32);
    int per_head = ceil_div_i(kReadoutTarget, s.BH);
    if (per_head > tiles) per_head = tiles;
    if (per_head < 1) per_head = 1;
    hipLaunchKernelGGL((readout_kernel<T, D>), dim3(per_head, s.BH), dim3(64 * Cfg::NWAVE), 0, st, Q, W, gs, gc,
                       out, s.L, s.Hq, s.Hkv, s.Hw, s.m, s.T);
  }
  if (hipGetLastError() != hipSuccess || !mk.mark(3, st)) return FAVOR_ERR_HIP;
  return FAVOR_OK;
}

template <class T, int D>
favor_status run_relu_bidirectional(const Plan& s, const T* Q, const T* K, const T* V, const float* W, T* out,
                                    char* ws, hipStream_t st) {
  float* gs = reinterpret_cast<float*>(ws + s.off_gs);
  float* gc = reinterpret_cast<float*>(ws + s.off_gc);
  const int units = s.BH * s.T, nfs = s.m / kFeatPerWave;
  hipLaunchKernelGGL((kv_summary_kernel<T, D, false, true>), dim3(8 * ceil_div_i(units, 8) * nfs),
                     dim3(64 * KvCfg<T, D>::KW), 0, st, K, V, W, s.L, s.Hkv, s.Hw, s.m, s.R, s.T, units, gs, gc,
                     nullptr, nullptr, nullptr);
  if (hipGetLastError() != hipSuccess) return FAVOR_ERR_HIP;
  using Cfg = ReadoutCfg<T, D>;
  const long long rows = (long long)s.G * s.L;
  const int tiles = ceil_div_i(rows, Cfg::NWAVE * Cfg::QN * 32);
  int per_head = ceil_div_i(kReadoutTarget, s.BH);
  if (per_head > tiles) per_head = tiles;
  if (per_head < 1) per_head = 1;
  hipLaunchKernelGGL((readout_kernel<T, D, true>), dim3(per_head, s.BH), dim3(64 * Cfg::NWAVE), 0, st, Q, W, gs, gc,
                     out, s.L, s.Hq, s.Hkv, s.Hw, s.m, s.T);
  return hipGetLastError() == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}

template <class T, int D>
favor_status run_causal(const Plan& s, const T* Q, const T* K, const T* V, const float* W, T* out, char* ws,
                        hipStream_t st, const Marks& mk) {
  float* gs = reinterpret_cast<float*>(ws + s.off_gs);
  float* gc = reinterpret_cast<float*>(ws + s.off_gc);
  if (!mk.mark(0, st)) return FAVOR_ERR_HIP;
  favor_status rc = launch_kv_summary<T, D>(s, K, V, W, gs, gc, ws, st);
  if (rc != FAVOR_OK || !mk.mark(1, st)) return rc != FAVOR_OK ? rc : FAVOR_ERR_HIP;
  // per-feature stabilisers: the scan's prefix maxima start each segment
  rc = launch_causal_scan_pf(s, ws, st);
  if (rc != FAVOR_OK) return rc;
  if (!mk.mark(2, st)) return FAVOR_ERR_HIP;
  if (causal_v_supported(s)) {
    // bf16 (d = 64, or m <= 256): the value columns split over the waves
    rc = launch_causal_v(s, Q, K, V, W, out, ws, st);
    if (rc != FAVOR_OK) return rc;
    return mk.mark(3, st) ? FAVOR_OK : FAVOR_ERR_HIP;
  }
  const auto* prefix = reinterpret_cast<const typename SumOf<T>::type*>(ws + s.off_p);
  const float* prefix_c = reinterpret_cast<const float*>(ws + s.off_pc);
  int* wide = reinterpret_cast<int*>(ws + s.off_wide);
  const int n_units = s.T * s.B * s.Hq;
  const dim3 grid(s.T, s.B * s.Hq);
  // the repair pass: one workgroup per CU at most, walking the segment flags
  const dim3 rgrid((unsigned)(n_units < kCUs ? n_units : kCUs));
  // one launch pair (first pass, repair) over nw waves from feature fbase
  auto pair = [&](auto first, auto repair, int nw, int fbase, float* part) {
    hipLaunchKernelGGL(first, grid, dim3(kWave * nw), 0, st, Q, K, V, W, prefix, prefix_c, out, s.L, s.Hq, s.Hkv,
                       s.Hw, s.m, s.R, s.T, fbase, part, wide, n_units);
    if (hipGetLastError() != hipSuccess) return false;
    hipLaunchKernelGGL(repair, rgrid, dim3(kWave * nw), 0, st, Q, K, V, W, prefix, prefix_c, out, s.L, s.Hq, s.Hkv,
                       s.Hw, s.m, s.R, s.T, fbase, part, wide, n_units);
    return hipGetLastError() == hipSuccess;
  };
  bool ok = false;
  if (D == 128 && s.m > 256) {
    // two launch pairs of one-tile waves over features [0, 256) and [256, m), merged per row
    // (the second pair's flags replace the first's once its repair has read them)
    if constexpr (D == 128) {
      float* part = reinterpret_cast<float*>(ws + s.off_part);
      ok = pair(causal_chunk_kernel<T, D, 1, 8, 1, false>, causal_chunk_kernel<T, D, 1, 8, 1, true>, 8, 0, part) &&
           pair(causal_chunk_kernel<T, D, 1, 8, 2, false>, causal_chunk_kernel<T, D, 1, 8, 2, true>,
                (s.m - 256) / 32, 256, part);
    }
  } else if constexpr (std::is_same<T, float>::value) {
    if (s.m <= 256) {
      // one 32-feature tile per wave: two waves per SIMD (a few spilled registers for d =
      // 128, still faster than two tiles per wave)
      ok = pair(causal_chunk_kernel<T, D, 1, 8, 0, false>, causal_chunk_kernel<T, D, 1, 8, 0, true>, s.m / 32, 0,
                nullptr);
    } else if constexpr (D == 64) {
      // m > 256 (5 to 8 waves): two 32-feature tiles per wave
      ok = pair(causal_chunk_kernel<T, D, 2, 8, 0, false>, causal_chunk_kernel<T, D, 2, 8, 0, true>, s.m / 64, 0,
                nullptr);
    } else {
      return FAVOR_ERR_UNSUPPORTED;  // not reached: d = 128 with m > 256 takes the split above
    }
  } else {
    return FAVOR_ERR_UNSUPPORTED;  // not reached: the other bf16 shapes take launch_causal_v
  }
  if (!ok || !mk.mark(3, st)) return FAVOR_ERR_HIP;
  return FAVOR_OK;
}

// ReLU attention, causal: the key side's segment summaries of ReLU(W k) [v, 1] (c = 0), their
// exclusive prefix (the per-feature scan reduces to a plain sum), then the chunk kernel in
// its ReLU mode -- one pass, no repair (no stabiliser moves, so no block is wide).
template <class T, int D>
favor_status run_relu_causal(const Plan& s, const T* Q, const T* K, const T* V, const float* W, T* out, char* ws,
                             hipStream_t st) {
  float* gs = reinterpret_cast<float*>(ws + s.off_gs);
  float* gc = reinterpret_cast<float*>(ws + s.off_gc);
  favor_status rc = launch_kv_segments<T, D, true>(s, K, V, W, gs, gc, st);
  if (rc != FAVOR_OK) return rc;
  rc = launch_causal_scan_pf(s, ws, st);
  if (rc != FAVOR_OK) return rc;
  const auto* prefix = reinterpret_cast<const typename SumOf<T>::type*>(ws + s.off_p);
  const float* prefix_c = reinterpret_cast<const float*>(ws + s.off_pc);
  int* wide = reinterpret_cast<int*>(ws + s.off_wide);
  const int n_units = s.T * s.B * s.Hq;
  const dim3 grid(s.T, s.B * s.Hq);
  auto pass = [&](auto kern, int nw, int fbase, float* part) {
    hipLaunchKernelGGL(kern, grid, dim3(kWave * nw), 0, st, Q, K, V, W, prefix, prefix_c, out, s.L, s.Hq, s.Hkv, s.Hw,
                       s.m, s.R, s.T, fbase, part, wide, n_units);
    return hipGetLastError() == hipSuccess;
  };
  bool ok = false;
  if (D == 128 && s.m > 256) {
    if constexpr (D == 128) {
      float* part = reinterpret_cast<float*>(ws + s.off_part);
      ok = pass(causal_chunk_kernel<T, D, 1, 8, 1, false, true>, 8, 0, part) &&
           pass(causal_chunk_kernel<T, D, 1, 8, 2, false, true>, (s.m - 256) / 32, 256, part);
    }
  } else if (s.m <= 256) {
    ok = pass(causal_chunk_kernel<T, D, 1, 8, 0, false, true>, s.m / 32, 0, nullptr);
  } else if constexpr (D == 64) {
    ok = pass(causal_chunk_kernel<T, D, 2, 8, 0, false, true>, s.m / 64, 0, nullptr);
  } else {
    return FAVOR_ERR_UNSUPPORTED;  // not reached: d = 128 with m > 256 takes the split above
  }
  return ok ? FAVOR_OK : FAVOR_ERR_HIP;
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

favor_status launch_key_summaries(const Plan& plan, const void* K, const void* V, const float* W, float* gs,
                                  float* gc, hipStream_t st) {
  if (plan.mode != FAVOR_BIDIRECTIONAL) return FAVOR_ERR_INVALID_ARG;
  Plan s = plan;
  s.img = false;  // float32 partials, never the readout's images
  if (s.dtype == FAVOR_BF16)
    return s.d == 64 ? launch_kv_summary<bf16, 64>(s, static_cast<const bf16*>(K), static_cast<const bf16*>(V), W, gs,
                                                   gc, nullptr, st)
                     : launch_kv_summary<bf16, 128>(s, static_cast<const bf16*>(K), static_cast<const bf16*>(V), W,
                                                    gs, gc, nullptr, st);
  return s.d == 64 ? launch_kv_summary<float, 64>(s, static_cast<const float*>(K), static_cast<const float*>(V), W,
                                                  gs, gc, nullptr, st)
                   : launch_kv_summary<float, 128>(s, static_cast<const float*>(K), static_cast<const float*>(V), W,
                                                   gs, gc, nullptr, st);
}

namespace {

template <class T>
favor_status run_relu_typed(const Plan& s, const void* Q, const void* K, const void* V, const float* W, void* out,
                            char* ws, hipStream_t st) {
  const T *q = static_cast<const T*>(Q), *k = static_cast<const T*>(K), *v = static_cast<const T*>(V);
  T* o = static_cast<T*>(out);
  if (s.mode == FAVOR_BIDIRECTIONAL)
    return s.d == 64 ? run_relu_bidirectional<T, 64>(s, q, k, v, W, o, ws, st)
                     : run_relu_bidirectional<T, 128>(s, q, k, v, W, o, ws, st);
  return s.d == 64 ? run_relu_causal<T, 64>(s, q, k, v, W, o, ws, st)
                   : run_relu_causal<T, 128>(s, q, k, v, W, o, ws, st);
}

}  // namespace

size_t relu_workspace_bytes(const Plan& s) { return s.mode == FAVOR_BIDIRECTIONAL ? s.off_p : s.bytes; }

favor_status launch_relu_attention(const Plan& s, const void* Q, const void* K, const void* V, const float* W,
                                   void* out, char* ws, hipStream_t st) {
  return s.dtype == FAVOR_BF16 ? run_relu_typed<bf16>(s, Q, K, V, W, out, ws, st)
                               : run_relu_typed<float>(s, Q, K, V, W, out, ws, st);
}

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

int32_t favor_attn_fwd_launches(const favor_problem* p) {
  favor::Plan s;
  if (favor::make_plan(p, &s) != FAVOR_OK) return 0;
  if (s.mode == FAVOR_BIDIRECTIONAL) return s.dtype == FAVOR_F32 && favor::small_f32_fused(s) ? 1 : 2;
  return s.d == 128 && s.m > 256 ? 6 : 4;
}

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

// ---- favor_attn_fwd_noalloc: the forward with the library's own device scratch ------
// For callers that cannot allocate device memory.  The scratch is one file-scope device
// array; every device the library runs on holds its own copy.  In host code `scratch` only
// names the symbol: its device address is looked up once per device (with that device
// current) and kept, and kernels and copies use that address only.
namespace {
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[FAVOR_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

favor_status favor_attn_fwd_noalloc(const favor_problem* p, const void* Q, const void* K, const void* V,
                                    const float* W, void* out, void* stream) {
  favor::Plan s;
  const favor_status st = favor::make_plan(p, &s);
  if (st != FAVOR_OK) return st;
  if (Q == nullptr || K == nullptr || V == nullptr || W == nullptr || out == nullptr) return FAVOR_ERR_INVALID_ARG;
  if (s.bytes > FAVOR_NOALLOC_SCRATCH_BYTES) return FAVOR_ERR_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FAVOR_ERR_HIP;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (hs != nullptr) {  // the scratch of the current device serves work on that device only
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(hs, &sdev) != hipSuccess) return FAVOR_ERR_HIP;
    if (sdev != dev) return FAVOR_ERR_INVALID_ARG;
  }
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
      void* addr = nullptr;
      if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) return FAVOR_ERR_HIP;
      g_scratch_ptr[dev] = addr;
    }
    ptr = g_scratch_ptr[dev];
  }
  return attn_fwd_impl(p, Q, K, V, W, out, ptr, FAVOR_NOALLOC_SCRATCH_BYTES, stream, favor::Marks{nullptr, 0});
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
