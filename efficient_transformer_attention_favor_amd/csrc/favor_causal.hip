// Causal FAVOR+ for bf16 problems on gfx950: the exclusive scan of the segment summaries
// with one running stabiliser per feature, and the chunked prefix pass -- causal_fg_kernel
// (d = 64: features split over the waves, intra-chunk blocks of 32..256 positions) and
// causal_v_kernel (d = 128, m <= 256: value columns and feature groups over the waves) --
// each followed by a repair pass for segments whose keys spread too far within a block.
//
// Method: "Rethinking Attention with Performers" (review page), "제안 방법": attention in
// linear order with positive random features; causal mode (inclusive mask j <= i) as the
// running sum S_i = sum_{j <= i} phi(k_j) [v_j, 1]^T, out_i = phi(q_i) S_v,i / phi(q_i) S_1,i.
// The sequence of one kv head is cut into segments; a segment starts from the exclusive
// prefix of the summaries of the segments before it (causal_scan_pf_kernel) and walks its
// 32-position blocks in order:
//   out_blk = phi(Q_blk) S_carry + tril(phi(Q_blk) phi(K_blk)^T) [V_blk, 1]
//   S_carry += phi(K_blk)^T [V_blk, 1]
// Exponents are in log2 units (W scaled by log2 e).  Keys carry one stabiliser c_f per
// feature: phi_K = 2^(w_f.k - |k|^2/2 - c_f), and c_f is added to the query exponent, so
// every product phi_Q phi_K is exact whatever c_f is.  c_f starts at the largest exponent of
// feature f over the earlier segments and rises (with the carry rescaled) when a block's
// keys exceed it by more than kTau; the query rows use their own maximum over the features.
#include <hip/hip_runtime.h>

#include <math.h>

#include <type_traits>

#include "favor_device.hpp"
#include "favor_ops.hpp"
#include "favor_plan.hpp"

namespace favor {

// ======================================================================================
// causal_scan_pf: per kv head bh and feature f, walking the segments in order,
//   P_t = sum_{t' < t} 2^(c_t'f - C_tf) S_t'f,   C_tf = max_{t' < t} c_t'f   (-inf for t = 0)
// in the summaries' layout [d+1][m] (rows in vperm order, row d the ones column; float32 or
// bf16 elements, accumulated in float32).  Grid (element groups of the [d+1][m] plane, B*Hkv); each thread owns 4 consecutive features of
// one row and keeps the running maximum of those features itself; the threads of row 0
// also write C_t.  TB segments' loads are in flight at a time.
// ======================================================================================
template <class ST>
__global__ void __launch_bounds__(256) causal_scan_pf_kernel(const ST* __restrict__ gs, const float* __restrict__ gc,
                                                             int T_ranges, int m, int D, ST* __restrict__ prefix,
                                                             float* __restrict__ prefix_c) {
  const int bh = blockIdx.y;
  const int e4 = blockIdx.x * 256 + threadIdx.x;  // group of 4 elements within the [d+1][m] plane
  if (e4 >= (D + 1) * m / 4) return;
  const int f = (e4 * 4) % m;
  const bool row0 = e4 * 4 < m;
  const size_t plane = (size_t)(D + 1) * m;
  const float* pc = gc + (size_t)bh * T_ranges * m;
  const ST* src = gs + (size_t)bh * T_ranges * plane + 4 * (size_t)e4;
  ST* dst = prefix + (size_t)bh * T_ranges * plane + 4 * (size_t)e4;
  float* dc = prefix_c + (size_t)bh * T_ranges * m + f;
  constexpr int TB = 8;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  f32x4 run = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  for (int t0 = 0; t0 < T_ranges; t0 += TB) {
    f32x4 sv[TB], cv[TB];
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int t = min(t0 + u, T_ranges - 1);
      sv[u] = load_sum4(src + (size_t)t * plane);
      cv[u] = *reinterpret_cast<const f32x4*>(pc + (size_t)t * m + f);
    }
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int t = t0 + u;
      if (t >= T_ranges) break;
      store_sum4(dst + (size_t)t * plane, acc);
      if (row0) *reinterpret_cast<f32x4*>(dc + (size_t)t * m) = run;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float nc = fmaxf(run[i], cv[u][i]);
        if (nc == -INFINITY) continue;  // nothing seen yet (an empty segment summary is zero)
        acc[i] = acc[i] * fast_exp2(run[i] - nc) + sv[u][i] * fast_exp2(cv[u][i] - nc);
        run[i] = nc;
      }
    }
  }
}

// ======================================================================================
// causal_v: the chunked prefix pass.  Grid (segments, B*Hq); NW = 2 d/32 waves.
//   Feature maps: the m/32 feature tiles are dealt to the waves (tile ft to wave ft % NW);
//   a wave computes the key and query exponents of its tiles on the MFMA (fp16 W x log2 e
//   in registers), the key features phi_K = 2^(. - c_f) into LDS as [feature][key], the
//   query exponents' row maxima into LDS; after a barrier the rows' maxima M are known and
//   phi_Q = 2^(. + c_f - M) goes to LDS in MFMA-operand order, with the wave's share of the
//   inter-block denominator phi_Q . S_1 and of the intra-block matrix A^T = phi_K phi_Q^T.
//   Products: wave (vt, fg) owns value columns [32 vt, 32 vt + 32) and group fg of the
//   features (NFG groups): it keeps that part of the carry S_v in registers (float32) and forms
//     num = S_v^T phi_Q^T (its features) [+ V^T tril(A)^T (fg = 0)],  S_v += phi_K^T V.
//   The fg > 0 waves hand their numerators to the fg = 0 wave, which divides by
//     den = sum of the waves' phi_Q . S_1 + the row sums of tril(A)
//   and stores the bf16 output.  S_1 (the ones column) lives in LDS, one float per feature.
// A block whose keys exceed their features' c_f by more than kTau raises those c_f first
// (carry and S_1 rescaled); the first block of the sequence sets them.
// ======================================================================================
// Largest spread (log2 units) of one feature's key exponents taken in one block: beyond it,
// or when a block's keys jump that far above c_f, the block runs one position at a time.
// Within it every query's own terms stay above 2^-kSpread of the largest, far from float32
// and bf16 underflow.
constexpr float kSpread = 100.f;

template <int D, int NFG> struct CausalV {
  static constexpr int NV = D / 32;       // value tiles
  static constexpr int NW = NFG * NV;     // waves: (value tile, feature group)
  static constexpr int LDK = D + 8;       // fp16 Q / K staging rows
  static constexpr int LDV = D + 16;      // bf16 V staging rows (transposed reads)
  static constexpr int LDP = 40;          // phi_K rows: 32 keys + pad (bf16)
  static constexpr int LDN = 36;          // numerator hand-over rows (float)
  // LDS bytes for at most 32 nft features
  static constexpr int bytes(int nft) {
    return 2 * 32 * LDK * 2 + 32 * LDV * 2 + 32 * nft * LDP * 2 + 32 * (32 * nft + 8) * 2 + NW * 1024 * 4 +
           NV * (NFG - 1) * 32 * LDN * 4 + 3 * 32 * nft * 4 + 2 * NW * 32 * 4 + 16;
  }
};

template <int D, int NFTMAX, int NFG, bool REPAIR>
__global__ void __launch_bounds__(64 * (D / 32) * NFG, (D / 32) * NFG == 4 && !REPAIR ? 2 : 1) causal_v_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V, const float* __restrict__ W,
    const bf16* __restrict__ prefix, const float* __restrict__ prefix_c, bf16* __restrict__ out, int L, int Hq,
    int Hkv, int Hw, int m, int R, int T_ranges, int* __restrict__ wide) {
  using Cfg = CausalV<D, NFG>;
  constexpr int NV = Cfg::NV, NW = Cfg::NW, LDK = Cfg::LDK, LDV = Cfg::LDV, LDP = Cfg::LDP, LDN = Cfg::LDN;
  constexpr int NKC = D / 16;
  constexpr int NMAP = (NFTMAX + NW - 1) / NW;  // feature tiles per wave in the map phase
  constexpr int NCT = NFTMAX / NFG;             // carry tiles per wave (its feature group)
  constexpr int NT = 64 * NW;
  const int NFT = m / 32;
  constexpr int LDQ = 32 * NFTMAX + 8;          // phi_Q rows (bf16)
  constexpr int MMAX = 32 * NFTMAX;

  __shared__ __attribute__((aligned(16))) char smem[Cfg::bytes(NFTMAX)];
  f16* Ql = reinterpret_cast<f16*>(smem);                       // [32][LDK]
  f16* Kl = Ql + 32 * LDK;                                      // [32][LDK]
  bf16* Vl = reinterpret_cast<bf16*>(Kl + 32 * LDK);            // [32][LDV]
  bf16* Pk = Vl + 32 * LDV;                                     // [m][LDP]
  bf16* Pq = Pk + (size_t)MMAX * LDP;                           // [32][LDQ]
  float* Ap = reinterpret_cast<float*>(Pq + 32 * LDQ);          // [NW][16][64] partial A^T
  float* Np = Ap + NW * 1024;                                   // [NV][NFG-1][32][LDN] numerator hand-over
  float* S1 = Np + NV * (NFG - 1) * 32 * LDN;                   // [m]
  float* Csh = S1 + MMAX;                                       // [m] c_f shift of the window
  float* S1b = Csh + MMAX;                                      // [m] S_1 before the window, rescaled
  float* Mr = S1b + MMAX;                                       // [NW][32] partial row maxima
  float* Dp = Mr + NW * 32;                                     // [NW][32] partial denominators
  int* flag = reinterpret_cast<int*>(Dp + NW * 32);             // [2]

  const int seg = blockIdx.x, bhq = blockIdx.y;
  // the repair pass redoes only the segments whose first pass met a wide block
  if (REPAIR && wide[(size_t)bhq * T_ranges + seg] == 0) return;
  const int b = bhq / Hq, hq = bhq % Hq, hkv = hq / (Hq / Hkv), bh = b * Hkv + hkv;
  const int wave = threadIdx.x >> 6, l = lane_id(), col = l & 31, g = l >> 5;
  const int vt = wave % NV, fg = wave / NV;
  const float* Wh = W + (size_t)(Hw == 1 ? 0 : hkv) * m * D;
  const bf16* Qh = Q + (size_t)bhq * L * D;
  bf16* Oh = out + (size_t)bhq * L * D;
  const bf16* Kh = K + (size_t)bh * L * D;
  const bf16* Vh = V + (size_t)bh * L * D;

  // ---- state -------------------------------------------------------------------------
  // map tiles of this wave: ft = wave + NW i; W fragments and c_f of feature 32 ft + col
  f16x8 wf[NMAP][NKC];
  float cf[NMAP];
#pragma unroll
  for (int i = 0; i < NMAP; ++i) {
    const int ft = wave + NW * i;
    if (ft < NFT) {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) load_w_frag(Wh + (size_t)(32 * ft + col) * D, kc, g, wf[i][kc]);
      cf[i] = prefix_c[((size_t)bh * T_ranges + seg) * m + 32 * ft + col];
    }
  }
  // carry of value tile vt, features of group fg: tile ct covers features 32 (fg nct + ct) + ..
  const int nct = NFT / NFG;
  const bf16* Pp = prefix + ((size_t)bh * T_ranges + seg) * (size_t)(D + 1) * m;
  f32x16 carry[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    carry[ct] = zero16();
    if (ct < nct) {
      const int fb = 32 * (fg * nct + ct);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 v = load_sum4(Pp + (size_t)(32 * vt + col) * m + fb + 8 * r4 + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) carry[ct][4 * r4 + i] = v[i];
      }
    }
  }
  for (int f = threadIdx.x; f < m; f += NT) S1[f] = (float)Pp[(size_t)D * m + f];

  // ---- staging: the block's Q, K (fp16) and V (bf16, columns permuted) ----------------
  // range-checked buffer loads: rows past L read as zero
  const unsigned head_bytes = (unsigned)L * (unsigned)D * 2u;
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void*)Qh, (short)0, (int)head_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, (int)head_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, (int)head_bytes, kBufWord3);
  constexpr int CPR = D / 8, NCH = 32 * CPR;            // 16-byte chunks per row, per block
  constexpr int PER = (NCH + NT - 1) / NT;
  f32x4 pq_[PER], pk_[PER], pv_[PER];
  auto prefetch = [&](int q0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + i * NT;
      const int row = c / CPR, c0 = (c % CPR) * 8;
      const unsigned off = c < NCH && q0 + row < L ? ((unsigned)(q0 + row) * D + c0) * 2u : head_bytes;
      pq_[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, (int)off, 0, 0));
      pk_[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, (int)off, 0, 0));
      pv_[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, (int)off, 0, 0));
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + i * NT;
      if (c < NCH) {
        const int row = c / CPR, c0 = (c % CPR) * 8;
        *reinterpret_cast<f16x8*>(Ql + row * LDK + c0) = to_wfrag(__builtin_bit_cast(bf16x8, pq_[i]));
        *reinterpret_cast<f16x8*>(Kl + row * LDK + c0) = to_wfrag(__builtin_bit_cast(bf16x8, pk_[i]));
        bf16* drow = Vl + row * LDV + (c0 & ~31);
        *reinterpret_cast<float2*>(drow + vperm_inv(c0 & 31)) = float2{pv_[i][0], pv_[i][1]};
        *reinterpret_cast<float2*>(drow + vperm_inv((c0 & 31) + 4)) = float2{pv_[i][2], pv_[i][3]};
      }
    }
  };

  const int p_begin = seg * R, p_end = min(p_begin + R, L);
  prefetch(p_begin);
  int wide_any = 0;
  bf16x2 one2;
  one2[0] = one2[1] = (bf16)1.f;

  for (int p0 = p_begin; p0 < p_end; p0 += 32) {
    __syncthreads();  // the previous block's readers of Ql / Kl / Vl are done
    stage();
    if (p0 + 32 < p_end) prefetch(p0 + 32);
    const int pend = min(p0 + 32, L);
    // The block is taken whole, or -- when its keys' exponents spread (or jump above c_f) by
    // more than kSpread for some feature -- one position at a time, so that no query's
    // terms can underflow against a later key of its own block.  Keys and queries outside
    // the window [lo, hi) are masked / not stored.
    // step(lo, hi, check): the positions [lo, hi) of the block.  check: look for a wide
    // block (see below); the repair pass then returns true having committed nothing, the
    // first pass records it and goes on.  The repair pass rewrites every output of the
    // segments it redoes.
    auto step = [&](const int lo, const int hi, const bool check) -> bool {
      if (threadIdx.x == 0) {
        flag[0] = 0;
        flag[1] = 0;
      }
      __syncthreads();  // staging done; the previous step's readers of Pk / Pq / Ap / Np done

      // ---- map phase 1: key features, their maxima, query exponents -----------------
      f16x8 kf[NKC];
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) kf[kc] = load_frag_k(Kl + col * LDK, kc, g);
      float nrm = sumsq(kf);
      nrm += partner32(nrm);
      const bool kin = p0 + col >= lo && p0 + col < hi;  // key col of the block in the window
      const f16x8 biasA = bias_rows(kin ? 0.5f * kLog2e * nrm : kMaskedRow, g, f16x8{});
      f32x16 cq[NMAP];
      float s1inc[NMAP], cnew[NMAP];
      float mloc = -INFINITY;
#pragma unroll
      for (int i = 0; i < NMAP; ++i) {
        const int ft = wave + NW * i;
        s1inc[i] = 0.f;
        cnew[i] = cf[i];
        if (ft >= NFT) continue;
        // key exponents relative to c_f: C[key][feature], lane = feature
        f32x16 ck = zero16();
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) ck = mma(kf[kc], wf[i][kc], ck);
        const bool init = cf[i] == -INFINITY;
        ck = mma(biasA, bias_cols(init ? 0.f : cf[i], g, f16x8{}), ck);
        // masked keys sit near -kMaskedRow: far below any key in the window
        float mx = ck[0], mn = ck[0] > -0.5f * kMaskedRow ? ck[0] : INFINITY;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
          mx = fmaxf(mx, ck[r]);
          mn = fminf(mn, ck[r] > -0.5f * kMaskedRow ? ck[r] : INFINITY);
        }
        mx = fmaxf(mx, partner32(mx));
        mn = fminf(mn, partner32(mn));
        // wide: the first keys of the sequence spread too far (an early query could see only
        // keys far below the block's largest), or a key jumps too far above c_f (the rescaled
        // carry of the queries before it would underflow).  Keys far below c_f are harmless
        // once there is a carry: it holds the key that set c_f.
        if (check && (init ? mx - mn > kSpread : mx > kSpread) && g == 0) flag[1] = 1;
        // c_f is set by the first keys of the sequence and raised when the window's keys
        // pass it by more than kTau; the carry and S_1 of a raised feature are rescaled by
        // 2^(old - new) (0 where it was unset).  Committed after the spread check.
        float shift = 0.f;
        if (init || mx > kTau) shift = mx;
        if (shift != 0.f) {
#pragma unroll
          for (int r = 0; r < 16; ++r) ck[r] -= shift;
          if (g == 0) flag[0] = 1;
        }
        if (g == 0) {
          Csh[32 * ft + col] = init ? -INFINITY : -shift;
          S1b[32 * ft + col] = init ? 0.f : (shift != 0.f ? S1[32 * ft + col] * fast_exp2(-shift) : S1[32 * ft + col]);
        }
        cnew[i] = (init ? 0.f : cf[i]) + shift;
        // key features to LDS [feature][key] and the window's S_1 increment of the feature
        bf16x8 ka[2];
        f32x16 e;
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = fast_exp2(ck[r]);
        acc_to_frags(e, ka);
        float sum = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            bf16x2 v2;
            v2[0] = ka[h][j];
            v2[1] = ka[h][j + 1];
            sum = __builtin_amdgcn_fdot2_f32_bf16(v2, one2, sum, false);
          }
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            bf16x4_t v;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = ka[h][4 * hh + q];
            *reinterpret_cast<bf16x4_t*>(Pk + (32 * ft + col) * LDP + 8 * (2 * h + hh) + 4 * g) = v;
          }
        }
        s1inc[i] = sum + partner32(sum);
      }
      // query exponents + c_f: C[feature][query], lane = query
      f16x8 qf[NKC];
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) qf[kc] = load_frag_k(Ql + col * LDK, kc, g);
#pragma unroll
      for (int i = 0; i < NMAP; ++i) {
        const int ft = wave + NW * i;
        if (ft >= NFT) continue;
        cq[i] = zero16();
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) cq[i] = mma(wf[i][kc], qf[kc], cq[i]);
        cq[i] = mma(bias_rows(-cnew[i], g, f16x8{}), bias_cols(0.f, g, f16x8{}), cq[i]);
        float qm = cq[i][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) qm = fmaxf(qm, cq[i][r]);
        mloc = fmaxf(mloc, qm);
      }
      mloc = fmaxf(mloc, partner32(mloc));
      if (g == 0) Mr[wave * 32 + col] = mloc;
      __syncthreads();
      if (check && __builtin_amdgcn_readfirstlane(flag[1]) != 0) {  // the same in every lane
        if (REPAIR) return true;  // nothing committed: the caller redoes the block position by position
        wide_any = 1;
      }
#pragma unroll
      for (int i = 0; i < NMAP; ++i) cf[i] = cnew[i];

      // ---- rescale the carry where c_f rose ---------------------------------------------
      if (__builtin_amdgcn_readfirstlane(flag[0]) != 0) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          if (ct >= nct) continue;
          const int fb = 32 * (fg * nct + ct);
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 sh = *reinterpret_cast<const f32x4*>(Csh + fb + 8 * r4 + 4 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i) carry[ct][4 * r4 + i] *= fast_exp2(sh[i]);
          }
        }
      }

      // ---- map phase 2: query features, the denominator share, A^T share --------------
      float M = Mr[col];
#pragma unroll
      for (int w = 1; w < NW; ++w) M = fmaxf(M, Mr[w * 32 + col]);
      float dsh = 0.f;
      f32x16 at = zero16();
#pragma unroll
      for (int i = 0; i < NMAP; ++i) {
        const int ft = wave + NW * i;
        if (ft >= NFT) continue;
        bf16x8 qa[2];
        f32x16 e;
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = fast_exp2(cq[i][r] - M);
        acc_to_frags(e, qa);
#pragma unroll
        for (int h = 0; h < 2; ++h) *reinterpret_cast<bf16x8*>(Pq + col * LDQ + 32 * ft + 16 * h + 8 * g) = qa[h];
        // phi_Q . S_1 over this tile's features (the bf16 values the numerator uses); S_1
        // of the positions before the window, relative to the window's c_f
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 sv = *reinterpret_cast<const f32x4*>(S1b + 32 * ft + 8 * r4 + 4 * g);
#pragma unroll
          for (int q = 0; q < 4; ++q) dsh = __builtin_fmaf((float)qa[r4 >> 1][4 * (r4 & 1) + q], sv[q], dsh);
        }
        // A^T[key][query] += phi_K phi_Q^T over this tile's features (keys through a
        // transposed read of the wave's own Pk rows)
#pragma unroll
        for (int h = 0; h < 2; ++h) at = mma(lds_frag_rows(Pk, LDP, 32 * ft, 0, h), qa[h], at);
      }
      dsh += partner32(dsh);
      if (g == 0) Dp[wave * 32 + col] = dsh;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<f32x4*>(Ap + (wave * 4 + r4) * 256 + 4 * l) =
            f32x4{at[4 * r4], at[4 * r4 + 1], at[4 * r4 + 2], at[4 * r4 + 3]};
      __syncthreads();

      // ---- S_1 of the positions up to the window's end (owners) -------------------------
#pragma unroll
      for (int i = 0; i < NMAP; ++i) {
        const int ft = wave + NW * i;
        if (ft < NFT && g == 0) S1[32 * ft + col] = S1b[32 * ft + col] + s1inc[i];
      }

      // ---- products of wave (vt, fg) ----------------------------------------------------
      // tril(A)^T with the rows summed in fixed order, and its row sums (denominator)
      f32x16 asum = zero16();
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(Ap + (w * 4 + r4) * 256 + 4 * l);
#pragma unroll
          for (int q = 0; q < 4; ++q) asum[4 * r4 + q] += v[q];
        }
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + 4 * g + (r & 3) > col) asum[r] = 0.f;
      bf16x8 ab[2];
      acc_to_frags(asum, ab);
      f32x16 num = zero16();
      // V^T operands of value tile vt (rows: keys in operand order)
      bf16x8 vo[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) vo[h] = lds_frag_rows(Vl, LDV, 0, 32 * vt, h);
      if (fg == 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) num = mma(vo[h], ab[h], num);
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        if (ct >= nct) continue;
        const int ftg = fg * nct + ct;
        bf16x8 ca[2];
        acc_to_frags(carry[ct], ca);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16x8 qb = *reinterpret_cast<const bf16x8*>(Pq + col * LDQ + 32 * ftg + 16 * h + 8 * g);
          num = mma(ca[h], qb, num);
        }
        // carry += phi_K^T V: phi_K rows of these features, keys in operand order
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16* prow = Pk + (32 * ftg + col) * LDP + 16 * h + 4 * g;
          const bf16x4_t plo = *reinterpret_cast<const bf16x4_t*>(prow);
          const bf16x4_t phi = *reinterpret_cast<const bf16x4_t*>(prow + 8);
          bf16x8 pa;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            pa[q] = plo[q];
            pa[q + 4] = phi[q];
          }
          carry[ct] = mma(pa, vo[h], carry[ct]);
        }
      }
      if (fg > 0) {
        float* np = Np + ((vt * (NFG - 1) + fg - 1) * 32 + col) * LDN + 16 * g;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *reinterpret_cast<f32x4*>(np + 4 * r4) = f32x4{num[4 * r4], num[4 * r4 + 1], num[4 * r4 + 2], num[4 * r4 + 3]};
      }
      float dintra = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) dintra += asum[r];
      dintra += partner32(dintra);
      __syncthreads();
      if (fg == 0) {
        float den = dintra;
#pragma unroll
        for (int w = 0; w < NW; ++w) den += Dp[w * 32 + col];
        const int pos = p0 + col;
        const float inv = __builtin_amdgcn_rcpf(den);
        if (pos >= lo && pos < hi) {
#pragma unroll
          for (int u = 1; u < NFG; ++u) {
            const float* np = Np + ((vt * (NFG - 1) + u - 1) * 32 + col) * LDN + 16 * g;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const f32x4 h = *reinterpret_cast<const f32x4*>(np + 4 * r4);
#pragma unroll
              for (int q = 0; q < 4; ++q) num[4 * r4 + q] += h[q];
            }
          }
          bf16x8 o0, o1;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            o0[j] = (bf16)(num[j] * inv);
            o1[j] = (bf16)(num[8 + j] * inv);
          }
          bf16* orow = Oh + (size_t)pos * D + 32 * vt + 16 * g;
          *reinterpret_cast<bf16x8*>(orow) = o0;
          *reinterpret_cast<bf16x8*>(orow + 8) = o1;
        }
      }
      return false;
    };
    if constexpr (REPAIR) {
      if (step(p0, pend, true))
        for (int q = p0; q < pend; ++q) step(q, q + 1, false);
    } else {
      step(p0, pend, true);
    }
  }
  if (!REPAIR && threadIdx.x == 0) wide[(size_t)bhq * T_ranges + seg] = wide_any;
}

// ======================================================================================
// causal_fg (d = 64): the chunked prefix pass with the features split over the waves.
// Grid (segments, B*Hq); NW waves, wave w owns features [64 w, 64 w + 64) (none when
// 64 w >= m) and works on them alone through a 32-position block:
//   key features  phi_K = 2^(w_f.k - |k|^2/2 - c_f), c_f per feature (set by the first keys
//                 of the sequence, raised with its carry rescaled when the block's keys pass
//                 it by more than kTau);
//   query features relative to the wave's own row maxima: phi_Q = 2^(w_f.q + c_f - M_w);
//   num_w = S_v,w^T phi_Q^T + V^T tril(phi_K phi_Q^T)^T    (its features, all 64 columns)
//   den_w = phi_Q . S_1,w + row sums of tril(phi_Q phi_K^T)
//   S_v,w += phi_K^T V,  S_1,w += the keys' sum of phi_K.
// The partials meet in LDS once per block: with M = max_w M_w,
//   out = sum_w 2^(M_w - M) num_w / sum_w 2^(M_w - M) den_w,
// each wave finishing 8 / NW of the block's eight 4-column groups of each value tile pair.
// Two barriers per block (staged Q / K / V ready; partials ready).  phi_K reaches the
// intra-block product through the wave's own LDS rows (a transposed read), which needs no
// barrier: one wave's LDS accesses complete in issue order.
// ======================================================================================
template <int NW, int NB> struct CausalFg {
  static constexpr int D = 64, LDK = D + 8, LDV = D + 16, LDP = 40;
  // Q (fp16) of a block; K (fp16) and V (bf16) of the NB blocks of a chunk
  static constexpr int STAGE = 32 * LDK * 2 + NB * (32 * LDK * 2 + 32 * LDV * 2);
  static constexpr int PK = 64 * LDP * 2;                        // per wave: phi_K [64 features][keys]
  static constexpr int RED = 2 * 4 * 64 * 16;                    // per wave: numerator partial
  static constexpr int DM = 32 * 8;                              // per wave: (den_w, M_w) per query
  static constexpr int VEC = 2 * 64 * 4;                         // per wave: S_1 before the block, c_f shifts
  static constexpr int BYTES = STAGE + NW * (PK + RED + DM + VEC) + 64;
};

template <int NW, int NB, bool REPAIR>
__global__ void __launch_bounds__(64 * NW, REPAIR || NW < 4 || NB > 1 ? 1 : 8 / NW) causal_fg_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V, const float* __restrict__ W,
    const bf16* __restrict__ prefix, const float* __restrict__ prefix_c, bf16* __restrict__ out, int L, int Hq,
    int Hkv, int Hw, int m, int R, int T_ranges, int* __restrict__ wide, int n_units) {
  using Cfg = CausalFg<NW, NB>;
  static_assert(NB == 1 || !REPAIR, "the repair pass takes the chunk as 32 positions");
  constexpr int D = 64, NKC = D / 16, LDK = Cfg::LDK, LDV = Cfg::LDV, LDP = Cfg::LDP, NT = 64 * NW;
  constexpr int UPW = 8 / NW;  // 4-column output groups a wave finishes per block
  __shared__ __attribute__((aligned(16))) char smem[Cfg::BYTES];
  const int wave = threadIdx.x >> 6, l = lane_id(), col = l & 31, g = l >> 5;
  f16* Ql = reinterpret_cast<f16*>(smem);                            // [32][LDK]
  f16* Kc = Ql + 32 * LDK;                                           // [NB][32][LDK]
  bf16* Vc = reinterpret_cast<bf16*>(Kc + NB * 32 * LDK);            // [NB][32][LDV], columns permuted
  char* wb = smem + Cfg::STAGE;
  bf16* Pk = reinterpret_cast<bf16*>(wb + wave * Cfg::PK);           // own [64][LDP]
  float* Red = reinterpret_cast<float*>(wb + NW * Cfg::PK);          // [NW][2][4][64] x f32x4
  float2* Dm = reinterpret_cast<float2*>(wb + NW * (Cfg::PK + Cfg::RED));  // [NW][32]
  float* S1v = reinterpret_cast<float*>(wb + NW * (Cfg::PK + Cfg::RED + Cfg::DM)) + wave * 128;  // own [64]
  float* Csh = S1v + 64;                                                                          // own [64]
  int* flagw = reinterpret_cast<int*>(wb + NW * (Cfg::PK + Cfg::RED + Cfg::DM + Cfg::VEC));       // [NW]

  // One segment (seg, bhq) from its prefix.  First pass: one per workgroup.  Repair pass:
  // the workgroups walk the n_units = B Hq T flags and redo the segments whose first pass
  // met a wide block.
  auto run_segment = [&](const int seg, const int bhq) {
  const int b = bhq / Hq, hq = bhq % Hq, hkv = hq / (Hq / Hkv), bh = b * Hkv + hkv;
  const int f0 = 64 * wave;
  const bool active = f0 < m;
  const float* Wh = W + (size_t)(Hw == 1 ? 0 : hkv) * m * D;
  const bf16* Qh = Q + (size_t)bhq * L * D;
  bf16* Oh = out + (size_t)bhq * L * D;
  const bf16* Kh = K + (size_t)bh * L * D;
  const bf16* Vh = V + (size_t)bh * L * D;

  // ---- state of the wave's features: W x log2 e (fp16), c_f, S_1 (lane = feature
  // 32 i + col), the carry S_v [feature][value] of tile i and value tile vt --------------
  f16x8 wf[2][NKC];
  float cf[2], s1r[2];
  f32x16 carry[2][2];
  // bias operands of c_f: key side -(c_f) on the feature columns (0 while c_f is unset),
  // query side +c_f on the feature rows; rebuilt only when c_f moves
  f16x8 bk[2], bq[2];
  const bf16* Pp = prefix + ((size_t)bh * T_ranges + seg) * (size_t)(D + 1) * m;
  const float* Pc = prefix_c + ((size_t)bh * T_ranges + seg) * m;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    cf[i] = 0.f;
    s1r[i] = 0.f;
#pragma unroll
    for (int vt = 0; vt < 2; ++vt) carry[i][vt] = zero16();
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) wf[i][kc] = zero_frag(f16x8{});
    if (active) {
      const int f = f0 + 32 * i;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) load_w_frag(Wh + (size_t)(f + col) * D, kc, g, wf[i][kc]);
      cf[i] = Pc[f + col];
      s1r[i] = (float)Pp[(size_t)D * m + f + col];
#pragma unroll
      for (int vt = 0; vt < 2; ++vt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 v = load_sum4(Pp + (size_t)(32 * vt + col) * m + f + 8 * r4 + 4 * g);
#pragma unroll
          for (int q = 0; q < 4; ++q) carry[i][vt][4 * r4 + q] = v[q];
        }
    }
    bk[i] = bias_cols(cf[i] == -INFINITY ? 0.f : cf[i], g, f16x8{});
    bq[i] = bias_rows(cf[i] == -INFINITY ? 0.f : -cf[i], g, f16x8{});
  }

  // ---- staging: the block's Q, K (fp16) and V (bf16, columns permuted) ----------------
  // range-checked buffer loads: rows past L read as zero
  const unsigned head_bytes = (unsigned)L * (unsigned)D * 2u;
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void*)Qh, (short)0, (int)head_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, (int)head_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, (int)head_bytes, kBufWord3);
  constexpr int CPR = D / 8, NCH = 32 * CPR;  // 16-byte chunks per row, per block
  constexpr int PER = (NCH + NT - 1) / NT;
  f32x4 pq_[PER], pk_[PER], pv_[PER];
  auto prefetch = [&](int q0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + i * NT;
      const int row = c / CPR, c0 = (c % CPR) * 8;
      const unsigned off = c < NCH && q0 + row < L ? ((unsigned)(q0 + row) * D + c0) * 2u : head_bytes;
      pq_[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, (int)off, 0, 0));
      pk_[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, (int)off, 0, 0));
      pv_[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, (int)off, 0, 0));
    }
  };
  auto stage = [&](f16* Kl, bf16* Vl) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + i * NT;
      if (c < NCH) {
        const int row = c / CPR, c0 = (c % CPR) * 8;
        *reinterpret_cast<f16x8*>(Ql + row * LDK + c0) = to_wfrag(__builtin_bit_cast(bf16x8, pq_[i]));
        *reinterpret_cast<f16x8*>(Kl + row * LDK + c0) = to_wfrag(__builtin_bit_cast(bf16x8, pk_[i]));
        bf16* drow = Vl + row * LDV + (c0 & ~31);
        *reinterpret_cast<float2*>(drow + vperm_inv(c0 & 31)) = float2{pv_[i][0], pv_[i][1]};
        *reinterpret_cast<float2*>(drow + vperm_inv((c0 & 31) + 4)) = float2{pv_[i][2], pv_[i][3]};
      }
    }
  };

  bf16x2 one2;
  one2[0] = one2[1] = (bf16)1.f;
  // tril masks of the intra-block product's operand words: slot j of operand h carries key
  // 16 h + 8 (j/4) + 4 g + j%4 of query col; a 16-bit half is kept when key <= col
  u32x4 tril[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k0 = 16 * h + 8 * ((2 * j) >> 2) + 4 * g + ((2 * j) & 3);
      tril[h][j] = (k0 <= col ? 0x0000FFFFu : 0u) | (k0 + 1 <= col ? 0xFFFF0000u : 0u);
    }
  bool wide_w = false;  // first pass: a block of this wave's features was wide

  // Key exponents of tile i relative to c_f (C[key][feature], lane = feature).
  auto key_exp = [&](const f16x8 (&kf)[NKC], const f16x8& biasA, int i) {
    f32x16 ck = zero16();
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) ck = mma(kf[kc], wf[i][kc], ck);
    return mma(biasA, bk[i], ck);
  };
  // A block is wide when one feature's key exponents spread by more than kSpread over the
  // first keys of the sequence (an early query may see only keys far below the block's
  // largest), or when a key passes c_f by more than kSpread (the rescaled carry of the
  // queries before it would underflow).  Keys far below c_f are harmless once there is a
  // carry: it holds the key that set c_f.  Masked keys sit near -kMaskedRow.
  auto is_wide = [&](const f32x16& ck, float mx, bool init) {
    if (!init) return mx > kSpread;
    float mn = INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mn = fminf(mn, ck[r] > -0.5f * kMaskedRow ? ck[r] : INFINITY);
    mn = pair_min(mn);
    return mx - mn > kSpread;
  };
  auto row_max = [&](const f32x16& c) {
    float mx = c[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, c[r]);
    return pair_max(mx);
  };

  // bf16 operands of the chunk-start carry S_v (NB > 1): converted once per chunk
  bf16x8 ca[2][2][2];

  const int p_begin = seg * R, p_end = min(p_begin + R, L);
  prefetch(p_begin);

  for (int p0 = p_begin; p0 < p_end; p0 += 32) {
    // block `slot` of its chunk (segments start on chunk boundaries)
    const int slot = NB == 1 ? 0 : ((p0 - p_begin) >> 5) % NB;
    f16* Kl = Kc + slot * 32 * LDK;
    bf16* Vl = Vc + slot * 32 * LDV;
    // every wave is past the previous block's second barrier: its staging reads are done
    stage(Kl, Vl);
    if (p0 + 32 < p_end) prefetch(p0 + 32);
    __syncthreads();
    const int pend = min(p0 + 32, L);
    // step(lo, hi, check): the positions [lo, hi) of the block (keys outside masked, rows
    // outside not stored).  The repair pass first tests the whole block (check) and
    // returns true, having changed nothing, when it is wide; the caller then takes the
    // block one position at a time.
    auto step = [&](const int lo, const int hi, const bool check) -> bool {
      if (REPAIR && !check) __syncthreads();  // the previous position's partials are read
      f16x8 kf[NKC];
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) kf[kc] = load_frag_k(Kl + col * LDK, kc, g);
      const float nrm = pair_sum(sumsq(kf));
      const bool kin = p0 + col >= lo && p0 + col < hi;
      const f16x8 biasA = bias_rows(kin ? 0.5f * kLog2e * nrm : kMaskedRow, g, f16x8{});
      if (REPAIR && check) {
        bool wd = false;
        if (active) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const bool init = cf[i] == -INFINITY;
            const f32x16 ck = key_exp(kf, biasA, i);
            wd = wd || is_wide(ck, row_max(ck), init);
          }
        }
        const bool any = wave_any(wd);
        if (l == 0) flagw[wave] = any ? 1 : 0;
        __syncthreads();
        int a = 0;
#pragma unroll
        for (int p = 0; p < NW; ++p) a |= flagw[p];
        if (a != 0) return true;
      }

      // the wave's partial to LDS: numerator (registers 4 r4 .. of value tile vt), den_w, M_w
      auto put = [&](const f32x16 (&num)[2], float den, float Mw) {
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            *reinterpret_cast<f32x4*>(Red + ((size_t)((wave * 2 + vt) * 4 + r4) * 64 + l) * 4) =
                f32x4{num[vt][4 * r4], num[vt][4 * r4 + 1], num[vt][4 * r4 + 2], num[vt][4 * r4 + 3]};
        if (g == 0) Dm[wave * 32 + col] = float2{den, Mw};
      };
      if (!active) {
        f32x16 num[2];
        num[0] = num[1] = zero16();
        put(num, 0.f, -INFINITY);
      } else {
        f32x16 num[2];
        float Mw = -INFINITY;
        // ---- key features: c_f, phi_K to the wave's LDS rows, S_1 ------------------------
        bool shifted = false;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const bool init = cf[i] == -INFINITY;
          f32x16 ck = key_exp(kf, biasA, i);
          const float mx = row_max(ck);
          if (!REPAIR && check) wide_w = wide_w || is_wide(ck, mx, init);
          // c_f := c_f + shift; the carry and S_1 of the feature scale by 2^-shift (0 when
          // it was unset)
          const float shift = init || mx > kTau ? mx : 0.f;
          if (g == 0) Csh[32 * i + col] = init ? -INFINITY : -shift;
          s1r[i] = init ? 0.f : (shift != 0.f ? s1r[i] * fast_exp2(-shift) : s1r[i]);
          // S_1 at the chunk start (the query side's inter-chunk denominator)
          if (g == 0) {
            if (slot == 0)
              S1v[32 * i + col] = s1r[i];
            else if (shift != 0.f)
              S1v[32 * i + col] *= fast_exp2(-shift);
          }
          if (init || shift != 0.f) {
            cf[i] = (init ? 0.f : cf[i]) + shift;
            bk[i] = bias_cols(cf[i], g, f16x8{});
            bq[i] = bias_rows(-cf[i], g, f16x8{});
          }
          shifted = shifted || shift != 0.f;
          if (shift != 0.f) {
#pragma unroll
            for (int r = 0; r < 16; ++r) ck[r] -= shift;
          }
          f32x16 e;
#pragma unroll
          for (int r = 0; r < 16; ++r) e[r] = fast_exp2(ck[r]);
          bf16x8 ka[2];
          acc_to_frags(e, ka);
          float sum = 0.f;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
              bf16x2 v2;
              v2[0] = ka[h][j];
              v2[1] = ka[h][j + 1];
              sum = __builtin_amdgcn_fdot2_f32_bf16(v2, one2, sum, false);
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              bf16x4_t v;
#pragma unroll
              for (int q = 0; q < 4; ++q) v[q] = ka[h][4 * hh + q];
              *reinterpret_cast<bf16x4_t*>(Pk + (32 * i + col) * LDP + 8 * (2 * h + hh) + 4 * g) = v;
            }
          }
          s1r[i] += pair_sum(sum);
        }
        asm volatile("" ::: "memory");  // the wave's LDS writes above before its reads below
        if (wave_any(shifted)) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const f32x4 sh = *reinterpret_cast<const f32x4*>(Csh + 32 * i + 8 * r4 + 4 * g);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float fct = fast_exp2(sh[q]);
#pragma unroll
                for (int vt = 0; vt < 2; ++vt) {
                  carry[i][vt][4 * r4 + q] *= fct;
                  // element 4 (r4 % 2) + q of operand r4 / 2 is carry register 4 r4 + q
                  if (NB > 1 && slot > 0) {
                    const int j = 4 * (r4 & 1) + q;
                    ca[i][vt][r4 >> 1][j] = (bf16)((float)ca[i][vt][r4 >> 1][j] * fct);
                  }
                }
              }
            }
        }
        if (NB > 1 && slot == 0) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) acc_to_frags(carry[i][vt], ca[i][vt]);
        }

        // ---- query features (C[feature][query], lane = query) ----------------------------
        f16x8 qf[NKC];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) qf[kc] = load_frag_k(Ql + col * LDK, kc, g);
        f32x16 cq[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          cq[i] = zero16();
#pragma unroll
          for (int kc = 0; kc < NKC; ++kc) cq[i] = mma(wf[i][kc], qf[kc], cq[i]);
          cq[i] = mma(bq[i], bias_cols(0.f, g, f16x8{}), cq[i]);
          Mw = fmaxf(Mw, row_max(cq[i]));
        }
        bf16x8 qa[2][2];
        float dsh = 0.f;
        // -M_w enters as one more MFMA per tile (the query columns' bias)
        const f16x8 bm = bias_cols(Mw, g, f16x8{});
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          cq[i] = mma(bias_unit_rows(g, f16x8{}), bm, cq[i]);
          f32x16 e;
#pragma unroll
          for (int r = 0; r < 16; ++r) e[r] = fast_exp2(cq[i][r]);
          acc_to_frags(e, qa[i]);
          // phi_Q . S_1 (S_1 of the positions before the block, at the block's c_f)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 sv = *reinterpret_cast<const f32x4*>(S1v + 32 * i + 8 * r4 + 4 * g);
#pragma unroll
            for (int q = 0; q < 4; ++q) dsh = __builtin_fmaf(e[4 * r4 + q], sv[q], dsh);
          }
        }
        dsh = pair_sum(dsh);

        // ---- tril(phi_K phi_Q^T) over the wave's features: C[key][query] -----------------
        f32x16 at = zero16();
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int h = 0; h < 2; ++h) at = mma(lds_frag_rows(Pk, LDP, 32 * i, 0, h), qa[i][h], at);
        // keep key <= query: the bf16 operand masked word by word, its row sums by dot2 (the
        // values the numerator uses)
        float dint = 0.f;
        {
          bf16x8 ab[2];
          acc_to_frags(at, ab);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            u32x4 w = __builtin_bit_cast(u32x4, ab[h]);
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] &= tril[h][j];
            ab[h] = __builtin_bit_cast(bf16x8, w);
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
              bf16x2 v2;
              v2[0] = ab[h][j];
              v2[1] = ab[h][j + 1];
              dint = __builtin_amdgcn_fdot2_f32_bf16(v2, one2, dint, false);
            }
          }
#pragma unroll
          for (int vt = 0; vt < 2; ++vt)
            num[vt] = mma(lds_frag_rows(Vl, LDV, 0, 32 * vt, 1), ab[1],
                          mma(lds_frag_rows(Vl, LDV, 0, 32 * vt, 0), ab[0], zero16()));
        }
        // ---- the chunk's earlier blocks i < slot (NB > 1): phi_Q phi_K,i^T [V_i, 1] ------
        // phi_K,i comes straight in the operand layout (C[feature][key], lane = key) from
        // the chunk's staged K at the current c_f.
        if constexpr (NB > 1) {
          if (slot > 0) {
            f16x8 br[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) br[t] = bias_rows(cf[t], g, f16x8{});
            for (int bi = 0; bi < slot; ++bi) {
              const f16* Ki = Kc + bi * 32 * LDK;
              f16x8 kfi[NKC];
#pragma unroll
              for (int kc = 0; kc < NKC; ++kc) kfi[kc] = load_frag_k(Ki + col * LDK, kc, g);
              const f16x8 bcol = bias_cols(0.5f * kLog2e * pair_sum(sumsq(kfi)), g, f16x8{});
              f32x16 ai = zero16();
#pragma unroll
              for (int t = 0; t < 2; ++t) {
                f32x16 e = zero16();
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc) e = mma(wf[t][kc], kfi[kc], e);
                e = mma(br[t], bcol, e);
#pragma unroll
                for (int r = 0; r < 16; ++r) e[r] = fast_exp2(e[r]);
                bf16x8 kt[2];
                acc_to_frags(e, kt);
#pragma unroll
                for (int h = 0; h < 2; ++h) ai = mma(kt[h], qa[t][h], ai);
              }
#pragma unroll
              for (int r = 0; r < 16; ++r) dint += ai[r];
              bf16x8 abi[2];
              acc_to_frags(ai, abi);
              const bf16* Vi = Vc + bi * 32 * LDV;
#pragma unroll
              for (int vt = 0; vt < 2; ++vt)
                num[vt] = mma(lds_frag_rows(Vi, LDV, 0, 32 * vt, 1), abi[1],
                              mma(lds_frag_rows(Vi, LDV, 0, 32 * vt, 0), abi[0], num[vt]));
            }
          }
        }
        const float den = dsh + pair_sum(dint);

        // ---- inter-chunk numerator and carry update per value tile -------------------------
#pragma unroll
        for (int vt = 0; vt < 2; ++vt) {
          bf16x8 vo[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) vo[h] = lds_frag_rows(Vl, LDV, 0, 32 * vt, h);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            if constexpr (NB == 1) {
              bf16x8 cb[2];
              acc_to_frags(carry[i][vt], cb);
#pragma unroll
              for (int h = 0; h < 2; ++h) num[vt] = mma(cb[h], qa[i][h], num[vt]);
            } else {
#pragma unroll
              for (int h = 0; h < 2; ++h) num[vt] = mma(ca[i][vt][h], qa[i][h], num[vt]);
            }
          }
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const bf16* prow = Pk + (32 * i + col) * LDP + 16 * h + 4 * g;
              const bf16x4_t plo = *reinterpret_cast<const bf16x4_t*>(prow);
              const bf16x4_t phi = *reinterpret_cast<const bf16x4_t*>(prow + 8);
              bf16x8 pa;
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                pa[q] = plo[q];
                pa[q + 4] = phi[q];
              }
              carry[i][vt] = mma(pa, vo[h], carry[i][vt]);
            }
        }
        asm volatile("" ::: "memory");  // this block's LDS reads before the next block's writes
        put(num, den, Mw);
      }
      // ---- the partials meet ----------------------------------------------------------------
      __syncthreads();
      float M = -INFINITY;
#pragma unroll
      for (int p = 0; p < NW; ++p) M = fmaxf(M, Dm[p * 32 + col].y);
      float sc[NW];
      float dd = 0.f;
#pragma unroll
      for (int p = 0; p < NW; ++p) {
        const float2 dm = Dm[p * 32 + col];
        sc[p] = fast_exp2(dm.y - M);  // 0 for a wave without features (M_w = -inf)
        dd = __builtin_fmaf(sc[p], dm.x, dd);
      }
      const float inv = __builtin_amdgcn_rcpf(dd);
      const int pos = p0 + col;
      if (pos >= lo && pos < hi) {
        // group u = wave UPW + j: value tile u / 4, registers 4 (u % 4) .. + 3 = columns
        // 32 (u / 4) + 16 g + 4 (u % 4) .. + 3
        bf16x4_t o[UPW];
#pragma unroll
        for (int j = 0; j < UPW; ++j) {
          const int u = wave * UPW + j, vt = u >> 2, r4 = u & 3;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < NW; ++p) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(Red + ((size_t)((p * 2 + vt) * 4 + r4) * 64 + l) * 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(sc[p], v[q], acc[q]);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) o[j][q] = (bf16)(acc[q] * inv);
        }
        bf16* orow = Oh + (size_t)pos * D + 16 * g;
        if constexpr (UPW == 1) {
          const int u = wave;
          *reinterpret_cast<bf16x4_t*>(orow + 32 * (u >> 2) + 4 * (u & 3)) = o[0];
        } else {
#pragma unroll
          for (int j = 0; j < UPW; j += 2) {
            const int u = wave * UPW + j;
            bf16x8 o8;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              o8[q] = o[j][q];
              o8[q + 4] = o[j + 1][q];
            }
            *reinterpret_cast<bf16x8*>(orow + 32 * (u >> 2) + 4 * (u & 3)) = o8;
          }
        }
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
    if (l == 0) flagw[wave] = any ? 1 : 0;
    __syncthreads();
    if (threadIdx.x == 0) {
      int a = 0;
#pragma unroll
      for (int p = 0; p < NW; ++p) a |= flagw[p];
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

// Exclusive scan of the segment summaries gs / gc with per-feature stabilisers into the
// prefix region of the workspace.
favor_status launch_causal_scan_pf(const Plan& s, char* ws, hipStream_t st) {
  const float* gc = reinterpret_cast<const float*>(ws + s.off_gc);
  float* prefix_c = reinterpret_cast<float*>(ws + s.off_pc);
  const dim3 grid((unsigned)(((size_t)(s.d + 1) * s.m / 4 + 255) / 256), s.BH);
  if (s.dtype == FAVOR_BF16)
    hipLaunchKernelGGL(causal_scan_pf_kernel<bf16>, grid, dim3(256), 0, st, reinterpret_cast<const bf16*>(ws + s.off_gs),
                       gc, s.T, s.m, s.d, reinterpret_cast<bf16*>(ws + s.off_p), prefix_c);
  else
    hipLaunchKernelGGL(causal_scan_pf_kernel<float>, grid, dim3(256), 0, st, reinterpret_cast<const float*>(ws + s.off_gs),
                       gc, s.T, s.m, s.d, reinterpret_cast<float*>(ws + s.off_p), prefix_c);
  return hipGetLastError() == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}

bool causal_v_supported(const Plan& s) { return s.dtype == FAVOR_BF16 && (s.d == 64 || s.m <= 256); }

bool causal_chunk_supported(const Plan& s) {
  if (s.chunk == 32) return true;
  // intra-chunk blocks above 32 positions: bf16 d = 64, and 256 only up to m = 256 (the
  // chunk's staged K and V beside the partials of eight waves do not fit in LDS)
  return s.dtype == FAVOR_BF16 && s.d == 64 && (s.chunk < 256 || s.m <= 256);
}

namespace {

template <int NW, int NB, bool RP>
void launch_fg(const Plan& s, dim3 grid, const bf16* q, const bf16* k, const bf16* v, const float* W,
               const bf16* prefix, const float* prefix_c, bf16* o, int* wide, hipStream_t st) {
  const int n_units = s.T * s.B * s.Hq;
  // the repair pass: one workgroup per CU at most, walking the segment flags
  const dim3 g = RP ? dim3((unsigned)(n_units < kCUs ? n_units : kCUs)) : grid;
  hipLaunchKernelGGL((causal_fg_kernel<NW, NB, RP>), g, dim3(64 * NW), 0, st, q, k, v, W, prefix, prefix_c, o, s.L,
                     s.Hq, s.Hkv, s.Hw, s.m, s.R, s.T, wide, n_units);
}

template <int NB, bool RP>
void launch_fg_nw(const Plan& s, dim3 grid, const bf16* q, const bf16* k, const bf16* v, const float* W,
                  const bf16* prefix, const float* prefix_c, bf16* o, int* wide, hipStream_t st) {
  // one wave per 64 features, NW rounded up to 1, 2, 4 or 8
  const int nw = s.m / 64;
  if (nw <= 1)
    launch_fg<1, NB, RP>(s, grid, q, k, v, W, prefix, prefix_c, o, wide, st);
  else if (nw <= 2)
    launch_fg<2, NB, RP>(s, grid, q, k, v, W, prefix, prefix_c, o, wide, st);
  else if (nw <= 4)
    launch_fg<4, NB, RP>(s, grid, q, k, v, W, prefix, prefix_c, o, wide, st);
  else if constexpr (NB < 8)
    launch_fg<8, NB, RP>(s, grid, q, k, v, W, prefix, prefix_c, o, wide, st);
}

}  // namespace

// The chunked pass (causal_fg_kernel for d = 64, causal_v_kernel for d = 128) from the
// prefixes launch_causal_scan_pf wrote: the first pass over every segment, then the repair
// pass (its workgroups return at once unless their segment met a wide block), which takes
// the chunk as 32 positions.
favor_status launch_causal_v(const Plan& s, const void* Q, const void* K, const void* V, const float* W, void* out,
                             char* ws, hipStream_t st) {
  if (!causal_v_supported(s) || !causal_chunk_supported(s)) return FAVOR_ERR_UNSUPPORTED;
  const bf16* prefix = reinterpret_cast<const bf16*>(ws + s.off_p);
  const float* prefix_c = reinterpret_cast<const float*>(ws + s.off_pc);
  const bf16* q = static_cast<const bf16*>(Q);
  const bf16* k = static_cast<const bf16*>(K);
  const bf16* v = static_cast<const bf16*>(V);
  bf16* o = static_cast<bf16*>(out);
  int* wide = reinterpret_cast<int*>(ws + s.off_wide);
  const dim3 grid(s.T, s.B * s.Hq);
  if (s.d == 64) {
    switch (s.chunk) {
      case 32: launch_fg_nw<1, false>(s, grid, q, k, v, W, prefix, prefix_c, o, wide, st); break;
      case 64: launch_fg_nw<2, false>(s, grid, q, k, v, W, prefix, prefix_c, o, wide, st); break;
      case 128: launch_fg_nw<4, false>(s, grid, q, k, v, W, prefix, prefix_c, o, wide, st); break;
      default: launch_fg_nw<8, false>(s, grid, q, k, v, W, prefix, prefix_c, o, wide, st); break;
    }
    if (hipGetLastError() != hipSuccess) return FAVOR_ERR_HIP;
    launch_fg_nw<1, true>(s, grid, q, k, v, W, prefix, prefix_c, o, wide, st);
    return hipGetLastError() == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
  }
  hipLaunchKernelGGL((causal_v_kernel<128, 8, 2, false>), grid, dim3(64 * 4 * 2), 0, st, q, k, v, W, prefix, prefix_c,
                     o, s.L, s.Hq, s.Hkv, s.Hw, s.m, s.R, s.T, wide);
  if (hipGetLastError() != hipSuccess) return FAVOR_ERR_HIP;
  hipLaunchKernelGGL((causal_v_kernel<128, 8, 2, true>), grid, dim3(64 * 4 * 2), 0, st, q, k, v, W, prefix, prefix_c,
                     o, s.L, s.Hq, s.Hkv, s.Hw, s.m, s.R, s.T, wide);
  return hipGetLastError() == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}

}  // namespace favor
