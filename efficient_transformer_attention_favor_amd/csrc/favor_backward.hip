// Gradients of bidirectional FAVOR+ (the favor_attn_bwd entry point).
//
// "Rethinking Attention with Performers" (review page), section "제안 방법": out = D^-1 A_hat V
// in linear order with positive random features phi.  The pages give no backward pass; the
// gradients below follow from that definition by the chain rule (W is a fixed input).  Per kv
// head, with the G query heads of that head taken as one sequence of G*L query rows,
// S = phi(K)^T [V, 1] = [S_v, S_1] and, per query row i, D_i = phi(q_i) . S_1:
//   g_i  = dout_i / D_i,   h_i = -(dout_i . out_i) / D_i,          G1 = [g, h]   (rows x (d+1))
//   dphi(Q) = G1 S^T,      dS = phi(Q)^T G1,
//   dphi(K) = [V, 1] dS^T, dV = phi(K) dS_v,
//   dX = (dphi(X) * phi(X)) W - X * rowsum(dphi(X) * phi(X))   for X = Q, K
// (d phi(x)_f / dx = phi(x)_f (w_f - x)); for X = Q the row sums are exactly 0 (out_i does not
// change when phi(q_i) is scaled), so that term is left out.  The feature matrices are scaled by any per-row
// (queries) or per-head (keys) constant, as the feature kernels leave them: every product
// above is invariant under those scalings.
//
// Implementation: the feature kernels write phi(Q) and phi(K) as float32 matrices, then seven
// batched float32 GEMMs on the matrix cores (one batch entry per (batch, kv head)) and row
// kernels.  The GEMMs that form dphi(Q) and dphi(K) multiply by phi in their epilogue, so
// they write T = dphi * phi directly (and, for keys, T's row sums in 32-feature partials).
// All arithmetic is float32; bf16 problems round only their inputs and returned gradients.
//
// Causal (inclusive mask j <= i): the positions of each head are cut into chunks of C = 64
// (the last one zero-padded), S_<c is the exclusive prefix of the chunk summaries
// phi(K_c)^T [V_c, 1] and R_>c the exclusive suffix, over later chunks and the G query heads,
// of phi(Q_c)^T G1_c.  Per chunk, with tril() keeping j <= i:
//   P_c = tril(phi(Q_c) phi(K_c)^T),  A_c = tril(G1_c [V_c, 1]^T)
//   [N, D]_c   = P_c [V_c, 1] + phi(Q_c) S_<c           (the forward, for G1)
//   dphi(Q_c)  = A_c phi(K_c) + G1_c S_<c^T
//   dphi(K_c)  = sum_g A_g,c^T phi(Q_g,c) + [V_c, 1] R_>c^T
//   dV_c       = sum_g P_g,c^T g_g,c + phi(K_c) R_>c,v
// as batched 64 x 64 chunk products, then the same feature and row steps as above.
#include <hip/hip_runtime.h>

#include <math.h>

#include "favor_device.hpp"
#include "favor_gemm.hpp"
#include "favor_ops.hpp"
#include "favor_plan.hpp"

namespace favor {
namespace {

// From ND = phi(Q) S ([rows][D+1], numerators then D_i): G1 = [dout/D, -(dout . out)/D]
// (rows padded; padding rows of G1 all zero).
template <class T, int D>
__global__ void __launch_bounds__(256)
    output_grads(const float* __restrict__ ND, const T* __restrict__ dout, float* __restrict__ G1, long long rows,
                 int L, int Lp) {
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int l = threadIdx.x & 63;
  float* g = G1 + r * (D + 1);
  bool real;
  const long long u = unpadded_row(r, L, Lp, &real);
  if (!real) {
    for (int c = l; c <= D; c += 64) g[c] = 0.f;
    return;
  }
  const float* nd = ND + r * (D + 1);
  const float inv = 1.f / nd[D];
  float dot = 0.f;
  for (int c = l; c < D; c += 64) dot = fmaf((float)dout[u * D + c], nd[c] * inv, dot);
  dot = wave_sum(dot);
  for (int c = l; c < D; c += 64) g[c] = (float)dout[u * D + c] * inv;
  if (l == 0) g[D] = -dot * inv;
}

// dX = P - X * rowsum(T), in the input dtype (rows: the user's; P and the row sums padded).
// The row sums of T = dphi * phi arrive as nt partial sums per row (one per 32 features,
// written by the GEMM that forms T), added here in feature order.
template <class T, int D>
__global__ void __launch_bounds__(256)
    input_grads(const float* __restrict__ P, const T* __restrict__ X, const float* __restrict__ rowp, int nt,
                T* __restrict__ dX, long long rows, int L, int Lp) {
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int l = threadIdx.x & 63;
  const long long p = padded_row(r, L, Lp);
  // lane j < nt holds partial j; the wave sum adds them in a fixed order
  const float t = wave_sum(l < nt ? rowp[p * nt + l] : 0.f);
  for (int c = l; c < D; c += 64) dX[r * D + c] = (T)(P[p * D + c] - (float)X[r * D + c] * t);
}

template <class T, int D>
__global__ void __launch_bounds__(256)
    to_dtype(const float* __restrict__ P, T* __restrict__ dX, long long rows, int L, int Lp) {
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int l = threadIdx.x & 63;
  const long long p = padded_row(r, L, Lp);
  for (int c = l; c < D; c += 64) dX[r * D + c] = (T)P[p * D + c];
}

// ---- chunk scans (causal) --------------------------------------------------------------

// Rx[h][c] = sum over c' > c (from the last chunk down) and over the G query heads g of
// kv head h (in order) of Rc[h G + g][c'].
__global__ void __launch_bounds__(256)
    chunk_suffix(const float* __restrict__ Rc, float* __restrict__ Rx, int NC, int G, int n) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  const size_t h = blockIdx.y;
  float run = 0.f;
  for (int c = NC - 1; c >= 0; --c) {
    Rx[(h * NC + c) * n + e] = run;
    for (int g = 0; g < G; ++g) run += Rc[((h * G + g) * NC + c) * n + e];
  }
}

// ---- workspace -----------------------------------------------------------------------

struct BwdLayout {
  size_t phq, cq, phk, ck, v1, S, ND, G1, dphq, Pq, dS, dphk, tk, Pk, dVf, part, bytes;
  int split_k, split_q;  // contraction splits of S = phi(K)^T [V, 1] and dS = phi(Q)^T G1
};


BwdLayout bwd_layout(const Plan& s) {
  const size_t Rq = (size_t)s.B * s.Hq * s.L, Rk = (size_t)s.B * s.Hkv * s.L;
  const size_t m = s.m, d1 = s.d + 1, f = sizeof(float);
  BwdLayout w;
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off = a256(off + n * f);
    return o;
  };
  w.phq = take(Rq * m);
  w.cq = take(Rq);
  w.phk = take(Rk * m);
  w.ck = take(s.BH);
  w.v1 = take(Rk * d1);
  w.S = take((size_t)s.BH * m * d1);
  w.ND = take(Rq * d1);
  w.G1 = take(Rq * d1);
  w.dphq = take(Rq * m);
  w.Pq = take(Rq * s.d);
  w.dS = take((size_t)s.BH * m * d1);
  w.dphk = take(Rk * m);
  w.tk = take(Rk * (m / 32));
  w.Pk = take(Rk * s.d);
  w.dVf = take(Rk * s.d);
  w.split_k = ksplit_for(s.m, s.d + 1, s.L, s.BH);
  w.split_q = ksplit_for(s.m, s.d + 1, s.G * s.L, s.BH);
  w.part = take((size_t)(w.split_k > w.split_q ? w.split_k : w.split_q) * s.BH * m * d1);
  w.bytes = off;
  return w;
}


#define FAVOR_TRY(x)        \
  if ((rc = (x)) != FAVOR_OK) return rc
#define FAVOR_LAUNCHED() \
  if (hipGetLastError() != hipSuccess) return FAVOR_ERR_HIP

template <class T, int D>
favor_status run_bwd(const Plan& s, const void* Qv, const void* Kv, const void* Vv, const float* W, const void* dOv,
                     void* dQv, void* dKv, void* dVv, char* ws, hipStream_t st) {
  const T* Q = static_cast<const T*>(Qv);
  const T* K = static_cast<const T*>(Kv);
  const T* V = static_cast<const T*>(Vv);
  const T* dO = static_cast<const T*>(dOv);
  const BwdLayout w = bwd_layout(s);
  auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  float *phq = F(w.phq), *phk = F(w.phk), *v1 = F(w.v1), *S = F(w.S), *ND = F(w.ND), *G1 = F(w.G1);
  float *dphq = F(w.dphq), *Pq = F(w.Pq), *dS = F(w.dS), *dphk = F(w.dphk), *tk = F(w.tk);
  float *Pk = F(w.Pk), *dVf = F(w.dVf);
  const long long Rq = (long long)s.B * s.Hq * s.L, Rk = (long long)s.B * s.Hkv * s.L;
  const int m = s.m, D1 = D + 1, GL = s.G * s.L, L = s.L, BH = s.BH;
  // W of batch entry z (= b * Hkv + hkv): head hkv, or the shared one
  const int wmod = s.Hw == 1 ? 1 : s.Hkv;
  const long long wstride = s.Hw == 1 ? 0 : (long long)m * D;
  favor_status rc;
  FAVOR_TRY(launch_features(s, 0, Q, W, phq, F(w.cq), st));
  FAVOR_TRY(launch_features(s, 1, K, W, phk, F(w.ck), st));
  hipLaunchKernelGGL((ones_column<T, D>), dim3(row_blocks(Rk)), dim3(256), 0, st, V, v1, Rk, L, L);
  FAVOR_LAUNCHED();
  // S = phi(K)^T [V, 1]                                    (m x D+1, contraction over L)
  FAVOR_TRY((gemm_split<true, false>(phk, v1, S, F(w.part), m, D1, L, m, D1, (long long)L * m, (long long)L * D1,
                                     kIdent, kIdent, BH, w.split_k, st)));
  // ND = phi(Q) S                                          (G L x D+1)
  FAVOR_TRY((gemm<false, false>(phq, S, ND, GL, D1, m, m, D1, D1, (long long)GL * m, (long long)m * D1,
                                (long long)GL * D1, kIdent, kIdent, BH, st)));
  hipLaunchKernelGGL((output_grads<T, D>), dim3(row_blocks(Rq)), dim3(256), 0, st, ND, dO, G1, Rq, L, L);
  FAVOR_LAUNCHED();
  // T = dphi(Q) * phi(Q) with dphi(Q) = G1 S^T                 (G L x m)
  Epi eq;
  eq.aux = phq;
  FAVOR_TRY((gemm<false, true>(G1, S, dphq, GL, m, D1, D1, D1, m, (long long)GL * D1, (long long)m * D1,
                               (long long)GL * m, kIdent, kIdent, BH, st, kMulAux, eq)));
  // dQ = T W: the term -Q * rowsum(T) vanishes for queries (rowsum(T)_i = g_i . N_i +
  // h_i D_i = 0, since scaling phi(q_i) leaves out_i unchanged), and dropping it avoids
  // subtracting the rounding noise of that cancellation
  FAVOR_TRY((gemm<false, false>(dphq, W, Pq, GL, D, m, m, D, D, (long long)GL * m, wstride, (long long)GL * D,
                                kIdent, modulo(wmod), BH, st)));
  hipLaunchKernelGGL((to_dtype<T, D>), dim3(row_blocks(Rq)), dim3(256), 0, st, Pq, static_cast<T*>(dQv), Rq, L, L);
  FAVOR_LAUNCHED();
  // dS = phi(Q)^T G1                                       (m x D+1, contraction over G L)
  FAVOR_TRY((gemm_split<true, false>(phq, G1, dS, F(w.part), m, D1, GL, m, D1, (long long)GL * m,
                                     (long long)GL * D1, kIdent, kIdent, BH, w.split_q, st)));
  // T' = dphi(K) * phi(K) with dphi(K) = [V, 1] dS^T, and its row sums   (L x m)
  Epi ek;
  ek.aux = phk;
  ek.rowp = tk;
  ek.ldrp = m / 32;
  ek.srp = (long long)L * (m / 32);
  FAVOR_TRY((gemm<false, true>(v1, dS, dphk, L, m, D1, D1, D1, m, (long long)L * D1, (long long)m * D1,
                               (long long)L * m, kIdent, kIdent, BH, st, kMulAux | kRowSum, ek)));
  FAVOR_TRY((gemm<false, false>(dphk, W, Pk, L, D, m, m, D, D, (long long)L * m, wstride, (long long)L * D, kIdent,
                                modulo(wmod), BH, st)));
  hipLaunchKernelGGL((input_grads<T, D>), dim3(row_blocks(Rk)), dim3(256), 0, st, Pk, K, tk, m / 32,
                     static_cast<T*>(dKv), Rk, L, L);
  FAVOR_LAUNCHED();
  // dV = phi(K) dS_v                                       (L x D; dS rows have stride D+1)
  FAVOR_TRY((gemm<false, false>(phk, dS, dVf, L, D, m, m, D1, D, (long long)L * m, (long long)m * D1,
                                (long long)L * D, kIdent, kIdent, BH, st)));
  hipLaunchKernelGGL((to_dtype<T, D>), dim3(row_blocks(Rk)), dim3(256), 0, st, dVf, static_cast<T*>(dVv), Rk, L,
                     L);
  FAVOR_LAUNCHED();
  return FAVOR_OK;
}

// ---- causal ----------------------------------------------------------------------------

constexpr int kBwdChunk = GT;  // one 64 x 64 tile per chunk product

struct CausalLayout {
  size_t phq, cq, phk, ck, v1, Sx, Pm, ND, G1, A, dphq, Pq, Rc, Rx, dphk, tk, Pk, dVf, bytes;
  int NC, Lp;  // chunks per head, padded positions per head
};

CausalLayout causal_layout(const Plan& s) {
  CausalLayout w;
  w.NC = (s.L + kBwdChunk - 1) / kBwdChunk;
  w.Lp = w.NC * kBwdChunk;
  const size_t Rq = (size_t)s.B * s.Hq * w.Lp, Rk = (size_t)s.B * s.Hkv * w.Lp;
  const size_t m = s.m, d1 = s.d + 1, C = kBwdChunk, f = sizeof(float);
  const size_t Zq = (size_t)s.B * s.Hq * w.NC, Zk = (size_t)s.BH * w.NC;
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off = a256(off + n * f);
    return o;
  };
  w.phq = take(Rq * m);
  w.cq = take(Rq);
  w.phk = take(Rk * m);
  w.ck = take(s.BH);
  w.v1 = take(Rk * d1);
  w.Sx = take(Zk * m * d1);
  w.Pm = take(Rq * C);
  w.ND = take(Rq * d1);
  w.G1 = take(Rq * d1);
  w.A = take(Rq * C);
  w.dphq = take(Rq * m);
  w.Pq = take(Rq * s.d);
  w.Rc = take(Zq * m * d1);
  w.Rx = take(Zk * m * d1);
  w.dphk = take(Rk * m);
  w.tk = take(Rk * (m / 32));
  w.Pk = take(Rk * s.d);
  w.dVf = take(Rk * s.d);
  w.bytes = off;
  return w;
}

template <class T, int D>
favor_status run_bwd_causal(const Plan& s, const void* Qv, const void* Kv, const void* Vv, const float* W,
                            const void* dOv, void* dQv, void* dKv, void* dVv, char* ws, hipStream_t st) {
  const T* K = static_cast<const T*>(Kv);
  const CausalLayout w = causal_layout(s);
  auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  float *phq = F(w.phq), *phk = F(w.phk), *v1 = F(w.v1), *Sx = F(w.Sx), *Pm = F(w.Pm), *ND = F(w.ND);
  float *G1 = F(w.G1), *A = F(w.A), *dphq = F(w.dphq), *Pq = F(w.Pq), *Rc = F(w.Rc);
  float *Rx = F(w.Rx), *dphk = F(w.dphk), *tk = F(w.tk), *Pk = F(w.Pk), *dVf = F(w.dVf);
  const int C = kBwdChunk, NC = w.NC, Lp = w.Lp, L = s.L, m = s.m, D1 = D + 1, G = s.G;
  const int BHk = s.BH, BHq = s.B * s.Hq, Zq = BHq * NC, Zk = BHk * NC;
  const long long Rqp = (long long)BHq * Lp, Rkp = (long long)BHk * Lp;
  const long long Rq = (long long)BHq * L, Rk = (long long)BHk * L;
  const long long cm = (long long)C * m, cd1 = (long long)C * D1, cc = (long long)C * C, sm = (long long)m * D1;
  const long long cd = (long long)C * D;
  // query chunk z = (b Hq + hq) NC + c reads key chunk (b Hkv + hq / G) NC + c; key chunk
  // z = bhk NC + c reads query chunk (bhk G + g) NC + c of group member g (base offset g NC)
  const BMap key_of_q{G * NC, 0x7fffffff, NC, NC};
  const BMap q_of_k{NC, 0x7fffffff, G * NC, NC};
  const long long wstride = s.Hw == 1 ? 0 : (long long)m * D;
  const BMap w_of_q{G, s.Hkv, 1, 1}, w_of_k = modulo(s.Hkv);
  const dim3 scan_grid((unsigned)((sm + 255) / 256), (unsigned)BHk);
  favor_status rc;

  FAVOR_TRY(launch_features(s, 0, Qv, W, phq, F(w.cq), st, Lp));
  FAVOR_TRY(launch_features(s, 1, Kv, W, phk, F(w.ck), st, Lp));
  hipLaunchKernelGGL((ones_column<T, D>), dim3(row_blocks(Rkp)), dim3(256), 0, st, static_cast<const T*>(Vv), v1,
                     Rkp, L, Lp);
  FAVOR_LAUNCHED();
  // S_c = phi(K_c)^T [V_c, 1] per chunk, then exclusive prefixes S_<c in place
  FAVOR_TRY((gemm<true, false>(phk, v1, Sx, m, D1, C, m, D1, D1, cm, cd1, sm, kIdent, kIdent, Zk, st)));
  hipLaunchKernelGGL(chunk_prefix, scan_grid, dim3(256), 0, st, Sx, NC, (int)sm);
  FAVOR_LAUNCHED();
  // P = tril(phi(Q_c) phi(K_c)^T);  [N, D] = P [V_c, 1] + phi(Q_c) S_<c
  FAVOR_TRY((gemm<false, true>(phq, phk, Pm, C, C, m, m, m, C, cm, cm, cc, kIdent, key_of_q, Zq, st, kTril)));
  FAVOR_TRY((gemm<false, false>(Pm, v1, ND, C, D1, C, C, D1, D1, cc, cd1, cd1, kIdent, key_of_q, Zq, st)));
  FAVOR_TRY((gemm<false, false>(phq, Sx, ND, C, D1, m, m, D1, D1, cm, sm, cd1, kIdent, key_of_q, Zq, st, kAccum)));
  hipLaunchKernelGGL((output_grads<T, D>), dim3(row_blocks(Rqp)), dim3(256), 0, st, ND, static_cast<const T*>(dOv),
                     G1, Rqp, L, Lp);
  FAVOR_LAUNCHED();
  // A = tril(G1_c [V_c, 1]^T);  T = dphi(Q_c) * phi(Q_c), dphi(Q_c) = A phi(K_c) + G1_c S_<c^T
  Epi eq;
  eq.aux = phq;
  FAVOR_TRY((gemm<false, true>(G1, v1, A, C, C, D1, D1, D1, C, cd1, cd1, cc, kIdent, key_of_q, Zq, st, kTril)));
  FAVOR_TRY((gemm<false, false>(A, phk, dphq, C, m, C, C, m, m, cc, cm, cm, kIdent, key_of_q, Zq, st)));
  FAVOR_TRY((gemm<false, true>(G1, Sx, dphq, C, m, D1, D1, D1, m, cd1, sm, cm, kIdent, key_of_q, Zq, st,
                               kAccum | kMulAux, eq)));
  // dQ = T W (the row-sum term is 0 for queries, as in the bidirectional case)
  FAVOR_TRY((gemm<false, false>(dphq, W, Pq, Lp, D, m, m, D, D, (long long)Lp * m, wstride, (long long)Lp * D,
                                kIdent, w_of_q, BHq, st)));
  hipLaunchKernelGGL((to_dtype<T, D>), dim3(row_blocks(Rq)), dim3(256), 0, st, Pq, static_cast<T*>(dQv), Rq, L, Lp);
  FAVOR_LAUNCHED();
  // R_c = phi(Q_c)^T G1_c per query chunk; R_>c summed over later chunks and the G heads
  FAVOR_TRY((gemm<true, false>(phq, G1, Rc, m, D1, C, m, D1, D1, cm, cd1, sm, kIdent, kIdent, Zq, st)));
  hipLaunchKernelGGL(chunk_suffix, scan_grid, dim3(256), 0, st, Rc, Rx, NC, G, (int)sm);
  FAVOR_LAUNCHED();
  // T' = dphi(K_c) * phi(K_c) and its row sums, dphi(K_c) = [V_c, 1] R_>c^T + sum_g A_g,c^T phi(Q_g,c)
  Epi ek;
  ek.aux = phk;
  ek.rowp = tk;
  ek.ldrp = m / 32;
  ek.srp = (long long)C * (m / 32);
  FAVOR_TRY((gemm<false, true>(v1, Rx, dphk, C, m, D1, D1, D1, m, cd1, sm, cm, kIdent, kIdent, Zk, st)));
  for (int g = 0; g < G; ++g)
    FAVOR_TRY((gemm<true, false>(A + g * NC * cc, phq + g * NC * cm, dphk, C, m, C, C, m, m, cc, cm, cm, q_of_k,
                                 q_of_k, Zk, st, g == G - 1 ? kAccum | kMulAux | kRowSum : kAccum, ek)));
  FAVOR_TRY((gemm<false, false>(dphk, W, Pk, Lp, D, m, m, D, D, (long long)Lp * m, wstride, (long long)Lp * D,
                                kIdent, w_of_k, BHk, st)));
  hipLaunchKernelGGL((input_grads<T, D>), dim3(row_blocks(Rk)), dim3(256), 0, st, Pk, K, tk, m / 32,
                     static_cast<T*>(dKv), Rk, L, Lp);
  FAVOR_LAUNCHED();
  // dV_c = phi(K_c) R_>c,v + sum_g P_g,c^T g_g,c          (R and G1 rows have stride D+1)
  FAVOR_TRY((gemm<false, false>(phk, Rx, dVf, C, D, m, m, D1, D, cm, sm, cd, kIdent, kIdent, Zk, st)));
  for (int g = 0; g < G; ++g)
    FAVOR_TRY((gemm<true, false>(Pm + g * NC * cc, G1 + g * NC * cd1, dVf, C, D, C, C, D1, D, cc, cd1, cd, q_of_k,
                                 q_of_k, Zk, st, kAccum)));
  hipLaunchKernelGGL((to_dtype<T, D>), dim3(row_blocks(Rk)), dim3(256), 0, st, dVf, static_cast<T*>(dVv), Rk, L,
                     Lp);
  FAVOR_LAUNCHED();
  return FAVOR_OK;
}
#undef FAVOR_TRY
#undef FAVOR_LAUNCHED

size_t bwd_bytes(const Plan& s) {
  return s.mode == FAVOR_CAUSAL ? causal_layout(s).bytes : bwd_layout(s).bytes;
}

// Validation as for the forward; the causal backward uses its own chunk of 64 whatever the
// problem's chunk field asks of the forward.
favor_status bwd_plan(const favor_problem* p, Plan* s) { return make_plan(p, s); }

}  // namespace
}  // namespace favor

extern "C" size_t favor_bwd_workspace_bytes(const favor_problem* p) {
  favor::Plan s;
  if (p == nullptr || favor::bwd_plan(p, &s) != FAVOR_OK) return 0;
  return favor::bwd_bytes(s);
}

extern "C" favor_status favor_attn_bwd(const favor_problem* p, const void* Q, const void* K, const void* V,
                                       const float* W, const void* dout, void* dQ, void* dK, void* dV,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  favor::Plan s;
  if (p == nullptr) return FAVOR_ERR_INVALID_ARG;
  const favor_status st = favor::bwd_plan(p, &s);
  if (st != FAVOR_OK) return st;
  if (Q == nullptr || K == nullptr || V == nullptr || W == nullptr || dout == nullptr || dQ == nullptr ||
      dK == nullptr || dV == nullptr)
    return FAVOR_ERR_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < favor::bwd_bytes(s) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return FAVOR_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (s.mode == FAVOR_CAUSAL) {
    if (s.dtype == FAVOR_BF16)
      return s.d == 64 ? favor::run_bwd_causal<favor::bf16, 64>(s, Q, K, V, W, dout, dQ, dK, dV, ws, hs)
                       : favor::run_bwd_causal<favor::bf16, 128>(s, Q, K, V, W, dout, dQ, dK, dV, ws, hs);
    return s.d == 64 ? favor::run_bwd_causal<float, 64>(s, Q, K, V, W, dout, dQ, dK, dV, ws, hs)
                     : favor::run_bwd_causal<float, 128>(s, Q, K, V, W, dout, dQ, dK, dV, ws, hs);
  }
  if (s.dtype == FAVOR_BF16)
    return s.d == 64 ? favor::run_bwd<favor::bf16, 64>(s, Q, K, V, W, dout, dQ, dK, dV, ws, hs)
                     : favor::run_bwd<favor::bf16, 128>(s, Q, K, V, W, dout, dQ, dK, dV, ws, hs);
  return s.d == 64 ? favor::run_bwd<float, 64>(s, Q, K, V, W, dout, dQ, dK, dV, ws, hs)
                   : favor::run_bwd<float, 128>(s, Q, K, V, W, dout, dQ, dK, dV, ws, hs);
}
