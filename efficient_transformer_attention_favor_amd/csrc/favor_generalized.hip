// Kernelised attention with a feature map other than softmax's (the favor_attn_fwd_generalized
// entry point).
//
// "Rethinking Attention with Performers" (review page), section "ABSTRACT": FAVOR+ can also
// model kernelisable attention mechanisms beyond softmax.  The same linear-order evaluation
// D^-1 A V, A = phi(Q) phi(K)^T ("KDEformer" review page, "提出的方法" for D^-1 A V), holds
// for any non-negative feature map; here phi(x) = ReLU(W x) / sqrt(m) (FAVOR_FEATURE_RELU),
// whose kernel is the first-order arc-cosine kernel.  Without an exponential there is no
// stabiliser, and a row whose weights are all zero (every feature of its query, or of its
// keys, zero) gets a zero output.
//
// Implementation.  Bidirectional: the softmax forward's generic key-side and readout
// kernels with ReLU in place of the exponential -- the features stay on chip, S =
// phi(K)^T [V, 1] per position range by MFMA (bf16 problems: fp16 W contraction, bf16
// features and products, float32 accumulation), then out = phi(Q) S_v / phi(Q) S_1.
// Causal: the feature matrices are materialised in float32 (the features kernel in its
// ReLU mode), then float32 batched products over 64-position chunks, S_<c the exclusive
// prefix of the chunk summaries, [N, D]_c = tril(phi(Q_c) phi(K_c)^T) [V_c, 1] +
// phi(Q_c) S_<c, and a row kernel writes out = N / D in the problem's dtype.
#include <hip/hip_runtime.h>

#include "favor_device.hpp"
#include "favor_gemm.hpp"
#include "favor_ops.hpp"
#include "favor_plan.hpp"

namespace favor {
namespace {

constexpr int kGenChunk = GT;

struct GenLayout {
  size_t phq, phk, v1, S, Pm, ND, bytes;
  int Lp, NC;
};

GenLayout gen_layout(const Plan& s) {
  GenLayout w{};
  if (s.mode != FAVOR_CAUSAL) {  // bidirectional: the plan's range summaries gs and gc
    w.bytes = s.off_p;
    return w;
  }
  w.NC = (s.L + kGenChunk - 1) / kGenChunk;
  w.Lp = w.NC * kGenChunk;
  const size_t Rq = (size_t)s.B * s.Hq * w.Lp, Rk = (size_t)s.B * s.Hkv * w.Lp;
  const size_t m = s.m, d1 = s.d + 1, f = sizeof(float);
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off = a256(off + n * f);
    return o;
  };
  w.phq = take(Rq * m);
  w.phk = take(Rk * m);
  w.v1 = take(Rk * d1);
  w.S = take((size_t)s.BH * w.NC * m * d1);
  w.Pm = take(Rq * kGenChunk);
  w.ND = take(Rq * d1);
  w.bytes = off;
  return w;
}

// out = N / D (0 where D = 0), rows: the user's; ND padded.
template <class T, int D>
__global__ void __launch_bounds__(256)
    ratio_out(const float* __restrict__ ND, T* __restrict__ out, long long rows, int L, int Lp) {
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int l = threadIdx.x & 63;
  const float* nd = ND + padded_row(r, L, Lp) * (D + 1);
  const float den = nd[D];
  const float inv = den > 0.f ? 1.f / den : 0.f;
  for (int c = l; c < D; c += 64) out[r * D + c] = (T)(nd[c] * inv);
}

#define FAVOR_TRY(x)        \
  if ((rc = (x)) != FAVOR_OK) return rc
#define FAVOR_LAUNCHED() \
  if (hipGetLastError() != hipSuccess) return FAVOR_ERR_HIP

template <class T, int D>
favor_status run_generalized(const Plan& s, const void* Q, const void* K, const void* V, const float* W, void* out,
                             char* ws, hipStream_t st) {
  if (s.mode != FAVOR_CAUSAL) return launch_relu_bidirectional(s, Q, K, V, W, out, ws, st);
  const GenLayout w = gen_layout(s);
  auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  float *phq = F(w.phq), *phk = F(w.phk), *v1 = F(w.v1), *S = F(w.S), *ND = F(w.ND), *Pm = F(w.Pm);
  const int L = s.L, Lp = w.Lp, NC = w.NC, m = s.m, D1 = D + 1, G = s.G, BH = s.BH;
  const long long Rq = (long long)s.B * s.Hq * L, Rkp = (long long)BH * Lp;
  const long long sm = (long long)m * D1;
  favor_status rc;
  FAVOR_TRY(launch_relu_features(s, 0, Q, W, phq, st, Lp));
  FAVOR_TRY(launch_relu_features(s, 1, K, W, phk, st, Lp));
  hipLaunchKernelGGL((ones_column<T, D>), dim3(row_blocks(Rkp)), dim3(256), 0, st, static_cast<const T*>(V), v1,
                     Rkp, L, Lp);
  FAVOR_LAUNCHED();
  const int C = kGenChunk, Zq = s.B * s.Hq * NC, Zk = BH * NC;
  const long long cm = (long long)C * m, cd1 = (long long)C * D1, cc = (long long)C * C;
  const BMap key_of_q{G * NC, 0x7fffffff, NC, NC};
  FAVOR_TRY((gemm<true, false>(phk, v1, S, m, D1, C, m, D1, D1, cm, cd1, sm, kIdent, kIdent, Zk, st)));
  hipLaunchKernelGGL(chunk_prefix, dim3((unsigned)((sm + 255) / 256), (unsigned)BH), dim3(256), 0, st, S, NC,
                     (int)sm);
  FAVOR_LAUNCHED();
  FAVOR_TRY((gemm<false, true>(phq, phk, Pm, C, C, m, m, m, C, cm, cm, cc, kIdent, key_of_q, Zq, st, kTril)));
  FAVOR_TRY((gemm<false, false>(Pm, v1, ND, C, D1, C, C, D1, D1, cc, cd1, cd1, kIdent, key_of_q, Zq, st)));
  FAVOR_TRY((gemm<false, false>(phq, S, ND, C, D1, m, m, D1, D1, cm, sm, cd1, kIdent, key_of_q, Zq, st, kAccum)));
  hipLaunchKernelGGL((ratio_out<T, D>), dim3(row_blocks(Rq)), dim3(256), 0, st, ND, static_cast<T*>(out), Rq, L,
                     Lp);
  FAVOR_LAUNCHED();
  return FAVOR_OK;
}
#undef FAVOR_TRY
#undef FAVOR_LAUNCHED

favor_status gen_plan(const favor_problem* p, int32_t fn, Plan* s) {
  if (p == nullptr) return FAVOR_ERR_INVALID_ARG;
  const favor_status st = make_plan(p, s);
  if (st != FAVOR_OK) return st;
  return fn == FAVOR_FEATURE_RELU ? FAVOR_OK : FAVOR_ERR_UNSUPPORTED;
}

}  // namespace
}  // namespace favor

extern "C" size_t favor_generalized_workspace_bytes(const favor_problem* p, int32_t fn) {
  favor::Plan s;
  if (favor::gen_plan(p, fn, &s) != FAVOR_OK) return 0;
  return favor::gen_layout(s).bytes;
}

extern "C" favor_status favor_attn_fwd_generalized(const favor_problem* p, int32_t fn, const void* Q, const void* K,
                                                   const void* V, const float* W, void* out, void* workspace,
                                                   size_t workspace_bytes, void* stream) {
  favor::Plan s;
  const favor_status st = favor::gen_plan(p, fn, &s);
  if (st != FAVOR_OK) return st;
  if (Q == nullptr || K == nullptr || V == nullptr || W == nullptr || out == nullptr) return FAVOR_ERR_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < favor::gen_layout(s).bytes ||
      (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return FAVOR_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (s.dtype == FAVOR_BF16)
    return s.d == 64 ? favor::run_generalized<favor::bf16, 64>(s, Q, K, V, W, out, ws, hs)
                     : favor::run_generalized<favor::bf16, 128>(s, Q, K, V, W, out, ws, hs);
  return s.d == 64 ? favor::run_generalized<float, 64>(s, Q, K, V, W, out, ws, hs)
                   : favor::run_generalized<float, 128>(s, Q, K, V, W, out, ws, hs);
}
