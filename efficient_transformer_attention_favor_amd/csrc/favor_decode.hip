// Causal decoding, one position per call (the favor_attn_decode entry point).
//
// "Rethinking Attention with Performers" (review page), section "제안 방법": attention in
// linear order through positive random features, phi(x) = exp(W x - |x|^2/2 - c)/sqrt(m).
// With the inclusive causal mask the summary of the positions seen so far,
// S = sum_j phi(k_j) [v_j, 1]^T, is all a new query needs; "Fast Transformer Decoding: One
// Write-Head is All You Need" (review page), "ABSTRACT": incremental decoding is bound by
// reloading the key/value history, which this m x (d+1) summary per kv head replaces.
//
// The state keeps one stabiliser per slice of m / kDecSplit features (any constant per
// feature cancels once it is folded into the query exponent, as in the forward readout), so
// the slices never need each other.  Two small kernels per step:
//   decode_update   kDecSplit workgroups per (batch, kv head), workgroup s owning features
//                   [s m/8, (s+1) m/8) and their rows of S: the new key's exponents
//                   e_f = log2e (w_f.k - |k|^2/2), c_s' = max(c_s, max over its f of e_f),
//                   S_f <- 2^(c_s - c_s') S_f + 2^(e_f - c_s') [v, 1]   (float32, VALU).
//   decode_readout  one workgroup per (batch, query head): p_f = 2^(log2e w_f.q + c_s(f) - M),
//                   M the row maximum, out = sum_f p_f S_v,f / sum_f p_f S_1,f.
// Both are latency-bound (a few hundred KB of state per call); the arithmetic is float32 on
// the VALU, so bf16 problems round only their inputs and outputs.
//
// A prompt enters the state in one call (favor_decode_prefill): the key side of the forward
// pass summarises the prompt's positions over ranges (float32 partials with per-feature
// stabilisers c_tf), then prefill_state merges them into the state format:
//   c_s = max of c_tf over t and the features f of slice s,
//   S[f][col] = sum_t 2^(c_tf - c_s(f)) partial_t[col][f],  n = L.
#include <hip/hip_runtime.h>

#include <math.h>

#include "favor_device.hpp"
#include "favor_ops.hpp"
#include "favor_plan.hpp"

namespace favor {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecSplit = 8;  // summary slices per (batch, kv head), one workgroup each

template <class T> __device__ __forceinline__ float to_f(T x) { return (float)x; }

// Block-wide maximum / sum over kDecThreads threads: within each wave by shuffles, then
// across the waves through LDS (red: at least kDecThreads / 64 floats).
__device__ __forceinline__ float block_max(float x, float* red) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x = fmaxf(x, __shfl_xor(x, s));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kDecThreads / 64; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}
__device__ __forceinline__ float block_sum(float x, float* red) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x += __shfl_xor(x, s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kDecThreads / 64; ++w) r += red[w];
  __syncthreads();
  return r;
}

// w_f . x (log2e applied by the caller); x in LDS as float.
template <int D>
__device__ __forceinline__ float row_dot(const float* __restrict__ wrow, const float* x) {
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < D; i += 4) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(wrow + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = fmaf(w[j], x[i + j], acc[j]);
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

template <class T, int D>
__global__ void __launch_bounds__(kDecThreads)
    decode_update(const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ W, int Hkv, int Hw,
                  int m, float* __restrict__ S, float* __restrict__ cst, unsigned* __restrict__ count) {
  static_assert(512 / kDecSplit <= 64, "a slice's features must fit one wave");
  __shared__ float kl[D], vl[D + 1], phi[512 / kDecSplit], sc;
  const int bh = blockIdx.x / kDecSplit, part = blockIdx.x % kDecSplit, hkv = bh % Hkv;
  const int mf = m / kDecSplit, fb = part * mf;  // this workgroup's features (at most 64)
  const float* Wh = W + (size_t)(Hw == 1 ? 0 : hkv) * m * D;
  const int t = threadIdx.x;
  // wave 0 owns the features, one per lane: its W row and the slice's stabiliser are
  // loaded before the key arrives
  const bool feat = t < mf;
  f32x4 wr[D / 4];
  if (feat) {
#pragma unroll
    for (int i = 0; i < D / 4; ++i) wr[i] = *reinterpret_cast<const f32x4*>(Wh + (size_t)(fb + t) * D + 4 * i);
  }
  const unsigned seen = count[bh * kDecSplit + part];
  const float c_prev = cst[bh * kDecSplit + part];
  if (t < D) {
    kl[t] = to_f(k[(size_t)bh * D + t]);
    vl[t] = to_f(v[(size_t)bh * D + t]);
  }
  if (t == 0) vl[D] = 1.f;  // the ones column carries the normaliser
  __syncthreads();
  if (t < 64) {  // wave 0: norm, exponents, maximum and stabiliser by shuffles
    float nrm = 0.f;
    for (int i = t; i < D; i += 64) nrm = fmaf(kl[i], kl[i], nrm);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) nrm += __shfl_xor(nrm, o);
    float e = -INFINITY;
    if (feat) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < D / 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = fmaf(wr[i][j], kl[4 * i + j], acc[j]);
      e = kLog2e * (((acc[0] + acc[1]) + (acc[2] + acc[3])) - 0.5f * nrm);
    }
    float mx = e;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    // an empty state (no position yet) takes the new key's maximum as its constant; after
    // that c only grows, so S never overflows and never has to be scaled up
    const float c_old = seen ? c_prev : mx;
    const float c_new = fmaxf(c_old, mx);
    if (feat) phi[t] = fast_exp2(e - c_new);
    if (t == 0) {
      sc = fast_exp2(c_old - c_new);
      cst[bh * kDecSplit + part] = c_new;
      count[bh * kDecSplit + part] = seen + 1u;
    }
  }
  __syncthreads();
  const float scale = sc;

  // this workgroup's rows of S [m][D+1] (mf (D+1) floats, a multiple of 4): 4 consecutive
  // elements per thread and step, two steps' loads in flight
  const int n = mf * (D + 1);
  float* Sh = S + (size_t)bh * m * (D + 1) + (size_t)part * n;
  auto upd = [&](int i, f32x4 x) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = i + u, f = e / (D + 1), j = e - f * (D + 1);
      x[u] = fmaf(x[u], scale, phi[f] * vl[j]);
    }
    *reinterpret_cast<f32x4*>(Sh + i) = x;
  };
  int i = 4 * t;
  for (; i + 4 * kDecThreads < n; i += 8 * kDecThreads) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(Sh + i);
    const f32x4 b = *reinterpret_cast<const f32x4*>(Sh + i + 4 * kDecThreads);
    upd(i, a);
    upd(i + 4 * kDecThreads, b);
  }
  if (i < n) upd(i, *reinterpret_cast<const f32x4*>(Sh + i));
}

template <class T, int D>
__global__ void __launch_bounds__(kDecThreads)
    decode_readout(const T* __restrict__ q, const float* __restrict__ W, const float* __restrict__ S,
                   const float* __restrict__ cst, int Hq, int Hkv, int Hw, int m, T* __restrict__ out) {
  constexpr int FG = kDecThreads / D;  // feature groups (threads per value column)
  __shared__ float ql[D], p[512], red[kDecThreads], part[FG][D];
  const int bhq = blockIdx.x, b = bhq / Hq, hq = bhq % Hq, hkv = hq / (Hq / Hkv);
  const int bh = b * Hkv + hkv;
  const float* Wh = W + (size_t)(Hw == 1 ? 0 : hkv) * m * D;
  const float* Sh = S + (size_t)bh * m * (D + 1);
  const int t = threadIdx.x;
  if (t < D) ql[t] = to_f(q[(size_t)bhq * D + t]);
  __syncthreads();

  float mx = -INFINITY;
  const int mf = m / kDecSplit;
  for (int f = t; f < m; f += kDecThreads) {
    // the slice's stabiliser joins the query exponent
    const float e = kLog2e * row_dot<D>(Wh + (size_t)f * D, ql) + cst[bh * kDecSplit + f / mf];
    p[f] = e;
    mx = fmaxf(mx, e);
  }
  mx = block_max(mx, red);  // the row stabiliser (cancels in the ratio)
  float den = 0.f;
  for (int f = t; f < m; f += kDecThreads) {
    p[f] = fast_exp2(p[f] - mx);
    den = fmaf(p[f], Sh[(size_t)f * (D + 1) + D], den);
  }
  den = block_sum(den, red);  // also orders the p[] writes before the reads below

  // thread (fg, j): features fg, fg + FG, ... of value column j
  const int j = t % D, fg = t / D;
  // m / FG is a multiple of 16: 16 independent loads in flight per step
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int f = fg; f < m; f += 16 * FG) {
    float sv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) sv[u] = Sh[(size_t)(f + u * FG) * (D + 1) + j];
#pragma unroll
    for (int u = 0; u < 16; ++u) acc[u & 3] = fmaf(p[f + u * FG], sv[u], acc[u & 3]);
  }
  part[fg][j] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (t < D) {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < FG; ++g) s += part[g][t];
    out[(size_t)bhq * D + t] = (T)(s / den);
  }
}

// d = 128: wave w takes features [w m/NW, (w+1) m/NW) for every value column (two per
// lane), relative to its own maximum; the NW partials are merged by their maxima after one
// barrier.  (For d = 64 the kernel above, which splits value columns over threads, is faster.)
template <class T, int D>
__global__ void __launch_bounds__(kDecThreads)
    decode_readout_waves(const T* __restrict__ q, const float* __restrict__ W, const float* __restrict__ S,
                         const float* __restrict__ cst, int Hq, int Hkv, int Hw, int m, T* __restrict__ out) {
  constexpr int NW = kDecThreads / 64, CPL = D / 64;  // waves; value columns per lane
  __shared__ float ql[D], p[512], part[NW][D + 2];
  const int bhq = blockIdx.x, b = bhq / Hq, hq = bhq % Hq, hkv = hq / (Hq / Hkv);
  const int bh = b * Hkv + hkv;
  const float* Wh = W + (size_t)(Hw == 1 ? 0 : hkv) * m * D;
  const float* Sh = S + (size_t)bh * m * (D + 1);
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  if (t < D) ql[t] = to_f(q[(size_t)bhq * D + t]);
  __syncthreads();

  const int fpw = m / NW, f0 = w * fpw, mf = m / kDecSplit;  // fpw <= 128: two per lane
  float e[2], Mw = -INFINITY;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int f = f0 + lane + 64 * h;
    e[h] = -INFINITY;
    if (lane + 64 * h < fpw) {
      // the slice's stabiliser joins the query exponent
      e[h] = kLog2e * row_dot<D>(Wh + (size_t)f * D, ql) + cst[bh * kDecSplit + f / mf];
      Mw = fmaxf(Mw, e[h]);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) Mw = fmaxf(Mw, __shfl_xor(Mw, o));
  float den = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (lane + 64 * h < fpw) {
      const int f = f0 + lane + 64 * h;
      const float pf = fast_exp2(e[h] - Mw);
      p[f] = pf;
      den = fmaf(pf, Sh[(size_t)f * (D + 1) + D], den);
    }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's p[] writes have landed
  __builtin_amdgcn_wave_barrier();

  // numerator columns lane + 64 c over the wave's features: rows of S read whole, 16 in flight
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  for (int f = f0; f < f0 + fpw; f += 16) {  // fpw is a multiple of 16
    float sv[16][CPL];
#pragma unroll
    for (int u = 0; u < 16; ++u)
#pragma unroll
      for (int c = 0; c < CPL; ++c) sv[u][c] = Sh[(size_t)(f + u) * (D + 1) + lane + 64 * c];
#pragma unroll
    for (int u = 0; u < 16; ++u)
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = fmaf(p[f + u], sv[u][c], acc[c]);
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) part[w][lane + 64 * c] = acc[c];
  if (lane == 0) {
    part[w][D] = den;
    part[w][D + 1] = Mw;
  }
  __syncthreads();
  if (t < D) {
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, part[v][D + 1]);
    float num = 0.f, dsum = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float sc = fast_exp2(part[v][D + 1] - M);
      num = fmaf(sc, part[v][t], num);
      dsum = fmaf(sc, part[v][D], dsum);
    }
    out[(size_t)bhq * D + t] = (T)(num / dsum);
  }
}

template <class T, int D>
favor_status run_decode(const Plan& s, const void* q, const void* k, const void* v, const float* W, float* state,
                        void* out, hipStream_t st) {
  float* S = state;
  float* cst = state + (size_t)s.BH * s.m * (s.d + 1);
  unsigned* count = reinterpret_cast<unsigned*>(cst + (size_t)s.BH * kDecSplit);
  hipLaunchKernelGGL((decode_update<T, D>), dim3(s.BH * kDecSplit), dim3(kDecThreads), 0, st, static_cast<const T*>(k),
                     static_cast<const T*>(v), W, s.Hkv, s.Hw, s.m, S, cst, count);
  if (hipGetLastError() != hipSuccess) return FAVOR_ERR_HIP;
  if constexpr (D == 128)
    hipLaunchKernelGGL((decode_readout_waves<T, D>), dim3(s.B * s.Hq), dim3(kDecThreads), 0, st,
                       static_cast<const T*>(q), W, S, cst, s.Hq, s.Hkv, s.Hw, s.m, static_cast<T*>(out));
  else
    hipLaunchKernelGGL((decode_readout<T, D>), dim3(s.B * s.Hq), dim3(kDecThreads), 0, st,
                       static_cast<const T*>(q), W, S, cst, s.Hq, s.Hkv, s.Hw, s.m, static_cast<T*>(out));
  return hipGetLastError() == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}

// One workgroup per (batch, kv head, slice of m/8 features): the merged state rows of its
// T range partials.
__global__ void __launch_bounds__(kDecThreads)
    prefill_state(const float* __restrict__ gs, const float* __restrict__ gc, int T, int d, int m, int L,
                  float* __restrict__ S, float* __restrict__ cst, unsigned* __restrict__ count) {
  // one workgroup per (batch, kv head, slice): the slice's mf <= 64 features, one per lane of
  // the first wave for the maxima
  __shared__ float scale[512 / kDecSplit], cs;
  const int bh = blockIdx.x / kDecSplit, sl = blockIdx.x % kDecSplit, t0 = threadIdx.x;
  const int mf = m / kDecSplit, fb = sl * mf;
  const float* gch = gc + (size_t)bh * T * m;
  if (t0 < 64) {
    float c = -INFINITY;
    if (t0 < mf)
      for (int t = 0; t < T; ++t) c = fmaxf(c, gch[(size_t)t * m + fb + t0]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) c = fmaxf(c, __shfl_xor(c, o));
    if (t0 == 0) cs = c;
  }
  __syncthreads();
  const float c_s = cs;
  const int d1 = d + 1;
  const float* gsh = gs + (size_t)bh * T * d1 * m;
  float* Sh = S + (size_t)bh * m * d1;
  for (int t = 0; t < T; ++t) {
    if (t0 < mf) scale[t0] = fast_exp2(gch[(size_t)t * m + fb + t0] - c_s);
    __syncthreads();
    // element (f, col) of the slice's state rows, f fastest (reads of the partial are contiguous)
    for (int e = t0; e < mf * d1; e += kDecThreads) {
      const int col = e / mf, fl = e - col * mf, f = fb + fl;
      const int row = col == d ? d : 32 * (col >> 5) + vperm_inv(col & 31);
      const float v = scale[fl] * gsh[((size_t)t * d1 + row) * m + f];
      float* dst = Sh + (size_t)f * d1 + col;
      *dst = t == 0 ? v : *dst + v;
    }
    __syncthreads();
  }
  if (t0 == 0) {
    cst[bh * kDecSplit + sl] = c_s;
    count[bh * kDecSplit + sl] = (unsigned)L;
  }
}

favor_status decode_plan(const favor_problem* p, Plan* s) {
  if (p == nullptr) return FAVOR_ERR_INVALID_ARG;
  favor_problem one = *p;
  one.chunk = 0;  // no segments in decoding
  const favor_status st = make_plan(&one, s);
  if (st != FAVOR_OK) return st;
  if (p->mode != FAVOR_CAUSAL || p->seq_len != 1) return FAVOR_ERR_INVALID_ARG;
  return FAVOR_OK;
}

// The prompt's problem as a bidirectional key-side pass over its L positions (the chunk
// field is validated as for the forward and otherwise ignored).
favor_status prefill_plan(const favor_problem* p, Plan* s) {
  if (p == nullptr) return FAVOR_ERR_INVALID_ARG;
  const favor_status st = make_plan(p, s);  // validation of the problem as given
  if (st != FAVOR_OK) return st;
  if (p->mode != FAVOR_CAUSAL) return FAVOR_ERR_INVALID_ARG;
  favor_problem q = *p;
  q.mode = FAVOR_BIDIRECTIONAL;
  q.chunk = 0;
  return make_plan(&q, s);
}

}  // namespace
}  // namespace favor

extern "C" size_t favor_decode_prefill_workspace_bytes(const favor_problem* p) {
  favor::Plan s;
  if (favor::prefill_plan(p, &s) != FAVOR_OK) return 0;
  return s.off_p;  // the range partials gs and their stabilisers gc
}

extern "C" favor_status favor_decode_prefill(const favor_problem* p, const void* K, const void* V, const float* W,
                                             float* state, void* workspace, size_t workspace_bytes, void* stream) {
  favor::Plan s;
  const favor_status st = favor::prefill_plan(p, &s);
  if (st != FAVOR_OK) return st;
  if (K == nullptr || V == nullptr || W == nullptr || state == nullptr) return FAVOR_ERR_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < s.off_p || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return FAVOR_ERR_WORKSPACE;
  if (s.m > 512) return FAVOR_ERR_UNSUPPORTED;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* gs = reinterpret_cast<float*>(ws + s.off_gs);
  float* gc = reinterpret_cast<float*>(ws + s.off_gc);
  const favor_status rc = favor::launch_key_summaries(s, K, V, W, gs, gc, hs);
  if (rc != FAVOR_OK) return rc;
  float* cst = state + (size_t)s.BH * s.m * (s.d + 1);
  unsigned* count = reinterpret_cast<unsigned*>(cst + (size_t)s.BH * favor::kDecSplit);
  hipLaunchKernelGGL(favor::prefill_state, dim3(s.BH * favor::kDecSplit), dim3(favor::kDecThreads), 0, hs, gs, gc,
                     s.T, s.d, s.m, s.L, state, cst, count);
  return hipGetLastError() == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}

extern "C" size_t favor_decode_state_bytes(const favor_problem* p) {
  favor::Plan s;
  if (favor::decode_plan(p, &s) != FAVOR_OK) return 0;
  const size_t n = (size_t)s.BH * s.m * (s.d + 1) + 2 * (size_t)s.BH * favor::kDecSplit;
  return (n * sizeof(float) + 255) & ~size_t(255);
}

extern "C" favor_status favor_attn_decode(const favor_problem* p, const void* q, const void* k, const void* v,
                                          const float* W, float* state, void* out, void* stream) {
  favor::Plan s;
  const favor_status st = favor::decode_plan(p, &s);
  if (st != FAVOR_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || W == nullptr || state == nullptr || out == nullptr)
    return FAVOR_ERR_INVALID_ARG;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (s.dtype == FAVOR_BF16)
    return s.d == 64 ? favor::run_decode<favor::bf16, 64>(s, q, k, v, W, state, out, hs)
                     : favor::run_decode<favor::bf16, 128>(s, q, k, v, W, state, out, hs);
  return s.d == 64 ? favor::run_decode<float, 64>(s, q, k, v, W, state, out, hs)
                   : favor::run_decode<float, 128>(s, q, k, v, W, state, out, hs);
}
