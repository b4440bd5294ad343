// Device building blocks for the FAVOR+ kernels on gfx950 (CDNA4, wave64).
//
// All contractions use the 32x32 MFMA accumulator tile.  Lane layouts (checked on the
// device against a host matmul):
//   v_mfma_f32_32x32x16_bf16  A[i][k]: lane (i = l%32), k = 8*(l/32) + j   (j = 0..7)
//                             B[k][n]: lane (n = l%32), k = 8*(l/32) + j
//   v_mfma_f32_32x32x2_f32    A[i][k]: lane (i = l%32), k = l/32;  B likewise
//   accumulator C[i][n]:      lane (n = l%32), register r holds row 8*(r/4) + 4*(l/32) + r%4
// So an accumulator feeds a later MFMA directly as an operand whose contraction index is
// its row index: for bf16, registers 8h..8h+7 form operand h and slot j of lane group g
// carries contraction index kappa(h,g,j) = 16h + 8(j/4) + 4g + j%4; for fp32, register r
// is operand r with index 8(r/4) + 4g + r%4.  The other operand of such a product must
// present the same index order; ds_read_b64_tr_b16 delivers it from a row-major LDS tile
// (each 16-lane group reads a 4x16 block and lane i receives column i).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace favor {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr float kLog2e = 1.4426950408889634f;
// Lazy stabiliser slack in log2 units: exponents are kept <= kTau, so features never
// exceed 2^kTau and a running maximum is only moved when a new block exceeds it by kTau.
constexpr float kTau = 8.0f;

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// Value held by lane l ^ 32.
__device__ __forceinline__ float partner32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(lane_id() < 32 ? r[1] : r[0]);
}

// x + partner32(x) and max(x, partner32(x)) in every lane: the two halves of one swap.
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_min(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0; }

// Causal segment summaries and their prefixes are stored in float32 for float32 problems and
// in bf16 for bf16 problems (their consumers accumulate in float32 either way).
template <class T> struct SumOf { using type = float; };
template <> struct SumOf<bf16> { using type = bf16; };
// four consecutive elements (16-byte aligned for float32, 8-byte for bf16)
__device__ __forceinline__ f32x4 load_sum4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 load_sum4(const bf16* p) {
  const bf16x4_t v = *reinterpret_cast<const bf16x4_t*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ void store_sum4(float* p, const f32x4& v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void store_sum4(bf16* p, const f32x4& v) {
  bf16x4_t h;
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = (bf16)v[i];
  *reinterpret_cast<bf16x4_t*>(p) = h;
}

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Per-precision traits.  T is the element type of Q, K, V and out.
//   frag   operand of the feature-side contractions (phi with S or with [V, 1])
//   wfrag  operand of the W contraction.  bf16 problems contract in fp16: bf16 Q and K
//          values convert to fp16 exactly (|x| < 65504; below 2^-14 they lose low bits,
//          an absolute error under 2^-25), and W * log2(e) rounds to fp16's 11-bit
//          significand, so the exponent is 8x more accurate than with bf16 W.
template <class T> struct Prec;

template <> struct Prec<bf16> {
  using frag = bf16x8;
  using wfrag = f16x8;
  using welem = f16;
  static constexpr int KS = 16;     // contraction length of one MFMA
  static constexpr int NF32 = 2;    // operands per 32-deep contraction
};

template <> struct Prec<float> {
  using frag = float;
  using wfrag = float;
  using welem = float;
  static constexpr int KS = 2;
  static constexpr int NF32 = 16;
};

__device__ __forceinline__ bf16x8 zero_frag(bf16x8) {
  bf16x8 z;
#pragma unroll
  for (int j = 0; j < 8; ++j) z[j] = (bf16)0.f;
  return z;
}
__device__ __forceinline__ f16x8 zero_frag(f16x8) {
  f16x8 z;
#pragma unroll
  for (int j = 0; j < 8; ++j) z[j] = (f16)0.f;
  return z;
}
__device__ __forceinline__ float zero_frag(float) { return 0.f; }

// Q / K operand of the W contraction.
__device__ __forceinline__ f16x8 to_wfrag(bf16x8 x) {
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (f16)(float)x[j];
  return r;
}
__device__ __forceinline__ float to_wfrag(float x) { return x; }

// ---- accumulator -> operand (contraction index = accumulator row) --------------------

__device__ __forceinline__ void acc_to_frags(const f32x16& c, bf16x8 (&f)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) f[h][j] = (bf16)c[8 * h + j];
}
__device__ __forceinline__ void acc_to_frags(const f32x16& c, float (&f)[16]) {
#pragma unroll
  for (int r = 0; r < 16; ++r) f[r] = c[r];
}

// ---- operands with the contraction index contiguous in memory ------------------------
// Row `row` of a row-major matrix, contraction chunk kc.

__device__ __forceinline__ bf16x8 load_frag_k(const bf16* row, int kc, int g) {
  return *reinterpret_cast<const bf16x8*>(row + 16 * kc + 8 * g);
}
__device__ __forceinline__ f16x8 load_frag_k(const f16* row, int kc, int g) {
  return *reinterpret_cast<const f16x8*>(row + 16 * kc + 8 * g);
}
__device__ __forceinline__ float load_frag_k(const float* row, int kc, int g) {
  return row[2 * kc + g];
}

// W row (float32 in global memory) scaled by log2(e), as a W-contraction operand.
__device__ __forceinline__ void load_w_frag(const float* wrow, int kc, int g, f16x8& f) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(wrow + 16 * kc + 8 * g);
  const f32x4 b = *reinterpret_cast<const f32x4*>(wrow + 16 * kc + 8 * g + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = (f16)(a[j] * kLog2e);
    f[j + 4] = (f16)(b[j] * kLog2e);
  }
}
__device__ __forceinline__ void load_w_frag(const float* wrow, int kc, int g, float& f) {
  f = wrow[2 * kc + g] * kLog2e;
}

// ---- operands with the contraction index along LDS rows ------------------------------
// X: row-major LDS tile with leading dimension ld.  Returns the operand whose lane column
// is col0 + l%32 and whose contraction rows follow the accumulator order of operand h
// (bf16) / register r (fp32) starting at row0.

__device__ __forceinline__ bf16x8 lds_frag_rows(const bf16* X, int ld, int row0, int col0, int h) {
  const int l = lane_id(), q = l >> 4, i = l & 15, g = l >> 5;
  const bf16* p0 = X + (row0 + 16 * h + 4 * g + (i >> 2)) * ld + col0 + 16 * (q & 1) + 4 * (i & 3);
  const bf16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)p0);
  const bf16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p0 + 8 * ld));
  bf16x8 f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = a[j];
    f[j + 4] = b[j];
  }
  return f;
}
__device__ __forceinline__ float lds_frag_rows(const float* X, int ld, int row0, int col0, int r) {
  const int l = lane_id(), g = l >> 5;
  return X[(row0 + 8 * (r >> 2) + 4 * g + (r & 3)) * ld + col0 + (l & 31)];
}

// ---- the bias operand: adds -(r_row + c_col) to a feature exponent in the MFMA --------
// A side (rows): per-row value r (e.g. |k|^2/2 in log2 units); B side (cols): per-column
// stabiliser c.  fp16: r and c are each carried as three fp16 pieces (exact to far below
// float32 rounding for |values| < 65504).

// x = f[i0] + f[i0+1] + f[i0+2] to float32 accuracy.
__device__ __forceinline__ void split3(float x, f16x8& f, int i0) {
  const f16 a = (f16)x;
  const float r1 = x - (float)a;
  const f16 b = (f16)r1;
  f[i0] = a;
  f[i0 + 1] = b;
  f[i0 + 2] = (f16)(r1 - (float)b);
}

__device__ __forceinline__ f16x8 bias_rows(float r, int g, f16x8) {
  f16x8 f = zero_frag(f16x8{});
  if (g == 0) {
    split3(r, f, 0);
    f[3] = f[4] = f[5] = (f16)1.f;
  }
  return f;
}
__device__ __forceinline__ f16x8 bias_cols(float c, int g, f16x8) {
  f16x8 f = zero_frag(f16x8{});
  if (g == 0) {
    f[0] = f[1] = f[2] = (f16)-1.f;
    split3(-c, f, 3);
  }
  return f;
}
__device__ __forceinline__ float bias_rows(float r, int g, float) { return g == 0 ? r : 1.f; }
// A-side operand that picks up only the stabiliser part of bias_cols: rows get -c_col.
__device__ __forceinline__ f16x8 bias_unit_rows(int g, f16x8) {
  f16x8 f = zero_frag(f16x8{});
  if (g == 0) f[3] = f[4] = f[5] = (f16)1.f;
  return f;
}
__device__ __forceinline__ float bias_unit_rows(int g, float) { return g == 0 ? 0.f : 1.f; }
__device__ __forceinline__ float bias_cols(float c, int g, float) { return g == 0 ? -1.f : -c; }
// Row bias that removes a row from a contraction (its features become 2^-30000 = 0).
constexpr float kMaskedRow = 30000.0f;
// Word 3 of a raw buffer descriptor for untyped loads (data format 32, no swizzle).
constexpr int kBufWord3 = 0x00020000;

// Sum of squares of the contraction values a lane holds in its row operands.
template <int N>
__device__ __forceinline__ float sumsq(const bf16x8 (&f)[N]) {
  float s[4] = {0.f, 0.f, 0.f, 0.f};  // four independent accumulation chains
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      bf16x2 v;
      v[0] = f[i][j];
      v[1] = f[i][j + 1];
      s[j / 2] = __builtin_amdgcn_fdot2_f32_bf16(v, v, s[j / 2], false);
    }
  return (s[0] + s[1]) + (s[2] + s[3]);
}
template <int N>
__device__ __forceinline__ float sumsq(const f16x8 (&f)[N]) {
  float s[4] = {0.f, 0.f, 0.f, 0.f};  // four independent accumulation chains
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      typedef f16 f16x2 __attribute__((ext_vector_type(2)));
      f16x2 v;
      v[0] = f[i][j];
      v[1] = f[i][j + 1];
      s[j / 2] = __builtin_amdgcn_fdot2(v, v, s[j / 2], false);
    }
  return (s[0] + s[1]) + (s[2] + s[3]);
}
template <int N>
__device__ __forceinline__ float sumsq(const float (&f)[N]) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) s = __builtin_fmaf(f[i], f[i], s);
  return s;
}

// Column permutation applied to value tiles so that an accumulator lane ends up holding
// 16 consecutive value columns: accumulator row rho of a 32-column tile carries value
// column vperm(rho); a value column c sits at tile row vperm_inv(c).
__host__ __device__ constexpr int vperm(int rho) {
  return 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3);
}
__host__ __device__ constexpr int vperm_inv(int c) {
  return 8 * ((c & 15) >> 2) + 4 * (c >> 4) + (c & 3);
}

}  // namespace favor
