// device_common.hpp -- element types, conversions and the fused epilogue shared
// by every gemm15 kernel (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace g15 {

enum : uint32_t { EPI_BIAS = 1u, EPI_GELU = 2u, EPI_RESID = 4u, EPI_SCALE = 8u };
enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

// Storage tags for the input types. The two 16-bit types are moved around as
// raw 16-bit patterns; only the MFMA and the scalar widening differ.
struct f32_t {
  static constexpr int code = DT_F32;
};
struct bf16_t {
  static constexpr int code = DT_BF16;
};
struct f16_t {
  static constexpr int code = DT_F16;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- widening of one 16-bit pattern to float (exact) ----
__device__ __forceinline__ float widen(bf16_t, uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ float widen(f16_t, uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return static_cast<float>(v);
}

// ---- narrowing of float to a 16-bit pattern, round to nearest even ----
__device__ __forceinline__ uint16_t narrow_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  uint16_t h;
  __builtin_memcpy(&h, &b, 2);
  return h;
}
__device__ __forceinline__ uint16_t narrow_f16(float f) {
  _Float16 v = static_cast<_Float16>(f);
  uint16_t h;
  __builtin_memcpy(&h, &v, 2);
  return h;
}

// Everything the epilogue needs, passed by value to each kernel.
struct Epi {
  uint32_t flags;     // EPI_* bits
  float scale;        // used when EPI_SCALE
  const float* bias;  // [N] fp32, used when EPI_BIAS
  const void* resid;  // [M x N] row-major in out_dtype, used when EPI_RESID
  int out_dtype;      // DT_F32 / DT_F16 / DT_BF16
};

// erfc(z) for z >= 0 in the Chebyshev-fitted form of Press et al., Numerical
// Recipes (function erfcc): erfc(z) = t exp(-z^2 + P(t)), t = 1 / (1 + z / 2),
// P of degree 9, relative error below 1.2e-7 for every z >= 0. One reciprocal,
// one exponential and nine fused multiply-adds, with no branch (the library
// erff takes two divergent polynomial branches and about 40 instructions).
__device__ __forceinline__ float erfc_nonneg(float z) {
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.5f, z, 1.0f));
  float p = 0.17087277f;
  p = __builtin_fmaf(p, t, -0.82215223f);
  p = __builtin_fmaf(p, t, 1.48851587f);
  p = __builtin_fmaf(p, t, -1.13520398f);
  p = __builtin_fmaf(p, t, 0.27886807f);
  p = __builtin_fmaf(p, t, -0.18628806f);
  p = __builtin_fmaf(p, t, 0.09678418f);
  p = __builtin_fmaf(p, t, 0.37409196f);
  p = __builtin_fmaf(p, t, 1.00002368f);
  p = __builtin_fmaf(p, t, -1.26551223f);
  return t * __expf(__builtin_fmaf(-z, z, p));
}

// GELU(v) = v Phi(v), Phi the standard normal CDF = 1 - erfc(v / sqrt 2) / 2 for
// v >= 0 and erfc(-v / sqrt 2) / 2 below (no cancellation in the negative tail).
// Absolute error about 1e-7 |v| against the exact-erf form.
__device__ __forceinline__ float gelu(float v) {
  const float ec = erfc_nonneg(__builtin_fabsf(v) * 0.70710678118654752f);
  const float phi = v >= 0.f ? __builtin_fmaf(-0.5f, ec, 1.0f) : 0.5f * ec;
  return v * phi;
}

// GELU for results that are rounded to 16 bits (bf16 / fp16 output), about half
// the VALU work of gelu(): with h = erfc(|v| / sqrt 2) / 2, GELU(v) = v (1 - h) for
// v >= 0 and v h below, i.e. max(v, 0) - |v| h in both cases (no select). With
// s = 1 / (2 + |v| / sqrt 2) (= t / 2 in the form above), |v| h = (|v| s) 2^(-log2(e) v^2 / 2
// + Q(s)), where Q is a degree-5 polynomial fitted (minimax, erfc_fit16.py beside
// this file) to log2(erfc(z) / 2s) + log2(e) z^2 over all z >= 0: erfc to 5.1e-5
// relative, GELU to 2.5e-5 |v| absolute and 6.1e-5 relative, a few percent of the
// 16-bit rounding step. One reciprocal, one base-2 exponential, eight fused
// multiply-adds / multiplies, a min and a max. GELU(+inf) = +inf, GELU(-inf) = 0.
__device__ __forceinline__ float gelu16(float v) {
  const float av = __builtin_fabsf(v);
  const float s = __builtin_amdgcn_rcpf(__builtin_fmaf(av, 0.70710678f, 2.0f));
  float p = 8.29845524f;
  p = __builtin_fmaf(p, s, -13.1949415f);
  p = __builtin_fmaf(p, s, 3.82766771f);
  p = __builtin_fmaf(p, s, 1.85619426f);
  p = __builtin_fmaf(p, s, 2.89719629f);
  p = __builtin_fmaf(p, s, -1.82582092f);
  const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(v, v * -0.72134752f, p));
  // |v| s tends to sqrt 2; the min keeps it finite (inf * 0) for infinite v
  const float q = __builtin_fminf(av * s, 1.41421356f);
  return __builtin_fmaf(-q, e, __builtin_fmaxf(v, 0.f));
}

__device__ __forceinline__ float load_out_elem(const void* p, int dt, int64_t idx) {
  if (dt == DT_F32) return static_cast<const float*>(p)[idx];
  const uint16_t h = static_cast<const uint16_t*>(p)[idx];
  return dt == DT_BF16 ? widen(bf16_t{}, h) : widen(f16_t{}, h);
}

__device__ __forceinline__ void store_out_elem(void* p, int dt, int64_t idx, float v) {
  if (dt == DT_F32)
    static_cast<float*>(p)[idx] = v;
  else if (dt == DT_BF16)
    static_cast<uint16_t*>(p)[idx] = narrow_bf16(v);
  else
    static_cast<uint16_t*>(p)[idx] = narrow_f16(v);
}

// Epilogue on one accumulator: scale, then bias, then GELU, then residual.
// `bias_n` is bias[col] when EPI_BIAS is on (the caller loads it once per column).
__device__ __forceinline__ float apply_epi(const Epi& e, float acc, float bias_n, const void* resid,
                                           int64_t idx) {
  float v = acc;
  if (e.flags & EPI_SCALE) v *= e.scale;
  if (e.flags & EPI_BIAS) v += bias_n;
  if (e.flags & EPI_GELU) v = gelu(v);
  if (e.flags & EPI_RESID) v += load_out_elem(resid, e.out_dtype, idx);
  return v;
}

}  // namespace g15
