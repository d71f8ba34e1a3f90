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

// GELU(v) = v * Phi(v) = 0.5 v (1 + erf(v / sqrt 2)), exact-erf form; erff is
// the device math library's.
__device__ __forceinline__ float gelu(float v) {
  return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
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
