// kernel_softmax.hip -- row softmax in fp32 between the two batched products of
// attention: P = softmax(scale * S) row by row, S the fp32 scores of Q K^T,
// P then multiplied by V (tutorial page, section 2: attention is Q K^T, a
// softmax, and the product with V; DeepGEMM page, section 3.4: the softmax
// denominator is a sum that must be accumulated wide).
//
// One wave per row. Rows of up to 1024 columns (multiples of 4, aligned) are
// held in registers: one read, the row maximum and then the sum of exp(x - max)
// reduced across the wave with XOR shuffles, P written as 8- or 16-byte stores.
// Other rows: each lane keeps a running (max, sum of exp(x - max)) pair over its
// share of the row (one pass; a larger element rescales the sum), the pairs are
// merged across the wave, and a second pass (the row is in L1/L2 by then) writes
// exp(x - max) / sum. fp32 throughout, P rounded once to the output type; exp is
// the hardware exp2 with its argument scaled by log2(e). The work is HBM-bound:
// the scores are read once and P written once.
#include "kernels.hpp"
#include "softmax.hpp"

namespace g15 {
namespace {

constexpr int SM_WAVES = 4;  // rows per workgroup

struct MS {
  float m, s;
};

__device__ __forceinline__ MS ms_merge(MS a, MS b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return MS{m, 0.f};  // both empty
  return MS{m, a.s * __expf(a.m - m) + b.s * __expf(b.m - m)};
}

__device__ __forceinline__ void ms_add(MS& a, float y) {
  if (y > a.m) {
    a.s = a.s * __expf(a.m - y) + 1.f;  // exp(-inf) = 0 for the first element
    a.m = y;
  } else {
    a.s += __expf(y - a.m);
  }
}

__device__ __forceinline__ void put_p(void* P, int dt, int64_t idx, float v) {
  if (dt == DT_F32)
    static_cast<float*>(P)[idx] = v;
  else if (dt == DT_BF16)
    static_cast<uint16_t*>(P)[idx] = narrow_bf16(v);
  else
    static_cast<uint16_t*>(P)[idx] = narrow_f16(v);
}

// Rows of at most 64 * 4 * NV columns (cols % 4 == 0, 16-byte aligned rows): each
// lane loads its NV float4 chunks once and keeps them in registers, so the row is
// read from memory once; a 16-bit P leaves as one 8-byte store per chunk.
template <int NV>
__global__ __launch_bounds__(64 * SM_WAVES) void softmax_rows_reg_kernel(
    const float* S, int64_t rows, int64_t cols, int64_t lds, float scale, void* P, int64_t ldp,
    int out_dt) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * SM_WAVES + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole waves only: no barrier below
  const f32x4* x4 = reinterpret_cast<const f32x4*>(S + row * lds);
  const int nc = static_cast<int>(cols / 4);
  f32x4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    v[i] = c < nc ? x4[c] * scale : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) m = fmaxf(m, v[i][t]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v[i][t] = __expf(v[i][t] - m);  // exp(-inf) = 0 for the padding past cols
      sum += v[i][t];
    }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  const float inv = 1.f / sum;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c >= nc) continue;
    const int64_t at = row * ldp + 4 * c;
    if (out_dt == DT_F32) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(P) + at) =
          f32x4{v[i][0] * inv, v[i][1] * inv, v[i][2] * inv, v[i][3] * inv};
    } else {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      uint16_t h[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        h[t] = out_dt == DT_BF16 ? narrow_bf16(v[i][t] * inv) : narrow_f16(v[i][t] * inv);
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(P) + at) =
          u32x2{h[0] | (static_cast<uint32_t>(h[1]) << 16),
                h[2] | (static_cast<uint32_t>(h[3]) << 16)};
    }
  }
}

// Any row: VEC (cols % 4 == 0 and 16-byte aligned rows) reads float4 chunks; a
// running (max, sum) per lane in one pass, a second pass for the output.
template <bool VEC>
__global__ __launch_bounds__(64 * SM_WAVES) void softmax_rows_kernel(
    const float* S, int64_t rows, int64_t cols, int64_t lds, float scale, void* P, int64_t ldp,
    int out_dt) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * SM_WAVES + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole waves only: no barrier below
  const float* x = S + row * lds;
  MS a{-INFINITY, 0.f};
  if constexpr (VEC) {
    const f32x4* x4 = reinterpret_cast<const f32x4*>(x);
    for (int64_t c = lane; c < cols / 4; c += 64) {
      const f32x4 v = x4[c];
      ms_add(a, scale * v[0]);
      ms_add(a, scale * v[1]);
      ms_add(a, scale * v[2]);
      ms_add(a, scale * v[3]);
    }
  } else {
    for (int64_t c = lane; c < cols; c += 64) ms_add(a, scale * x[c]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    MS b;
    b.m = __shfl_xor(a.m, o);
    b.s = __shfl_xor(a.s, o);
    a = ms_merge(a, b);
  }
  const float inv = 1.f / a.s;
  const int64_t pr = row * ldp;
  if constexpr (VEC) {
    const f32x4* x4 = reinterpret_cast<const f32x4*>(x);
    for (int64_t c = lane; c < cols / 4; c += 64) {
      const f32x4 v = x4[c];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        put_p(P, out_dt, pr + 4 * c + t, __expf(scale * v[t] - a.m) * inv);
    }
  } else {
    for (int64_t c = lane; c < cols; c += 64)
      put_p(P, out_dt, pr + c, __expf(scale * x[c] - a.m) * inv);
  }
}

}  // namespace

hipError_t launch_softmax_rows(const float* S, int64_t rows, int64_t cols, int64_t lds,
                               float scale, void* P, int64_t ldp, int out_dt, hipStream_t s) {
  const int64_t blocks = (rows + SM_WAVES - 1) / SM_WAVES;
  const bool vec = cols % 4 == 0 && lds % 4 == 0 && (reinterpret_cast<uintptr_t>(S) & 15) == 0;
  // the register form also needs P rows aligned for its 8- or 16-byte stores
  const int pb = out_dt == DT_F32 ? 4 : 2;
  const bool pvec = (reinterpret_cast<uintptr_t>(P) & (pb == 4 ? 15 : 7)) == 0 && ldp % 4 == 0;
  if (vec && pvec && cols <= 64 * 4 * 4) {
    if (cols <= 64 * 4 * 2)
      hipLaunchKernelGGL(softmax_rows_reg_kernel<2>, dim3(static_cast<unsigned>(blocks)),
                         dim3(64 * SM_WAVES), 0, s, S, rows, cols, lds, scale, P, ldp, out_dt);
    else
      hipLaunchKernelGGL(softmax_rows_reg_kernel<4>, dim3(static_cast<unsigned>(blocks)),
                         dim3(64 * SM_WAVES), 0, s, S, rows, cols, lds, scale, P, ldp, out_dt);
  } else if (vec)
    hipLaunchKernelGGL(softmax_rows_kernel<true>, dim3(static_cast<unsigned>(blocks)),
                       dim3(64 * SM_WAVES), 0, s, S, rows, cols, lds, scale, P, ldp, out_dt);
  else
    hipLaunchKernelGGL(softmax_rows_kernel<false>, dim3(static_cast<unsigned>(blocks)),
                       dim3(64 * SM_WAVES), 0, s, S, rows, cols, lds, scale, P, ldp, out_dt);
  return hipGetLastError();
}

}  // namespace g15
