// kernel_simple.hip -- the universal fallback: an LDS-tiled scalar GEMM that
// takes any shape, any alignment and any of the three input types.
//
// It follows the tiled kernel of the tutorial page (section 4.2: a block stages
// an A tile and a B tile in shared memory, zero-fills out-of-range elements,
// synchronises, accumulates, synchronises, and guards the final store) with the
// register tile of section 4.3 (each thread owns a 4 x 4 block of C). The
// accumulation is fp32 in k order for every element.
#include "kernels.hpp"

namespace g15 {
namespace {

constexpr int ST = 64;  // C tile is ST x ST
constexpr int SK = 16;  // k-slice staged per step
constexpr int SNT = 256;

template <typename T>
__device__ __forceinline__ float ld_in(const void* p, int64_t i);
template <>
__device__ __forceinline__ float ld_in<f32_t>(const void* p, int64_t i) {
  return static_cast<const float*>(p)[i];
}
template <>
__device__ __forceinline__ float ld_in<bf16_t>(const void* p, int64_t i) {
  return widen(bf16_t{}, static_cast<const uint16_t*>(p)[i]);
}
template <>
__device__ __forceinline__ float ld_in<f16_t>(const void* p, int64_t i) {
  return widen(f16_t{}, static_cast<const uint16_t*>(p)[i]);
}

template <typename T>
__global__ __launch_bounds__(SNT) void gemm_simple_kernel(LaunchArgs a) {
  // As is stored k-major so the 16 rows a thread row reads sit in one LDS row.
  __shared__ float As[SK][ST + 1];
  __shared__ float Bs[SK][ST + 1];

  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t z = blockIdx.z;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * ST;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * ST;
  const int64_t M = a.M, N = a.N, K = a.K;
  const char* Ab = static_cast<const char*>(a.A);
  const char* Bb = static_cast<const char*>(a.B);
  const int64_t in_bytes = (T::code == DT_F32) ? 4 : 2;
  const void* Ap = Ab + z * a.sA * in_bytes;
  const void* Bp = Bb + z * a.sB * in_bytes;

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int64_t k0 = 0; k0 < K; k0 += SK) {
#pragma unroll
    for (int i = 0; i < (ST * SK) / SNT; ++i) {
      const int e = tid + i * SNT;
      // A: e -> (row, k) with k fastest, so neighbouring lanes read neighbouring k
      const int ar = e / SK, ak = e % SK;
      const int64_t gm = m0 + ar, gk = k0 + ak;
      As[ak][ar] = (gm < M && gk < K) ? ld_in<T>(Ap, gm * K + gk) : 0.f;
      // B: e -> (k, col) with col fastest
      const int bk = e / ST, bc = e % ST;
      const int64_t gk2 = k0 + bk, gn = n0 + bc;
      Bs[bk][bc] = (gk2 < K && gn < N) ? ld_in<T>(Bp, gk2 * N + gn) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < SK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }

  const Epi& e = a.epi;
  const int64_t out_bytes = e.out_dtype == DT_F32 ? 4 : 2;
  void* Cp = static_cast<char*>(a.C) + z * a.sC * out_bytes;
  const void* Rp = (e.flags & EPI_RESID) ? static_cast<const char*>(e.resid) + z * a.sR * out_bytes
                                         : nullptr;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t gn = n0 + tx + 16 * j;
    if (gn >= N) continue;
    const float bn = (e.flags & EPI_BIAS) ? e.bias[gn] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t gm = m0 + ty + 16 * i;
      if (gm >= M) continue;
      const int64_t idx = gm * N + gn;
      store_out_elem(Cp, e.out_dtype, idx, apply_epi(e, acc[i][j], bn, Rp, idx));
    }
  }
}

template <typename T>
hipError_t launch_simple(const LaunchArgs& a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>((a.N + ST - 1) / ST), static_cast<unsigned>((a.M + ST - 1) / ST),
            static_cast<unsigned>(a.batch));
  hipLaunchKernelGGL(gemm_simple_kernel<T>, grid, dim3(SNT), 0, s, a);
  return hipGetLastError();
}

const KernelEntry kSimple[] = {
    {"simple_f32", KIND_SIMPLE, DT_F32, ST, ST, SK, SNT, 2 * SK * (ST + 1) * 4, 0, 0,
     launch_simple<f32_t>},
    {"simple_f16", KIND_SIMPLE, DT_F16, ST, ST, SK, SNT, 2 * SK * (ST + 1) * 4, 0, 0,
     launch_simple<f16_t>},
    {"simple_bf16", KIND_SIMPLE, DT_BF16, ST, ST, SK, SNT, 2 * SK * (ST + 1) * 4, 0, 0,
     launch_simple<bf16_t>},
};
}  // namespace

int simple_entries(const KernelEntry** out) {
  *out = kSimple;
  return static_cast<int>(sizeof(kSimple) / sizeof(kSimple[0]));
}

}  // namespace g15
