// kernel_ladder.hip -- the optimisation ladder of the DeepGEMM page (section 4.1)
// rebuilt as separate kernels, so that each step's effect can be measured on
// this chip, plus the accumulation-precision variant of its section 3.4.
//
//  V0  one thread per element of C; both operands read straight from global
//      memory (neighbouring threads take neighbouring columns, so B reads
//      coalesce and A reads broadcast)
//  V1  shared-memory tiling: a 16 x 16 block stages a 16 x 16 tile of A and of B
//      per 16-deep k step and reads the operands from LDS, one element per thread
//  V2  register tiling: 64 x 64 block tile, 256 threads, each a 4 x 4 block of
//      C held in registers and fed from LDS values reused 4 times; A is staged
//      k-major (transposed on the way in), rows of exactly 64 floats
//  V3  V2 with the LDS rows padded to 65 floats: the transposed A stores of 16
//      neighbouring k go to 16 different banks instead of one, but the rows are
//      no longer 16-byte aligned, so the four consecutive floats a thread reads
//      per operand take four LDS reads instead of one (the trap the page's
//      section 5.2 describes: padding against vector access)
//  V3a V2 with rows padded to 68 floats: 16-byte aligned rows keep the vector
//      reads, the A stores spread over 8 banks (the page's fix: padding that
//      keeps 16-byte alignment)
//  V4  matrix instructions on the same 64 x 64 tile: the mfma16_{t}_64x64_w2x2
//      (and for fp32 f32_64x64_w2x2) configurations of the other kernel files
//
//  V3acc16 (fp16 inputs only): V3 with every accumulator held in fp16, one fused
//      multiply-add rounded to fp16 per k. It exists to show the error the page
//      warns about (FP16 accumulation against FP32); it does not meet the fp32
//      accumulation tolerance.
//
// All of them take any shape, row alignment and batch, accumulate in k order per
// element, apply the fused epilogue per element and store element by element.
// They are never chosen automatically (kind KIND_LADDER); a plan gets one only
// when its configuration is forced by name.
#include <type_traits>

#include "kernels.hpp"

namespace g15 {
namespace {

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

constexpr int LT = 256;  // threads per block, every rung

template <typename T>
__device__ __forceinline__ int64_t in_bytes() {
  return T::code == DT_F32 ? 4 : 2;
}

// C[m][n] of item z: epilogue and store of one element
__device__ __forceinline__ void put(const LaunchArgs& a, int64_t z, int64_t m, int64_t n,
                                    float acc) {
  const Epi& e = a.epi;
  const int64_t ob = e.out_dtype == DT_F32 ? 4 : 2;
  void* Cp = static_cast<char*>(a.C) + z * a.sC * ob;
  const void* Rp =
      (e.flags & EPI_RESID) ? static_cast<const char*>(e.resid) + z * a.sR * ob : nullptr;
  const int64_t idx = m * a.ldc + n;
  const float bn = (e.flags & EPI_BIAS) ? e.bias[n] : 0.f;
  store_out_elem(Cp, e.out_dtype, idx, apply_epi(e, acc, bn, Rp, idx));
}

// ---- V0: one thread per output element, global memory only
template <typename T>
__global__ __launch_bounds__(LT) void ladder_v0_kernel(LaunchArgs a) {
  const int64_t tiles_n = (a.N + 15) / 16;
  const int64_t m = static_cast<int64_t>(blockIdx.x) / tiles_n * 16 + (threadIdx.x >> 4);
  const int64_t n = static_cast<int64_t>(blockIdx.x) % tiles_n * 16 + (threadIdx.x & 15);
  const int64_t z = blockIdx.y;
  if (m >= a.M || n >= a.N) return;
  const char* Ap = static_cast<const char*>(a.A) + z * a.sA * in_bytes<T>();
  const char* Bp = static_cast<const char*>(a.B) + z * a.sB * in_bytes<T>();
  float acc = 0.f;
  for (int64_t k = 0; k < a.K; ++k)
    acc = __builtin_fmaf(ld_in<T>(Ap, m * a.lda + k), ld_in<T>(Bp, k * a.ldb + n), acc);
  put(a, z, m, n, acc);
}

// ---- V1: 16 x 16 LDS tiles, one output element per thread
template <typename T>
__global__ __launch_bounds__(LT) void ladder_v1_kernel(LaunchArgs a) {
  __shared__ float As[16][16];
  __shared__ float Bs[16][16];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t tiles_n = (a.N + 15) / 16;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) / tiles_n * 16;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) % tiles_n * 16;
  const int64_t z = blockIdx.y;
  const char* Ap = static_cast<const char*>(a.A) + z * a.sA * in_bytes<T>();
  const char* Bp = static_cast<const char*>(a.B) + z * a.sB * in_bytes<T>();
  const int64_t m = m0 + ty, n = n0 + tx;
  float acc = 0.f;
  for (int64_t k0 = 0; k0 < a.K; k0 += 16) {
    // thread (ty, tx) fetches A[m0 + ty][k0 + tx] and B[k0 + ty][n0 + tx], zero past the edges
    As[ty][tx] = (m < a.M && k0 + tx < a.K) ? ld_in<T>(Ap, m * a.lda + k0 + tx) : 0.f;
    Bs[ty][tx] = (k0 + ty < a.K && n < a.N) ? ld_in<T>(Bp, (k0 + ty) * a.ldb + n) : 0.f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc = __builtin_fmaf(As[ty][kk], Bs[kk][tx], acc);
    __syncthreads();
  }
  if (m < a.M && n < a.N) put(a, z, m, n, acc);
}

// ---- V2 / V3 / V3a (PAD = 0 / 1 / 4) and V3acc16 (ACC16): 64 x 64 tile, 4 x 4 per thread
template <typename T, int PAD, bool ACC16>
__global__ __launch_bounds__(LT) void ladder_v23_kernel(LaunchArgs a) {
  constexpr int BT = 64, BKD = 16;
  __shared__ float As[BKD][BT + PAD];  // k-major: As[k][row]
  __shared__ float Bs[BKD][BT + PAD];  // Bs[k][col]
  typedef typename std::conditional<ACC16, _Float16, float>::type acc_t;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t tiles_n = (a.N + BT - 1) / BT;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) / tiles_n * BT;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) % tiles_n * BT;
  const int64_t z = blockIdx.y;
  const char* Ap = static_cast<const char*>(a.A) + z * a.sA * in_bytes<T>();
  const char* Bp = static_cast<const char*>(a.B) + z * a.sB * in_bytes<T>();

  acc_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = static_cast<acc_t>(0.f);

  for (int64_t k0 = 0; k0 < a.K; k0 += BKD) {
#pragma unroll
    for (int r = 0; r < (BT * BKD) / LT; ++r) {
      const int e = tid + r * LT;
      // A: e -> (row, k) with k fastest (neighbouring lanes read neighbouring k and
      // store to LDS rows BT + PAD floats apart)
      const int ar = e / BKD, ak = e % BKD;
      const int64_t gm = m0 + ar, gk = k0 + ak;
      As[ak][ar] = (gm < a.M && gk < a.K) ? ld_in<T>(Ap, gm * a.lda + gk) : 0.f;
      // B: e -> (k, col) with col fastest
      const int bk = e / BT, bc = e % BT;
      const int64_t gk2 = k0 + bk, gn = n0 + bc;
      Bs[bk][bc] = (gk2 < a.K && gn < a.N) ? ld_in<T>(Bp, gk2 * a.ldb + gn) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKD; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (ACC16)  // fp16 inputs: the conversions are exact
            acc[i][j] = __builtin_fmaf16(static_cast<_Float16>(av[i]),
                                         static_cast<_Float16>(bv[j]), acc[i][j]);
          else
            acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t gm = m0 + ty * 4 + i;
    if (gm >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t gn = n0 + tx * 4 + j;
      if (gn < a.N) put(a, z, gm, gn, static_cast<float>(acc[i][j]));
    }
  }
}

template <int TILE, typename K>
hipError_t launch_ladder(K kernel, const LaunchArgs& a, hipStream_t s) {
  const int64_t tiles = ((a.M + TILE - 1) / TILE) * ((a.N + TILE - 1) / TILE);
  dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(a.batch));
  hipLaunchKernelGGL(kernel, grid, dim3(LT), 0, s, a);
  return hipGetLastError();
}
template <typename T>
hipError_t launch_v0(const LaunchArgs& a, hipStream_t s) {
  return launch_ladder<16>(ladder_v0_kernel<T>, a, s);
}
template <typename T>
hipError_t launch_v1(const LaunchArgs& a, hipStream_t s) {
  return launch_ladder<16>(ladder_v1_kernel<T>, a, s);
}
template <typename T, int PAD, bool ACC16>
hipError_t launch_v23(const LaunchArgs& a, hipStream_t s) {
  return launch_ladder<64>(ladder_v23_kernel<T, PAD, ACC16>, a, s);
}

#define G15_LADDER(T, TN)                                                                        \
  {"ladder_v0_" TN "_16x16", KIND_LADDER, T::code, 16, 16, 1, LT, 0, 0, 0, launch_v0<T>},          \
  {"ladder_v1_" TN "_16x16x16", KIND_LADDER, T::code, 16, 16, 16, LT, 2 * 16 * 16 * 4, 0, 0,       \
   launch_v1<T>},                                                                                 \
  {"ladder_v2_" TN "_64x64x16", KIND_LADDER, T::code, 64, 64, 16, LT, 2 * 16 * 64 * 4, 0, 0,       \
   launch_v23<T, 0, false>},                                                                      \
  {"ladder_v3_" TN "_64x64x16", KIND_LADDER, T::code, 64, 64, 16, LT, 2 * 16 * 65 * 4, 0, 0,       \
   launch_v23<T, 1, false>},                                                                      \
  {"ladder_v3a_" TN "_64x64x16", KIND_LADDER, T::code, 64, 64, 16, LT, 2 * 16 * 68 * 4, 0, 0,      \
   launch_v23<T, 4, false>}

const KernelEntry kLadder[] = {
    G15_LADDER(f16_t, "f16"),
    G15_LADDER(bf16_t, "bf16"),
    G15_LADDER(f32_t, "f32"),
    {"ladder_v3acc16_f16_64x64x16", KIND_LADDER, DT_F16, 64, 64, 16, LT, 2 * 16 * 65 * 4, 0, 0,
     launch_v23<f16_t, 1, true>},
};

}  // namespace

int ladder_entries(const KernelEntry** out) {
  *out = kLadder;
  return static_cast<int>(sizeof(kLadder) / sizeof(kLadder[0]));
}

}  // namespace g15
