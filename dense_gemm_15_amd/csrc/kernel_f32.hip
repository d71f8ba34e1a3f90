// kernel_f32.hip -- fp32 SGEMM on the gfx950 matrix cores (v_mfma_f32_32x32x2_f32),
// fused epilogue.
//
// This is the wave-level output tiling of the SGEMM page (sections 2.1 and 3.2:
// a warp owns a sub-tile of C, each thread a block of accumulators that stay in
// registers, operands reused from registers) with the double-buffered shared
// staging of its section 2.3, mapped onto CDNA4: a 64-lane wave owns a
// (BM/WGM) x (BN/WGN) sub-tile built from 32 x 32 matrix-core blocks, and
// products are exact-fp32 fused multiply-adds done by the matrix core instead of
// the vector ALU (there is no reduced-precision fp32 mode on this path).
//
// One 32x32x2 step sums two k values; lane half h (lanes 32h .. 32h+31) supplies
// the second. Inside every group of 8 k the four steps s = 0..3 pair
// k = 8g + s (half 0) with k = 8g + 4 + s (half 1). A lane therefore needs k =
// 8g + 4h .. 8g + 4h + 3 of its A row: one 16-byte LDS read feeds four steps, and
// A is staged row-major exactly as it sits in memory (no transpose).
//
// B is staged row-major too. Column j of matrix-core block f of a wave is mapped
// to C column (j * FN + f) of the wave's sub-tile, so each lane reads its FN
// columns of one B row as one contiguous 4*FN-byte LDS read, and later writes its
// FN results of one C row as one contiguous store.
//
// LDS: A slice = BM rows of 32 floats (8 chunks of 16 bytes, chunk c of row r
// stored at position c ^ (r & 7)); B slice = 32 rows of BN floats. Two slices.
#include "kernels.hpp"

namespace g15 {
namespace {

constexpr int FBK = 32;  // k per LDS slice

__device__ __forceinline__ int fswz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

__device__ __forceinline__ void ftile_coords(int wid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  if ((total & 7) == 0) wid = (wid & 7) * (total >> 3) + (wid >> 3);
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int group = wid / per_group;
  const int first = group * GM;
  const int gsz = min(tiles_m - first, GM);
  const int in = wid - group * per_group;
  tm = first + in % gsz;
  tn = in / gsz;
}

template <int FN>
struct FVec;
template <>
struct FVec<1> {
  typedef float type;
};
template <>
struct FVec<2> {
  typedef float type __attribute__((ext_vector_type(2)));
};
template <>
struct FVec<4> {
  typedef float type __attribute__((ext_vector_type(4)));
};

template <int FN>
__device__ __forceinline__ float vget(const typename FVec<FN>::type& v, int i) {
  if constexpr (FN == 1)
    return v;
  else
    return v[i];
}

template <int BM, int BN, int WGM, int WGN, bool VA, bool VB>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_f32_kernel(LaunchArgs a) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int NA = BM * 8 / NT;          // A 16-byte chunks per thread per slice
  constexpr int BCH = BN / 4;              // 16-byte chunks per B row
  constexpr int NB = FBK * BCH / NT;       // B chunks per thread per slice
  static_assert(BM * 8 % NT == 0 && FBK * BCH % NT == 0, "staging must divide evenly");
  static_assert(FN == 1 || FN == 2 || FN == 4, "FN must be 1, 2 or 4");
  typedef typename FVec<FN>::type bvec;

  __shared__ f32x4 ldsA[2][BM * 8];
  __shared__ f32x4 ldsB[2][FBK * BCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int64_t M = a.M, N = a.N, K = a.K;
  const int tiles_m = static_cast<int>((M + BM - 1) / BM);
  const int tiles_n = static_cast<int>((N + BN - 1) / BN);
  int tm, tn;
  ftile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = static_cast<int64_t>(tm) * BM, n0 = static_cast<int64_t>(tn) * BN;
  const int64_t z = blockIdx.y;
  const float* Ap = static_cast<const float*>(a.A) + z * a.sA;
  const float* Bp = static_cast<const float*>(a.B) + z * a.sB;

  f32x4 ra[NA], rb[NB];

  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int c = tid + i * NT;
      const int row = c >> 3, kc = c & 7;
      const int64_t gm = m0 + row, gk = k0 + kc * 4;
      if constexpr (VA) {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (gm < M && gk < K) v = *reinterpret_cast<const f32x4*>(Ap + gm * K + gk);
        ra[i] = v;
      } else {
        f32x4 v;
#pragma unroll
        for (int p = 0; p < 4; ++p) v[p] = (gm < M && gk + p < K) ? Ap[gm * K + gk + p] : 0.f;
        ra[i] = v;
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int c = tid + i * NT;
      const int kr = c / BCH, nc = c % BCH;
      const int64_t gk = k0 + kr, gn = n0 + nc * 4;
      if constexpr (VB) {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (gk < K && gn < N) v = *reinterpret_cast<const f32x4*>(Bp + gk * N + gn);
        rb[i] = v;
      } else {
        f32x4 v;
#pragma unroll
        for (int p = 0; p < 4; ++p) v[p] = (gk < K && gn + p < N) ? Bp[gk * N + gn + p] : 0.f;
        rb[i] = v;
      }
    }
  };

  auto stash = [&](int s) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int c = tid + i * NT;
      ldsA[s][fswz(c >> 3, c & 7)] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) ldsB[s][tid + i * NT] = rb[i];
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = static_cast<int>((K + FBK - 1) / FBK);
  fetch(0);
  stash(0);
  if (nk > 1) fetch(FBK);

  const int lrow = lane & 31, lhalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    if (kt + 1 < nk) {
      stash((kt + 1) & 1);
      if (kt + 2 < nk) fetch(static_cast<int64_t>(kt + 2) * FBK);
    }
    const f32x4* As = ldsA[kt & 1];
    const float* Bs = reinterpret_cast<const float*>(ldsB[kt & 1]);
#pragma unroll
    for (int g = 0; g < FBK / 8; ++g) {
      f32x4 fa[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[i] = As[fswz(wm * WTM + i * 32 + lrow, 2 * g + lhalf)];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kr = 8 * g + 4 * lhalf + s;
        const bvec fb = *reinterpret_cast<const bvec*>(Bs + kr * BN + wn * WTN + lrow * FN);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][s], vget<FN>(fb, j), acc[i][j],
                                                             0, 0, 0);
      }
    }
  }

  // lane holds, for block (i, j), C[row][col] with
  // row = 8 * (r / 4) + 4 * (lane / 32) + r % 4 and col = (lane % 32) * FN + j.
  const Epi& e = a.epi;
  const int64_t ob = e.out_dtype == DT_F32 ? 4 : 2;
  void* Cp = static_cast<char*>(a.C) + z * a.sC * ob;
  const void* Rp =
      (e.flags & EPI_RESID) ? static_cast<const char*>(e.resid) + z * a.sR * ob : nullptr;
  const int64_t colbase = n0 + wn * WTN + lrow * FN;
  float bn[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j)
    bn[j] = ((e.flags & EPI_BIAS) && colbase + j < N) ? e.bias[colbase + j] : 0.f;
  const bool fast = (e.flags == 0) && (e.out_dtype == DT_F32) && VB && (colbase + FN <= N);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
      if (row >= M) continue;
      if (fast) {
        bvec v;
        if constexpr (FN == 1) {
          v = acc[i][0][r];
        } else {
#pragma unroll
          for (int j = 0; j < FN; ++j) v[j] = acc[i][j][r];
        }
        *reinterpret_cast<bvec*>(static_cast<float*>(Cp) + row * N + colbase) = v;
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t col = colbase + j;
          if (col < N) {
            const int64_t idx = row * N + col;
            store_out_elem(Cp, e.out_dtype, idx, apply_epi(e, acc[i][j][r], bn[j], Rp, idx));
          }
        }
      }
    }
  }
}

template <int BM, int BN, int WGM, int WGN, bool VA, bool VB>
hipError_t launch_f32(const LaunchArgs& a, hipStream_t s) {
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(a.batch));
  hipLaunchKernelGGL((gemm_f32_kernel<BM, BN, WGM, WGN, VA, VB>), grid, dim3(64 * WGM * WGN), 0, s,
                     a);
  return hipGetLastError();
}

#define G15_F32(BM, BN, WGM, WGN, VA, VB, SUF)                                                   \
  {"f32_" #BM "x" #BN "_w" #WGM "x" #WGN SUF, KIND_F32, DT_F32, BM, BN, FBK, 64 * WGM * WGN,     \
   2 * (BM * 8 + FBK * BN / 4) * 16, VA, VB, launch_f32<BM, BN, WGM, WGN, VA, VB>}

const KernelEntry kF32[] = {
    G15_F32(128, 128, 2, 2, 1, 1, ""),
    G15_F32(256, 128, 2, 2, 1, 1, ""),
    G15_F32(128, 256, 2, 2, 1, 1, ""),
    G15_F32(256, 256, 2, 2, 1, 1, ""),
    G15_F32(64, 64, 2, 2, 1, 1, ""),
    G15_F32(128, 128, 2, 2, 0, 0, "_scalar"),
    G15_F32(64, 64, 2, 2, 0, 0, "_scalar"),
};

}  // namespace

int f32_entries(const KernelEntry** out) {
  *out = kF32;
  return static_cast<int>(sizeof(kF32) / sizeof(kF32[0]));
}

}  // namespace g15
