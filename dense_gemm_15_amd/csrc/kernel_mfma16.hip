// kernel_mfma16.hip -- bf16 / fp16 GEMM on the gfx950 matrix cores, fp32
// accumulation, fused epilogue.
//
// Structure (the three-level tiling of the DeepGEMM page, section 2.2, and the
// double-buffered K loop of the SGEMM page, section 2.3, re-laid for CDNA4):
//  * a workgroup owns a BM x BN tile of C and walks K in slices of 64;
//  * each slice of A (BM x 64) and of B (64 x BN) is staged in LDS, two slices
//    deep: while the waves multiply slice k out of one LDS buffer, slice k+1 sits
//    in registers on its way in and slice k+2 is being fetched from memory;
//  * each wave owns a (BM/WGM) x (BN/WGN) sub-tile made of 32 x 32 blocks, each
//    block accumulated by v_mfma_f32_32x32x16_{bf16,f16} into 16 fp32 values per
//    lane; accumulators never leave registers until the epilogue
//    (DeepGEMM page, sections 3.1 and 3.3);
//  * inputs stay 16-bit up to the matrix core, products and sums are fp32
//    (DeepGEMM page, section 3.4).
//
// The matrix core wants, per lane, 8 consecutive k of one row of A and 8
// consecutive k of one column of B. A is row-major (k contiguous) and is staged
// as is. B is row-major (n contiguous), so each thread fetches an 8 (k) x 8 (n)
// block, transposes it in registers and stores it n-major, k contiguous.
//
// LDS layout: both tiles are rows of 64 k-values = 128 bytes = 8 chunks of 16
// bytes; chunk c of row r lives at chunk position c ^ (r & 7). Eight lanes that
// read the same chunk index of eight consecutive rows (the operand fetch), or
// eight chunks of one row (the staging store), then hit eight different 16-byte
// bank groups (the padding-versus-alignment trade of the DeepGEMM page, section
// 5.2, solved by a permutation instead of padding so 16-byte accesses stay
// aligned; the SGEMM page, section 6, names this XOR form).
//
// Edges: rows >= M, columns >= N and k >= K are zero-filled on load and masked
// on store (tutorial page, sections 4.2 and 4.3). When a row of A (or of B) is
// not 16-byte aligned the VA (VB) = false variant loads element by element.
#include "kernels.hpp"

namespace g15 {
namespace {

constexpr int BK = 64;  // k per LDS slice: 8 chunks of 8 elements

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

template <typename T>
__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mfma<bf16_t>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma<f16_t>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Tile index -> (tile row, tile col). Workgroups are handed to the 8 XCDs in
// turn, so consecutive ids land on different L2s; remap so each XCD gets a
// contiguous run of tiles, then walk that run in groups of GM tile rows so the
// tiles resident together share A rows and B columns.
__device__ __forceinline__ void tile_coords(int wid, int tiles_m, int tiles_n, int& tm, int& tn) {
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

template <typename T, int BM, int BN, int WGM, int WGN, bool VA, bool VB>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_mfma16_kernel(LaunchArgs a) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int NA = BM * 8 / NT;                 // A chunks per thread per slice
  constexpr int NB = (BN + NT - 1) / NT;          // B 8x8 blocks per thread per slice
  static_assert(BM * 8 % NT == 0, "A staging must divide evenly");
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold a 32x32 block");

  __shared__ u32x4 lds[2][(BM + BN) * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int64_t M = a.M, N = a.N, K = a.K;
  const int tiles_m = static_cast<int>((M + BM - 1) / BM);
  const int tiles_n = static_cast<int>((N + BN - 1) / BN);
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = static_cast<int64_t>(tm) * BM, n0 = static_cast<int64_t>(tn) * BN;
  const int64_t z = blockIdx.y;
  const uint16_t* Ap = static_cast<const uint16_t*>(a.A) + z * a.sA;
  const uint16_t* Bp = static_cast<const uint16_t*>(a.B) + z * a.sB;

  u32x4 ra[NA];
  u32x4 rb[NB][8];

  // ---- global -> registers for slice starting at k0 ----
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int c = tid + i * NT;
      const int row = c >> 3, kc = c & 7;
      const int64_t gm = m0 + row, gk = k0 + kc * 8;
      if constexpr (VA) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (gm < M && gk < K) v = *reinterpret_cast<const u32x4*>(Ap + gm * K + gk);
        ra[i] = v;
      } else {
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t lo = (gm < M && gk + 2 * p < K) ? Ap[gm * K + gk + 2 * p] : 0u;
          const uint32_t hi = (gm < M && gk + 2 * p + 1 < K) ? Ap[gm * K + gk + 2 * p + 1] : 0u;
          w[p] = lo | (hi << 16);
        }
        ra[i] = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int b = tid + i * NT;
      if (NB * NT > BN && b >= BN) break;
      const int kb = b & 7, nb = b >> 3;
      const int64_t gn = n0 + nb * 8;
      if constexpr (VB) {
        // rows k0+kb*8 .. +7, columns gn .. gn+7 ; then transpose 8x8 of 16-bit
        u32x4 v[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int64_t gk = k0 + kb * 8 + r;
          u32x4 t = {0u, 0u, 0u, 0u};
          if (gk < K && gn < N) t = *reinterpret_cast<const u32x4*>(Bp + gk * N + gn);
          v[r] = t;
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          uint32_t w[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t x0 = v[2 * p][c >> 1], x1 = v[2 * p + 1][c >> 1];
            w[p] = (c & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
          }
          rb[i][c] = u32x4{w[0], w[1], w[2], w[3]};
        }
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          uint32_t w[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int64_t gk = k0 + kb * 8 + 2 * p;
            const bool okn = gn + c < N;
            const uint32_t lo = (okn && gk < K) ? Bp[gk * N + gn + c] : 0u;
            const uint32_t hi = (okn && gk + 1 < K) ? Bp[(gk + 1) * N + gn + c] : 0u;
            w[p] = lo | (hi << 16);
          }
          rb[i][c] = u32x4{w[0], w[1], w[2], w[3]};
        }
      }
    }
  };

  // ---- registers -> LDS buffer s ----
  auto stash = [&](int s) {
    u32x4* As = lds[s];
    u32x4* Bs = lds[s] + BM * 8;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int c = tid + i * NT;
      As[swz(c >> 3, c & 7)] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int b = tid + i * NT;
      if (NB * NT > BN && b >= BN) break;
      const int kb = b & 7, nb = b >> 3;
#pragma unroll
      for (int c = 0; c < 8; ++c) Bs[swz(nb * 8 + c, kb)] = rb[i][c];
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = static_cast<int>((K + BK - 1) / BK);
  fetch(0);
  stash(0);
  if (nk > 1) fetch(BK);

  const int lrow = lane & 31, lhalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    if (kt + 1 < nk) {
      stash((kt + 1) & 1);
      if (kt + 2 < nk) fetch(static_cast<int64_t>(kt + 2) * BK);
    }
    const u32x4* As = lds[kt & 1];
    const u32x4* Bs = lds[kt & 1] + BM * 8;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      u32x4 fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[i] = As[swz(wm * WTM + i * 32 + lrow, ks * 2 + lhalf)];
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = Bs[swz(wn * WTN + j * 32 + lrow, ks * 2 + lhalf)];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma<T>(fa[i], fb[j], acc[i][j]);
    }
  }

  // ---- epilogue in registers, then a masked store ----
  // lane holds, for block (i, j), C[row][col] with col = lane % 32 and
  // row = 8 * (r / 4) + 4 * (lane / 32) + r % 4 for its 16 values r.
  const Epi& e = a.epi;
  const int64_t ob = e.out_dtype == DT_F32 ? 4 : 2;
  void* Cp = static_cast<char*>(a.C) + z * a.sC * ob;
  const void* Rp =
      (e.flags & EPI_RESID) ? static_cast<const char*>(e.resid) + z * a.sR * ob : nullptr;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t col = n0 + wn * WTN + j * 32 + lrow;
    const bool okc = col < N;
    const float bn = ((e.flags & EPI_BIAS) && okc) ? e.bias[col] : 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
        if (okc && row < M) {
          const int64_t idx = row * N + col;
          store_out_elem(Cp, e.out_dtype, idx, apply_epi(e, acc[i][j][r], bn, Rp, idx));
        }
      }
    }
  }
}

template <typename T, int BM, int BN, int WGM, int WGN, bool VA, bool VB>
hipError_t launch_mfma16(const LaunchArgs& a, hipStream_t s) {
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(a.batch));
  hipLaunchKernelGGL((gemm_mfma16_kernel<T, BM, BN, WGM, WGN, VA, VB>), grid, dim3(64 * WGM * WGN),
                     0, s, a);
  return hipGetLastError();
}

#define G15_M16(T, TN, BM, BN, WGM, WGN, VA, VB, SUF)                                          \
  {"mfma16_" TN "_" #BM "x" #BN "_w" #WGM "x" #WGN SUF, KIND_MFMA16, T::code, BM, BN, BK,     \
   64 * WGM * WGN, 2 * (BM + BN) * 128, VA, VB, launch_mfma16<T, BM, BN, WGM, WGN, VA, VB>}

#define G15_M16_ALL(T, TN)                                       \
  G15_M16(T, TN, 256, 256, 2, 2, 1, 1, ""),                      \
  G15_M16(T, TN, 256, 128, 2, 2, 1, 1, ""),                      \
  G15_M16(T, TN, 128, 256, 2, 2, 1, 1, ""),                      \
  G15_M16(T, TN, 128, 128, 2, 2, 1, 1, ""),                      \
  G15_M16(T, TN, 128, 64, 2, 2, 1, 1, ""),                       \
  G15_M16(T, TN, 64, 64, 2, 2, 1, 1, ""),                        \
  G15_M16(T, TN, 128, 128, 2, 2, 0, 0, "_scalar"),               \
  G15_M16(T, TN, 64, 64, 2, 2, 0, 0, "_scalar")

const KernelEntry kMfma16[] = {
    G15_M16_ALL(bf16_t, "bf16"),
    G15_M16_ALL(f16_t, "f16"),
};

}  // namespace

int mfma16_entries(const KernelEntry** out) {
  *out = kMfma16;
  return static_cast<int>(sizeof(kMfma16) / sizeof(kMfma16[0]));
}

}  // namespace g15
