// kernel_mfma16_pipe.hip -- the software-pipelined bf16 / fp16 matrix-core GEMM
// for 16-byte aligned rows (the large-shape path).
//
// Same tiling as kernel_mfma16.hip (block tile of C per workgroup, wave
// sub-tiles of 32 x 32 matrix-core blocks, v_mfma_f32_32x32x16 with fp32
// accumulators in registers, B transposed 8 x 8 in registers on its way into an
// n-major LDS tile, XOR-permuted 16-byte chunks), with the memory side re-cut
// so the matrix core never waits on it:
//  * every global access is a buffer load or store through a resource
//    descriptor; an access that falls outside the matrix (row >= M, column >=
//    N, k >= K) gets an offset beyond the descriptor's extent, which the
//    hardware turns into a zero load or a dropped store. The K loop therefore
//    has no branches: edge tiles run the same instruction stream as interior
//    ones (the zero-filled edge of the tutorial page, sections 4.2-4.3, done by
//    the address unit);
//  * one barrier per K slice. Right after it, each wave stores the slice it
//    fetched one iteration earlier into the other LDS buffer and issues the
//    fetch of the slice after that into registers (the prefetch of the SGEMM
//    page, section 2.3, one slice deeper);
//  * operand fragments for k-step s+1 are read from LDS while the matrix core
//    works on k-step s, and the instruction order inside the iteration is laid
//    out explicitly (matrix-core ops interleaved with LDS reads, LDS writes
//    and global loads) so each wave keeps its matrix core fed.
#include "kernels.hpp"

namespace g15 {
namespace {

constexpr uint32_t OOB = 0x80000000u;  // offset past every descriptor extent used here

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

template <typename T>
__device__ __forceinline__ f32x16 mfma16(u32x4 a, u32x4 b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mfma16<bf16_t>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma16<f16_t>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Instruction-order plan for one K slice: N matrix-core ops, each followed by
// its share of LDS reads, LDS writes and global loads (spread evenly).
template <int I, int N, int NDR, int NDW, int NVM>
__device__ __forceinline__ void sched_slice() {
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int dr = (I + 1) * NDR / N - I * NDR / N;
    constexpr int dw = (I + 1) * NDW / N - I * NDW / N;
    constexpr int vm = (I + 1) * NVM / N - I * NVM / N;
    if constexpr (dr > 0) __builtin_amdgcn_sched_group_barrier(0x100, dr, 0);
    if constexpr (dw > 0) __builtin_amdgcn_sched_group_barrier(0x200, dw, 0);
    if constexpr (vm > 0) __builtin_amdgcn_sched_group_barrier(0x020, vm, 0);
    sched_slice<I + 1, N, NDR, NDW, NVM>();
  }
}

__device__ __forceinline__ void tile_xy(int wid, int tiles_m, int tiles_n, int& tm, int& tn) {
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

template <typename T, int BM, int BN, int BK, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_m16p_kernel(LaunchArgs a) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int CH = BK / 8;             // 16-byte chunks per LDS row
  constexpr int RPL = 8 / CH;            // LDS rows per 128-byte line
  constexpr int KS = BK / 16;            // matrix-core k-steps per slice
  constexpr int NA = BM * CH / NT;       // A chunks per thread
  constexpr int KB = BK / 8;             // 8-row groups of B per slice
  constexpr int NBB = KB * (BN / 8);     // 8x8 blocks of B per slice
  constexpr int NB = (NBB + NT - 1) / NT;
  static_assert(BM * CH % NT == 0, "A staging must divide evenly");
  static_assert(CH == 4 || CH == 8, "BK must be 32 or 64");
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold a 32x32 block");

  __shared__ u32x4 lds[2][(BM + BN) * CH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int M = static_cast<int>(a.M), N = static_cast<int>(a.N), K = static_cast<int>(a.K);
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_xy(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t z = blockIdx.y;
  const auto rA = rsrc(static_cast<const uint16_t*>(a.A) + z * a.sA,
                       static_cast<uint32_t>(static_cast<int64_t>(M) * K * 2));
  const auto rB = rsrc(static_cast<const uint16_t*>(a.B) + z * a.sB,
                       static_cast<uint32_t>(static_cast<int64_t>(K) * N * 2));

  auto swz = [](int row, int c) { return row * CH + (c ^ ((row / RPL) & (CH - 1))); };

  u32x4 ra[NA];
  u32x4 rb[NB][8];

  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int c = tid + i * NT;
      const int gm = m0 + c / CH, gk = k0 + (c % CH) * 8;
      const uint32_t off = (gm < M && gk < K) ? static_cast<uint32_t>(gm * K + gk) * 2u : OOB;
      ra[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, off, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int b = tid + i * NT;
      const bool act = (NB * NT == NBB) || b < NBB;
      const int kb = b % KB, nb = b / KB;
      const int gn = n0 + nb * 8;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int gk = k0 + kb * 8 + r;
        const uint32_t off =
            (act && gk < K && gn < N) ? static_cast<uint32_t>(gk * N + gn) * 2u : OOB;
        rb[i][r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rB, off, 0, 0));
      }
    }
  };

  auto stash = [&](int s) {
    u32x4* As = lds[s];
    u32x4* Bs = lds[s] + BM * CH;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int c = tid + i * NT;
      As[swz(c / CH, c % CH)] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int b = tid + i * NT;
      if (NB * NT != NBB && b >= NBB) break;
      const int kb = b % KB, nb = b / KB;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t x0 = rb[i][2 * p][c >> 1], x1 = rb[i][2 * p + 1][c >> 1];
          w[p] = (c & 1) ? __builtin_amdgcn_perm(x1, x0, 0x07060302u)
                         : __builtin_amdgcn_perm(x1, x0, 0x05040100u);
        }
        Bs[swz(nb * 8 + c, kb)] = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (K + BK - 1) / BK;
  fetch(0);
  stash(0);
  fetch(BK);

  const int lrow = lane & 31, lhalf = lane >> 5;
  int arow[FM], brow[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) arow[i] = wm * WTM + i * 32 + lrow;
#pragma unroll
  for (int j = 0; j < FN; ++j) brow[j] = BM + wn * WTN + j * 32 + lrow;

  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    const u32x4* L = lds[kt & 1];
    u32x4 fa[2][FM], fb[2][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[0][i] = L[swz(arow[i], lhalf)];
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[0][j] = L[swz(brow[j], lhalf)];
    // next slice: registers -> other LDS buffer, then the one after -> registers.
    // Past the end both are harmless: the loads read zeros (out-of-range
    // offsets) and the buffer written is never read again.
    stash((kt + 1) & 1);
    fetch((kt + 2) * BK);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s + 1 < KS) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[(s + 1) & 1][i] = L[swz(arow[i], 2 * (s + 1) + lhalf)];
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[(s + 1) & 1][j] = L[swz(brow[j], 2 * (s + 1) + lhalf)];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma16<T>(fa[s & 1][i], fb[s & 1][j], acc[i][j]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
    sched_slice<0, FM * FN * KS, (FM + FN) * (KS - 1), NA + 8 * NB, NA + 8 * NB>();
  }

  // ---- epilogue: lane holds C[row][col] for block (i, j), col = lane % 32,
  // row = 8 (r / 4) + 4 (lane / 32) + r % 4. Out-of-range lanes store to an
  // out-of-range offset (dropped).
  const Epi& e = a.epi;
  const int ob = e.out_dtype == DT_F32 ? 4 : 2;
  const auto rC = rsrc(static_cast<char*>(a.C) + z * a.sC * ob,
                       static_cast<uint32_t>(static_cast<int64_t>(M) * N * ob));
  const bool has_r = (e.flags & EPI_RESID) != 0;
  const auto rR = rsrc(has_r ? static_cast<const char*>(e.resid) + z * a.sR * ob
                             : static_cast<const char*>(a.C),
                       static_cast<uint32_t>(static_cast<int64_t>(M) * N * ob));
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int col = n0 + wn * WTN + j * 32 + lrow;
    const bool okc = col < N;
    const float bn = ((e.flags & EPI_BIAS) && okc) ? e.bias[col] : 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
        const uint32_t idx = static_cast<uint32_t>(row * N + col);
        const uint32_t off = (okc && row < M) ? idx * ob : OOB;
        float v = acc[i][j][r];
        if (e.flags & EPI_SCALE) v *= e.scale;
        if (e.flags & EPI_BIAS) v += bn;
        if (e.flags & EPI_GELU) v = gelu(v);
        if (has_r) {
          if (ob == 4) {
            v += __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rR, off, 0, 0));
          } else {
            const uint16_t h = __builtin_amdgcn_raw_buffer_load_b16(rR, off, 0, 0);
            v += e.out_dtype == DT_BF16 ? widen(bf16_t{}, h) : widen(f16_t{}, h);
          }
        }
        if (ob == 4)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rC, off, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b16(
              e.out_dtype == DT_BF16 ? narrow_bf16(v) : narrow_f16(v), rC, off, 0, 0);
      }
    }
  }
}

template <typename T, int BM, int BN, int BK, int WGM, int WGN>
hipError_t launch_m16p(const LaunchArgs& a, hipStream_t s) {
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(a.batch));
  hipLaunchKernelGGL((gemm_m16p_kernel<T, BM, BN, BK, WGM, WGN>), grid, dim3(64 * WGM * WGN), 0, s,
                     a);
  return hipGetLastError();
}

#define G15_M16P(T, TN, BM, BN, BK, WGM, WGN)                                                    \
  {"m16p_" TN "_" #BM "x" #BN "x" #BK "_w" #WGM "x" #WGN, KIND_MFMA16, T::code, BM, BN, BK,       \
   64 * WGM * WGN, 2 * (BM + BN) * BK * 2, 1, 1, launch_m16p<T, BM, BN, BK, WGM, WGN>, 1}

#define G15_M16P_ALL(T, TN)                 \
  G15_M16P(T, TN, 256, 256, 64, 2, 2),      \
  G15_M16P(T, TN, 256, 256, 64, 2, 4),      \
  G15_M16P(T, TN, 256, 256, 32, 2, 2),      \
  G15_M16P(T, TN, 256, 128, 64, 2, 2),      \
  G15_M16P(T, TN, 256, 128, 32, 2, 2),      \
  G15_M16P(T, TN, 128, 128, 64, 2, 2),      \
  G15_M16P(T, TN, 128, 64, 64, 2, 2),       \
  G15_M16P(T, TN, 64, 64, 64, 2, 2)

const KernelEntry kM16P[] = {
    G15_M16P_ALL(bf16_t, "bf16"),
    G15_M16P_ALL(f16_t, "f16"),
};

}  // namespace

int mfma16_pipe_entries(const KernelEntry** out) {
  *out = kM16P;
  return static_cast<int>(sizeof(kM16P) / sizeof(kM16P[0]));
}

}  // namespace g15
