// kernel_f32_dlds.hip -- fp32 SGEMM on v_mfma_f32_32x32x2_f32 with both operands
// streamed global -> LDS by buffer_load ... lds into a ring of slices.
//
// The wave-level output tiling of the SGEMM page (sections 2.1 and 3.2: each
// warp owns a sub-tile, accumulators stay in registers, operands are reused
// from registers) on the gfx950 matrix core, with the prefetch of its section
// 2.3 made a ring of SA slices deep. For fp32 neither operand needs a transpose
// on the way in:
//  * one 32x32x2 step sums two k values, lane half h supplying the second. In
//    each group of 8 k the four steps pair k = 8g + s (half 0) with 8g + 4 + s
//    (half 1), so a lane needs k = 8g + 4h .. 8g + 4h + 3 of its A row: one
//    16-byte LDS read feeds four steps and A stays row-major;
//  * column j of matrix-core block f of a wave maps to C column j * FN + f of
//    the wave's sub-tile, so a lane reads its FN columns of one B row as one
//    contiguous LDS read and later stores FN contiguous results;
//  * A rows of an LDS slice are 64 bytes (16 k); chunk c of row r sits at
//    c ^ ((r >> 2) & 3), which keeps a fragment read (32 consecutive rows, one
//    chunk) free of bank conflicts on gfx950's LDS (with (r >> 1) & 3 every read
//    took two passes: 8.5 against 4.4 cycles measured).
// Every global access goes through a buffer descriptor: rows past M, columns
// past N and k past K read zeros, stores past the edge are dropped. One barrier
// per slice; fragments of the next k-group are read during the current one.
#include <type_traits>

#include "kernels.hpp"

namespace g15 {
namespace {

constexpr uint32_t FOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t frsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

typedef __attribute__((address_space(3))) void flds_void;

template <int n>
__device__ __forceinline__ void fwait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void flds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void ftile(int wid, int tiles_m, int tiles_n, int& tm, int& tn) {
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
struct FV;
template <>
struct FV<2> {
  typedef float type __attribute__((ext_vector_type(2)));
};
template <>
struct FV<4> {
  typedef float type __attribute__((ext_vector_type(4)));
};

template <int BM, int BN, int WGM, int WGN, int SA, bool BNK>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_f32d_kernel(LaunchArgs a) {
  constexpr int BK = 16;                    // k per slice
  constexpr int NW = WGM * WGN, NT = 64 * NW;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_CH = BM * 4;              // 16-byte chunks of an A slice (64 B rows)
  constexpr int B_CH = BK * BN / 4;         // 16-byte chunks of a B slice
  constexpr int AI = A_CH / 64 / NW;        // direct A loads per wave per slice
  constexpr int BI = B_CH / 64 / NW;        // direct B loads per wave per slice
  constexpr int STAGE = A_CH + B_CH;
  static_assert(A_CH % (64 * NW) == 0 && B_CH % (64 * NW) == 0 && AI >= 1 && BI >= 1,
                "slices must split evenly into 1 KB loads over the waves");
  static_assert(FN == 2 || FN == 4, "FN must be 2 or 4");
  static_assert(SA >= 2, "ring of two slices at least");
  typedef typename FV<FN>::type bvec;

  __shared__ f32x4 lds[SA * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: LDS slot addresses in SGPRs
  const int wm = wave / WGN, wn = wave % WGN;
  const int M = static_cast<int>(a.M), N = static_cast<int>(a.N), K = static_cast<int>(a.K);
  // row strides of A and B: K and N, or those rounded up to 4 (operands copied into
  // zero-padded rows)
  const int LDA = static_cast<int>(a.lda), LDB = static_cast<int>(a.ldb);
  const int LDC = static_cast<int>(a.ldc);  // C (and residual) row stride, N unless a block of C
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  ftile(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t z = blockIdx.y;
  const float* Abase = static_cast<const float*>(a.A) + z * a.sA;
  const float* Bbase = static_cast<const float*>(a.B) + z * a.sB;

  // A: instruction i of this wave fills 16 rows r0 .. r0+15 (lane l -> slot
  // r0*4 + l, i.e. row r0 + l/4, position l%4). Position p of row r holds chunk
  // p ^ ((r >> 2) & 3); r0 is a multiple of 16, so that is (l%4) ^ ((l/16) & 3).
  const int a_row = lane >> 2, a_chunk = (lane & 3) ^ ((lane >> 4) & 3);
  uint32_t a_voff[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int gm = m0 + (wave * AI + i) * 16 + a_row;
    a_voff[i] = gm < M ? static_cast<uint32_t>(gm * LDA + a_chunk * 4) * 4u : FOOB;
  }
  // B: instruction i of this wave fills 64 chunks of the slice: row q / (BN/4),
  // chunk q % (BN/4), for q = (wave*BI + i)*64 + lane. B given transposed (Bt
  // [N x K], BNK): the slice is BN rows (n) of 16 k laid out like A's, filled like A.
  uint32_t b_voff[BI];
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    if constexpr (BNK) {
      const int gn = n0 + (wave * BI + i) * 16 + a_row;
      b_voff[i] = gn < N ? static_cast<uint32_t>(gn * LDB + a_chunk * 4) * 4u : FOOB;
    } else {
      const int q = (wave * BI + i) * 64 + lane;
      const int r = q / (BN / 4), gn = n0 + (q % (BN / 4)) * 4;
      b_voff[i] = gn < N ? static_cast<uint32_t>(r * LDB + gn) * 4u : FOOB;
    }
  }
  // A lane whose load falls outside the matrix leaves its LDS slot untouched,
  // so it stores zeros there itself (only k past K matters: stale rows past M or
  // columns past N only reach outputs that are never stored).
  const int b_row = ((wave * BI) * 64 + lane) / (BN / 4);  // row of instruction 0; +64/(BN/4) per i
  // TAIL: the slice may reach past K (masked chunks, zeroed slots); otherwise the
  // issue is branch-free.
  auto issue = [&](int k0, int stage, auto TailC) {
    constexpr bool TAIL = decltype(TailC)::value;
    const int64_t aleft = static_cast<int64_t>(M) * LDA - k0;
    const auto ra = frsrc(Abase + k0, static_cast<uint32_t>(aleft > 0 ? aleft * 4 : 0));
    const bool kin = !TAIL || k0 + a_chunk * 4 < K;  // k past K inside a row would read the next row
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const uint32_t off = kin ? a_voff[i] : FOOB;
      f32x4* slot = lds + stage * STAGE + (wave * AI + i) * 64;
      if (TAIL && !kin) slot[lane] = f32x4{0.f, 0.f, 0.f, 0.f};
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (flds_void*)slot, 16, off, 0, 0, 0);
    }
    if constexpr (BNK) {
      const int64_t bleft = static_cast<int64_t>(N) * LDB - k0;
      const auto rb = frsrc(Bbase + k0, static_cast<uint32_t>(bleft > 0 ? bleft * 4 : 0));
#pragma unroll
      for (int i = 0; i < BI; ++i) {
        const uint32_t off = kin ? b_voff[i] : FOOB;
        f32x4* slot = lds + stage * STAGE + A_CH + (wave * BI + i) * 64;
        if (TAIL && !kin) slot[lane] = f32x4{0.f, 0.f, 0.f, 0.f};
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (flds_void*)slot, 16, off, 0, 0, 0);
      }
      return;
    }
    const int64_t bleft = static_cast<int64_t>(K - k0) * LDB;
    const auto rb = frsrc(Bbase + static_cast<int64_t>(k0) * LDB,
                          static_cast<uint32_t>(bleft > 0 ? bleft * 4 : 0));
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const uint32_t off = b_voff[i];
      f32x4* slot = lds + stage * STAGE + A_CH + (wave * BI + i) * 64;
      if (TAIL && k0 + b_row + i * (64 / (BN / 4)) >= K) slot[lane] = f32x4{0.f, 0.f, 0.f, 0.f};
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (flds_void*)slot, 16, off, 0, 0, 0);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int lrow = lane & 31, lhalf = lane >> 5;
  // A fragment of k-group g, block i: row wm*WTM + 32 i + lrow, chunk 2g + lhalf
  const int a_fbase = (wm * WTM + lrow) * 4;
  const int a_fperm = (lrow >> 2) & 3;
  auto afrag = [&](const f32x4* L, int g, f32x4 (&fa)[FM]) {
    const int c = (2 * g + lhalf) ^ a_fperm;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = L[a_fbase + i * 128 + c];
  };
  // B fragment of step s of group g: row 8g + 4 lhalf + s, FN floats at wn*WTN + lrow*FN
  auto bfrag = [&](const f32x4* L, int g, int s) {
    const float* Bs = reinterpret_cast<const float*>(L + A_CH);
    return *reinterpret_cast<const bvec*>(Bs + (8 * g + 4 * lhalf + s) * BN + wn * WTN + lrow * FN);
  };
  // BNK: B fragment of k-group g, block j: Bt row wn*WTN + 32 j + lrow (C column
  // 32 j + lrow of the wave's sub-tile), chunk 2g + lhalf: four k, one per step
  const int b_fbase = (wn * WTN + lrow) * 4;
  auto bfrag_nk = [&](const f32x4* L, int g, f32x4 (&fb)[FN]) {
    const int c = (2 * g + lhalf) ^ a_fperm;
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = L[A_CH + b_fbase + j * 128 + c];
  };

  const int nk = (K + BK - 1) / BK;
#pragma unroll
  for (int s = 0; s < SA - 1; ++s) issue(s * BK, s, std::true_type{});
  constexpr int PER = AI + BI;
  fwait_vm<PER * (SA - 2)>();  // slice 0 has landed
  flds_barrier();

  int cur = 0;
  // one K slice; TailC: whether the slice issued here (kt + SA - 1) may reach past K
  auto slice = [&](int kt, auto TailC) {
    const f32x4* L = lds + cur * STAGE;
    const int far = cur == 0 ? SA - 1 : cur - 1;  // slot of slice kt-1, refilled with kt+SA-1
    issue((kt + SA - 1) * BK, far, TailC);
    f32x4 fa0[FM], fa1[FM];
    afrag(L, 0, fa0);
    afrag(L, 1, fa1);
#pragma unroll
    for (int g = 0; g < BK / 8; ++g) {
      f32x4 fbk[BNK ? FN : 1];
      if constexpr (BNK) bfrag_nk(L, g, fbk);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bvec fb;
        if constexpr (BNK) {
#pragma unroll
          for (int j = 0; j < FN; ++j) fb[j] = fbk[j][s];
        } else {
          fb = bfrag(L, g, s);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(g == 0 ? fa0[i][s] : fa1[i][s], fb[j],
                                                             acc[i][j], 0, 0, 0);
      }
    }
    // slice kt+1 landed (everything but the last SA-2 slices' loads) and every
    // wave is done with slice kt-1's slot before anyone refills it
    fwait_vm<PER * (SA - 2)>();
    flds_barrier();
    cur = cur + 1 == SA ? 0 : cur + 1;
  };
  int kt = 0;
  for (; kt < nk && (kt + SA) * BK <= K; ++kt) slice(kt, std::false_type{});
  for (; kt < nk; ++kt) slice(kt, std::true_type{});

  // lane holds, for block (i, j), C[row][col] with row = 8 (r / 4) + 4 (lane / 32)
  // + r % 4 and col = (lane % 32) * FN + j of the wave's sub-tile (BNK: 32 j +
  // lane % 32).
  const Epi& e = a.epi;
  const int ob = e.out_dtype == DT_F32 ? 4 : 2;
  const auto rC = frsrc(static_cast<char*>(a.C) + z * a.sC * ob,
                        static_cast<uint32_t>(static_cast<int64_t>(M) * LDC * ob));
  const bool has_r = (e.flags & EPI_RESID) != 0;
  const auto rR = frsrc(has_r ? static_cast<const char*>(e.resid) + z * a.sR * ob
                              : static_cast<const char*>(a.C),
                        static_cast<uint32_t>(static_cast<int64_t>(M) * LDC * ob));
  const int colbase = n0 + wn * WTN + lrow * FN;
  auto col_of = [&](int j) { return BNK ? n0 + wn * WTN + 32 * j + lrow : colbase + j; };
  float bn[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j)
    bn[j] = ((e.flags & EPI_BIAS) && col_of(j) < N) ? e.bias[col_of(j)] : 0.f;
  const bool plain = e.flags == 0 && ob == 4;
  // a lane's FN consecutive columns leave as one vector store (rows whose start is not
  // FN-aligned, C's row stride not a multiple of FN: a vector store to a 4-byte aligned
  // address, which the memory system serves like an aligned one)
  const bool vec_ok = !BNK && (N % FN) == 0;
  const bool vec_aligned = (LDC % FN) == 0;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
      if (plain && vec_ok) {
        // plain vector store (a buffer store of a register pair built from
        // accumulators miscompiled here: every row received the first row's data)
        if (row < M && colbase < N) {
          bvec v;
#pragma unroll
          for (int j = 0; j < FN; ++j) v[j] = acc[i][j][r];
          float* dst = static_cast<float*>(a.C) + z * a.sC + static_cast<int64_t>(row) * LDC + colbase;
          if (vec_aligned)
            *reinterpret_cast<bvec*>(dst) = v;
          else
            __builtin_memcpy(dst, &v, sizeof(v));
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = col_of(j);
          const uint32_t off =
              (row < M && col < N) ? static_cast<uint32_t>(row * LDC + col) * ob : FOOB;
          float v = acc[i][j][r];
          if (e.flags & EPI_SCALE) v *= e.scale;
          if (e.flags & EPI_BIAS) v += bn[j];
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
}

template <int BM, int BN, int WGM, int WGN, int SA, bool BNK>
hipError_t launch_f32d(const LaunchArgs& a, hipStream_t s) {
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(a.batch));
  hipLaunchKernelGGL((gemm_f32d_kernel<BM, BN, WGM, WGN, SA, BNK>), grid, dim3(64 * WGM * WGN), 0,
                     s, a);
  return hipGetLastError();
}

// SFX "" for B [K x N], "_nk" for B given transposed (Bt [N x K])
#define G15_F32D(BM, BN, WGM, WGN, SA, BNK, SFX)                                               \
  {"f32d_" #BM "x" #BN "x16_w" #WGM "x" #WGN "_a" #SA SFX, KIND_F32, DT_F32, BM, BN, 16,       \
   64 * WGM * WGN, SA * (BM * 64 + 16 * BN * 4), 1, 1, launch_f32d<BM, BN, WGM, WGN, SA, BNK>, \
   1, BNK ? 1 : 0}
#define G15_F32D_ALL(BNK, SFX)                                                               \
  G15_F32D(128, 128, 2, 2, 4, BNK, SFX), G15_F32D(128, 128, 2, 2, 3, BNK, SFX),               \
      G15_F32D(256, 128, 4, 2, 4, BNK, SFX), G15_F32D(128, 256, 2, 4, 4, BNK, SFX),           \
      G15_F32D(256, 256, 4, 2, 3, BNK, SFX)

const KernelEntry kF32D[] = {G15_F32D_ALL(false, ""), G15_F32D_ALL(true, "_nk")};

}  // namespace

int f32_dlds_entries(const KernelEntry** out) {
  *out = kF32D;
  return static_cast<int>(sizeof(kF32D) / sizeof(kF32D[0]));
}

}  // namespace g15
