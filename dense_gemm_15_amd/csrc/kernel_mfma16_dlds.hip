// kernel_mfma16_dlds.hip -- bf16 / fp16 matrix-core GEMM with A streamed straight
// into LDS and B prefetched two slices ahead through registers.
//
// Tiling as in kernel_mfma16.hip: a workgroup owns a BM x BN tile of C, waves
// own (BM/WGM) x (BN/WGN) sub-tiles of 32 x 32 blocks accumulated by
// v_mfma_f32_32x32x16 into fp32 registers, K walked in 64-wide slices
// (DeepGEMM page, sections 2.2 and 3.1). What changes is how far ahead the
// memory side runs (the prefetch of the SGEMM page, section 2.3, made deep
// enough for this chip's cache-miss latency):
//  * A slices go global -> LDS with buffer_load ... lds (no registers, no LDS
//    store instructions) into a ring of SA LDS buffers, issued SA-1 slices
//    ahead of use;
//  * B slices must be transposed (the matrix core wants k contiguous per lane,
//    B is n contiguous), so they land in registers one or two slices ahead (one
//    or two register sets), are transposed in registers per thread block of
//    4 x 8 or 8 x 8 (k x n) and stored into one of two n-major LDS buffers;
//  * a single barrier per slice; the wait before it only covers the loads
//    issued two slices earlier, so two slices of loads stay in flight;
//  * operand fragments of k-step s+1 are read while the matrix core runs k-step
//    s, and the instruction order is laid out explicitly.
// Chunks of 16 bytes in every LDS row (64 k values) are XOR-permuted by the row
// index so fragment reads and staging writes spread over all banks. Rows past
// M, columns past N and k past K read as zeros (buffer loads beyond the
// descriptor extent) and stores past the edge are dropped.
#include "m16_common.hpp"

namespace g15 {
namespace {


template <typename T, int BM, int BN, int WGM, int WGN, int SA, int KR, int NSB>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_m16d_kernel(LaunchArgs a) {
  constexpr int BK = 64;
  constexpr int NW = WGM * WGN;
  constexpr int NT = 64 * NW;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int KS = BK / 16;
  constexpr int AI = BM / 8 / NW;   // direct A loads per wave per slice (8 rows each)
  constexpr int NBB = (BK / KR) * (BN / 8);  // KR x 8 blocks of B per slice
  constexpr int NB = NBB / NT;               // per thread
  constexpr int A_STAGE = BM * 8;    // 16-byte chunks per A buffer
  constexpr int B_STAGE = BN * 8;
  static_assert(BM % (8 * NW) == 0 && AI >= 1, "A rows must split evenly over the waves");
  static_assert(NBB % NT == 0 && NB >= 1, "B blocks must split evenly over the threads");
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold a 32x32 block");
  static_assert(SA >= 2, "A ring needs two buffers at least");
  static_assert(NSB == 1 || NSB == 2, "one or two B register sets");
  static_assert(KR == 8 || (KR == 4 && NBB == NT), "B staging: 8x8 blocks, or one 4x8 block per thread");
  static_assert(BK / 16 == 4, "the K loop below is written for four k-steps per slice");

  __shared__ u32x4 lds[SA * A_STAGE + 2 * B_STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index as a scalar: LDS slot addresses derived from it stay in SGPRs
  // (the direct-to-LDS loads take their LDS address in M0)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int M = static_cast<int>(a.M), N = static_cast<int>(a.N), K = static_cast<int>(a.K);
  const int LDA = static_cast<int>(a.lda), LDB = static_cast<int>(a.ldb),
            LDC = static_cast<int>(a.ldc);
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  int64_t z;
  batch_tile_of(tiles_m, tiles_n, tm, tn, z);
  const int m0 = tm * BM, n0 = tn * BN;

  // 16-byte chunk c of LDS row `row` (A and B alike) sits at c ^ (row & 7) ^
  // ((row >> 3) & 3). A fragment read (32 consecutive rows, one chunk) is then free
  // of bank conflicts on gfx950's LDS; row & 7 alone leaves rows 8 apart on the same
  // banks and halves the read rate (measured: 8.4 against 4.4 cycles per read). The
  // permutation does not change when the row moves by a multiple of 32, so all
  // fragments of one k-step share one per-lane chunk offset.
  auto swzb = [](int row, int c) { return row * 8 + (c ^ (row & 7) ^ ((row >> 3) & 3)); };

  // A: instruction i of this wave fills LDS rows r0 .. r0+7 (1 KB, lane l -> slot
  // r0*8 + l), r0 = 8 (wave AI + i). Slot (row, p) holds logical chunk
  // p ^ (row & 7) ^ ((row >> 3) & 3) (as for B), so lane l fetches chunk
  // (l & 7) ^ (l >> 3) ^ ((r0 >> 3) & 3) of row r0 + (l >> 3).
  const int a_lrow = lane >> 3;
  int a_chk[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) a_chk[i] = (lane & 7) ^ (lane >> 3) ^ ((wave * AI + i) & 3);
  // Per-thread byte offsets are fixed for the whole K loop; each slice only moves
  // the descriptor base along K (scalar work). A row past M gets an offset past
  // every extent; B rows past K fall beyond the shrinking extent on their own.
  const uint16_t* Abase = static_cast<const uint16_t*>(a.A) + z * a.sA;
  const uint16_t* Bbase = static_cast<const uint16_t*>(a.B) + z * a.sB;
  uint32_t a_voff[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int gm = m0 + (wave * AI + i) * 8 + a_lrow;
    a_voff[i] = gm < M ? static_cast<uint32_t>(gm * LDA + a_chk[i] * 8) * 2u : OOB;
  }
  // TAIL: the slice may reach past K (chunks past K are masked and their slots
  // zeroed); otherwise every chunk is inside K and the issue is branch-free.
  auto issue_a = [&](int k0, int stage, auto TailC) {
    constexpr bool TAIL = decltype(TailC)::value;
    const int64_t left = static_cast<int64_t>(M) * LDA - k0;
    const auto r = rsrc(Abase + k0, static_cast<uint32_t>(left > 0 ? left * 2 : 0));
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const bool kin = !TAIL || k0 + a_chk[i] * 8 < K;  // k past K inside a row would read the next row
      const int r0 = (wave * AI + i) * 8;
      const uint32_t off = kin ? a_voff[i] : OOB;
      u32x4* slot = lds + stage * A_STAGE + r0 * 8;
      // an out-of-range load leaves its LDS slot untouched: zero it here so the
      // K tail multiplies zeros, never stale or uninitialised LDS contents
      if (TAIL && !kin) slot[lane] = u32x4{0u, 0u, 0u, 0u};
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)slot, 16, off, 0, 0, 0);
    }
  };

  // B: thread block b covers KR rows (k) x 8 columns (n) of the slice. KR = 8:
  // (kb, nb) = (b & 7, b >> 3). KR = 4 (one block per thread): the bits of b, from
  // the lowest, give nb bits 0-1, kq bit 0, kq bit 3, the other nb bits, kq bits
  // 1-2 (kq = k / 4). The transposed store of column c writes row 8 nb + c at chunk
  // kq / 2 (permuted by nb & 3), half kq & 1; gfx950's LDS takes 16 lanes of an
  // 8-byte store per pass over 32 banks, and these 16 lanes then hit 16 different
  // (chunk, half) slots: no bank conflicts (nb & 7 on the low lanes had 2-way
  // conflicts in every store). Each load still reads 256 contiguous bytes of a row
  // with 16 lanes. The block is transposed in registers and stored n-major.
  u32x4 rb[NSB][NB][KR];
  constexpr int NBH = BN == 256 ? 3 : BN == 128 ? 2 : 1;  // nb bits above the lowest two
  static_assert(KR == 8 || BN / 32 == (1 << NBH), "KR = 4 mapping: BN of 64, 128 or 256");
  auto b_coords = [&](int b, int& kr0, int& nb) {
    if constexpr (KR == 8) {
      kr0 = (b & 7) * 8;
      nb = b >> 3;
    } else {
      const int kq = ((b >> 2) & 1) | (((b >> 3) & 1) << 3) | (((b >> (4 + NBH)) & 3) << 1);
      kr0 = kq * 4;
      nb = (b & 3) | (((b >> 4) & ((1 << NBH) - 1)) << 2);
    }
  };
  uint32_t b_voff[NB][KR];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    int kr0, nb;
    b_coords(tid + i * NT, kr0, nb);
    const int gn = n0 + nb * 8;
#pragma unroll
    for (int r = 0; r < KR; ++r)
      b_voff[i][r] = gn < N ? static_cast<uint32_t>((kr0 + r) * LDB + gn) * 2u : OOB;
  }
  auto issue_b = [&](int k0, int set) {
    const int64_t left = static_cast<int64_t>(K - k0) * LDB;
    const auto r = rsrc(Bbase + static_cast<int64_t>(k0) * LDB,
                        static_cast<uint32_t>(left > 0 ? left * 2 : 0));
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int q = 0; q < KR; ++q)
        rb[set][i][q] =
            __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, b_voff[i][q], 0, 0));
  };
  auto stash_b = [&](int set, int stage) {
    u32x4* Bs = lds + SA * A_STAGE + stage * B_STAGE;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      int kr0, nb;
      b_coords(tid + i * NT, kr0, nb);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        uint32_t w[KR / 2];
#pragma unroll
        for (int p = 0; p < KR / 2; ++p) {
          const uint32_t x0 = rb[set][i][2 * p][c >> 1], x1 = rb[set][i][2 * p + 1][c >> 1];
          w[p] = (c & 1) ? __builtin_amdgcn_perm(x1, x0, 0x07060302u)
                         : __builtin_amdgcn_perm(x1, x0, 0x05040100u);
        }
        const int row = nb * 8 + c;
        if constexpr (KR == 8) {
          Bs[swzb(row, kr0 / 8)] = u32x4{w[0], w[1], w[2], w[3]};
        } else {
          typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
          u32x2* half = reinterpret_cast<u32x2*>(Bs + swzb(row, kr0 / 8)) + ((kr0 / 4) & 1);
          *half = u32x2{w[0], w[1]};
        }
      }
    }
  };

  // With four waves, no clearing: k-step 0 of slice 0 takes a zero accumulator
  // operand (an inline constant), which saves one register write per accumulator
  // element (measured 3-5% at 512^3 and 1024^3). With eight waves (256 registers,
  // no accumulation registers) the separate first slice makes the compiler spill
  // more (measured 2% slower at 8192^3): those clear the accumulators up front.
  constexpr bool PEEL = NW <= 4;
  f32x16 acc[FM][FN];
  if constexpr (!PEEL) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }

  const int nk = (K + BK - 1) / BK;
  const int lrow = lane & 31, lhalf = lane >> 5;

  // fragment rows: A row wm*WTM + 32 i + lrow, B row wn*WTN + 32 j + lrow
  const int a_base = (wm * WTM + lrow) * 8, b_base = (wn * WTN + lrow) * 8;
  const int a_perm = (lrow & 7) ^ ((lrow >> 3) & 3);
  const int b_perm = (lrow & 7) ^ (((wn * WTN + lrow) >> 3) & 3);
  auto frags = [&](const u32x4* LA, const u32x4* LB, int s, u32x4 (&fa)[FM], u32x4 (&fb)[FN]) {
    const int ca = (2 * s + lhalf) ^ a_perm, cb = (2 * s + lhalf) ^ b_perm;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = LA[a_base + i * 256 + ca];
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = LB[b_base + j * 256 + cb];
  };
  // matrix-core ops of one k-step on rows [I0, I1) of the wave's blocks; ZERO: the
  // first k-step (accumulators start from zero)
  auto mmas = [&](auto ZeroC, const u32x4 (&fa)[FM], const u32x4 (&fb)[FN], int i0, int i1) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i < i0 || i >= i1) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (decltype(ZeroC)::value)
          acc[i][j] = mma<T>(fa[i], fb[j], f32x16{});
        else
          acc[i][j] = mma<T>(fa[i], fb[j], acc[i][j]);
      }
    }
  };
  const std::false_type acc_in{};

  // Prologue: A slices 0 .. SA-2 into the ring, B slices 0, 1 into registers,
  // slice 0 of B into LDS, slice 2 of B into the freed registers, then the
  // step-0 fragments of slice 0.
#pragma unroll
  for (int s = 0; s < SA - 1; ++s) issue_a(s * BK, s, std::true_type{});
  if constexpr (NSB == 2) {
    issue_b(0, 0);
    issue_b(BK, 1);
    stash_b(0, 0);
    issue_b(2 * BK, 0);
  } else {
    issue_b(0, 0);
    stash_b(0, 0);
    issue_b(BK, 0);
  }
  wait_vm<KR * NB>();  // all but the last B slice: A(0) .. A(SA-2) have landed
  lds_barrier();
  u32x4 f0a[FM], f0b[FN], f1a[FM], f1b[FN];
  frags(lds, lds + SA * A_STAGE, 0, f0a, f0b);

  // loads issued per slice, per thread: AI (A, direct) + KR NB (B)
  constexpr int PER_SLICE = AI + KR * NB;
  constexpr int HALF = FM / 2;
  int cur = 0;  // ring slot of A(kt)
  // One K slice. P = kt & 1 selects the B register set and LDS buffer at compile
  // time (register arrays cannot be indexed at run time without going to memory).
  auto slice = [&](auto Pc, auto TailC, auto FirstC, int kt) {
    constexpr int P = decltype(Pc)::value;
    const int nxt = cur + 1 == SA ? 0 : cur + 1;  // slot of A(kt+1)
    const int far = cur == 0 ? SA - 1 : cur - 1;   // slot of A(kt-1), refilled with A(kt+SA-1)
    const u32x4* LA = lds + cur * A_STAGE;
    const u32x4* LB = lds + SA * A_STAGE + P * B_STAGE;

    // k-step 0: fragments of step 1; B(kt+1) registers -> the other B buffer
    frags(LA, LB, 1, f1a, f1b);
    stash_b(NSB == 2 ? P ^ 1 : 0, P ^ 1);
    mmas(FirstC, f0a, f0b, 0, FM);
    plan_slice<0, FM * FN, FM + FN, 8 * NB, 0>();
    __builtin_amdgcn_sched_barrier(0);

    // k-step 1: fragments of step 2; B(kt+3) into the freed registers, A(kt+SA-1)
    // into the ring slot A(kt-1) used (past the end: zeros into unused buffers)
    frags(LA, LB, 2, f0a, f0b);
    if constexpr (NSB == 2)
      issue_b((kt + 3) * BK, P ^ 1);
    else
      issue_b((kt + 2) * BK, 0);
    issue_a((kt + SA - 1) * BK, far, TailC);
    mmas(acc_in, f1a, f1b, 0, FM);
    plan_slice<0, FM * FN, FM + FN, 0, PER_SLICE>();
    __builtin_amdgcn_sched_barrier(0);

    // k-step 2: fragments of step 3
    frags(LA, LB, 3, f1a, f1b);
    mmas(acc_in, f0a, f0b, 0, FM);
    plan_slice<0, FM * FN, FM + FN, 0, 0>();
    __builtin_amdgcn_sched_barrier(0);

    // k-step 3: half the blocks, then the slice boundary (A(kt+1) landed, B(kt+1)
    // stored by every wave), step-0 fragments of slice kt+1 under the other half
    mmas(acc_in, f1a, f1b, 0, HALF);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<PER_SLICE * (SA - 2)>();
    lds_barrier();
    frags(lds + nxt * A_STAGE, lds + SA * A_STAGE + (P ^ 1) * B_STAGE, 0, f0a, f0b);
    mmas(acc_in, f1a, f1b, HALF, FM);
    plan_slice<0, (FM - HALF) * FN, FM + FN, 0, 0>();
    __builtin_amdgcn_sched_barrier(0);
    cur = nxt;
  };
  // Slice 0 (K >= 1, so there is one) starts the accumulators when PEEL. Slices
  // whose A issue (slice kt + SA - 1) lies wholly inside K run the branch-free
  // issue; the last few take the masked one. Slices go in pairs so that the B
  // register set (kt & 1) stays a compile-time choice.
  using Full = std::false_type;
  using Tail = std::true_type;
  const std::integral_constant<int, 0> p0{};
  const std::integral_constant<int, 1> p1{};
  int kt = 0;
  if constexpr (PEEL) {
    if (SA * BK <= K)
      slice(p0, Full{}, std::true_type{}, 0);
    else
      slice(p0, Tail{}, std::true_type{}, 0);
    kt = 1;
    for (; kt + 1 < nk && (kt + SA + 1) * BK <= K; kt += 2) {
      slice(p1, Full{}, acc_in, kt);
      slice(p0, Full{}, acc_in, kt + 1);
    }
    for (; kt + 1 < nk; kt += 2) {
      slice(p1, Tail{}, acc_in, kt);
      slice(p0, Tail{}, acc_in, kt + 1);
    }
    if (kt < nk) slice(p1, Tail{}, acc_in, kt);
  } else {
    for (; kt + 1 < nk && (kt + SA + 1) * BK <= K; kt += 2) {
      slice(p0, Full{}, acc_in, kt);
      slice(p1, Full{}, acc_in, kt + 1);
    }
    for (; kt + 1 < nk; kt += 2) {
      slice(p0, Tail{}, acc_in, kt);
      slice(p1, Tail{}, acc_in, kt + 1);
    }
    if (kt < nk) slice(p0, Tail{}, acc_in, kt);
  }

  // ---- epilogue (store_tile_rt)
  wait_vm<0>();
  lds_barrier();  // every wave is done with the operand ring; LDS is free
  store_tile_rt<FM, FN, WTM, WTN, NW, static_cast<int>(sizeof(lds))>(
      a, acc, reinterpret_cast<float*>(lds), m0, n0, wm, wn, wave, lane, z);
}

template <typename T, int BM, int BN, int WGM, int WGN, int SA, int KR, int NSB>
hipError_t launch_m16d(const LaunchArgs& a, hipStream_t s) {
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(a.batch));
  hipLaunchKernelGGL((gemm_m16d_kernel<T, BM, BN, WGM, WGN, SA, KR, NSB>), grid,
                     dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}

#define G15_M16D(T, TN, BM, BN, WGM, WGN, SA, KR, NSB)                                        \
  {"m16d_" TN "_" #BM "x" #BN "x64_w" #WGM "x" #WGN "_a" #SA "_b" #KR "_r" #NSB, KIND_MFMA16,     \
   T::code, BM, BN, 64, 64 * WGM * WGN, (SA * BM + 2 * BN) * 128, 1, 1,                        \
   launch_m16d<T, BM, BN, WGM, WGN, SA, KR, NSB>, 1}

#define G15_M16D_ALL(T, TN)                    \
  G15_M16D(T, TN, 256, 256, 2, 4, 3, 4, 2),    \
  G15_M16D(T, TN, 256, 256, 2, 4, 3, 4, 1),    \
  G15_M16D(T, TN, 256, 256, 4, 2, 3, 4, 1),    \
  G15_M16D(T, TN, 256, 256, 2, 2, 3, 8, 2),    \
  G15_M16D(T, TN, 256, 256, 2, 2, 3, 8, 1),    \
  G15_M16D(T, TN, 256, 128, 2, 2, 4, 4, 2),    \
  G15_M16D(T, TN, 256, 128, 2, 2, 4, 4, 1),    \
  G15_M16D(T, TN, 128, 256, 2, 4, 3, 4, 1),    \
  G15_M16D(T, TN, 128, 128, 2, 2, 3, 4, 2),    \
  G15_M16D(T, TN, 128, 128, 2, 2, 3, 4, 1),    \
  G15_M16D(T, TN, 128, 128, 2, 2, 4, 4, 2),    \
  G15_M16D(T, TN, 64, 128, 2, 2, 4, 4, 2)

const KernelEntry kM16D[] = {
    G15_M16D_ALL(bf16_t, "bf16"),
    G15_M16D_ALL(f16_t, "f16"),
};

}  // namespace

int mfma16_dlds_entries(const KernelEntry** out) {
  *out = kM16D;
  return static_cast<int>(sizeof(kM16D) / sizeof(kM16D[0]));
}

}  // namespace g15
