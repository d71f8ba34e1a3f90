// kernel_mfma16_nt.hip -- bf16 / fp16 matrix-core GEMMs with both operands
// streamed global -> LDS directly:
//  * m16n: the right operand given transposed, C = epi(A x Bt^T), A [M x K] and
//    Bt [N x K] row-major (a linear layer's weight in [out, in] order, or K of
//    attention scores Q K^T);
//  * m16t: the plain layout, B [K x N] row-major, with B slices stored in LDS as
//    they come (k rows of n) and B fragments read with the gfx950 transposing
//    LDS read (ds_read_b64_tr_b16), two per fragment.
//
// Same tiling and schedule as kernel_mfma16_dlds.hip (DeepGEMM page, sections
// 2.2 and 3.1; prefetch of the SGEMM page, section 2.3), but both operands now
// arrive k-contiguous, which is what the matrix core reads: Bt slices go global
// -> LDS directly (buffer_load ... lds) exactly like A, into their own ring, and
// B fragments are read like A fragments. No register staging, no transpose, no
// LDS stores in the main loop.
//
// For m16t the transposing read returns, in lane i of each group of 16 lanes, 4
// consecutive k of column n0 + i when source lane t of the group addresses row
// k0 + t / 4, columns n0 + 4 (t % 4) .. +3; a fragment (8 k of one column per
// lane) takes two such reads. B rows of 2 BN bytes permute 16-byte chunk c to
// c ^ (4 (k & 3)), which keeps those reads free of bank conflicts (measured 2.9
// cycles per read, like an untransposed 8-byte read).
//
// LDS: an A ring of SA slices and a B ring of SB slices (BM x 128 and BN x 128
// bytes per slice). With SB = SA - 1 (the 256 x 256 tile, whose rings would not
// fit otherwise) B is fetched one slice ahead, A two; the B loads of a slice are
// issued before its A loads so the wait at the slice boundary can leave the
// newest A loads in flight. The compiler makes an LDS read that may alias a
// direct-to-LDS load in flight wait for every load (vmcnt(0)); each slice takes
// its read and load slots as separate restrict parameters, so that wait is gone
// and the A loads keep their lead across the slice boundary.
#include "m16_common.hpp"

namespace g15 {
namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

template <typename T, int BM, int BN, int WGM, int WGN, int SA, int SB, bool BROW>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_m16n_kernel(LaunchArgs a) {
  constexpr int BK = 64;
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int AI = BM / 8 / NW;  // direct A loads per wave per slice (8 rows each)
  constexpr int BI = BN / 8 / NW;  // direct B loads per wave per slice
  constexpr int A_STAGE = BM * 8;  // 16-byte chunks per A slice
  constexpr int B_STAGE = BN * 8;
  static_assert(BM % (8 * NW) == 0 && AI >= 1, "A rows must split evenly over the waves");
  static_assert(BN % (8 * NW) == 0 && BI >= 1, "B rows must split evenly over the waves");
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold a 32x32 block");
  static_assert(SB >= 2 && (SA == SB || SA == SB + 1), "rings: SA = SB or SA = SB + 1");
  static_assert(BK / 16 == 4, "the K loop below is written for four k-steps per slice");
  // B row-major (m16t): a slice is 64 rows of BN/8 chunks; one load fills RPI rows
  constexpr int CPR_B = BN / 8, RPI = 64 / CPR_B;
  static_assert(!BROW || (CPR_B >= 16 && 64 % CPR_B == 0), "m16t: BN of 128 or 256");
  constexpr int RING = SA * A_STAGE + SB * B_STAGE;
  constexpr int STG = (NW * 32 * (WTN + 8) * 4 + 15) / 16;  // epilogue staging, 16-byte units
  __shared__ u32x4 lds[RING > STG ? RING : STG];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index as a scalar: LDS slot addresses derived from it stay in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int M = static_cast<int>(a.M), N = static_cast<int>(a.N), K = static_cast<int>(a.K);
  const int LDA = static_cast<int>(a.lda), LDB = static_cast<int>(a.ldb);
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  int64_t z;
  batch_tile_of(tiles_m, tiles_n, tm, tn, z);
  const int m0 = tm * BM, n0 = tn * BN;

  // 16-byte chunk c of an LDS row sits at c ^ (row & 7) ^ ((row >> 3) & 3) in both
  // rings (conflict-free fragment reads). Instruction i of a wave fills 8 rows
  // r0 .. r0+7 (lane l -> slot r0*8 + l), so lane l fetches logical chunk
  // (l & 7) ^ (l >> 3) ^ ((r0 >> 3) & 3) of row r0 + (l >> 3).
  const uint16_t* Abase = static_cast<const uint16_t*>(a.A) + z * a.sA;
  const uint16_t* Bbase = static_cast<const uint16_t*>(a.B) + z * a.sB;
  int a_chk[AI], b_chk[BI];
  uint32_t a_voff[AI], b_voff[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    a_chk[i] = (lane & 7) ^ (lane >> 3) ^ ((wave * AI + i) & 3);
    const int gm = m0 + (wave * AI + i) * 8 + (lane >> 3);
    a_voff[i] = gm < M ? static_cast<uint32_t>(gm * LDA + a_chk[i] * 8) * 2u : OOB;
  }
  int b_row[BI];  // m16t: the slice row this lane fills in load i
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    if constexpr (!BROW) {
      b_chk[i] = (lane & 7) ^ (lane >> 3) ^ ((wave * BI + i) & 3);
      const int gn = n0 + (wave * BI + i) * 8 + (lane >> 3);
      b_voff[i] = gn < N ? static_cast<uint32_t>(gn * LDB + b_chk[i] * 8) * 2u : OOB;
      b_row[i] = 0;
    } else {
      // load q = wave BI + i fills rows q RPI .. +RPI-1; lane l -> row q RPI + l / CPR_B,
      // slot chunk l % CPR_B, which holds logical chunk (l % CPR_B) ^ (4 (row & 3))
      const int row = (wave * BI + i) * RPI + lane / CPR_B;
      const int gn = n0 + ((lane % CPR_B) ^ (4 * (row & 3))) * 8;
      b_row[i] = row;
      b_chk[i] = 0;
      b_voff[i] = gn < N ? static_cast<uint32_t>(row * LDB + gn) * 2u : OOB;
    }
  }
  // One operand's slice k0 into ring slot `slot`. TAIL: the slice may reach past K
  // (chunks past K are masked and their slots zeroed, since an out-of-range
  // direct load leaves its LDS slot untouched); otherwise the issue is branch-free.
  auto issue = [&](const uint16_t* base, int rows, int ld, const uint32_t* voff,
                   const int* chk, u32x4* ring, int per_wave, int k0, int slot, auto TailC,
                   auto NC) {
    constexpr bool TAIL = decltype(TailC)::value;
    constexpr int NI = decltype(NC)::value;
    const int64_t left = static_cast<int64_t>(rows) * ld - k0;
    const auto r = rsrc(base + k0, static_cast<uint32_t>(left > 0 ? left * 2 : 0));
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bool kin = !TAIL || k0 + chk[i] * 8 < K;  // k past K inside a row would read the next row
      const uint32_t off = kin ? voff[i] : OOB;
      u32x4* dst = ring + slot * (per_wave * NW * 64) + (wave * per_wave + i) * 64;
      if (TAIL && !kin) dst[lane] = u32x4{0u, 0u, 0u, 0u};
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, off, 0, 0, 0);
    }
  };
  u32x4* const ringA = lds;
  u32x4* const ringB = lds + SA * A_STAGE;
  auto issue_a = [&](int k0, int slot, auto TailC) {
    issue(Abase, M, LDA, a_voff, a_chk, ringA, AI, k0, slot, TailC,
          std::integral_constant<int, AI>{});
  };
  auto issue_b = [&](int k0, int slot, auto TailC) {
    if constexpr (!BROW) {
      issue(Bbase, N, LDB, b_voff, b_chk, ringB, BI, k0, slot, TailC,
            std::integral_constant<int, BI>{});
    } else {
      // rows past K fall beyond the slice's descriptor extent (read as zeros; the
      // tail zeroes their slots, which such a load leaves untouched)
      constexpr bool TAIL = decltype(TailC)::value;
      const int64_t left = static_cast<int64_t>(K - k0) * LDB;
      const auto r = rsrc(Bbase + static_cast<int64_t>(k0) * LDB,
                          static_cast<uint32_t>(left > 0 ? left * 2 : 0));
#pragma unroll
      for (int i = 0; i < BI; ++i) {
        u32x4* dst = ringB + slot * B_STAGE + (wave * BI + i) * 64;
        if (TAIL && k0 + b_row[i] >= K) dst[lane] = u32x4{0u, 0u, 0u, 0u};
        // (an array element written straight into the builtin's arguments makes the
        // host compilation drop this kernel's launch stub; go through a local)
        const uint32_t off = b_voff[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, off, 0, 0, 0);
      }
    }
  };

  // no clearing: the first k-step of slice 0 takes a zero accumulator operand (an
  // inline constant), which saves one register write per accumulator element
  f32x16 acc[FM][FN];

  const int nk = (K + BK - 1) / BK;
  const int lrow = lane & 31, lhalf = lane >> 5;
  // fragment rows: A row wm*WTM + 32 i + lrow, B row wn*WTN + 32 j + lrow; the
  // chunk permutation depends on the row modulo 32 only
  const int a_base = (wm * WTM + lrow) * 8, b_base = (wn * WTN + lrow) * 8;
  const int perm = (lrow & 7) ^ ((lrow >> 3) & 3);
  // m16t: byte offset in a B slice of this lane's first transposing read of block
  // j at k-step 0 (group g = lane / 16, t = lane % 16: row 8 (g / 2) + t / 4,
  // column wn WTN + 32 j + 16 (g % 2) + 4 (t % 4)); k-step s adds 16 s rows, the
  // second read of a fragment 4 rows, neither of which changes row & 3
  int btr[FN];
  {
    const int g = lane >> 4, t = lane & 15;
    const int kr = 8 * (g >> 1) + (t >> 2);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = wn * WTN + 32 * j + 16 * (g & 1) + 4 * (t & 3);
      btr[j] = kr * (BN * 2) + (((n >> 3) ^ (4 * (kr & 3))) << 4) + (n & 7) * 2;
    }
  }
  // Fragment read r of k-step s, in the order the ops of a k-step consume them:
  // A block 0, B blocks 0 .. FN-1, then A blocks 1 .. FM-1.
  auto read_frag = [&](const lds_char* LA, const lds_char* LB, int s, int r, u32x4 (&fa)[FM],
                       u32x4 (&fb)[FN]) __attribute__((always_inline)) {
    const int c = (2 * s + lhalf) ^ perm;
    if (r == 0 || r > FN) {
      const int i = r == 0 ? 0 : r - FN;
      fa[i] = *(const lds_u32x4*)(LA + (a_base + i * 256 + c) * 16);
      return;
    }
    const int j = r - 1;
    if constexpr (!BROW) {
      fb[j] = *(const lds_u32x4*)(LB + (b_base + j * 256 + c) * 16);
    } else {
      const lds_char* Lb = LB + 16 * s * (BN * 2) + btr[j];
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)Lb);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Lb + 4 * (BN * 2)));
      fb[j] = u32x4{__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                    __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                    __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1)),
                    __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3))};
    }
  };
  auto frags = [&](const lds_char* LA, const lds_char* LB, int s, u32x4 (&fa)[FM],
                   u32x4 (&fb)[FN]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < FM + FN; ++r) read_frag(LA, LB, s, r, fa, fb);
  };
  lds_char* const L8 = (lds_char*)lds;
  auto slotA8 = [&](int sl) __attribute__((always_inline)) { return L8 + sl * A_STAGE * 16; };
  auto slotB8 = [&](int sl) __attribute__((always_inline)) {
    return L8 + (SA * A_STAGE + sl * B_STAGE) * 16;
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

  // Prologue: B slices 0 .. SB-2 and A slices 0 .. SA-2 (B of a slice before its A).
  for (int s = 0; s < SA - 1; ++s) {
    if (s < SB - 1) issue_b(s * BK, s, std::true_type{});
    issue_a(s * BK, s, std::true_type{});
  }
  wait_vm<0>();
  lds_barrier();
  u32x4 f0a[FM], f0b[FN], f1a[FM], f1b[FN];
  frags(slotA8(0), slotB8(0), 0, f0a, f0b);

  // m16n: the instruction order of a slice is fixed here, op by op: each
  // matrix-core op is followed by the fragment reads and direct loads assigned to
  // it, and a scheduling fence keeps the compiler from gathering those into one
  // block that leaves the matrix core idle (measured: 4% fewer cycles at 4096^3).
  //  * k-steps 0-2: the FM + FN fragment reads of the next k-step spread over the
  //    first half of the ops (they land well before the next k-step needs them);
  //    the slice's NV = BI + AI direct loads (B first) spread over the 3 FM FN ops
  //    of the three k-steps;
  //  * k-step 3: HALF FN ops, the slice boundary (A(kt+1), B(kt+1) landed, every
  //    wave done with slice kt), one op, all of the next slice's step-0 reads, and
  //    the rest of the ops, which cover their latency.
  constexpr int NM = FM * FN, NR = FM + FN, NV = AI + BI;
  constexpr int HALF = FM / 2;
  constexpr int Q3 = HALF * FN;  // ops of k-step 3 before the boundary
  static_assert(NV <= 3 * NM, "one direct load per op at most");
  // loads left in flight at a slice boundary: everything issued after B(kt+1)
  constexpr int WAITN = SA == SB ? NV * (SA - 2) : NV * (SB - 2) + AI;
  int ca = 0, cb = 0;  // ring slots of A(kt), B(kt)
  auto slice = [&](auto TailC, auto FirstC, int kt) {
    constexpr bool TAIL = decltype(TailC)::value;
    const int na = ca + 1 == SA ? 0 : ca + 1, nb = cb + 1 == SB ? 0 : cb + 1;
    const int fa = ca == 0 ? SA - 1 : ca - 1;  // slot of A(kt-1), refilled with A(kt+SA-1)
    const int fb = cb == 0 ? SB - 1 : cb - 1;  // slot of B(kt-1), refilled with B(kt+SB-1)
    // Slot pointers of this slice (reads of slice kt, of slice kt+1 after the
    // boundary, loads of the slices kt+SA-1 / kt+SB-1) passed as restrict parameters:
    // the compiler then does not make the transposing reads wait for the loads in
    // flight (each slot it reads has been waited for explicitly before the barrier).
    auto body = [&](const lds_char* __restrict__ LA, const lds_char* __restrict__ LB,
                    const lds_char* __restrict__ NA, const lds_char* __restrict__ NB,
                    lds_char* __restrict__ WA, lds_char* __restrict__ WB)
                    __attribute__((always_inline)) {
    // descriptors of this slice's direct loads (scalar work)
    const int k0a = (kt + SA - 1) * BK, k0b = (kt + SB - 1) * BK;
    const int64_t lefta = static_cast<int64_t>(M) * LDA - k0a;
    const auto rA = rsrc(Abase + k0a, static_cast<uint32_t>(lefta > 0 ? lefta * 2 : 0));
    int64_t leftb;
    const uint16_t* Bk;
    if constexpr (!BROW) {
      leftb = static_cast<int64_t>(N) * LDB - k0b;
      Bk = Bbase + k0b;
    } else {
      leftb = static_cast<int64_t>(K - k0b) * LDB;
      Bk = Bbase + static_cast<int64_t>(k0b) * LDB;
    }
    const auto rB = rsrc(Bk, static_cast<uint32_t>(leftb > 0 ? leftb * 2 : 0));
    auto dma = [&](int v) {
      if (v < BI) {
        const int i = v;
        lds_char* dst = WB + (wave * BI + i) * 1024;
        bool kin;
        if constexpr (!BROW)
          kin = !TAIL || k0b + b_chk[i] * 8 < K;
        else
          kin = !TAIL || k0b + b_row[i] < K;
        const uint32_t off = kin ? b_voff[i] : OOB;
        if (TAIL && !kin) ((lds_u32x4*)dst)[lane] = u32x4{0u, 0u, 0u, 0u};
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void*)dst, 16, off, 0, 0, 0);
      } else {
        const int i = v - BI;
        lds_char* dst = WA + (wave * AI + i) * 1024;
        const bool kin = !TAIL || k0a + a_chk[i] * 8 < K;
        const uint32_t off = kin ? a_voff[i] : OOB;
        if (TAIL && !kin) ((lds_u32x4*)dst)[lane] = u32x4{0u, 0u, 0u, 0u};
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void*)dst, 16, off, 0, 0, 0);
      }
    };
    // k-step s (0..2) on fragments (xa, xb), reading step s+1 into (ya, yb)
    auto step = [&](auto ZeroC, int s, const u32x4 (&xa)[FM], const u32x4 (&xb)[FN],
                    u32x4 (&ya)[FM], u32x4 (&yb)[FN]) {
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        if constexpr (decltype(ZeroC)::value)
          acc[q / FN][q % FN] = mma<T>(xa[q / FN], xb[q % FN], f32x16{});
        else
          acc[q / FN][q % FN] = mma<T>(xa[q / FN], xb[q % FN], acc[q / FN][q % FN]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < NR; ++r)
          if (r * NM / (2 * NR) == q) read_frag(LA, LB, s + 1, r, ya, yb);
#pragma unroll
        for (int v = 0; v < NV; ++v)
          if (v * 3 * NM / NV == s * NM + q) dma(v);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if constexpr (BROW) {
      // m16t keeps the grouped order (measured faster for it): each k-step's
      // fragment reads, then its ops, with the direct loads in k-step 1
      frags(LA, LB, 1, f1a, f1b);
      mmas(FirstC, f0a, f0b, 0, FM);
      plan_slice<0, FM * FN, FM + FN, 0, 0>();
      __builtin_amdgcn_sched_barrier(0);
      // the B fragments of k-step 3 are read here too, before the slice's direct
      // loads (measured order; with the slots as restrict parameters the compiler no
      // longer makes these reads wait for the loads in flight, so this order is not
      // required for that any more)
      u32x4 f3b[FN];
      frags(LA, LB, 2, f0a, f0b);
#pragma unroll
      for (int j = 0; j < FN; ++j) read_frag(LA, LB, 3, 1 + j, f1a, f3b);
#pragma unroll
      for (int v = 0; v < NV; ++v) dma(v);
      mmas(acc_in, f1a, f1b, 0, FM);
      plan_slice<0, FM * FN, FM + 2 * FN, 0, NV>();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < FM + FN; ++r)
        if (r == 0 || r > FN) read_frag(LA, LB, 3, r, f1a, f1b);
#pragma unroll
      for (int j = 0; j < FN; ++j) f1b[j] = f3b[j];
      mmas(acc_in, f0a, f0b, 0, FM);
      plan_slice<0, FM * FN, FM, 0, 0>();
      __builtin_amdgcn_sched_barrier(0);
      mmas(acc_in, f1a, f1b, 0, HALF);
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<WAITN>();
      lds_barrier();
      frags(NA, NB, 0, f0a, f0b);
      mmas(acc_in, f1a, f1b, HALF, FM);
      plan_slice<0, (FM - HALF) * FN, FM + FN, 0, 0>();
      __builtin_amdgcn_sched_barrier(0);
      return;
    }
    step(FirstC, 0, f0a, f0b, f1a, f1b);
    step(acc_in, 1, f1a, f1b, f0a, f0b);
    step(acc_in, 2, f0a, f0b, f1a, f1b);
#pragma unroll
    for (int q = 0; q < Q3; ++q) {
      acc[q / FN][q % FN] = mma<T>(f1a[q / FN], f1b[q % FN], acc[q / FN][q % FN]);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vm<WAITN>();
    lds_barrier();
#pragma unroll
    for (int q = Q3; q < NM; ++q) {
      acc[q / FN][q % FN] = mma<T>(f1a[q / FN], f1b[q % FN], acc[q / FN][q % FN]);
      __builtin_amdgcn_sched_barrier(0);
      if (q == Q3) frags(NA, NB, 0, f0a, f0b);
      __builtin_amdgcn_sched_barrier(0);
    }
    };
    body(slotA8(ca), slotB8(cb), slotA8(na), slotB8(nb), slotA8(fa), slotB8(fb));
    ca = na;
    cb = nb;
  };
  // Slice 0 (K >= 1, so there is one) starts the accumulators. Slices whose issues
  // (A(kt + SA - 1), B(kt + SB - 1)) lie wholly inside K run the branch-free issue;
  // the last few take the masked one.
  if (SA * BK <= K)
    slice(std::false_type{}, std::true_type{}, 0);
  else
    slice(std::true_type{}, std::true_type{}, 0);
  int kt = 1;
  for (; kt < nk && (kt + SA) * BK <= K; ++kt) slice(std::false_type{}, acc_in, kt);
  for (; kt < nk; ++kt) slice(std::true_type{}, acc_in, kt);

  wait_vm<0>();
  lds_barrier();  // every wave is done with the rings; LDS is free
  store_tile<FM, FN, WTM, WTN, NW, static_cast<int>(sizeof(lds))>(
      a, acc, reinterpret_cast<float*>(lds), m0, n0, wm, wn, wave, lane, z);
}

template <typename T, int BM, int BN, int WGM, int WGN, int SA, int SB, bool BROW>
hipError_t launch_m16n(const LaunchArgs& a, hipStream_t s) {
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(a.batch));
  hipLaunchKernelGGL((gemm_m16n_kernel<T, BM, BN, WGM, WGN, SA, SB, BROW>), grid,
                     dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}

#define G15_M16N(T, TN, BM, BN, WGM, WGN, SA, SB) G15_M16X(T, TN, "m16n_", false, BM, BN, WGM, WGN, SA, SB)
#define G15_M16T(T, TN, BM, BN, WGM, WGN, SA, SB) G15_M16X(T, TN, "m16t_", true, BM, BN, WGM, WGN, SA, SB)
#define G15_M16X(T, TN, PFX, BROW, BM, BN, WGM, WGN, SA, SB)                                      \
  {PFX TN "_" #BM "x" #BN "x64_w" #WGM "x" #WGN "_a" #SA "_b" #SB, KIND_MFMA16, T::code, BM,       \
   BN, 64, 64 * WGM * WGN,                                                                        \
   static_cast<int>(sizeof(u32x4)) *                                                              \
       ((SA * BM + SB * BN) * 8 > (WGM * WGN * 32 * (BN / WGN + 8) * 4 + 15) / 16                  \
            ? (SA * BM + SB * BN) * 8                                                             \
            : (WGM * WGN * 32 * (BN / WGN + 8) * 4 + 15) / 16),                                   \
   1, 1, launch_m16n<T, BM, BN, WGM, WGN, SA, SB, BROW>, 1, BROW ? 0 : 1}

#define G15_M16N_ALL(T, TN)                     \
  G15_M16N(T, TN, 256, 256, 4, 2, 3, 2),        \
  G15_M16N(T, TN, 256, 256, 2, 4, 3, 2),        \
  G15_M16N(T, TN, 256, 128, 2, 2, 3, 3),        \
  G15_M16N(T, TN, 128, 256, 2, 4, 3, 3),        \
  G15_M16N(T, TN, 128, 128, 2, 2, 3, 3),        \
  G15_M16N(T, TN, 128, 128, 2, 2, 2, 2),        \
  G15_M16N(T, TN, 64, 128, 2, 2, 4, 4),        \
  G15_M16N(T, TN, 64, 128, 2, 2, 3, 3)

#define G15_M16T_ALL(T, TN)                     \
  G15_M16T(T, TN, 256, 256, 4, 2, 3, 2),        \
  G15_M16T(T, TN, 256, 256, 2, 4, 3, 2),        \
  G15_M16T(T, TN, 256, 128, 2, 2, 3, 3),        \
  G15_M16T(T, TN, 128, 256, 2, 4, 3, 3),        \
  G15_M16T(T, TN, 128, 128, 2, 2, 3, 3),        \
  G15_M16T(T, TN, 128, 128, 2, 2, 2, 2),        \
  G15_M16T(T, TN, 64, 128, 2, 2, 3, 3)

const KernelEntry kM16N[] = {
    G15_M16N_ALL(bf16_t, "bf16"), G15_M16N_ALL(f16_t, "f16"),
    G15_M16T_ALL(bf16_t, "bf16"), G15_M16T_ALL(f16_t, "f16"),
};

}  // namespace

int mfma16_nt_entries(const KernelEntry** out) {
  *out = kM16N;
  return static_cast<int>(sizeof(kM16N) / sizeof(kM16N[0]));
}

}  // namespace g15
