// kernel_mfma16_k1.hip -- bf16 / fp16 matrix-core GEMM for products whose K fits
// one 64-deep slice: the attention scores S = Q K^T of heads of dimension 64 (the
// tutorial page's attention, section 2: a batched Q K^T whose output the softmax
// then reads). With K = 64 a 128 x 128 tile reads 32 KB of operands and writes
// 64 KB of fp32 C, so the writes are the work: each workgroup walks a strided list
// of tiles (batch items included) and keeps the next tile's operands loading while
// it multiplies and stores the current one, instead of one tile per workgroup with
// its loads, products and stores in sequence.
//
// Per tile: wait for its operands (and the previous tile's stores), barrier, read
// every A fragment (16-byte LDS reads) and every B fragment (the transposing read
// ds_read_b64_tr_b16, two per fragment) of the four 16-deep k-steps, issue the
// direct-to-LDS loads of the next tile into the other slot, run the products, and
// store C straight from the accumulators (DeepGEMM page, section 3.1: the tile's
// accumulators leave once; the 16-bit forms without LDS staging, which would need
// the slot being filled). All B fragments are read before the next tile's loads
// go out because the compiler makes a transposing read that follows a direct load
// wait for every load in flight.
//
// LDS (as in kernel_mfma16_nt.hip for m16t): an A slot is BM rows of 64 k, 16-byte
// chunk c of row r at c ^ (r & 7) ^ ((r >> 3) & 3); a B slot is 64 rows (k) of BN
// columns, chunk c of row k at c ^ (4 (k & 3)). Slots of k at or past K are zeroed
// once (K is the same for every tile and the loads never write them); rows past M
// and columns past N keep whatever the slot held, which only reaches outputs that
// are not stored.
//
// Tile order: with 8 or more batch items, every tile of a batch item goes to one
// XCD (workgroups reach the 8 XCDs round-robin), so each item's operands are
// fetched into one L2; otherwise the tiles of the single product are strided over
// the workgroups in the XCD-aware order of tile_of.
#include "m16_common.hpp"
#include "attention.hpp"

namespace g15 {
namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

// Row reduction of 32 values per lane over the 32 lanes of each half-wave, by
// halving: in the round for lane bit b a lane keeps the half of its values that
// bit b selects and combines it with its partner's copy of that half; the partner
// differs in bit b and agrees in the bits of the earlier rounds, so it holds the
// same values. Rounds: bit 4 with v_permlane16_swap (lanes 16 apart), then bit 3,
// 2, 1, 0 with DPP moves from lane l ^ 15 (row_mirror), l ^ 7 (row_half_mirror),
// l ^ 2 and l ^ 1 (quad permutations); 31 exchanges, no LDS. The result is the
// reduction of value index lane % 32, in a fixed order.
template <bool MAXOP>
__device__ __forceinline__ float comb(float a, float b) {
  return MAXOP ? fmaxf(a, b) : a + b;
}

// m ? a : b as a bit select (v_bfi_b32) behind inline assembly: written as a
// conditional, the compiler turns the choice into a lane-dependent index into the
// 32 registers, i.e. a 32-way compare-and-select chain per value.
__device__ __forceinline__ float bit_pick(uint32_t m, float a, float b) {
  float r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(a), "v"(b));
  return r;
}

template <bool MAXOP, int H, int CTRL>
__device__ __forceinline__ void halve_dpp(float (&x)[32], int lane) {
  const uint32_t up = (lane & H) != 0 ? 0xffffffffu : 0u;
#pragma unroll
  for (int q = 0; q < H; ++q) {
    const float send = bit_pick(up, x[q], x[q + H]);
    const float keep = bit_pick(up, x[q + H], x[q]);
    const float recv =
        __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(send), CTRL, 0xf, 0xf, false));
    x[q] = comb<MAXOP>(keep, recv);
  }
}

template <bool MAXOP>
__device__ __forceinline__ float halve32(float (&x)[32], int lane) {
  // v_permlane16_swap exchanges the odd 16-lane rows of its first operand with the
  // even rows of its second: from (x[q], x[q + 16]) a lane of an even row gets its
  // own and its partner's x[q], a lane of an odd row both copies of x[q + 16]
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[q]), __float_as_uint(x[q + 16]),
                                                    false, false);
    x[q] = comb<MAXOP>(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  halve_dpp<MAXOP, 8, 0x140>(x, lane);  // row_mirror
  halve_dpp<MAXOP, 4, 0x141>(x, lane);  // row_half_mirror
  halve_dpp<MAXOP, 2, 0x4E>(x, lane);   // quad_perm 2 3 0 1
  halve_dpp<MAXOP, 1, 0xB1>(x, lane);   // quad_perm 1 0 3 2
  return x[0];
}

template <typename T, int BM, int BN, int WGM, int WGN, bool BROW, bool SMAX>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_m16s_kernel(LaunchArgs a) {
  constexpr int BK = 64;
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int AI = BM / 8 / NW;                    // A loads per wave per tile (8 rows each)
  constexpr int CPR_B = BN / 8, RPI = 64 / CPR_B;    // B: 16-byte chunks per row, rows per load
  constexpr int BI = BN / 8 / NW;                    // B loads per wave per tile
  constexpr int A_STAGE = BM * 8, B_STAGE = BN * 8;  // 16-byte chunks per slot
  static_assert(BM % (8 * NW) == 0 && AI >= 1, "A rows must split evenly over the waves");
  static_assert(BN % (8 * NW) == 0 && BI >= 1, "B chunks must split evenly over the waves");
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold a 32x32 block");
  static_assert(!BROW || (CPR_B >= 16 && 64 % CPR_B == 0), "row-major B: 128 or 256 columns");
  __shared__ u32x4 lds[2 * (A_STAGE + B_STAGE)];
  // SMAX: every row of the tile lies in one tile (N <= BN) and in every wave (WGM = 1)
  static_assert(!SMAX || (WGM == 1 && FM == 2 && FN == 2), "softmax tile: 64 rows, 64 columns a wave");
  __shared__ float2 sm_part[SMAX ? NW * BM : 1];         // per wave and row: (max, sum)
  __shared__ __align__(16) float sm_w[SMAX ? NW * BM : 1];  // per wave and row, wave-private
  u32x4* const ringA = lds;
  u32x4* const ringB = lds + 2 * A_STAGE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int M = static_cast<int>(a.M), N = static_cast<int>(a.N), K = static_cast<int>(a.K);
  const int LDA = static_cast<int>(a.lda), LDB = static_cast<int>(a.ldb);
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int64_t per_item = static_cast<int64_t>(tiles_m) * tiles_n;
  const int64_t batch = a.batch;

  // Tile-independent parts of this lane's load offsets. A: load i of the wave fills
  // slot rows 8 (wave AI + i) .. +7, lane l row + l / 8, logical chunk a_chk[i].
  // B: load i fills rows (wave BI + i) RPI .. +RPI-1, lane l row + l / CPR_B, slot
  // chunk l % CPR_B, which holds logical chunk (l % CPR_B) ^ (4 (row & 3)).
  int a_row[AI];
  uint32_t a_koff[AI];
  bool a_kin[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int chk = (lane & 7) ^ (lane >> 3) ^ ((wave * AI + i) & 3);
    a_row[i] = (wave * AI + i) * 8 + (lane >> 3);
    a_koff[i] = static_cast<uint32_t>(chk * 8);
    a_kin[i] = chk * 8 < K;  // K is a multiple of 8: a chunk is wholly inside K or past it
  }
  // B given transposed (Bt [N x K], !BROW) loads like A: rows n, chunks of k.
  int b_row[BI], b_col[BI];
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    if constexpr (BROW) {
      const int row = (wave * BI + i) * RPI + lane / CPR_B;
      b_row[i] = row;
      b_col[i] = ((lane % CPR_B) ^ (4 * (row & 3))) * 8;
    } else {
      // slot row (wave BI + i) 8 + l / 8 is n within the tile; b_row holds the k of
      // this lane's chunk, or K for a chunk past K
      const int chk = (lane & 7) ^ (lane >> 3) ^ ((wave * BI + i) & 3);
      b_col[i] = (wave * BI + i) * 8 + (lane >> 3);
      b_row[i] = chk * 8 < K ? chk * 8 : K;
    }
  }
  // k at or past K: zero those chunks of both slots once
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int i = 0; i < AI; ++i)
      if (!a_kin[i]) ringA[s * A_STAGE + (wave * AI + i) * 64 + lane] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < BI; ++i)
      if (b_row[i] >= K) ringB[s * B_STAGE + (wave * BI + i) * 64 + lane] = u32x4{0u, 0u, 0u, 0u};
  }

  // The q-th tile of this workgroup: batch item z and tile origin (m0, n0), or false
  // past the end. Workgroup w runs on XCD w % 8.
  const int64_t G = gridDim.x;
  const bool by_item = batch >= 8 && G % 8 == 0;
  auto tile = [&](int64_t q, int64_t& z, int& m0, int& n0) -> bool {
    int64_t r;
    if (by_item) {
      // XCD x takes the items z = x, x + 8, ...; its G / 8 workgroups stride over the
      // concatenated tiles of those items
      const int64_t x = blockIdx.x % 8, gx = G / 8;
      const int64_t u = blockIdx.x / 8 + q * gx;
      const int64_t zi = u / per_item;
      z = zi * 8 + x;
      r = u - zi * per_item;
      if (z >= batch) return false;
    } else {
      const int64_t t = blockIdx.x + q * G;
      z = t / per_item;
      r = t - z * per_item;
      if (z >= batch) return false;
    }
    int tm, tn;
    if (by_item) {
      tm = static_cast<int>(r / tiles_n);
      tn = static_cast<int>(r - static_cast<int64_t>(tm) * tiles_n);
    } else {
      tile_of(static_cast<int>(r), tiles_m, tiles_n, tm, tn);
    }
    m0 = tm * BM;
    n0 = tn * BN;
    return true;
  };
  // Direct-to-LDS loads of one tile into slot `slot`. A row past M, a column past N,
  // a chunk or row past K get an offset past the extent (the slot is left as it is).
  auto issue = [&](int64_t z, int m0, int n0, int slot) {
    const uint16_t* Az = static_cast<const uint16_t*>(a.A) + z * a.sA;
    const uint16_t* Bz = static_cast<const uint16_t*>(a.B) + z * a.sB;
    const auto rA = rsrc(Az, static_cast<uint32_t>(static_cast<int64_t>(M) * LDA * 2));
    const auto rB = rsrc(Bz, static_cast<uint32_t>(static_cast<int64_t>(BROW ? K : N) * LDB * 2));
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int gm = m0 + a_row[i];
      const uint32_t off =
          (a_kin[i] && gm < M) ? static_cast<uint32_t>(gm * LDA) * 2u + a_koff[i] * 2u : OOB;
      u32x4* dst = ringA + slot * A_STAGE + (wave * AI + i) * 64;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void*)dst, 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int gn = n0 + b_col[i];
      // row-major B: row b_row (k), column gn; transposed: row gn (n), k chunk at b_row
      const uint32_t off =
          (b_row[i] < K && gn < N)
              ? static_cast<uint32_t>(BROW ? b_row[i] * LDB + gn : gn * LDB + b_row[i]) * 2u
              : OOB;
      u32x4* dst = ringB + slot * B_STAGE + (wave * BI + i) * 64;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void*)dst, 16, off, 0, 0, 0);
    }
  };

  // fragment addresses: A row wm*WTM + 32 i + (lane & 31), k chunk 2 s + lane / 32;
  // B as in m16t (group g = lane / 16, t = lane % 16: row 8 (g / 2) + t / 4, column
  // wn WTN + 32 j + 16 (g % 2) + 4 (t % 4); k-step s adds 16 s rows, the second read
  // of a fragment 4 rows, neither of which changes row & 3)
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int a_base = (wm * WTM + lrow) * 8;
  const int perm = (lrow & 7) ^ ((lrow >> 3) & 3);
  // transposed B: fragment row wn*WTN + 32 j + (lane & 31), laid out like A
  const int b_base = (wn * WTN + lrow) * 8;
  const int bperm = (lrow & 7) ^ (((wn * WTN + lrow) >> 3) & 3);
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

  LaunchArgs out = a;
  out.c_vec = 0;  // 16-bit C straight from the registers: LDS holds the next tile's operands

  f32x16 acc[FM][FN];
  // SMAX with a 16-bit P of even N: a tile's P leaves one tile later, right after
  // the next tile's loads are issued, so the loop-top wait for every load and store
  // in flight finds the stores a tile old instead of just issued. Registers 2p and
  // 2p+1 of a block are rows R and R+1 of one column and lanes l, l^1 hold
  // neighbouring columns: after one exchange the even lane holds columns (c, c+1)
  // of row R and the odd lane (c-1, c) of row R+1, one 4-byte store each.
  // Without the softmax the same delay applies to fp32 C with no epilogue on the
  // 8-wave tiles (their registers have room for the held tile).
  constexpr bool HOLD = !SMAX && NW == 8;
  const bool defer = SMAX ? (a.epi.out_dtype != DT_F32 && (N & 1) == 0 && (a.ldc & 1) == 0)
                          : (HOLD && a.epi.out_dtype == DT_F32 && a.epi.flags == 0);
  uint32_t pk[SMAX ? FM : 1][SMAX ? FN : 1][8];
  f32x16 held[HOLD ? FM : 1][HOLD ? FN : 1];
  bool pend = false;
  int64_t zp = 0;
  int m0p = 0, n0p = 0;
  const bool odd_lane = (lane & 1) != 0;
  const uint32_t odd_mask = odd_lane ? 0xffffffffu : 0u;
  auto pack = [&]() {
    const bool bf = a.epi.out_dtype == DT_BF16;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const float e0 = acc[i][j][2 * p], e1 = acc[i][j][2 * p + 1];
          // DPP quad_perm [1, 0, 3, 2]: the neighbour's row R (odd lane) or R+1 (even)
          const float recv = __uint_as_float(__builtin_amdgcn_mov_dpp(
              __float_as_uint(bit_pick(odd_mask, e0, e1)), 0xB1, 0xf, 0xf, false));
          const float lo = bit_pick(odd_mask, recv, e0);
          const float hi = bit_pick(odd_mask, e1, recv);
          pk[i][j][p] = bf ? (static_cast<uint32_t>(narrow_bf16(lo)) |
                              (static_cast<uint32_t>(narrow_bf16(hi)) << 16))
                           : (static_cast<uint32_t>(narrow_f16(lo)) |
                              (static_cast<uint32_t>(narrow_f16(hi)) << 16));
        }
  };
  auto put = [&](int64_t zz, int mm, int nn) {
    const int LDC = static_cast<int>(a.ldc);
    char* Cz = static_cast<char*>(a.C) + zz * a.sC * 2;
    const auto rC = rsrc(Cz, static_cast<uint32_t>(static_cast<int64_t>(M) * LDC * 2));
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int ce = (nn + wn * WTN + 32 * j + lrow) & ~1;
        const int rb = mm + wm * WTM + 32 * i + 4 * lhalf + (odd_lane ? 1 : 0);
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const int row = rb + 8 * (p >> 1) + 2 * (p & 1);
          const uint32_t off = (row < M && ce < N) ? static_cast<uint32_t>(row * LDC + ce) * 2u : OOB;
          __builtin_amdgcn_raw_buffer_store_b32(pk[i][j][p], rC, off, 0, 0);
        }
      }
  };

  auto put32 = [&](int64_t zz, int mm, int nn) {
    const int LDC = static_cast<int>(a.ldc);
    char* Cz = static_cast<char*>(a.C) + zz * a.sC * 4;
    const auto rC = rsrc(Cz, static_cast<uint32_t>(static_cast<int64_t>(M) * LDC * 4));
#pragma unroll
    for (int i = 0; i < (HOLD ? FM : 0); ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int cl = nn + wn * WTN + 32 * j + lrow;
        const int rb = mm + wm * WTM + 32 * i + 4 * lhalf;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rb + 8 * (r >> 2) + (r & 3);
          const uint32_t off = (row < M && cl < N) ? static_cast<uint32_t>(row * LDC + cl) * 4u : OOB;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(held[i][j][r]), rC, off, 0, 0);
        }
      }
  };

  int64_t z;
  int m0, n0;
  bool have = tile(0, z, m0, n0);
  if (have) issue(z, m0, n0, 0);
  int slot = 0;
  for (int64_t q = 0; have; ++q) {
    int64_t zn;
    int m0n, n0n;
    const bool next = tile(q + 1, zn, m0n, n0n);
    wait_vm<0>();  // this tile's operands (and the previous tile's stores) are complete
    lds_barrier();  // every wave's loads have landed; every wave is done with the other slot

    const u32x4* LA = ringA + slot * A_STAGE;
    const u32x4* LB = ringB + slot * B_STAGE;
    const int bslot = (static_cast<int>(ringB - lds) + slot * B_STAGE) * 16;
    u32x4 fa[4][FM], fb[4][FN];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (!BROW) {
          fb[s][j] = LB[b_base + j * 256 + ((2 * s + lhalf) ^ bperm)];
          continue;
        }
        const lds_char* Lb = (const lds_char*)lds + bslot + 16 * s * (BN * 2) + btr[j];
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)Lb);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Lb + 4 * (BN * 2)));
        fb[s][j] = u32x4{__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3))};
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[s][i] = LA[a_base + i * 256 + ((2 * s + lhalf) ^ perm)];
    }
    __builtin_amdgcn_sched_barrier(0);
    if (next) issue(zn, m0n, n0n, slot ^ 1);
    if (pend) {  // the previous tile's C
      if constexpr (SMAX) put(zp, m0p, n0p);
      if constexpr (HOLD) put32(zp, m0p, n0p);
    }
    pend = false;
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mma<T>(fa[s][i], fb[s][j], acc[i][j]);

    if constexpr (SMAX) {
      // P = softmax(scale S) along each row, columns past N at -inf. Each wave
      // reduces its own 64 columns: the row maximum m_w (halving exchange, so lane
      // `own` holds row own), then e = exp(s - m_w) and the sum s_w of e. After one
      // barrier the lane owning a row merges the 8 waves' (m_w, s_w) as the online
      // softmax does: M = max m_w, S = sum s_w exp(m_w - M), and scales its wave's
      // e by exp(m_w - M) / S. Per-row values reach the other lanes of the wave
      // through the wave's own LDS row (a wave's LDS accesses complete in order).
      // exp is the hardware exp2 of the argument times log2(e).
      const float scl = a.epi.scale;
      const int h = lane >> 5, q = lane & 31;
      const int own = 32 * (q >> 4) + 8 * ((q & 15) >> 2) + 4 * h + (q & 3);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const bool cin = n0 + wn * WTN + 32 * j + lrow < N;
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = cin ? acc[i][j][r] * scl : -INFINITY;
        }
      float* const wrow = sm_w + wave * BM;
      float rv[FM][16];
      auto row_values = [&]() {  // wrow at the rows of this lane's registers
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(wrow + 32 * i + 8 * r4 + 4 * h);
#pragma unroll
            for (int t = 0; t < 4; ++t) rv[i][4 * r4 + t] = v[t];
          }
      };
      float x[32];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[16 * i + r] = fmaxf(acc[i][0][r], acc[i][1][r]);
      const float mw = halve32<true>(x, lane);
      // a wave whose columns are all past N has m_w = -inf: subtract 0 instead (e = 0)
      wrow[own] = mw == -INFINITY ? 0.f : mw;
      row_values();
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = __expf(acc[i][j][r] - rv[i][r]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[16 * i + r] = acc[i][0][r] + acc[i][1][r];
      const float sw = halve32<false>(x, lane);
      sm_part[wave * BM + own] = float2{mw, sw};
      lds_barrier();
      float2 pw[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) pw[w] = sm_part[w * BM + own];
      float mx = pw[0].x;
#pragma unroll
      for (int w = 1; w < NW; ++w) mx = fmaxf(mx, pw[w].x);
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += pw[w].y * __expf(pw[w].x - mx);
      wrow[own] = __expf(mw - mx) * (1.f / sum);
      row_values();
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] *= rv[i][r];
    }
    if (defer) {
      if constexpr (SMAX) pack();
      if constexpr (HOLD) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) held[i][j] = acc[i][j];
      }
      pend = true;
      zp = z;
      m0p = m0;
      n0p = n0;
    } else {
      store_tile<FM, FN, WTM, WTN, NW, static_cast<int>(sizeof(lds))>(
          out, acc, reinterpret_cast<float*>(lds), m0, n0, wm, wn, wave, lane, z);
    }
    have = next;
    z = zn;
    m0 = m0n;
    n0 = n0n;
    slot ^= 1;
  }
  if (pend) {
    if constexpr (SMAX) put(zp, m0p, n0p);
    if constexpr (HOLD) put32(zp, m0p, n0p);
  }
}

template <typename T, int BM, int BN, int WGM, int WGN, bool BROW, bool SMAX = false>
hipError_t launch_m16s(const LaunchArgs& a, hipStream_t s) {
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * a.batch;
  // a.split: the workgroups the device keeps resident (set at plan time); a multiple
  // of 8 so each XCD gets the same number
  int64_t g = a.split > 1 ? a.split : 512;
  if (tiles < g) g = (tiles + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_m16s_kernel<T, BM, BN, WGM, WGN, BROW, SMAX>), dim3(static_cast<unsigned>(g)),
                     dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}

// SFX "" for row-major B [K x N], "_nk" for B given transposed [N x K]
#define G15_M16S(T, TN, BM, BN, WGM, WGN, BROW, SFX)                                           \
  {"m16s_" TN "_" #BM "x" #BN "x64_w" #WGM "x" #WGN SFX, KIND_K1, T::code, BM, BN, 64,          \
   64 * WGM * WGN, 2 * (BM + BN) * 128, 1, 1, launch_m16s<T, BM, BN, WGM, WGN, BROW>, 1,        \
   BROW ? 0 : 1}
#define G15_M16S_ALL(T, TN, BROW, SFX)                                      \
  G15_M16S(T, TN, 128, 128, 2, 2, BROW, SFX), G15_M16S(T, TN, 128, 256, 2, 4, BROW, SFX), \
      G15_M16S(T, TN, 256, 128, 4, 2, BROW, SFX)

const KernelEntry kM16S[] = {
    G15_M16S_ALL(bf16_t, "bf16", true, ""),    G15_M16S_ALL(f16_t, "f16", true, ""),
    G15_M16S_ALL(bf16_t, "bf16", false, "_nk"), G15_M16S_ALL(f16_t, "f16", false, "_nk"),
};

}  // namespace

hipError_t launch_attention_probs(const LaunchArgs& a, bool bf16, bool b_rowmajor, hipStream_t s) {
  if (a.K > 64 || a.N > 512 || a.epi.flags != 0) return hipErrorInvalidValue;
  if (bf16)
    return b_rowmajor ? launch_m16s<bf16_t, 64, 512, 1, 8, true, true>(a, s)
                      : launch_m16s<bf16_t, 64, 512, 1, 8, false, true>(a, s);
  return b_rowmajor ? launch_m16s<f16_t, 64, 512, 1, 8, true, true>(a, s)
                    : launch_m16s<f16_t, 64, 512, 1, 8, false, true>(a, s);
}

int mfma16_k1_entries(const KernelEntry** out) {
  *out = kM16S;
  return static_cast<int>(sizeof(kM16S) / sizeof(kM16S[0]));
}

}  // namespace g15
