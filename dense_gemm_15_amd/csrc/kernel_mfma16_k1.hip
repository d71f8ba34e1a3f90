// kernel_mfma16_k1.hip -- bf16 / fp16 matrix-core GEMM for products whose K fits
// one 64-deep slice: the attention scores S = Q K^T of heads of dimension 64 (the
// tutorial page's attention, section 2: a batched Q K^T whose output the softmax
// then reads). With K = 64 a 128 x 128 tile reads 32 KB of operands and writes
// 64 KB of fp32 C, so the writes are the work: each workgroup walks a strided list
// of tiles (batch items included) and keeps the next tile's operands loading while
// it multiplies and stores the current one, instead of one tile per workgroup with
// its loads, products and stores in sequence.
//
// Per tile: wait for its operands, barrier, read every A fragment (16-byte LDS
// reads) and every B fragment (the transposing read ds_read_b64_tr_b16, two per
// fragment) of the four 16-deep k-steps, issue the direct-to-LDS loads of the next
// tile into the other slot, run the products, and store C straight from the
// accumulators (DeepGEMM page, section 3.1: the tile's accumulators leave once; the
// 16-bit forms without LDS staging, which would need the slot being filled). All B
// fragments are read before the next tile's loads go out because the compiler makes
// a transposing read that follows a direct load wait for every load in flight. With
// fp32 C and no epilogue the 8-wave tiles hold a tile's C in registers and store it
// while the next tile's products run.
//
// Register-load form (the "_u" configurations): rows of any 2-byte alignment, so K
// or the row strides need not be multiples of 8 elements (4095 x 4097 x 63 without
// padded copies). Each lane loads the chunks the direct loads would fill into
// registers and writes them to the other slot after the products.
//
// LDS (as in kernel_mfma16_nt.hip for m16t): an A slot is BM rows of 64 k, 16-byte
// chunk c of row r at c ^ (r & 7) ^ ((r >> 3) & 3); a B slot is 64 rows (k) of BN
// columns, chunk c of row k at c ^ (4 (k & 3)). Slots of k at or past K are zeroed
// once (K is the same for every tile and the loads never write them); rows past M
// and columns past N keep whatever the slot held, which only reaches outputs that
// are not stored.
//
// Tile order (see `tile` below): whole batch items per XCD, else whole tile rows per
// XCD, so that each XCD's stores fill contiguous stretches of C.
#include "m16_common.hpp"

namespace g15 {
namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

template <typename T, int BM, int BN, int WGM, int WGN, bool BROW, bool UN>
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
    a_kin[i] = chk * 8 < K;  // a chunk is wholly inside K or past it: K is a multiple of 8,
                             // or A arrives in rows zero-padded to one (the padded-copy mode)
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
  // k at or past K: zero those chunks of both slots once (the register-load form
  // writes every chunk of a slot for every tile)
#pragma unroll
  for (int s = 0; s < (UN ? 0 : 2); ++s) {
#pragma unroll
    for (int i = 0; i < AI; ++i)
      if (!a_kin[i]) ringA[s * A_STAGE + (wave * AI + i) * 64 + lane] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < BI; ++i)
      if (b_row[i] >= K) ringB[s * B_STAGE + (wave * BI + i) * 64 + lane] = u32x4{0u, 0u, 0u, 0u};
  }

  // The q-th tile of this workgroup: batch item z and tile origin (m0, n0), or false
  // past the end. Workgroup w runs on XCD w % 8; C leaves fastest when each XCD
  // writes contiguous regions (measured with stores alone, 4096 x 4096 fp32 C in
  // 256 x 128 tiles: 11.3 us with whole tile rows per XCD against 13.2 us for
  // 8 x 4 tile blocks). Three orders:
  //  * 8 or more batch items: XCD x takes the items x, x + 8, ...;
  //  * else with 8 or more tile rows (in all items), 32 or more or a multiple of 8:
  //    XCD x takes the tile rows x, x + 8, ..., its workgroups walking them row by
  //    row;
  //  * else the tiles in the XCD-aware order of tile_of.
  // In the last two a thin last tile column (N % BN at most BN / 4) goes after every
  // other tile of the XCD (or of the grid): the last round of a workgroup's tiles is
  // then the cheap one (at 4095 x 4097 on 256 x 128 tiles, 512 full tiles in two
  // rounds of 256 workgroups and the 16 one-column tiles after them, not 16 full
  // tiles in a third round). The tile_of order also puts a thin last tile row last.
  const int64_t G = gridDim.x;
  const bool by_item = batch >= 8 && G % 8 == 0;
  const int64_t trows = batch * tiles_m;
  const bool by_row = !by_item && G % 8 == 0 && trows >= 8 && (trows % 8 == 0 || trows >= 32);
  const int mn = (N % BN != 0 && N > BN && N % BN <= BN / 4) ? N / BN : tiles_n;
  const int mm = (!by_row && M % BM != 0 && M > BM && M % BM <= BM / 4) ? M / BM : tiles_m;
  const int64_t main_per_item = static_cast<int64_t>(mm) * mn;
  auto tile = [&](int64_t q, int64_t& z, int& m0, int& n0) -> bool {
    int tm, tn;
    if (by_item) {
      // XCD x takes the items z = x, x + 8, ...; its G / 8 workgroups stride over the
      // concatenated tiles of those items
      const int64_t x = blockIdx.x % 8, gx = G / 8;
      const int64_t u = blockIdx.x / 8 + q * gx;
      const int64_t zi = u / per_item;
      z = zi * 8 + x;
      const int64_t r = u - zi * per_item;
      if (z >= batch) return false;
      tm = static_cast<int>(r / tiles_n);
      tn = static_cast<int>(r - static_cast<int64_t>(tm) * tiles_n);
    } else if (by_row) {
      // XCD x takes the tile rows x, x + 8, ... (row R is tile row R % tiles_m of item
      // R / tiles_m): first their tiles left of a thin last column, then those
      const int64_t x = blockIdx.x % 8, gx = G / 8;
      const int64_t u = blockIdx.x / 8 + q * gx;
      const int64_t rows_x = (trows - x + 7) / 8;
      const int64_t thin = tiles_n - mn;
      int64_t ri;
      if (u < rows_x * mn) {
        ri = u / mn;
        tn = static_cast<int>(u - ri * mn);
      } else {
        const int64_t e = u - rows_x * mn;
        if (e >= rows_x * thin) return false;
        ri = e / thin;
        tn = mn + static_cast<int>(e - ri * thin);
      }
      const int64_t R = x + 8 * ri;
      z = R / tiles_m;
      tm = static_cast<int>(R - z * tiles_m);
    } else {
      const int64_t t = blockIdx.x + q * G;
      if (t >= batch * per_item) return false;
      if (t < batch * main_per_item) {
        z = t / main_per_item;
        tile_of(static_cast<int>(t - z * main_per_item), mm, mn, tm, tn);
      } else {
        // the thin strips: last tile column (every tile row), then last tile row
        const int64_t edge = per_item - main_per_item;
        const int64_t e = t - batch * main_per_item;
        z = e / edge;
        const int r = static_cast<int>(e - z * edge);
        if (mn < tiles_n && r < tiles_m) {
          tm = r;
          tn = mn;
        } else {
          tm = mm;
          tn = mn < tiles_n ? r - tiles_m : r;
        }
      }
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

  // Register-load form (rows of any 2-byte alignment: K or the row stride not a
  // multiple of 8 elements, or an unaligned base): each lane loads the same 16-byte
  // chunks the direct loads would, as 16-byte loads from 2-byte aligned addresses
  // (which the memory system serves like aligned ones), and writes them to the slot
  // after the tile's products. A chunk that straddles the end of a row (v < 8 of its
  // elements inside) loads instead the 8 elements that end the row and shifts them
  // down by 8 - v elements, zeros coming in at the top: one load per chunk either
  // way, and no address outside the row. Rows shorter than 8 elements take element
  // loads. Chunks past M, N or K are zero.
  u32x4 ra[UN ? AI : 1], rb[UN ? BI : 1];
  auto shift_down = [](u32x4 w, int v) -> u32x4 {
    // w holds elements e .. e + 7 of which the top v are wanted at the bottom
    const int sh = 8 - v;  // 1 .. 7 elements
    const int d = sh >> 1;
    uint32_t y[5];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x1 = i + 1 < 4 ? w[i + 1] : 0u, x2 = i + 2 < 4 ? w[i + 2] : 0u;
      const uint32_t x3 = i + 3 < 4 ? w[i + 3] : 0u;
      y[i] = d == 0 ? w[i] : d == 1 ? x1 : d == 2 ? x2 : x3;
    }
    y[4] = 0u;
    const uint32_t bits = (sh & 1) ? 16u : 0u;
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_alignbit(y[i + 1], y[i], bits);
    return r;
  };
  // the chunk at p with `valid` (0 .. 8) leading elements inside a row of row_len
  auto chunk = [&](const uint16_t* p, int valid, int row_len) -> u32x4 {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row_len >= 8) {
      if (valid > 0) {
        __builtin_memcpy(&v, valid >= 8 ? p : p + valid - 8, 16);
        if (valid < 8) v = shift_down(v, valid);
      }
    } else if (valid > 0) {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = e < valid ? p[e] : 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = h[2 * e] | (h[2 * e + 1] << 16);
    }
    return v;
  };
  auto load_regs = [&](int64_t z, int m0, int n0) {
    const uint16_t* Az = static_cast<const uint16_t*>(a.A) + z * a.sA;
    const uint16_t* Bz = static_cast<const uint16_t*>(a.B) + z * a.sB;
#pragma unroll
    for (int i = 0; i < (UN ? AI : 0); ++i) {
      const int gm = m0 + a_row[i];
      const int k0 = static_cast<int>(a_koff[i]);
      const int valid = gm < M ? min(max(K - k0, 0), 8) : 0;
      ra[i] = chunk(Az + static_cast<int64_t>(gm < M ? gm : 0) * LDA + k0, valid, K);
    }
#pragma unroll
    for (int i = 0; i < (UN ? BI : 0); ++i) {
      const int gn = n0 + b_col[i];
      if constexpr (BROW) {
        const int valid = b_row[i] < K ? min(max(N - gn, 0), 8) : 0;
        rb[i] = chunk(Bz + static_cast<int64_t>(b_row[i] < K ? b_row[i] : 0) * LDB + gn, valid, N);
      } else {
        const int valid = gn < N ? min(max(K - b_row[i], 0), 8) : 0;
        rb[i] = chunk(Bz + static_cast<int64_t>(gn < N ? gn : 0) * LDB + b_row[i], valid, K);
      }
    }
  };
  auto commit_regs = [&](int slot) {
#pragma unroll
    for (int i = 0; i < (UN ? AI : 0); ++i) ringA[slot * A_STAGE + (wave * AI + i) * 64 + lane] = ra[i];
#pragma unroll
    for (int i = 0; i < (UN ? BI : 0); ++i) ringB[slot * B_STAGE + (wave * BI + i) * 64 + lane] = rb[i];
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
  // fp32 C without epilogue on the 8-wave tiles (their registers have room for the
  // held tile): a tile's C leaves one tile later, right after the next tile's loads
  // are issued, and is in flight during that tile's products. (Spreading the stores
  // between the k-steps measured slower. The memory system takes this layout's
  // 4-byte stores, two 128-byte row pieces per instruction, at full write bandwidth:
  // 6.3 TB/s measured with stores alone for a 4096 x 4096 fp32 C.)
  constexpr bool HOLD = NW == 8;
  const bool defer = HOLD && a.epi.out_dtype == DT_F32 && a.epi.flags == 0;
  // The tile loop, compiled separately for the held-C form (DEFER) and the other:
  // with the choice known at compile time the held registers are live only from
  // the copy at a tile's end to their stores in the next iteration.
  auto run = [&](auto defer_tag) {
    constexpr bool DEFER = decltype(defer_tag)::value;
    f32x16 held[HOLD ? FM : 1][HOLD ? FN : 1];
    bool pend = false;
    int64_t zp = 0;
    int m0p = 0, n0p = 0;
    // block b (row i = b / FN, column j = b % FN of the wave's blocks) of the held tile
    auto put_block = [&](int64_t zz, int mm, int nn, int b) {
      const int LDC = static_cast<int>(a.ldc);
      char* Cz = static_cast<char*>(a.C) + zz * a.sC * 4;
      const auto rC = rsrc(Cz, static_cast<uint32_t>(static_cast<int64_t>(M) * LDC * 4));
      const int i = b / FN, j = b % FN;
      const int cl = nn + wn * WTN + 32 * j + lrow;
      const int rb = mm + wm * WTM + 32 * i + 4 * lhalf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rb + 8 * (r >> 2) + (r & 3);
        const uint32_t off = (row < M && cl < N) ? static_cast<uint32_t>(row * LDC + cl) * 4u : OOB;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(held[HOLD ? i : 0][HOLD ? j : 0][r]), rC,
                                              off, 0, 0);
      }
    };

    int64_t z;
    int m0, n0;
    bool have = tile(0, z, m0, n0);
    if (have) {
      if constexpr (UN) {
        load_regs(z, m0, n0);
        commit_regs(0);
      } else {
        issue(z, m0, n0, 0);
      }
    }
    int slot = 0;
    bool stored = false;  // the previous iteration issued the held tile's stores
    for (int64_t q = 0; have; ++q) {
      int64_t zn;
      int m0n, n0n;
      const bool next = tile(q + 1, zn, m0n, n0n);
      // Direct loads: this tile's operands have landed once at most the held tile's
      // stores, issued after them, are still in flight (vmcnt counts loads and stores
      // in issue order; 63 is its largest value). The register-load form wrote its
      // operands to the slot in the previous iteration.
      if constexpr (!UN) {
        if (DEFER && stored)
          wait_vm<(FM * FN * 16 < 63 ? FM * FN * 16 : 63)>();
        else
          wait_vm<0>();
      }
      lds_barrier();  // every wave's operands are in the slot; every wave is done with the other slot
      if constexpr (UN) {
        if (next) load_regs(zn, m0n, n0n);
      }
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
      if constexpr (!UN) {
        if (next) issue(zn, m0n, n0n, slot ^ 1);
      }
      __builtin_amdgcn_sched_barrier(0);

#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
      // the held tile's C, then the products (the stores are in flight meanwhile)
      const bool put = DEFER && pend;
      if constexpr (DEFER) {
        if (put) {
#pragma unroll
          for (int b = 0; b < FM * FN; ++b) put_block(zp, m0p, n0p, b);
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mma<T>(fa[s][i], fb[s][j], acc[i][j]);
      stored = put;
      pend = false;
      // the next tile's operands into the other slot (every wave read it before this
      // iteration's barrier); the registers are free again for the epilogue
      if constexpr (UN) {
        if (next) commit_regs(slot ^ 1);
      }

      if constexpr (DEFER) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) held[i][j] = acc[i][j];
        pend = true;
        zp = z;
        m0p = m0;
        n0p = n0;
      } else {
        store_tile_rt<FM, FN, WTM, WTN, NW, static_cast<int>(sizeof(lds))>(
            out, acc, reinterpret_cast<float*>(lds), m0, n0, wm, wn, wave, lane, z);
      }
      have = next;
      z = zn;
      m0 = m0n;
      n0 = n0n;
      slot ^= 1;
    }
    if (pend) {
#pragma unroll
      for (int b = 0; b < FM * FN; ++b) put_block(zp, m0p, n0p, b);
    }
  };
  if constexpr (HOLD) {
    if (defer) {
      run(std::true_type{});
      return;
    }
  }
  run(std::false_type{});
}

template <typename T, int BM, int BN, int WGM, int WGN, bool BROW, bool UN>
hipError_t launch_m16s(const LaunchArgs& a, hipStream_t s) {
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * a.batch;
  // a.split: the workgroups the device keeps resident (set at plan time); a multiple
  // of 8 so each XCD gets the same number
  int64_t g = a.split > 1 ? a.split : 512;
  if (tiles < g) g = (tiles + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_m16s_kernel<T, BM, BN, WGM, WGN, BROW, UN>),
                     dim3(static_cast<unsigned>(g)), dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}

// SFX "" for row-major B [K x N], "_nk" for B given transposed [N x K]; the "_u"
// forms load rows of any alignment through registers (no 16-byte row requirement)
#define G15_M16S(T, TN, BM, BN, WGM, WGN, BROW, SFX, UN)                                       \
  {"m16s_" TN "_" #BM "x" #BN "x64_w" #WGM "x" #WGN SFX, KIND_K1, T::code, BM, BN, 64,          \
   64 * WGM * WGN, 2 * (BM + BN) * 128, UN ? 0 : 1, UN ? 0 : 1,                                 \
   launch_m16s<T, BM, BN, WGM, WGN, BROW, UN>, 1, BROW ? 0 : 1}
#define G15_M16S_ALL(T, TN, BROW, SFX)                                                    \
  G15_M16S(T, TN, 128, 128, 2, 2, BROW, SFX, false),                                      \
      G15_M16S(T, TN, 128, 256, 2, 4, BROW, SFX, false),                                  \
      G15_M16S(T, TN, 256, 128, 4, 2, BROW, SFX, false),                                  \
      G15_M16S(T, TN, 256, 128, 4, 2, BROW, SFX "_u", true)

const KernelEntry kM16S[] = {
    G15_M16S_ALL(bf16_t, "bf16", true, ""),    G15_M16S_ALL(f16_t, "f16", true, ""),
    G15_M16S_ALL(bf16_t, "bf16", false, "_nk"), G15_M16S_ALL(f16_t, "f16", false, "_nk"),
};

}  // namespace

int mfma16_k1_entries(const KernelEntry** out) {
  *out = kM16S;
  return static_cast<int>(sizeof(kM16S) / sizeof(kM16S[0]));
}

}  // namespace g15
