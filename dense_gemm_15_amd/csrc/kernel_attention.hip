// kernel_attention.hip -- the attention probabilities P = softmax(scale Q K^T) per
// batch item in one kernel (tutorial page, section 2: the product Q K^T and the row
// softmax that follows it; DeepGEMM page, section 3.4: the softmax denominator
// accumulated in FP32). With at most 512 keys a whole row of scores fits one
// workgroup, so the scores stay in registers and only P is written.
//
// Tile: 32 query rows x all 512 keys; 4 waves side by side, wave w owns keys
// 128 w .. 128 w + 127 (a 32 x 128 wave tile, four 32x32 MFMA blocks). The keys of
// one batch item (64 KB at D = 64) sit in one LDS slot for as long as the
// workgroup works on that item; the 32-row Q tiles are double-buffered (4 KB each).
// About 74 KB of LDS in all, so two workgroups share a CU and one's softmax and
// stores overlap the other's loads and products.
//
// Work split: the tiles in item-major order are cut into equal contiguous runs,
// one per workgroup; the runs of consecutive workgroups of one XCD (workgroups
// reach the 8 XCDs round-robin) are adjacent, so the workgroups that share an item
// share an L2. A workgroup reloads the keys only where its run crosses into the
// next item.
//
// Softmax per tile, in base 2 (exp(scale s) = 2^(c s), c = scale log2 e): each wave
// reduces its 128 keys to a per-row maximum m_w of c s and the sum s_w of
// e = 2^(c s - m_w) by a halving exchange over the 32 lanes that hold a row
// (v_permlane16_swap, then DPP moves; no LDS); after one barrier the lanes owning a
// row merge the waves' (m_w, s_w) as the online softmax does (M = max m_w,
// S = sum s_w 2^(m_w - M)) and the wave scales e by 2^(m_w - M) / S. A 16-bit P of
// even N is packed into registers and stored one tile late, after the next tile's
// loads are issued.
//
// LDS layouts (as the m16 kernels): a Q slot is 32 rows of 64 k, chunk c of row r
// at c ^ (r & 7) ^ ((r >> 3) & 3); keys as K^T [D x N]: 64 rows (k) of 512 keys,
// chunk c of row k at c ^ (4 (k & 3)), read with ds_read_b64_tr_b16; keys as
// stored [N x D]: 512 rows (keys) laid out like Q.
#include "attention.hpp"
#include "m16_common.hpp"

namespace g15 {
namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int BM = 32;   // query rows per tile
constexpr int BN = 512;  // keys per tile: every key of a row
constexpr int NW = 4;    // waves
constexpr int WTN = BN / NW, FN = WTN / 32;
constexpr int A_STAGE = BM * 8, B_STAGE = BN * 8;  // 16-byte chunks
constexpr int BI = B_STAGE / 64 / NW;               // key loads per wave

enum { OP_MAX = 0, OP_MIN = 1, OP_ADD = 2 };
template <int OP>
__device__ __forceinline__ float comb(float a, float b) {
  return OP == OP_MAX ? fmaxf(a, b) : OP == OP_MIN ? fminf(a, b) : a + b;
}

// m ? a : b as a bit select (v_bfi_b32) behind inline assembly: written as a
// conditional, the compiler turns the choice into a lane-dependent index into the
// value registers, i.e. a compare-and-select chain per value.
__device__ __forceinline__ float bit_pick(uint32_t m, float a, float b) {
  float r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(a), "v"(b));
  return r;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(v), CTRL, 0xf, 0xf, false));
}

// One halving round: a lane keeps the half of its H-value pairs that lane bit BIT
// selects and combines it with the partner's copy (partner: the DPP pattern CTRL,
// which differs in bit BIT and agrees in the bits of the earlier rounds).
template <int OP, int H, int BIT, int CTRL>
__device__ __forceinline__ void halve_round(float (&x)[16], int lane) {
  const uint32_t up = (lane & BIT) != 0 ? 0xffffffffu : 0u;
#pragma unroll
  for (int q = 0; q < H; ++q) {
    const float send = bit_pick(up, x[q], x[q + H]);
    const float keep = bit_pick(up, x[q + H], x[q]);
    x[q] = comb<OP>(keep, dpp<CTRL>(send));
  }
}

// Reduction of 16 values per lane over the 32 lanes of each half-wave: lane bit 4
// by v_permlane16_swap (it exchanges the odd 16-lane rows of its first operand with
// the even rows of its second), bits 3, 2, 1 by DPP moves from lane l ^ 15
// (row_mirror), l ^ 7 (row_half_mirror) and l ^ 2, bit 0 by a full exchange with
// lane l ^ 1. Lanes 2i and 2i+1 of each half end with the reduction of value i, in
// a fixed order.
template <int OP>
__device__ __forceinline__ float halve16(float (&x)[16], int lane) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[q]), __float_as_uint(x[q + 8]),
                                                    false, false);
    x[q] = comb<OP>(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  halve_round<OP, 4, 8, 0x140>(x, lane);  // row_mirror
  halve_round<OP, 2, 4, 0x141>(x, lane);  // row_half_mirror
  halve_round<OP, 1, 2, 0x4E>(x, lane);   // quad_perm 2 3 0 1
  return comb<OP>(x[0], dpp<0xB1>(x[0]));  // quad_perm 1 0 3 2
}

// two workgroups per CU: at most 256 registers per lane (2 waves per SIMD)
template <typename T, bool BROW>
__global__ __launch_bounds__(64 * NW, 2) void attention_probs_kernel(LaunchArgs a) {
  __shared__ u32x4 lds[2 * A_STAGE + B_STAGE];
  __shared__ float2 sm_part[NW * BM];                // per wave and row: (max, sum)
  __shared__ __align__(16) float sm_w[NW * BM];      // per wave and row, wave-private
  u32x4* const ringA = lds;
  u32x4* const Bs = lds + 2 * A_STAGE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = static_cast<int>(a.M), N = static_cast<int>(a.N), K = static_cast<int>(a.K);
  const int LDA = static_cast<int>(a.lda), LDB = static_cast<int>(a.ldb);
  const int tiles_m = (M + BM - 1) / BM;
  const int64_t total = static_cast<int64_t>(tiles_m) * a.batch;
  // runs: virtual index v puts the G / 8 workgroups of one XCD on adjacent runs
  const int64_t G = gridDim.x;  // a multiple of 8
  const int64_t v = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;
  const int64_t t_begin = v * total / G, t_end = (v + 1) * total / G;
  if (t_begin >= t_end) return;

  // Q loads: wave w fills slot rows 8 w .. 8 w + 7, lane l row + l / 8, slot chunk
  // l % 8, which holds logical chunk a_chk.
  const int a_chk = (lane & 7) ^ (lane >> 3) ^ (wave & 3);
  const int a_row = wave * 8 + (lane >> 3);
  const bool a_kin = a_chk * 8 < K;  // K is a multiple of 8
  // key loads: load s = wave BI + i fills slot row s (k; keys as K^T, lane l key
  // chunk l ^ 4 (s & 3)) or slot rows 8 s .. 8 s + 7 (keys as stored: lane l key
  // 8 s + l / 8, k chunk (l & 7) ^ (l >> 3) ^ (s & 3)); both depend on s & 3 only
  // through the chunk, so each is computed where it is used
  auto k_chunk = [&](int s) -> int {  // k of this lane's chunk (keys as stored), or K past it
    const int chk = (lane & 7) ^ (lane >> 3) ^ (s & 3);
    return chk * 8 < K ? chk * 8 : K;
  };
  // k at or past K: zero those chunks once (the loads never write them)
#pragma unroll
  for (int s = 0; s < 2; ++s)
    if (!a_kin) ringA[s * A_STAGE + wave * 64 + lane] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int s = wave * BI + i;
    if (BROW ? s >= K : k_chunk(s) >= K) Bs[s * 64 + lane] = u32x4{0u, 0u, 0u, 0u};
  }

  auto issue_q = [&](int64_t z, int m0, int slot) {
    const uint16_t* Az = static_cast<const uint16_t*>(a.A) + z * a.sA;
    const auto rA = rsrc(Az, static_cast<uint32_t>(static_cast<int64_t>(M) * LDA * 2));
    const int gm = m0 + a_row;
    const uint32_t off = (a_kin && gm < M) ? static_cast<uint32_t>(gm * LDA + a_chk * 8) * 2u : OOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void*)(ringA + slot * A_STAGE + wave * 64), 16,
                                             off, 0, 0, 0);
  };
  auto issue_k = [&](int64_t z) {
    const uint16_t* Bz = static_cast<const uint16_t*>(a.B) + z * a.sB;
    const auto rB = rsrc(Bz, static_cast<uint32_t>(static_cast<int64_t>(BROW ? K : N) * LDB * 2));
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int s = wave * BI + i;
      uint32_t off;
      if constexpr (BROW) {
        const int gn = (lane ^ (4 * (s & 3))) * 8;
        off = (s < K && gn < N) ? static_cast<uint32_t>(s * LDB + gn) * 2u : OOB;
      } else {
        const int gn = s * 8 + (lane >> 3), kc = k_chunk(s);
        off = (kc < K && gn < N) ? static_cast<uint32_t>(gn * LDB + kc) * 2u : OOB;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void*)(Bs + s * 64), 16, off, 0, 0, 0);
    }
  };

  // fragment addresses (as the m16 kernels): Q row lane & 31, k chunk 2 s + lane / 32;
  // keys as K^T by the transposing read (group g = lane / 16, t = lane % 16: row
  // 8 (g / 2) + t / 4, key wave WTN + 32 j + 16 (g % 2) + 4 (t % 4)); keys as stored:
  // row wave WTN + 32 j + (lane & 31), laid out like Q
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int a_base = lrow * 8;
  const int perm = (lrow & 7) ^ ((lrow >> 3) & 3);
  const int b_base = (wave * WTN + lrow) * 8;
  const int bperm = (lrow & 7) ^ (((wave * WTN + lrow) >> 3) & 3);
  int btr[FN];
  {
    const int g = lane >> 4, t = lane & 15;
    const int kr = 8 * (g >> 1) + (t >> 2);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = wave * WTN + 32 * j + 16 * (g & 1) + 4 * (t & 3);
      btr[j] = kr * (BN * 2) + (((n >> 3) ^ (4 * (kr & 3))) << 4) + (n & 7) * 2;
    }
  }
  const int bbyte = static_cast<int>(Bs - lds) * 16;

  // deferred 16-bit P: registers 2p and 2p+1 of a block are rows R and R+1 of one
  // key and lanes l, l^1 hold neighbouring keys; after one exchange the even lane
  // holds keys (c, c+1) of row R and the odd lane (c-1, c) of row R+1
  const bool defer = a.epi.out_dtype != DT_F32 && (N & 1) == 0 && (a.ldc & 1) == 0;
  const bool bf_out = a.epi.out_dtype == DT_BF16;
  f32x16 acc[1][FN];
  uint32_t pk[FN][8];
  // rows R, R+1 of this lane's key converted as a pair (RNE), the neighbour's pair
  // fetched, and the row this lane stores picked bytewise: the even lane takes
  // (R, c) and (R, c+1), the odd lane (R+1, c-1) and (R+1, c). v_perm_b32 numbers
  // the bytes of its second operand 0-3 and of its first 4-7.
  const uint32_t pick = (lane & 1) != 0 ? 0x03020706u : 0x05040100u;
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  auto pack = [&]() {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const f32x2 e = {acc[0][j][2 * p], acc[0][j][2 * p + 1]};
        const uint32_t own2 = bf_out ? __builtin_bit_cast(uint32_t, __builtin_convertvector(e, bf16x2))
                                     : __builtin_bit_cast(uint32_t, __builtin_convertvector(e, f16x2));
        const uint32_t nb2 = __builtin_amdgcn_mov_dpp(own2, 0xB1, 0xf, 0xf, false);
        pk[j][p] = __builtin_amdgcn_perm(nb2, own2, pick);
      }
  };
  // a whole tile (32 rows inside M, all 512 keys): a per-lane byte offset fixed for
  // the kernel plus a uniform one per store (the row), no bounds checks
  uint32_t lane_off[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j)
    lane_off[j] = static_cast<uint32_t>((4 * lhalf + (lane & 1)) * static_cast<int>(a.ldc) +
                                        ((wave * WTN + 32 * j + lrow) & ~1)) * 2u;
  auto put = [&](int64_t zz, int mm) {
    const int LDC = static_cast<int>(a.ldc);
    char* Cz = static_cast<char*>(a.C) + zz * a.sC * 2;
    const auto rC = rsrc(Cz, static_cast<uint32_t>(static_cast<int64_t>(M) * LDC * 2));
    if (mm + BM <= M && N == BN) {
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const uint32_t row_off =
            static_cast<uint32_t>((mm + 8 * (p >> 1) + 2 * (p & 1)) * LDC) * 2u;  // uniform
#pragma unroll
        for (int j = 0; j < FN; ++j)
          __builtin_amdgcn_raw_buffer_store_b32(pk[j][p], rC, lane_off[j], row_off, 0);
      }
      return;
    }
    const int rb = mm + 4 * lhalf + (lane & 1);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int ce = (wave * WTN + 32 * j + lrow) & ~1;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int row = rb + 8 * (p >> 1) + 2 * (p & 1);
        const uint32_t off = (row < M && ce < N) ? static_cast<uint32_t>(row * LDC + ce) * 2u : OOB;
        __builtin_amdgcn_raw_buffer_store_b32(pk[j][p], rC, off, 0, 0);
      }
    }
  };
  LaunchArgs out = a;
  out.c_vec = 0;  // P straight from the registers

  int64_t t = t_begin;
  int64_t z = t / tiles_m;
  int m0 = static_cast<int>(t - z * tiles_m) * BM;
  int64_t zk = z;  // the item whose keys the slot holds
  issue_k(z);
  issue_q(z, m0, 0);
  int slot = 0;
  bool pend = false;
  int64_t zp = 0;
  int m0p = 0;
  // the softmax runs in base 2: exp(scale s) = 2^(c s) with c = scale log2(e), and
  // every exponential is the hardware exp2 (v_exp_f32)
  const float scl2 = a.epi.scale * 1.44269504088896341f;
  const int q = lane & 31;
  const int own = 8 * (q >> 3) + 4 * lhalf + ((q >> 1) & 3);  // the row this lane's reductions end on
  float* const wrow = sm_w + wave * BM;

  for (; t < t_end; ++t) {
    const bool next = t + 1 < t_end;
    const int64_t zn = (t + 1) / tiles_m;
    const int m0n = static_cast<int>(t + 1 - zn * tiles_m) * BM;
    wait_vm<0>();   // this tile's Q (and keys), and the stores of two tiles back
    lds_barrier();  // every wave's loads have landed; every wave is done with the other slot

    const u32x4* LA = ringA + slot * A_STAGE;
    u32x4 fa[4], fb[4][FN];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (!BROW) {
          fb[s][j] = Bs[b_base + j * 256 + ((2 * s + lhalf) ^ bperm)];
          continue;
        }
        const lds_char* Lb = (const lds_char*)lds + bbyte + 16 * s * (BN * 2) + btr[j];
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)Lb);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Lb + 4 * (BN * 2)));
        fb[s][j] = u32x4{__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3))};
      }
      fa[s] = LA[a_base + ((2 * s + lhalf) ^ perm)];
    }
    __builtin_amdgcn_sched_barrier(0);
    if (next) {
      if (zn != zk) {   // the run enters the next item: new keys, once every wave has
        lds_barrier();  // its key fragments in registers
        issue_k(zn);
        zk = zn;
      }
      issue_q(zn, m0n, slot ^ 1);
    }
    if (pend) put(zp, m0p);  // the previous tile's P
    pend = false;
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[0][j][r] = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[0][j] = mma<T>(fa[s], fb[s][j], acc[0][j]);

    // softmax of the 32 rows: lane l holds key wave WTN + 32 j + l % 32 of rows
    // 8 (r / 4) + 4 (l / 32) + r % 4, r = 0 .. 15
    // The scaled scores are c s with c = scale log2(e); their row maximum is c times
    // the maximum of s (the minimum for a negative scale), so s stays unscaled and
    // each exponential takes fma(s, c, -m). Keys past N (N < 512 only): s set to the
    // far end so the maximum ignores them, their exponentials to 0 afterwards.
    const bool neg = scl2 < 0.f;
    if (N < BN) {
      const float far = neg ? INFINITY : -INFINITY;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const bool cin = wave * WTN + 32 * j + lrow < N;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[0][j][r] = cin ? acc[0][j][r] : far;
      }
    }
    float x[16], rv[16];
    auto row_values = [&]() {  // wrow at the rows of this lane's registers
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 w4 = *reinterpret_cast<const f32x4*>(wrow + 8 * r4 + 4 * lhalf);
#pragma unroll
        for (int u = 0; u < 4; ++u) rv[4 * r4 + u] = w4[u];
      }
    };
    float m_raw;
    if (!neg) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float m = acc[0][0][r];
#pragma unroll
        for (int j = 1; j < FN; ++j) m = fmaxf(m, acc[0][j][r]);
        x[r] = m;
      }
      m_raw = halve16<OP_MAX>(x, lane);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float m = acc[0][0][r];
#pragma unroll
        for (int j = 1; j < FN; ++j) m = fminf(m, acc[0][j][r]);
        x[r] = m;
      }
      m_raw = halve16<OP_MIN>(x, lane);
    }
    // the wave's row maximum of c s: -inf when its keys all lie past N, and then 0 is
    // subtracted instead (e = 0); both lanes of a pair write the same value (a wave's
    // LDS accesses complete in order)
    const float mw = __builtin_isinf(m_raw) ? -INFINITY : m_raw * scl2;
    wrow[own] = mw == -INFINITY ? 0.f : mw;
    row_values();
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc[0][j][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[0][j][r], scl2, -rv[r]));
    if (N < BN) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const bool cin = wave * WTN + 32 * j + lrow < N;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[0][j][r] = cin ? acc[0][j][r] : 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float sm = acc[0][0][r];
#pragma unroll
      for (int j = 1; j < FN; ++j) sm += acc[0][j][r];
      x[r] = sm;
    }
    const float sw = halve16<OP_ADD>(x, lane);
    sm_part[wave * BM + own] = float2{mw, sw};
    lds_barrier();
    float mx = -INFINITY;
    float2 pw[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      pw[w] = sm_part[w * BM + own];
      mx = fmaxf(mx, pw[w].x);
    }
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum += pw[w].y * __builtin_amdgcn_exp2f(pw[w].x - mx);
    wrow[own] = __builtin_amdgcn_exp2f(mw - mx) * (1.f / sum);
    row_values();
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[0][j][r] *= rv[r];

    if (defer) {
      pack();
      pend = true;
      zp = z;
      m0p = m0;
    } else {
      store_tile_rt<1, FN, BM, WTN, NW, static_cast<int>(sizeof(lds))>(
          out, acc, reinterpret_cast<float*>(lds), m0, 0, 0, wave, wave, lane, z);
    }
    z = zn;
    m0 = m0n;
    slot ^= 1;
  }
  if (pend) put(zp, m0p);
}

template <typename T, bool BROW>
hipError_t launch(const LaunchArgs& a, hipStream_t s) {
  const int64_t total = ((a.M + BM - 1) / BM) * a.batch;
  // a.split: the workgroups the device keeps resident, a multiple of 8
  int64_t g = a.split >= 8 ? a.split : 512;
  if (total < g) g = (total + 7) / 8 * 8;
  hipLaunchKernelGGL((attention_probs_kernel<T, BROW>), dim3(static_cast<unsigned>(g)),
                     dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_probs(const LaunchArgs& a, bool bf16, bool b_rowmajor, hipStream_t s) {
  if (a.K > 64 || a.N > BN || a.epi.flags != 0) return hipErrorInvalidValue;
  if (bf16) return b_rowmajor ? launch<bf16_t, true>(a, s) : launch<bf16_t, false>(a, s);
  return b_rowmajor ? launch<f16_t, true>(a, s) : launch<f16_t, false>(a, s);
}

int attention_workgroups(int cu_count) { return (2 * cu_count + 7) / 8 * 8; }

}  // namespace g15
