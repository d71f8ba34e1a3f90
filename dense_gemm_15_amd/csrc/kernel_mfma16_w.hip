// kernel_mfma16_w.hip -- bf16 / fp16 matrix-core GEMM with one wave per SIMD:
// a 256 x 256 (or 256 x 128) tile on 4 waves, each wave a 128 x 128 (128 x 64)
// sub-tile of 16 x 16 blocks computed with v_mfma_f32_16x16x32_{bf16,f16}, its
// 256 (128) FP32 accumulators held in the accumulation registers (a wave alone on
// its SIMD has 512 registers per lane).
//
// Tiling follows the DeepGEMM page (sections 2.2, 3.1: block tile in shared
// memory, warp tile, per-thread register tile of accumulators; section 3.3:
// matrix instructions) and the SGEMM page's prefetch (section 2.3), re-cut for
// gfx950:
//  * K moves in 32-deep slices (one 16x16x32 k-step). A and B slices stream
//    global -> LDS directly (buffer_load ... lds) into a ring of R slots; the
//    slice read in slice kt is kt + 1, the one loaded is kt + R, so every load has
//    R - 1 slices of matrix work to land.
//  * One barrier per slice. Each wave waits for its own loads of slice kt + 1,
//    then the barrier makes every wave's loads visible and proves slot kt free.
//  * The slice's instruction order is fixed op by op (scheduling fences): a few
//    matrix ops, the barrier, then every op followed by its share of the next
//    slice's fragment reads and of the loads of slice kt + R.
//  * B row-major (the plain layout): slices land as stored (k rows of n) and B
//    fragments come from the transposing read ds_read_b64_tr_b16 (in each group
//    of 16 lanes, lane i gets 4 consecutive k of column n0 + i when lane t
//    addresses row k0 + t / 4, columns n0 + 4 (t % 4) .. +3), two per fragment.
//    B given transposed (Bt [N x K], "_nk") is loaded and read like A.
//  * The compiler makes an LDS read that may alias a direct-to-LDS load in flight
//    wait for every load (vmcnt(0)); the slice body takes its read and load slots
//    as separate restrict pointers, which tells it they do not alias, so the
//    loads of later slices stay in flight across the reads.
//
// LDS layouts (16-byte chunks, conflict-free for the 64-lane reads):
//  * A (and Bt) slot: rows of 64 bytes (32 k); chunk c of row r at c ^ ((r >> 1) & 3).
//    A fragment read: lane l reads row 16 i + (l & 15), chunk l >> 4. A 128-bit read
//    is served 16 lanes at a time; which row permutations keep those 16 lanes on
//    distinct banks was measured with an in-bounds probe of LDS access patterns
//    (this one: no extra cycle; ((r >> 2) & 3) and no permutation: one more).
//  * B slot (row-major): 32 k-rows of 2 BN bytes; chunk c of row k at c ^ h(k),
//    h(k) = 2 ((k & 3) | ((k >> 3) & 1) << 2): the 8 rows one 32-lane pass of the
//    transposing read touches get 8 distinct chunk pairs.
// Edges: rows past M, columns past N and k past K use out-of-range buffer offsets
// (loads return nothing, stores are dropped); an out-of-range direct load leaves
// its LDS slot untouched, so slots of k past K are zeroed by the loading wave.
#include "m16_common.hpp"

namespace g15 {
namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

template <typename T>
__device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mma16<bf16_t>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mma16<f16_t>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

constexpr int WBK = 32;  // K per slice

// f(integral_constant<int, I>) for I = B .. E-1, expanded at compile time (the
// slice body is too large for the loop unroller's limits)
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <int BM, int BN, int R>
struct WGeom {
  static constexpr int WTM = BM / 2, WTN = BN / 2;  // 2 x 2 waves
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static constexpr int A_SLOT = BM * WBK * 2, B_SLOT = BN * WBK * 2;  // bytes
  static constexpr int AI = A_SLOT / 4096, BI = B_SLOT / 4096;        // 1 KB loads per wave
  static constexpr int NV = AI + BI;
  static constexpr int RING = R * (A_SLOT + B_SLOT);
  static_assert(AI >= 1 && BI >= 1, "each wave loads at least 1 KB of each operand");
  static_assert(RING <= 163840, "ring exceeds gfx950 LDS");
};

// Epilogue of a wave's WTM x WTN sub-tile of 16 x 16 blocks at tile (m0, n0). The
// matrix ops take the B fragment as their first operand, so each block accumulates
// the transposed product and lane l holds four consecutive columns of one row:
// C[row][col + t], t = 0 .. 3, row = 16 i + l % 16, col = 16 j + 4 (l / 16). Scale,
// bias and GELU are applied in registers, the residual where the value is stored.
// With 16-byte aligned C rows (a.c_vec: C, the residual and their rows on 16 bytes,
// N % 8 == 0) a lane's four values leave as one 16-byte (fp32) or 8-byte (16-bit)
// store straight from the registers; otherwise one element at a time.
//
// The residual and the output type are template parameters, chosen once per
// launch: with a run-time residual test inside the store loop the compiler puts a
// wait for every vector-memory operation in flight where the two paths join, and
// on gfx950 stores count there too, so each block of stores would wait for the
// previous block's to reach memory.
// Scale, bias and GELU on a lane's four values of one block, each stage behind one
// uniform branch per block (sc is the scale, or 1 without EPI_SCALE; the bias reads
// as 0 without EPI_BIAS): with one wave per SIMD, per-element tests and selects in
// the store sequence cost more than the stores. 16-bit results take gelu16.
template <int OUT>
__device__ __forceinline__ f32x4 epi_block(const Epi& e, f32x4 v, f32x4 bias, float sc) {
  if (e.flags & (EPI_SCALE | EPI_BIAS)) {
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = v[t] * sc + bias[t];
  }
  if (e.flags & EPI_GELU) {
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = OUT == DT_F32 ? gelu(v[t]) : gelu16(v[t]);
  }
  return v;
}


template <int FM, int FN, int WTM, int WTN, bool HAS_R, int OUT>
__device__ __forceinline__ void store_tile_w(const LaunchArgs& a, f32x4 (&acc)[FM][FN], int m0,
                                             int n0, int wm, int wn, int lane, int64_t z) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const int M = static_cast<int>(a.M), N = static_cast<int>(a.N), LDC = static_cast<int>(a.ldc);
  const int lr = lane & 15, lg = lane >> 4;
  const Epi& e = a.epi;
  constexpr int ob = OUT == DT_F32 ? 4 : 2;
  char* Cz = static_cast<char*>(a.C) + z * a.sC * ob;
  const char* Rz = HAS_R ? static_cast<const char*>(e.resid) + z * a.sR * ob : Cz;
  const auto rC = rsrc(Cz, static_cast<uint32_t>(static_cast<int64_t>(M) * LDC * ob));
  const auto rR = rsrc(Rz, static_cast<uint32_t>(static_cast<int64_t>(M) * LDC * ob));
  const int row0 = m0 + wm * WTM + lr;      // + 16 i
  const int col0 = n0 + wn * WTN + 4 * lg;  // + 16 j + t
  // bias through a buffer descriptor: columns past N read as 0 with no branch (a
  // guarded load per element puts 32 divergent regions into the epilogue)
  f32x4 bj[FN];
  const auto rB = rsrc(e.bias, (e.flags & EPI_BIAS) ? static_cast<uint32_t>(N) * 4u : 0u);
  const float sc = (e.flags & EPI_SCALE) ? e.scale : 1.f;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const uint32_t col = static_cast<uint32_t>(col0 + 16 * j);
    if (a.c_vec) {  // N % 8 == 0: the four columns lie wholly inside or past N
      bj[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rB, col * 4u, 0, 0));
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        bj[j][t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rB, (col + t) * 4u, 0, 0));
    }
  }
  if (a.c_vec) {
    // Two neighbouring blocks j0 = 2p, j1 = 2p + 1 per step. Lanes 8 apart within
    // each 16-lane row exchange registers (DPP row rotate by 8) so that one store
    // covers rows 0-7 of the block row and the next rows 8-15, each row's 32 columns
    // j0, j1 by 8 lanes: whole 128-byte spans (fp32) instead of 64-byte halves.
    static_assert(FN % 2 == 0, "block pairs");
    const bool hi = lr >= 8;
    const int rlo = m0 + wm * WTM + (lr & 7);  // + 16 i (first store), + 8 (second)
    auto ror8 = [](float x) {
      return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
    };
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      uint32_t off[FN];  // [2p]: rows 0-7 of the pair, [2p + 1]: rows 8-15
      u32x4 res[FN];
#pragma unroll
      for (int q = 0; q < FN; ++q) {
        const int row = rlo + 16 * i + 8 * (q & 1);
        const int col = col0 + 16 * ((q & ~1) + (hi ? 1 : 0));  // N % 8 == 0: covers col + 3
        off[q] = (row < M && col < N) ? static_cast<uint32_t>(row * LDC + col) * ob : OOB;
        if constexpr (HAS_R) {  // the block row's residual loads all in flight at once
          if constexpr (OUT == DT_F32) {
            res[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rR, off[q], 0, 0));
          } else {
            const u32x2 h = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rR, off[q], 0, 0));
            res[q] = u32x4{h[0], h[1], 0u, 0u};
          }
        }
      }
#pragma unroll
      for (int p = 0; p < FN / 2; ++p) {
        const f32x4 v0 = epi_block<OUT>(e, acc[i][2 * p], bj[2 * p], sc);
        const f32x4 v1 = epi_block<OUT>(e, acc[i][2 * p + 1], bj[2 * p + 1], sc);
        f32x4 d[2];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float x = ror8(v1[t]), y = ror8(v0[t]);
          d[0][t] = hi ? x : v0[t];
          d[1][t] = hi ? v1[t] : y;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x4 v = d[h];
          const int q = 2 * p + h;
          if constexpr (OUT == DT_F32) {
            if constexpr (HAS_R)
#pragma unroll
              for (int t = 0; t < 4; ++t) v[t] += __uint_as_float(res[q][t]);
            __builtin_amdgcn_raw_buffer_store_b128(
                u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                      __float_as_uint(v[3])},
                rC, off[q], 0, 0);
          } else {
            if constexpr (HAS_R) {
              v[0] += widen16<OUT>(res[q][0] & 0xffffu);
              v[1] += widen16<OUT>(res[q][0] >> 16);
              v[2] += widen16<OUT>(res[q][1] & 0xffffu);
              v[3] += widen16<OUT>(res[q][1] >> 16);
            }
            const u32x2 w{pack16<OUT>(v[0], v[1]), pack16<OUT>(v[2], v[3])};
            __builtin_amdgcn_raw_buffer_store_b64(w, rC, off[q], 0, 0);
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = row0 + 16 * i;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      uint32_t off[4];
      float rv[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int col = col0 + 16 * j + t;
        off[t] = (row < M && col < N) ? static_cast<uint32_t>(row * LDC + col) * ob : OOB;
        if constexpr (HAS_R) {
          if constexpr (OUT == DT_F32)
            rv[t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rR, off[t], 0, 0));
          else
            rv[t] = widen16<OUT>(__builtin_amdgcn_raw_buffer_load_b16(rR, off[t], 0, 0));
        }
      }
      const f32x4 vb = epi_block<OUT>(e, acc[i][j], bj[j], sc);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float v = vb[t];
        if constexpr (HAS_R) v += rv[t];
        if constexpr (OUT == DT_F32)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rC, off[t], 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b16(narrow16<OUT>(v), rC, off[t], 0, 0);
      }
    }
  }
}

// Dispatch of the epilogue on (residual, output type), once per launch.
template <int FM, int FN, int WTM, int WTN>
__device__ __forceinline__ void store_w(const LaunchArgs& a, f32x4 (&acc)[FM][FN], int m0, int n0,
                                        int wm, int wn, int lane, int64_t z) {
  auto go = [&](auto HR, auto OD) __attribute__((always_inline)) {
    store_tile_w<FM, FN, WTM, WTN, decltype(HR)::value, decltype(OD)::value>(a, acc, m0, n0, wm,
                                                                             wn, lane, z);
  };
  auto by_out = [&](auto HR) __attribute__((always_inline)) {
    if (a.epi.out_dtype == DT_F32)
      go(HR, std::integral_constant<int, DT_F32>{});
    else if (a.epi.out_dtype == DT_BF16)
      go(HR, std::integral_constant<int, DT_BF16>{});
    else
      go(HR, std::integral_constant<int, DT_F16>{});
  };
  if (a.epi.flags & EPI_RESID)
    by_out(std::true_type{});
  else
    by_out(std::false_type{});
}

template <typename T, int BM, int BN, int R, bool BROW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_m16w_kernel(LaunchArgs a) {
  using G = WGeom<BM, BN, R>;
  constexpr int WTM = G::WTM, WTN = G::WTN, FM = G::FM, FN = G::FN;
  constexpr int A_SLOT = G::A_SLOT, B_SLOT = G::B_SLOT, AI = G::AI, BI = G::BI, NV = G::NV;
  constexpr int CPR_B = BN / 8;   // 16-byte chunks per row-major B row
  constexpr int RPI_B = 64 / CPR_B;  // B rows one 1 KB load fills
  static_assert(!BROW || (CPR_B >= 16 && 64 % CPR_B == 0), "row-major B: BN of 128 or 256");
  __shared__ u32x4 lds[G::RING / 16];
  lds_char* const L = (lds_char*)lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int M = static_cast<int>(a.M), N = static_cast<int>(a.N), K = static_cast<int>(a.K);
  const int LDA = static_cast<int>(a.lda), LDB = static_cast<int>(a.ldb);
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t z = blockIdx.y;
  const uint16_t* Abase = static_cast<const uint16_t*>(a.A) + z * a.sA;
  const uint16_t* Bbase = static_cast<const uint16_t*>(a.B) + z * a.sB;

  // Direct loads. Load q of a slot (q = wave * AI + i) fills its bytes q KB .. +1 KB.
  // A: rows 16 q .. +15, lane l -> row 16 q + l / 4, slot chunk l % 4, which holds
  // logical chunk (l % 4) ^ ((row >> 1) & 3).
  int a_col[AI];
  uint32_t a_voff[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int r = (wave * AI + i) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 1) & 3);
    a_col[i] = 8 * c;
    a_voff[i] = m0 + r < M ? static_cast<uint32_t>((m0 + r) * LDA + 8 * c) * 2u : OOB;
  }
  int b_key[BI];  // row-major B: the slot row (k within the slice); Bt: the k column
  uint32_t b_voff[BI];
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    if constexpr (BROW) {
      const int r = (wave * BI + i) * RPI_B + lane / CPR_B;
      const int h = 2 * ((r & 3) | (((r >> 3) & 1) << 2));
      const int gn = n0 + ((lane % CPR_B) ^ h) * 8;
      b_key[i] = r;
      b_voff[i] = gn < N ? static_cast<uint32_t>(r * LDB + gn) * 2u : OOB;
    } else {
      const int r = (wave * BI + i) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ ((r >> 1) & 3);
      b_key[i] = 8 * c;
      b_voff[i] = n0 + r < N ? static_cast<uint32_t>((n0 + r) * LDB + 8 * c) * 2u : OOB;
    }
  }

  // Loads of the slice at k0 into slots (wa, wb): `full` when the slice lies wholly
  // inside K (no per-chunk test); otherwise chunks (rows of B) past K are zeroed in
  // LDS and not loaded. Every call issues NV loads, so wait counts stay exact.
  auto dma = [&](lds_char* __restrict__ wa, lds_char* __restrict__ wb, int k0, int v, auto FullC) __attribute__((always_inline)) {
    constexpr bool full = decltype(FullC)::value;
    if (v < BI) {
      const int i = v;
      lds_char* dst = wb + (wave * BI + i) * 1024;
      bool kin;
      __amdgpu_buffer_rsrc_t r;
      if constexpr (BROW) {
        const int64_t left = static_cast<int64_t>(K - k0) * LDB;
        r = rsrc(Bbase + static_cast<int64_t>(k0) * LDB,
                 static_cast<uint32_t>(left > 0 ? left * 2 : 0));
        kin = full || k0 + b_key[i] < K;
      } else {
        const int64_t left = static_cast<int64_t>(N) * LDB - k0;
        r = rsrc(Bbase + k0, static_cast<uint32_t>(left > 0 ? left * 2 : 0));
        kin = full || k0 + b_key[i] < K;
      }
      const uint32_t off = kin ? b_voff[i] : OOB;
      if (!full && !kin) ((lds_u32x4*)dst)[lane] = u32x4{0u, 0u, 0u, 0u};
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, off, 0, 0, 0);
    } else {
      const int i = v - BI;
      lds_char* dst = wa + (wave * AI + i) * 1024;
      const int64_t left = static_cast<int64_t>(M) * LDA - k0;
      const auto r = rsrc(Abase + k0, static_cast<uint32_t>(left > 0 ? left * 2 : 0));
      const bool kin = full || k0 + a_col[i] < K;
      const uint32_t off = kin ? a_voff[i] : OOB;
      if (!full && !kin) ((lds_u32x4*)dst)[lane] = u32x4{0u, 0u, 0u, 0u};
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, off, 0, 0, 0);
    }
  };

  // Fragment reads. A block i: row wm WTM + 16 i + (l & 15), chunk l >> 4 (its slot
  // position does not depend on i: 16 i is a multiple of 4 rows).
  const int lr = lane & 15, lg = lane >> 4;
  const int a_rd = (wm * WTM + lr) * 64 + ((lg ^ ((lr >> 1) & 3)) << 4);
  // B block j, half h (row-major): lane t of group g addresses k row 8 g + 4 h + t / 4,
  // columns wn WTN + 16 j + 4 (t % 4) .. +3
  int b_rd[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    if constexpr (BROW) {
      const int t = lr;
      const int k = 8 * lg + (t >> 2);
      const int hk = 2 * ((k & 3) | (((k >> 3) & 1) << 2));
      const int n = wn * WTN + 16 * j + 4 * (t & 3);
      b_rd[j] = k * (BN * 2) + (((n >> 3) ^ hk) << 4) + (n & 7) * 2;
    } else {
      b_rd[j] = (wn * WTN + 16 * j + lr) * 64 + ((lg ^ ((lr >> 1) & 3)) << 4);
    }
  }
  struct Frag {
    u32x4 a[FM], b[FN];
  };
  // read r of a slice in the order the ops consume them: A 0, B 0 .. FN-1, A 1 ..
  // FM-1 (a row-major B fragment is two transposing reads)
  auto read_frag = [&](const lds_char* __restrict__ ra, const lds_char* __restrict__ rb, int r,
                       Frag& f) __attribute__((always_inline)) {
    if (r == 0 || r > FN) {
      const int i = r == 0 ? 0 : r - FN;
      f.a[i] = *(const lds_u32x4*)(ra + a_rd + i * 1024);
      return;
    }
    const int j = r - 1;
    if constexpr (BROW) {
      const lds_char* p = rb + b_rd[j];
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * (BN * 2)));
      f.b[j] = u32x4{__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                     __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                     __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1)),
                     __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3))};
    } else {
      f.b[j] = *(const lds_u32x4*)(rb + b_rd[j]);
    }
  };
  constexpr int NR = FM + FN;

  // no clearing: the first slice's ops take a zero accumulator operand (an inline
  // constant), which saves one register write per accumulator element per call
  f32x4 acc[FM][FN];

  // slot s holds A then B of one slice
  constexpr int SLOT = A_SLOT + B_SLOT;
  auto slotA = [&](int s) __attribute__((always_inline)) { return L + s * SLOT; };
  auto slotB = [&](int s) __attribute__((always_inline)) { return L + s * SLOT + A_SLOT; };
  const int nk = (K + WBK - 1) / WBK;

  // Prologue: slices 0 .. R-1 into slots 0 .. R-1, then slice 0's fragments.
#pragma unroll
  for (int s = 0; s < R; ++s) {
    if ((s + 1) * WBK <= K) {
#pragma unroll
      for (int v = 0; v < NV; ++v) dma(slotA(s), slotB(s), s * WBK, v, std::true_type{});
    } else {
#pragma unroll
      for (int v = 0; v < NV; ++v) dma(slotA(s), slotB(s), s * WBK, v, std::false_type{});
    }
  }
  wait_vm<(R - 1) * NV>();
  lds_barrier();
  Frag fx, fy;
#pragma unroll
  for (int r = 0; r < NR; ++r) read_frag(slotA(0), slotB(0), r, fx);

  // One slice: ops on cur (slice kt, in registers); the barrier (slice kt + 1 landed
  // everywhere, slot kt free); reads of slice kt + 1 into nxt; loads of slice kt + R
  // into slot kt. Q0 ops go before the barrier; the reads spread over the next
  // ops, the loads over the ops after them. The slots are runtime values, so each
  // slice forms its few read addresses itself rather than the compiler keeping one
  // register per (slot, fragment); slices alternate the roles of the two fragment
  // sets (no copies). FULL: the slice loaded lies wholly inside K.
  constexpr int NM = FM * FN;
  constexpr int Q0 = 4;
  constexpr int QR = NM * 9 / 16;  // ops that carry the NR reads
  static_assert(Q0 + QR + NV <= NM, "slice schedule");
  auto slice = [&](auto FullC, auto FirstC, const Frag& cur, Frag& nxt, lds_char* __restrict__ ra,
                   lds_char* __restrict__ rb, lds_char* __restrict__ wa, lds_char* __restrict__ wb,
                   int kt) __attribute__((always_inline)) {
    const int k0 = (kt + R) * WBK;
    static_for<0, NM>([&](auto QC) __attribute__((always_inline)) {
      constexpr int q = decltype(QC)::value;
      // B fragment first: the block accumulates C^T (rows along the lanes)
      if constexpr (decltype(FirstC)::value)
        acc[q / FN][q % FN] = mma16<T>(cur.b[q % FN], cur.a[q / FN], f32x4{0.f, 0.f, 0.f, 0.f});
      else
        acc[q / FN][q % FN] = mma16<T>(cur.b[q % FN], cur.a[q / FN], acc[q / FN][q % FN]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (q == Q0 - 1) {
        wait_vm<(R - 2) * NV>();
        lds_barrier();
      }
      if constexpr (q >= Q0 && q < Q0 + QR) {
        static_for<0, NR>([&](auto RC) __attribute__((always_inline)) {
          constexpr int r = decltype(RC)::value;
          if constexpr (r * QR / NR == q - Q0) read_frag(ra, rb, r, nxt);
        });
      }
      if constexpr (q >= Q0 + QR) {
        static_for<0, NV>([&](auto VC) __attribute__((always_inline)) {
          constexpr int v = decltype(VC)::value;
          if constexpr (v * (NM - Q0 - QR) / NV == q - Q0 - QR) dma(wa, wb, k0, v, FullC);
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  int ws = 0;  // slot of slice kt (loaded with slice kt + R during it)
  int kt = 0;
  auto step = [&](auto FullC, auto FirstC, const Frag& cur, Frag& nxt)
                  __attribute__((always_inline)) {
    const int rs = ws + 1 == R ? 0 : ws + 1;
    slice(FullC, FirstC, cur, nxt, slotA(rs), slotB(rs), slotA(ws), slotB(ws), kt);
    ws = rs;
    ++kt;
  };
  // slice 0 (K >= 1, so there is one), then the slices whose load (slice kt + R) lies
  // inside K, two at a time, then the rest
  const int nfull = K / WBK - R;
  if (nfull >= 1)
    step(std::true_type{}, std::true_type{}, fx, fy);
  else
    step(std::false_type{}, std::true_type{}, fx, fy);
  while (kt + 2 <= nfull) {
    step(std::true_type{}, std::false_type{}, fy, fx);
    step(std::true_type{}, std::false_type{}, fx, fy);
  }
  while (kt < nk) {
    step(std::false_type{}, std::false_type{}, fy, fx);
    if (kt >= nk) {
      fy = fx;
      break;
    }
    step(std::false_type{}, std::false_type{}, fx, fy);
  }

  wait_vm<0>();  // no direct load still writing LDS when the wave ends
  store_w<FM, FN, WTM, WTN>(a, acc, m0, n0, wm, wn, lane, z);
}

template <typename T, int BM, int BN, int R, bool BROW>
hipError_t launch_m16w(const LaunchArgs& a, hipStream_t s) {
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(a.batch));
  hipLaunchKernelGGL((gemm_m16w_kernel<T, BM, BN, R, BROW>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

#define G15_M16W(T, TN, BM, BN, R, BROW, SFX)                                                  \
  {"m16w_" TN "_" #BM "x" #BN "x32_r" #R SFX, KIND_MFMA16, T::code, BM, BN, 32, 256,            \
   WGeom<BM, BN, R>::RING, 1, 1, launch_m16w<T, BM, BN, R, BROW>, 1, BROW ? 0 : 1}

#define G15_M16W_ALL(T, TN)                       \
  G15_M16W(T, TN, 256, 256, 5, true, ""),         \
  G15_M16W(T, TN, 256, 256, 4, true, ""),         \
  G15_M16W(T, TN, 256, 128, 6, true, ""),         \
  G15_M16W(T, TN, 256, 256, 5, false, "_nk"),     \
  G15_M16W(T, TN, 256, 128, 6, false, "_nk")

const KernelEntry kM16W[] = {
    G15_M16W_ALL(bf16_t, "bf16"),
    G15_M16W_ALL(f16_t, "f16"),
};

}  // namespace

int mfma16_w_entries(const KernelEntry** out) {
  *out = kM16W;
  return static_cast<int>(sizeof(kM16W) / sizeof(kM16W[0]));
}

}  // namespace g15
