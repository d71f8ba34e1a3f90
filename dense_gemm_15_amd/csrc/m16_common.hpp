// m16_common.hpp -- pieces shared by the bf16 / fp16 matrix-core kernels that
// stream operands global -> LDS (kernel_mfma16_dlds.hip, kernel_mfma16_nt.hip):
// buffer descriptors, the 32x32x16 MFMA, wait and barrier helpers, instruction
// grouping, the XCD-aware tile order and the epilogue.
#pragma once

#include <type_traits>

#include "kernels.hpp"

namespace g15 {
namespace {

constexpr uint32_t OOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

typedef __attribute__((address_space(3))) void lds_void;

template <typename T>
__device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mma<bf16_t>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mma<f16_t>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for the LDS ring: this wave's LDS stores are complete, then
// s_barrier. Unlike __syncthreads() it does not drain the direct-to-LDS loads
// still in flight (their completion is waited for explicitly with wait_vm); the
// memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int I, int N, int NDR, int NDW, int NVM>
__device__ __forceinline__ void plan_slice() {
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int dr = (I + 1) * NDR / N - I * NDR / N;
    constexpr int dw = (I + 1) * NDW / N - I * NDW / N;
    constexpr int vm = (I + 1) * NVM / N - I * NVM / N;
    if constexpr (dr > 0) __builtin_amdgcn_sched_group_barrier(0x100, dr, 0);
    if constexpr (dw > 0) __builtin_amdgcn_sched_group_barrier(0x200, dw, 0);
    if constexpr (vm > 0) __builtin_amdgcn_sched_group_barrier(0x020, vm, 0);
    plan_slice<I + 1, N, NDR, NDW, NVM>();
  }
}

__device__ __forceinline__ void tile_in_groups(int wid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int group = wid / per_group;
  const int first = group * GM;
  const int gsz = min(tiles_m - first, GM);
  const int in = wid - group * per_group;
  tm = first + in % gsz;
  tn = in / gsz;
}

__device__ __forceinline__ void tile_of(int wid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  if ((total & 7) == 0) wid = (wid & 7) * (total >> 3) + (wid >> 3);
  tile_in_groups(wid, tiles_m, tiles_n, tm, tn);
}

// Tile and batch item of this workgroup in a (tiles, items) grid. Workgroups reach
// the 8 XCDs round-robin in dispatch order (x fastest), so with few tiles per item
// XCD k would take tile k of every item and its L2 would share no operand rows. With
// several items and a whole number of workgroups per XCD, the (item, tile) pairs are
// taken item by item and XCD x gets the x-th eighth of them: whole items where the
// items divide by 8 (measured: 64 items of 256 x 256 x 256 on 64 x 128 tiles 14.1 us
// in the tile-major order, 10.4 us so); otherwise the tile-major order of tile_of.
__device__ __forceinline__ void batch_tile_of(int tiles_m, int tiles_n, int& tm, int& tn,
                                              int64_t& z) {
  const int64_t per_item = static_cast<int64_t>(tiles_m) * tiles_n;  // gridDim.x
  const int64_t total = per_item * gridDim.y;
  if (gridDim.y > 1 && (total & 7) == 0) {
    const int64_t l = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
    const int64_t w = (l & 7) * (total >> 3) + (l >> 3);  // XCD l & 7 takes a contiguous run
    z = w / per_item;
    tile_in_groups(static_cast<int>(w - z * per_item), tiles_m, tiles_n, tm, tn);
    return;
  }
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  z = blockIdx.y;
}

// Epilogue of a wave's WTM x WTN sub-tile (FM x FN blocks of 32 x 32) of the tile
// at (m0, n0). In the accumulators lane l holds C[row][col] of block (i, j) with
// col = l % 32 and row = 8 (r / 4) + 4 (l / 32) + r % 4. Scale, bias and GELU are
// applied there (the bias is one value per lane and block column); the residual is
// added and the result rounded where it is stored. Three store forms, measured:
//  * fp32 output: straight from the registers. One register of a block is 32
//    consecutive columns of two rows, two whole 128-byte spans per store, and
//    regrouping would only add work (also for rows of any alignment).
//  * 16-bit output with a.c_vec (N a multiple of 8, 16-byte aligned rows): each
//    32-row block row goes through the wave's own LDS area and comes back as 8
//    consecutive columns per lane, 16-byte residual loads and C stores.
//  * other 16-bit output: straight from the registers, two columns per lane
//    after one exchange between neighbouring lanes (even LDC), else one.
// lds_f is the workgroup's LDS (LDS_BYTES bytes); every wave must have finished
// with its previous contents.
template <int OUT>
__device__ __forceinline__ uint16_t narrow16(float x) {
  return OUT == DT_BF16 ? narrow_bf16(x) : narrow_f16(x);
}
// Two values rounded to OUT in one instruction (v_cvt_pk_bf16_f32 /
// v_cvt_pk_f16_f32, the conversion narrow16 uses): x0 in the low half.
template <int OUT>
__device__ __forceinline__ uint32_t pack16(float x0, float x1) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  uint32_t w;
  if constexpr (OUT == DT_BF16) {
    const bf16x2 r = __builtin_convertvector(f32x2{x0, x1}, bf16x2);
    __builtin_memcpy(&w, &r, 4);
  } else {
    const f16x2 r = __builtin_convertvector(f32x2{x0, x1}, f16x2);
    __builtin_memcpy(&w, &r, 4);
  }
  return w;
}
template <int OUT>
__device__ __forceinline__ float widen16(uint32_t h) {
  return OUT == DT_BF16 ? widen(bf16_t{}, static_cast<uint16_t>(h))
                        : widen(f16_t{}, static_cast<uint16_t>(h));
}

// The store forms above for one output type and residual choice (template
// parameters, chosen once per launch: run-time tests of either inside the store
// loops become per-element selects, and a run-time residual test makes the
// compiler wait for every store in flight where the paths join). Scale and bias
// are one multiply-add per element (sc = 1 without EPI_SCALE; the bias reads as 0
// without EPI_BIAS, through a buffer descriptor, so no guarded loads), and each
// stage is one uniform branch per block. 16-bit results take gelu16.
template <int FM, int FN, int WTM, int WTN, int NW, int LDS_BYTES, int OUT, bool HAS_R>
__device__ __forceinline__ void store_tile_t(const LaunchArgs& a, f32x16 (&acc)[FM][FN],
                                             float* lds_f, int m0, int n0, int wm, int wn,
                                             int wave, int lane, int64_t z) {
  const int M = static_cast<int>(a.M), N = static_cast<int>(a.N), LDC = static_cast<int>(a.ldc);
  const int lrow = lane & 31, lhalf = lane >> 5;

  const Epi& e = a.epi;
  constexpr int ob = OUT == DT_F32 ? 4 : 2;
  char* Cz = static_cast<char*>(a.C) + z * a.sC * ob;
  const char* Rz = HAS_R ? static_cast<const char*>(e.resid) + z * a.sR * ob : Cz;
  const auto rC = rsrc(Cz, static_cast<uint32_t>(static_cast<int64_t>(M) * LDC * ob));
  const auto rR = rsrc(Rz, static_cast<uint32_t>(static_cast<int64_t>(M) * LDC * ob));
  const auto rB = rsrc(e.bias, (e.flags & EPI_BIAS) ? static_cast<uint32_t>(N) * 4u : 0u);
  const float sc = (e.flags & EPI_SCALE) ? e.scale : 1.f;
  float bj[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const uint32_t col = static_cast<uint32_t>(n0 + wn * WTN + j * 32 + lrow);
    bj[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rB, col * 4u, 0, 0));
  }
  auto epi = [&](f32x16& v, int j) __attribute__((always_inline)) {
    if (e.flags & (EPI_SCALE | EPI_BIAS)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = v[r] * sc + bj[j];
    }
    if (e.flags & EPI_GELU) {
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = OUT == DT_F32 ? gelu(v[r]) : gelu16(v[r]);
    }
  };

  if constexpr (OUT == DT_F32) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int cl = n0 + wn * WTN + 32 * j + lrow;
        const int rb = m0 + wm * WTM + 32 * i + 4 * lhalf;
        uint32_t off[16];
        float rv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rb + 8 * (r >> 2) + (r & 3);
          off[r] = (row < M && cl < N) ? static_cast<uint32_t>(row * LDC + cl) * 4u : OOB;
          if constexpr (HAS_R)  // the block's residual loads all in flight at once
            rv[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rR, off[r], 0, 0));
        }
        f32x16 v = acc[i][j];
        epi(v, j);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = v[r];
          if constexpr (HAS_R) x += rv[r];
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rC, off[r], 0, 0);
        }
      }
    return;
  } else {
    if (!a.c_vec) {
      // Registers 2p and 2p+1 of a block are rows R and R+1 of one column per lane
      // and lanes l, l^1 hold neighbouring columns: after one exchange the even lane
      // has columns (c, c+1) of row R and the odd lane columns (c-1, c) of row R+1,
      // 4 bytes per lane (4-byte aligned when LDC and N are even).
      const bool odd = (lane & 1) != 0;
      const bool pairs = ((LDC | N) & 1) == 0;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int cl = n0 + wn * WTN + 32 * j + lrow;
          const int rb = m0 + wm * WTM + 32 * i + 4 * lhalf;
          f32x16 v = acc[i][j];
          epi(v, j);
          if (pairs) {
            const int ce = cl & ~1;
            uint32_t off[8], res[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) {
              const int row = rb + 8 * (p >> 1) + 2 * (p & 1) + (odd ? 1 : 0);
              off[p] = (row < M && ce < N) ? static_cast<uint32_t>(row * LDC + ce) * 2u : OOB;
              if constexpr (HAS_R) res[p] = __builtin_amdgcn_raw_buffer_load_b32(rR, off[p], 0, 0);
            }
#pragma unroll
            for (int p = 0; p < 8; ++p) {
              // DPP quad_perm [1, 0, 3, 2]: each lane receives its neighbour's value
              const float recv = __int_as_float(__builtin_amdgcn_mov_dpp(
                  __float_as_int(odd ? v[2 * p] : v[2 * p + 1]), 0xB1, 0xF, 0xF, false));
              float lo = odd ? recv : v[2 * p];
              float hi = odd ? v[2 * p + 1] : recv;
              if constexpr (HAS_R) {
                lo += widen16<OUT>(res[p] & 0xffffu);
                hi += widen16<OUT>(res[p] >> 16);
              }
              __builtin_amdgcn_raw_buffer_store_b32(pack16<OUT>(lo, hi), rC, off[p], 0, 0);
            }
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = rb + 8 * (r >> 2) + (r & 3);
              const uint32_t o =
                  (row < M && cl < N) ? static_cast<uint32_t>(row * LDC + cl) * 2u : OOB;
              float x = v[r];
              if constexpr (HAS_R) x += widen16<OUT>(__builtin_amdgcn_raw_buffer_load_b16(rR, o, 0, 0));
              __builtin_amdgcn_raw_buffer_store_b16(narrow16<OUT>(x), rC, o, 0, 0);
            }
          }
        }
      return;
    }

    constexpr int EP = WTN + 8;    // floats per staged row: rows 4 apart land 32 banks apart
    constexpr int CPR = WTN / 8;   // 8-column chunks per row
    constexpr int RPP = 64 / CPR;  // rows per pass
    constexpr int PASSES = 32 / RPP;
    static_assert(NW * 32 * EP * 4 <= LDS_BYTES, "staging must fit in LDS");
    static_assert(64 % CPR == 0 && 32 % RPP == 0, "staging passes");
    float* stg = lds_f + wave * 32 * EP;
    const int q = lane % CPR;  // this lane's chunk within a staged row
    const int col = n0 + wn * WTN + 8 * q;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        f32x16 v = acc[i][j];
        epi(v, j);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          stg[(8 * (r >> 2) + 4 * lhalf + (r & 3)) * EP + 32 * j + lrow] = v[r];
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's staging writes are done

      uint32_t off[PASSES];
      u32x4 res[PASSES];
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        const int row = m0 + wm * WTM + 32 * i + p * RPP + lane / CPR;
        off[p] = (row < M && col < N) ? static_cast<uint32_t>(row * LDC + col) * 2u : OOB;
        if constexpr (HAS_R)  // every residual load of the block row in flight at once
          res[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rR, off[p], 0, 0));
      }
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        const float* src = stg + (p * RPP + lane / CPR) * EP + 8 * q;
        const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
        const float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float x0 = v[2 * t], x1 = v[2 * t + 1];
          if constexpr (HAS_R) {
            x0 += widen16<OUT>(res[p][t] & 0xffffu);
            x1 += widen16<OUT>(res[p][t] >> 16);
          }
          w[t] = pack16<OUT>(x0, x1);
        }
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[0], w[1], w[2], w[3]}, rC, off[p], 0, 0);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next block row
    }
  }
}

template <int FM, int FN, int WTM, int WTN, int NW, int LDS_BYTES>
__device__ __forceinline__ void store_tile(const LaunchArgs& a, f32x16 (&acc)[FM][FN], float* lds_f,
                                           int m0, int n0, int wm, int wn, int wave, int lane,
                                           int64_t z) {
  auto go = [&](auto OD, auto HR) __attribute__((always_inline)) {
    store_tile_t<FM, FN, WTM, WTN, NW, LDS_BYTES, decltype(OD)::value, decltype(HR)::value>(
        a, acc, lds_f, m0, n0, wm, wn, wave, lane, z);
  };
  auto by_out = [&](auto HR) __attribute__((always_inline)) {
    if (a.epi.out_dtype == DT_F32)
      go(std::integral_constant<int, DT_F32>{}, HR);
    else if (a.epi.out_dtype == DT_BF16)
      go(std::integral_constant<int, DT_BF16>{}, HR);
    else
      go(std::integral_constant<int, DT_F16>{}, HR);
  };
  if (a.epi.flags & EPI_RESID)
    by_out(std::true_type{});
  else
    by_out(std::false_type{});
}

// The same epilogue with the output type, residual and stages tested at run time
// inside one body: fewer registers than store_tile's per-launch variants, for
// kernels that already sit at the register limit (their variants would spill).
template <int FM, int FN, int WTM, int WTN, int NW, int LDS_BYTES>
__device__ __forceinline__ void store_tile_rt(const LaunchArgs& a, f32x16 (&acc)[FM][FN], float* lds_f,
                                              int m0, int n0, int wm, int wn, int wave, int lane,
                                              int64_t z) {
  const int M = static_cast<int>(a.M), N = static_cast<int>(a.N), LDC = static_cast<int>(a.ldc);
  const int lrow = lane & 31, lhalf = lane >> 5;

  const Epi& e = a.epi;
  const int ob = e.out_dtype == DT_F32 ? 4 : 2;
  char* Cz = static_cast<char*>(a.C) + z * a.sC * ob;
  const bool has_r = (e.flags & EPI_RESID) != 0;
  const char* Rz = has_r ? static_cast<const char*>(e.resid) + z * a.sR * ob : Cz;
  const auto rC = rsrc(Cz, static_cast<uint32_t>(static_cast<int64_t>(M) * LDC * ob));
  const auto rR = rsrc(Rz, static_cast<uint32_t>(static_cast<int64_t>(M) * LDC * ob));
  float bj[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int col = n0 + wn * WTN + j * 32 + lrow;
    bj[j] = ((e.flags & EPI_BIAS) && col < N) ? e.bias[col] : 0.f;
  }
  auto epi = [&](float v, int j) {
    if (e.flags & EPI_SCALE) v *= e.scale;
    if (e.flags & EPI_BIAS) v += bj[j];
    if (e.flags & EPI_GELU) v = gelu(v);
    return v;
  };

  if (e.out_dtype == DT_F32) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int cl = n0 + wn * WTN + 32 * j + lrow;
        const int rb = m0 + wm * WTM + 32 * i + 4 * lhalf;
        uint32_t off[16];
        float rv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rb + 8 * (r >> 2) + (r & 3);
          off[r] = (row < M && cl < N) ? static_cast<uint32_t>(row * LDC + cl) * 4u : OOB;
          if (has_r)  // the block's residual loads all in flight at once
            rv[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rR, off[r], 0, 0));
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = epi(acc[i][j][r], j);
          if (has_r) v += rv[r];
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rC, off[r], 0, 0);
        }
      }
    return;
  }

  const bool bf = e.out_dtype == DT_BF16;
  auto narrow = [&](float x) { return bf ? narrow_bf16(x) : narrow_f16(x); };
  auto widen16 = [&](uint32_t h) {
    return bf ? widen(bf16_t{}, static_cast<uint16_t>(h)) : widen(f16_t{}, static_cast<uint16_t>(h));
  };

  if (!a.c_vec) {
    // Registers 2p and 2p+1 of a block are rows R and R+1 of one column per lane
    // and lanes l, l^1 hold neighbouring columns: after one exchange the even lane
    // has columns (c, c+1) of row R and the odd lane columns (c-1, c) of row R+1,
    // 4 bytes per lane (4-byte aligned when LDC and N are even).
    const bool odd = (lane & 1) != 0;
    const bool pairs = ((LDC | N) & 1) == 0;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int cl = n0 + wn * WTN + 32 * j + lrow;
        const int rb = m0 + wm * WTM + 32 * i + 4 * lhalf;
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = epi(acc[i][j][r], j);
        if (pairs) {
          const int ce = cl & ~1;
          uint32_t off[8], res[8];
#pragma unroll
          for (int p = 0; p < 8; ++p) {
            const int row = rb + 8 * (p >> 1) + 2 * (p & 1) + (odd ? 1 : 0);
            off[p] = (row < M && ce < N) ? static_cast<uint32_t>(row * LDC + ce) * 2u : OOB;
            if (has_r) res[p] = __builtin_amdgcn_raw_buffer_load_b32(rR, off[p], 0, 0);
          }
#pragma unroll
          for (int p = 0; p < 8; ++p) {
            // DPP quad_perm [1, 0, 3, 2]: each lane receives its neighbour's value
            const float recv = __int_as_float(__builtin_amdgcn_mov_dpp(
                __float_as_int(odd ? v[2 * p] : v[2 * p + 1]), 0xB1, 0xF, 0xF, false));
            float lo = odd ? recv : v[2 * p];
            float hi = odd ? v[2 * p + 1] : recv;
            if (has_r) {
              lo += widen16(res[p] & 0xffffu);
              hi += widen16(res[p] >> 16);
            }
            const uint32_t w = static_cast<uint32_t>(narrow(lo)) | (static_cast<uint32_t>(narrow(hi)) << 16);
            __builtin_amdgcn_raw_buffer_store_b32(w, rC, off[p], 0, 0);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = rb + 8 * (r >> 2) + (r & 3);
            const uint32_t o = (row < M && cl < N) ? static_cast<uint32_t>(row * LDC + cl) * 2u : OOB;
            float x = v[r];
            if (has_r) x += widen16(__builtin_amdgcn_raw_buffer_load_b16(rR, o, 0, 0));
            __builtin_amdgcn_raw_buffer_store_b16(narrow(x), rC, o, 0, 0);
          }
        }
      }
    return;
  }

  constexpr int EP = WTN + 8;    // floats per staged row: rows 4 apart land 32 banks apart
  constexpr int CPR = WTN / 8;   // 8-column chunks per row
  constexpr int RPP = 64 / CPR;  // rows per pass
  constexpr int PASSES = 32 / RPP;
  static_assert(NW * 32 * EP * 4 <= LDS_BYTES, "staging must fit in LDS");
  static_assert(64 % CPR == 0 && 32 % RPP == 0, "staging passes");
  float* stg = lds_f + wave * 32 * EP;
  const int q = lane % CPR;  // this lane's chunk within a staged row
  const int col = n0 + wn * WTN + 8 * q;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        stg[(8 * (r >> 2) + 4 * lhalf + (r & 3)) * EP + 32 * j + lrow] = epi(acc[i][j][r], j);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's staging writes are done

    uint32_t off[PASSES];
    u32x4 res[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = m0 + wm * WTM + 32 * i + p * RPP + lane / CPR;
      off[p] = (row < M && col < N) ? static_cast<uint32_t>(row * LDC + col) * 2u : OOB;
      if (has_r)  // every residual load of the block row in flight at once
        res[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rR, off[p], 0, 0));
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const float* src = stg + (p * RPP + lane / CPR) * EP + 8 * q;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
      const float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      uint32_t w[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float x0 = v[2 * t], x1 = v[2 * t + 1];
        if (has_r) {
          x0 += widen16(res[p][t] & 0xffffu);
          x1 += widen16(res[p][t] >> 16);
        }
        w[t] = static_cast<uint32_t>(narrow(x0)) | (static_cast<uint32_t>(narrow(x1)) << 16);
      }
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[0], w[1], w[2], w[3]}, rC, off[p], 0, 0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next block row
  }
}

}  // namespace
}  // namespace g15
