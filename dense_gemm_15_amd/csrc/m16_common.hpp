// m16_common.hpp -- pieces shared by the bf16 / fp16 matrix-core kernels that
// stream operands global -> LDS (kernel_mfma16_dlds.hip, kernel_mfma16_nt.hip):
// buffer descriptors, the 32x32x16 MFMA, wait and barrier helpers, instruction
// grouping, the XCD-aware tile order and the LDS-staged epilogue.
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

__device__ __forceinline__ void tile_of(int wid, int tiles_m, int tiles_n, int& tm, int& tn) {
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

// Epilogue of a wave's WTM x WTN sub-tile (FM x FN blocks of 32 x 32) of the tile
// at (m0, n0). In the accumulators lane l holds C[row][col] of block (i, j) with
// col = l % 32 and row = 8 (r / 4) + 4 (l / 32) + r % 4: one column per lane, so
// direct stores would write 2 or 4 bytes per lane. Instead scale, bias and GELU
// are applied there (the bias is one value per lane and block column), then each
// 32-row block row of the sub-tile goes through the wave's own LDS area and comes
// back as 8 consecutive columns per lane: residual loads and C stores move 16 or
// 32 contiguous bytes per lane. That needs a.c_vec: N a multiple of 8 (a chunk of
// 8 columns is all inside or all outside the matrix) and 16-byte aligned rows;
// otherwise each lane moves single elements. lds_f is the workgroup's LDS
// (LDS_BYTES bytes); every wave must have finished with its previous contents.
template <int FM, int FN, int WTM, int WTN, int NW, int LDS_BYTES>
__device__ __forceinline__ void store_tile(const LaunchArgs& a, f32x16 (&acc)[FM][FN], float* lds_f,
                                           int m0, int n0, int wm, int wn, int wave, int lane,
                                           int64_t z) {
  const int M = static_cast<int>(a.M), N = static_cast<int>(a.N), LDC = static_cast<int>(a.ldc);
  const int lrow = lane & 31, lhalf = lane >> 5;
  constexpr int EP = WTN + 8;  // floats per staged row: rows 4 apart land 32 banks apart
  constexpr int CPR = WTN / 8;  // 8-column chunks per row
  constexpr int RPP = 64 / CPR;  // rows per pass
  constexpr int PASSES = 32 / RPP;
  static_assert(NW * 32 * EP * 4 <= LDS_BYTES, "staging must fit in LDS");
  static_assert(64 % CPR == 0 && 32 % RPP == 0, "staging passes");
  float* stg = lds_f + wave * 32 * EP;

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
  const int q = lane % CPR;  // this lane's chunk within a staged row
  const int col = n0 + wn * WTN + 8 * q;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = acc[i][j][r];
        if (e.flags & EPI_SCALE) v *= e.scale;
        if (e.flags & EPI_BIAS) v += bj[j];
        if (e.flags & EPI_GELU) v = gelu(v);
        stg[(8 * (r >> 2) + 4 * lhalf + (r & 3)) * EP + 32 * j + lrow] = v;
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's staging writes are done

    if (!a.c_vec) {
      // C rows not 16-byte aligned: the lanes take consecutive columns of one row
      // and move one element each (coalesced, no vector access)
      for (int rr = 0; rr < 32; ++rr) {
        const int row = m0 + wm * WTM + 32 * i + rr;
#pragma unroll
        for (int cc = lane; cc < WTN; cc += 64) {
          const int cl = n0 + wn * WTN + cc;
          if (row < M && cl < N) {
            const int64_t idx = static_cast<int64_t>(row) * LDC + cl;
            float v = stg[rr * EP + cc];
            if (has_r) v += load_out_elem(Rz, e.out_dtype, idx);
            store_out_elem(Cz, e.out_dtype, idx, v);
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      continue;
    }

    uint32_t off[PASSES];
    u32x4 res[PASSES][2];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = m0 + wm * WTM + 32 * i + p * RPP + lane / CPR;
      off[p] = (row < M && col < N) ? static_cast<uint32_t>(row * LDC + col) * ob : OOB;
      if (has_r) {  // every residual load of the block row in flight at once
        res[p][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rR, off[p], 0, 0));
        if (ob == 4)
          res[p][1] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(rR, off[p] + 16u, 0, 0));
      }
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const float* src = stg + (p * RPP + lane / CPR) * EP + 8 * q;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
      float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      if (ob == 4) {
        if (has_r)
#pragma unroll
          for (int t = 0; t < 8; ++t) v[t] += __uint_as_float(res[p][t >> 2][t & 3]);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]),
                                                     __float_as_uint(v[2]), __float_as_uint(v[3])},
                                               rC, off[p], 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]),
                                                     __float_as_uint(v[6]), __float_as_uint(v[7])},
                                               rC, off[p] + 16u, 0, 0);
      } else {
        const bool bf = e.out_dtype == DT_BF16;
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float x0 = v[2 * t], x1 = v[2 * t + 1];
          if (has_r) {
            const uint32_t rr = res[p][0][t];
            const uint16_t r0 = static_cast<uint16_t>(rr & 0xffffu), r1 = static_cast<uint16_t>(rr >> 16);
            x0 += bf ? widen(bf16_t{}, r0) : widen(f16_t{}, r0);
            x1 += bf ? widen(bf16_t{}, r1) : widen(f16_t{}, r1);
          }
          const uint16_t h0 = bf ? narrow_bf16(x0) : narrow_f16(x0);
          const uint16_t h1 = bf ? narrow_bf16(x1) : narrow_f16(x1);
          w[t] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
        }
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[0], w[1], w[2], w[3]}, rC, off[p], 0, 0);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next block row
  }
}

}  // namespace
}  // namespace g15
