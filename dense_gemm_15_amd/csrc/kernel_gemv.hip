// kernel_gemv.hip -- few-row products (M <= 8, e.g. one token through a layer):
// C[M x N] = epi(A[M x K] B[K x N]) as a split-K streaming kernel.
//
// With M this small the product is bound by reading B once from memory (the
// DeepGEMM page, section 4.3: at M = 1 no tiling helps; use a small-block path).
// The grid is (column strips of 128) x (S slices of K). Each workgroup streams
// its slice of K rows of its strip with 16-byte buffer loads (16 or 32 lanes per
// row: 256 contiguous bytes, several rows in flight per lane), multiplies by A
// values staged in LDS, and sums its row groups (cross-lane, then across the 4
// waves in LDS). With S = 1 it applies the epilogue and stores C. With S > 1 it
// stores its fp32 partial sums to the plan's workspace and a second small
// kernel adds the S partials in slice order, applies the epilogue and stores C.
// The kernel boundary orders the two: an in-kernel "last workgroup reduces"
// scheme needs a device-scope release and acquire per workgroup, which on this
// chip write back and invalidate the whole L2 of the XCD: measured 4x slower at
// 1 x 4096 x 4096 (42 us against 10 us for both kernels here). Without fences
// (partials written and read back with agent-scope atomic stores and loads, which
// go through to memory, and an agent-scope counter) it is still slower, 12.5
// against 8.7 us in a graph: the last workgroup of a strip waits for its stores to
// reach memory, the counter's round trip and the partials' reads in turn. No split at
// all (one workgroup per strip of 16, 32 or 64 columns over all of K, strips sharing
// cache lines on one XCD) measured 15-23 us at 1 x 4096 x 4096: too few workgroups,
// each walking all of K. Accumulation is fp32; the result does not depend on timing
// (fixed summation order).
#include "kernels.hpp"
#include "splitk.hpp"

namespace g15 {
namespace {

constexpr uint32_t GOOB = 0x80000000u;
constexpr int GNS = 128;  // columns per strip
constexpr int GNT = 256;  // threads per workgroup

__device__ __forceinline__ __amdgpu_buffer_rsrc_t grsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

template <typename T>
__device__ __forceinline__ float gload(const void* p, int64_t i);
template <>
__device__ __forceinline__ float gload<f32_t>(const void* p, int64_t i) {
  return static_cast<const float*>(p)[i];
}
template <>
__device__ __forceinline__ float gload<bf16_t>(const void* p, int64_t i) {
  return widen(bf16_t{}, static_cast<const uint16_t*>(p)[i]);
}
template <>
__device__ __forceinline__ float gload<f16_t>(const void* p, int64_t i) {
  return widen(f16_t{}, static_cast<const uint16_t*>(p)[i]);
}

template <typename T>
__device__ __forceinline__ void unpack(const u32x4& v, float (&x)[T::code == DT_F32 ? 4 : 8]);
template <>
__device__ __forceinline__ void unpack<f32_t>(const u32x4& v, float (&x)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(v[e]);
}
template <>
__device__ __forceinline__ void unpack<bf16_t>(const u32x4& v, float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(v[e] << 16);
    x[2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void unpack<f16_t>(const u32x4& v, float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = widen(f16_t{}, static_cast<uint16_t>(v[e] & 0xffffu));
    x[2 * e + 1] = widen(f16_t{}, static_cast<uint16_t>(v[e] >> 16));
  }
}

// Workspace layout: float partial[S][MR][N]. KMAX bounds the K rows one
// workgroup stages from A (the plan keeps ceil(K / S) <= KMAX by its choice of S).
template <typename T, int MR, int KMAX, int U>
__global__ __launch_bounds__(GNT) void gemv_kernel(LaunchArgs a, int64_t z0) {
  constexpr int EPL = T::code == DT_F32 ? 4 : 8;  // elements per 16-byte load
  constexpr int LPR = GNS / EPL;                  // lanes per B row segment
  constexpr int RPW = 64 / LPR;                   // row groups per wave
  constexpr int RG = 4 * RPW;                     // row groups per workgroup
  constexpr int SU = 4;                           // A values in flight per thread

  __shared__ float sa[MR][KMAX];
  __shared__ float red[4][MR][GNS];

  const int M = static_cast<int>(a.M), N = static_cast<int>(a.N), K = static_cast<int>(a.K);
  // row strides: A's (K unless rows of a padded copy), B's (N, likewise) and C's (N
  // unless a block of a larger C)
  const int64_t LDA = a.lda, LDB = a.ldb, LDC = a.ldc;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int strip = blockIdx.x, split = blockIdx.y, S = gridDim.y;
  const int64_t z = z0 + blockIdx.z;
  const int n0 = strip * GNS;
  const int kper = (K + S - 1) / S;
  const int kb = split * kper, ke = min(K, kb + kper);
  const int in_bytes = T::code == DT_F32 ? 4 : 2;
  const char* Ap = static_cast<const char*>(a.A) + z * a.sA * in_bytes;
  const char* Bp = static_cast<const char*>(a.B) + z * a.sB * in_bytes;

  const int rg = wave * RPW + lane / LPR;  // this lane's row group
  const int cl = (lane % LPR) * EPL;       // first column of this lane in the strip
  const auto rB = grsrc(Bp, static_cast<uint32_t>(static_cast<int64_t>(K) * LDB * in_bytes));
  const bool colok = n0 + cl < N;  // N is a multiple of EPL: a chunk is all in or all out

  // rows k0, k0 + RG, ..., k0 + (U - 1) RG of this lane's 16-byte column chunk
  u32x4 v[U];
  auto issue = [&](int k0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + u * RG;
      const uint32_t off = (colok && k < ke)
                               ? static_cast<uint32_t>((static_cast<int64_t>(k) * LDB + n0 + cl) * in_bytes)
                               : GOOB;
      v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rB, off, 0, 0));
    }
  };
  int k0 = kb + rg;
  issue(k0);  // the first B rows are in flight while A is staged

  // stage A[m][kb .. ke) as fp32, SU loads in flight per thread
  for (int m = 0; m < MR; ++m) {
    for (int j0 = tid; j0 < kper; j0 += SU * GNT) {
      float t[SU];
#pragma unroll
      for (int u = 0; u < SU; ++u) {
        const int k = j0 + u * GNT;
        t[u] = (m < M && kb + k < ke) ? gload<T>(Ap, static_cast<int64_t>(m) * LDA + kb + k) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < SU; ++u)
        if (j0 + u * GNT < kper) sa[m][j0 + u * GNT] = t[u];
    }
  }
  __syncthreads();

  float acc[MR][EPL];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[m][e] = 0.f;

  while (k0 < ke) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + u * RG;
      float x[EPL];
      unpack<T>(v[u], x);
      const int kk = min(k, ke - 1) - kb;
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const float am = k < ke ? sa[m][kk] : 0.f;  // rows past the slice add nothing
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[m][e] = __builtin_fmaf(am, x[e], acc[m][e]);
      }
    }
    k0 += U * RG;
    if (k0 < ke) issue(k0);
  }

  // sum the row groups: first across the wave's RPW groups, then across waves
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int e = 0; e < EPL; ++e)
#pragma unroll
      for (int d = LPR; d < 64; d *= 2) acc[m][e] += __shfl_xor(acc[m][e], d);
  if (lane < LPR) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int e = 0; e < EPL; ++e) red[wave][m][cl + e] = acc[m][e];
  }
  __syncthreads();
  // thread t owns column t % GNS and the rows m with m % 2 == t / GNS
  const int col = tid % GNS, mh = tid / GNS;
  const int gn = n0 + col;
  const bool cok = gn < N;
  const Epi& e = a.epi;
  auto finish = [&](int m, float v) {
    const int64_t ob = e.out_dtype == DT_F32 ? 4 : 2;
    void* Cp = static_cast<char*>(a.C) + z * a.sC * ob;
    const void* Rp =
        (e.flags & EPI_RESID) ? static_cast<const char*>(e.resid) + z * a.sR * ob : nullptr;
    const float bn = (e.flags & EPI_BIAS) ? e.bias[gn] : 0.f;
    const int64_t idx = static_cast<int64_t>(m) * LDC + gn;
    store_out_elem(Cp, e.out_dtype, idx, apply_epi(e, v, bn, Rp, idx));
  };

  if (S == 1) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
      if ((m & 1) == mh && m < M && cok)
        finish(m, red[0][m][col] + red[1][m][col] + red[2][m][col] + red[3][m][col]);
    return;
  }
  float* ws = static_cast<float*>(a.workspace);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if ((m & 1) != mh || m >= M || !cok) continue;
    ws[(static_cast<int64_t>(split) * MR + m) * N + gn] =
        red[0][m][col] + red[1][m][col] + red[2][m][col] + red[3][m][col];
  }
}

// Few columns (N <= 8: the strip of a product's last columns past a 256-column tile
// boundary): C[m][j] = epi(sum_k A[m][k] B[k][j]), j < N. Workgroup: 8 rows, 2 per
// wave (two workgroups per CU at 4096 rows; one row per wave measured slower, each
// workgroup staging all of B's strip); K in chunks of KC = 512. Lane l takes
// the EPL consecutive k at EPL (l + 64 i) of a chunk, one 16-byte load per row and i
// (A's rows must hold whole 16-byte chunks up to roundup(K, EPL): zero-padded copies,
// or K a multiple of EPL). B's chunk (KC rows x 8 columns, zeros past N and K; 16-byte
// loads of each row's columns, so B's rows too must hold whole 16-byte chunks up to N
// rounded up) goes through two LDS buffers, stored as [e][l][8] so that a lane's reads
// are contiguous:
// while chunk c is summed, the loads of chunk c + 1's B (into registers, written to the
// other buffer after the sums) and A are in flight. The 64 lanes' sums of each (row,
// column) are then added across the wave and lane 0 applies the epilogue. fp32
// accumulation in a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void gemv_cols_kernel(LaunchArgs a) {
  constexpr int EPL = T::code == DT_F32 ? 4 : 8;  // elements per 16-byte load
  constexpr int RW = 2, PER = 8 / EPL;             // KC = 512 rows of B per chunk
  constexpr int H = 8 / EPL;  // 16-byte chunks of a B row's 8 columns
  constexpr int KC = 64 * EPL * PER, BPT = KC * H / 256;
  __shared__ float bs[2][PER][EPL][64][8];  // chunk row kk = EPL (l + 64 i) + e at [i][e][l]
  const int M = static_cast<int>(a.M), N = static_cast<int>(a.N), K = static_cast<int>(a.K);
  const int64_t LDA = a.lda, LDB = a.ldb, LDC = a.ldc;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t z = blockIdx.y;
  const int in_bytes = T::code == DT_F32 ? 4 : 2;
  const char* Ap = static_cast<const char*>(a.A) + z * a.sA * in_bytes;
  const char* Bp = static_cast<const char*>(a.B) + z * a.sB * in_bytes;
  const int row0 = blockIdx.x * (4 * RW) + wave * RW;  // the same for the whole wave
  const int kpad = (K + EPL - 1) / EPL * EPL;
  __amdgpu_buffer_rsrc_t rA[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int m = row0 + r;
    rA[r] = grsrc(Ap + static_cast<int64_t>(m < M ? m : 0) * LDA * in_bytes,
                  m < M ? static_cast<uint32_t>(kpad * in_bytes) : 0u);
  }
  float acc[RW][8];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[r][j] = 0.f;
  // B's chunk row kk: its 8 columns as H 16-byte loads (B's rows start on 16 bytes and
  // hold whole chunks up to N rounded up); thread t takes loads t + 256 q (row / H,
  // chunk % H); chunks wholly past N or rows past K are zeros
  u32x4 bq[BPT];
  u32x4 av[RW][PER];
  auto load_b = [&](int kc) {
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      const int idx = tid + 256 * q, kk = idx / H, h = idx % H;
      bq[q] = u32x4{0u, 0u, 0u, 0u};
      if (kc + kk < K && h * EPL < N)
        bq[q] = *reinterpret_cast<const u32x4*>(
            Bp + (static_cast<int64_t>(kc + kk) * LDB + h * EPL) * in_bytes);
    }
  };
  auto store_b = [&](int buf) {
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      const int idx = tid + 256 * q, kk = idx / H, h = idx % H;
      const int e = kk % EPL, l = (kk / EPL) % 64, i = kk / (EPL * 64);
      float x[EPL];
      unpack<T>(bq[q], x);
#pragma unroll
      for (int c = 0; c < EPL; ++c) bs[buf][i][e][l][h * EPL + c] = x[c];
    }
  };
  auto load_a = [&](int kc) {
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const uint32_t off = static_cast<uint32_t>((kc + EPL * (lane + 64 * i)) * in_bytes);
        av[r][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rA[r], off, 0, 0));
      }
  };
  load_b(0);
  store_b(0);
  load_a(0);
  int buf = 0;
  for (int kc = 0; kc < K; kc += KC) {
    const bool more = kc + KC < K;
    if (more) load_b(kc + KC);  // in flight during this chunk's sums
    __syncthreads();            // chunk kc's B is in bs[buf]
    u32x4 an[RW][PER];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int i = 0; i < PER; ++i) an[r][i] = av[r][i];
    if (more) load_a(kc + KC);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      float x[RW][EPL];
#pragma unroll
      for (int r = 0; r < RW; ++r) unpack<T>(an[r][i], x[r]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(&bs[buf][i][e][lane][0]);
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(&bs[buf][i][e][lane][4]);
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[r][j] = __builtin_fmaf(x[r][e], b0[j], acc[r][j]);
            acc[r][j + 4] = __builtin_fmaf(x[r][e], b1[j], acc[r][j + 4]);
          }
      }
    }
    if (more) store_b(buf ^ 1);  // every wave read bs[buf ^ 1] before this chunk's barrier
    buf ^= 1;
  }
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int d = 1; d < 64; d *= 2) acc[r][j] += __shfl_xor(acc[r][j], d);
  if (lane != 0) return;
  const Epi& e = a.epi;
  const int64_t ob = e.out_dtype == DT_F32 ? 4 : 2;
  void* Cp = static_cast<char*>(a.C) + z * a.sC * ob;
  const void* Rp = (e.flags & EPI_RESID) ? static_cast<const char*>(e.resid) + z * a.sR * ob : nullptr;
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int m = row0 + r;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= N) continue;
      const float bn = (e.flags & EPI_BIAS) ? e.bias[j] : 0.f;
      const int64_t idx = static_cast<int64_t>(m) * LDC + j;
      store_out_elem(Cp, e.out_dtype, idx, apply_epi(e, acc[r][j], bn, Rp, idx));
    }
  }
}

// C[m][n] = epi(sum over s of partial[s][m][n]), s ascending; one thread per element
// (partial [split][rows][N]).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(LaunchArgs a, int64_t z, int64_t rows) {
  const int64_t N = a.N;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= a.M * N) return;
  const int64_t m = i / N, n = i - m * N;
  const int64_t o = m * a.ldc + n;  // C (and residual) index: row stride ldc
  const float* ws = static_cast<const float*>(a.workspace);
  const int64_t stride = rows * N;
  const float* p = ws + m * N + n;
  float s = 0.f;
  for (int s0 = 0; s0 < a.split; s0 += 32) {  // 32 loads in flight, summed in slice order
    float t[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) t[j] = s0 + j < a.split ? p[(s0 + j) * stride] : 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) s += t[j];
  }
  const Epi& e = a.epi;
  const int64_t ob = e.out_dtype == DT_F32 ? 4 : 2;
  void* Cp = static_cast<char*>(a.C) + z * a.sC * ob;
  const void* Rp =
      (e.flags & EPI_RESID) ? static_cast<const char*>(e.resid) + z * a.sR * ob : nullptr;
  const float bn = (e.flags & EPI_BIAS) ? e.bias[n] : 0.f;
  store_out_elem(Cp, e.out_dtype, o, apply_epi(e, s, bn, Rp, o));
}

template <typename T, int MR, int KMAX, int U>
hipError_t launch_gemv(const LaunchArgs& a, hipStream_t s) {
  const unsigned strips = static_cast<unsigned>((a.N + GNS - 1) / GNS);
  if (a.M > MR || a.split < 1 || (a.K + a.split - 1) / a.split > KMAX) return hipErrorInvalidValue;
  if (a.split == 1) {  // no workspace: every batch item in one launch
    hipLaunchKernelGGL((gemv_kernel<T, MR, KMAX, U>), dim3(strips, 1, static_cast<unsigned>(a.batch)),
                       dim3(GNT), 0, s, a, int64_t(0));
    return hipGetLastError();
  }
  if (!a.workspace ||
      a.workspace_bytes < static_cast<int64_t>(a.split) * MR * a.N * 4)
    return hipErrorInvalidValue;
  for (int64_t z = 0; z < a.batch; ++z) {  // batch items share the workspace, in stream order
    hipLaunchKernelGGL((gemv_kernel<T, MR, KMAX, U>), dim3(strips, static_cast<unsigned>(a.split)),
                       dim3(GNT), 0, s, a, z);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    err = launch_splitk_reduce(a, z, MR, s);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// bk holds KMAX, the most K rows one workgroup takes; U is the B rows each lane
// has in flight (4 where MR x 8 accumulators already fill the registers).
#define G15_GEMV(T, TN, MR, KMAX, U)                                                        \
  {"gemv_" TN "_m" #MR, KIND_GEMV, T::code, MR, GNS, KMAX, GNT,                             \
   static_cast<int>(sizeof(float) * (MR * KMAX + 4 * MR * GNS)), 0, 1,                      \
   launch_gemv<T, MR, KMAX, U>, 1}

const KernelEntry kGemv[] = {
    G15_GEMV(f16_t, "f16", 1, 4096, 8),   G15_GEMV(f16_t, "f16", 4, 1024, 4),
    G15_GEMV(f16_t, "f16", 8, 512, 4),    G15_GEMV(bf16_t, "bf16", 1, 4096, 8),
    G15_GEMV(bf16_t, "bf16", 4, 1024, 4), G15_GEMV(bf16_t, "bf16", 8, 512, 4),
    G15_GEMV(f32_t, "f32", 1, 4096, 8),   G15_GEMV(f32_t, "f32", 4, 1024, 4),
    G15_GEMV(f32_t, "f32", 8, 512, 4),
};

}  // namespace

hipError_t launch_splitk_reduce(const LaunchArgs& a, int64_t z, int64_t rows, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((a.M * a.N + 255) / 256);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, a, z, rows);
  return hipGetLastError();
}

int gemv_entries(const KernelEntry** out) {
  *out = kGemv;
  return static_cast<int>(sizeof(kGemv) / sizeof(kGemv[0]));
}

hipError_t launch_gemv_cols(const LaunchArgs& a, int in_dtype, hipStream_t s) {
  const int64_t es = in_dtype == DT_F32 ? 4 : 2, epl = 16 / es;
  if (a.N < 1 || a.N > 8 || a.M < 1 || a.batch < 1 || a.batch > 65535 ||
      (a.M + 7) / 8 > 0x7fffffff || (a.lda * es) % 16 != 0 || (a.sA * es) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(a.A) % 16 != 0 || a.lda < (a.K + epl - 1) / epl * epl ||
      a.K * es >= (int64_t(1) << 31) || (a.ldb * es) % 16 != 0 || (a.sB * es) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(a.B) % 16 != 0 || a.ldb < (a.N + epl - 1) / epl * epl)
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((a.M + 7) / 8), static_cast<unsigned>(a.batch));
  if (in_dtype == DT_F32)
    hipLaunchKernelGGL(gemv_cols_kernel<f32_t>, grid, dim3(256), 0, s, a);
  else if (in_dtype == DT_BF16)
    hipLaunchKernelGGL(gemv_cols_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  else if (in_dtype == DT_F16)
    hipLaunchKernelGGL(gemv_cols_kernel<f16_t>, grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace g15
