// kernels.hpp -- host-side view of the gemm15 kernel family: launch arguments
// and the registry of instantiated tile configurations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace g15 {

enum KernelKind : int {
  KIND_SIMPLE = 0,  // LDS-tiled scalar kernel, any shape / alignment / type
  KIND_MFMA16 = 1,  // bf16 / fp16 MFMA kernel
  KIND_F32 = 2,     // fp32 MFMA kernel
  KIND_GEMV = 3,    // few-row split-K kernel (M small)
  KIND_LADDER = 4,  // optimisation-ladder rungs: run only when forced by name
  KIND_K1 = 5,      // one K slice (K <= bk), workgroups streaming over tiles: taken
                    // by the measured shape table or by name, not the cost model
};

// One launch: a strided batch of row-major products C = epi(A x B).
struct LaunchArgs {
  int64_t M, N, K;
  int64_t batch;
  const void* A;
  int64_t sA;  // batch strides, in elements
  const void* B;
  int64_t sB;
  void* C;
  int64_t sC;
  int64_t sR;  // residual batch stride (elements of out_dtype)
  Epi epi;
  void* workspace;      // split-K partials (GEMV kind only)
  int64_t workspace_bytes;
  int split;            // split-K factor (GEMV kind); resident workgroups (K1 kind)
  // Row strides in elements. Every kernel handles lda = K, ldb = N, ldc = N; the
  // m16d, m16t/m16n, m16s and f32d kernels take other A and B strides (operands
  // packed into padded rows).
  int64_t lda, ldb, ldc;
  int c_vec;            // 1: C (and resid) base and rows 16-byte aligned, N % 8 == 0
                        // (read by the 16-bit staged epilogue of the m16 kernels)
};

// Copy a rows x cols matrix of 16-bit elements (row stride cols) into rows of
// ld_dst >= cols elements, zero-filling columns cols .. ld_dst-1.
hipError_t pack_rows16(const void* src, int64_t rows, int64_t cols, void* dst, int64_t ld_dst,
                       hipStream_t s);
// The same for fp32 elements, ld_dst a multiple of 4.
hipError_t pack_rows32(const void* src, int64_t rows, int64_t cols, void* dst, int64_t ld_dst,
                       hipStream_t s);

// Debug aid: fill `batch` items of a rows x cols output (row stride ld, batch stride
// `stride`, both in elements of out_dtype) with NaN, so elements a kernel leaves
// unwritten show. Needs C, row lengths, row and batch strides in 4-byte multiples
// (else hipErrorInvalidValue, nothing launched).
hipError_t poison_output(void* C, int64_t rows, int64_t cols, int64_t ld, int64_t batch,
                         int64_t stride, int out_dtype, hipStream_t s);

typedef hipError_t (*LaunchFn)(const LaunchArgs&, hipStream_t);

struct KernelEntry {
  const char* name;
  int kind;       // KernelKind
  int in_dtype;   // DT_* the kernel reads; -1: any
  int bm, bn, bk; // block tile
  int threads;    // workgroup size
  int lds_bytes;  // static LDS per workgroup
  int vec_a;      // 1: needs 16-byte aligned A rows (K multiple of 16 B / elem size)
  int vec_b;      // 1: needs 16-byte aligned B rows
  LaunchFn launch;
  int buf32 = 0;  // 1: addresses A, B, C with 32-bit byte offsets (each must be < 2 GiB)
  int b_nk = 0;   // 1: B is given transposed, Bt [N x K] row-major (row stride ldb)
};

// Each kernel file appends its instantiations.
int simple_entries(const KernelEntry** out);
int mfma16_entries(const KernelEntry** out);
int mfma16_dlds_entries(const KernelEntry** out);
int mfma16_nt_entries(const KernelEntry** out);
int f32_entries(const KernelEntry** out);
int f32_dlds_entries(const KernelEntry** out);
int gemv_entries(const KernelEntry** out);
int ladder_entries(const KernelEntry** out);
int mfma16_k1_entries(const KernelEntry** out);
int mfma16_w_entries(const KernelEntry** out);

}  // namespace g15
