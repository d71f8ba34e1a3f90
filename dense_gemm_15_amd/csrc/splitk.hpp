// splitk.hpp -- the second kernel of a split-K product: C = epi(sum of the fp32
// partial products in the plan's workspace), shared by the few-row kernel and the
// tile kernels run split along K.
#pragma once

#include "kernels.hpp"

namespace g15 {

// C[z][m][n] = epi(sum over s < a.split, ascending, of ws[s][m][n]) for m < a.M,
// n < a.N, with ws = a.workspace as float [a.split][rows][a.N] (rows >= a.M). Bias,
// residual (batch item z, stride a.sR), scale and output type come from a.epi; C is
// batch item z of a.C (stride a.sC), row stride a.ldc.
hipError_t launch_splitk_reduce(const LaunchArgs& a, int64_t z, int64_t rows, hipStream_t s);

// Few columns: C[z][m][j] = epi(sum_k A[z][m][k] B[z][k][j]) for m < a.M, j < a.N <= 8,
// A, B of type in_dtype (DT_*) with row strides a.lda, a.ldb, C and the residual with
// row stride a.ldc, bias[j]; every batch item in one launch. A's and B's rows must start
// on 16 bytes and hold whole 16-byte chunks up to K (A) and N (B) rounded up, zero past
// K (padded copies, or K a multiple of 16 bytes); hipErrorInvalidValue otherwise, for N
// outside 1..8 or another type.
hipError_t launch_gemv_cols(const LaunchArgs& a, int in_dtype, hipStream_t s);

}  // namespace g15
