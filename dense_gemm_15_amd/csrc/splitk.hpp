// splitk.hpp -- the second kernel of a split-K product: C = epi(sum of the fp32
// partial products in the plan's workspace), shared by the few-row kernel and the
// tile kernels run split along K.
#pragma once

#include "kernels.hpp"

namespace g15 {

// C[z][m][n] = epi(sum over s < a.split, ascending, of ws[s][m][n]) for m < a.M,
// n < a.N, with ws = a.workspace as float [a.split][rows][a.N] (rows >= a.M). Bias,
// residual (batch item z, stride a.sR), scale and output type come from a.epi; C is
// batch item z of a.C (stride a.sC).
hipError_t launch_splitk_reduce(const LaunchArgs& a, int64_t z, int64_t rows, hipStream_t s);

}  // namespace g15
