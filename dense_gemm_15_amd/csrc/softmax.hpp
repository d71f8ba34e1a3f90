// softmax.hpp -- entry of the row softmax kernel (kernel_softmax.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace g15 {

// P = softmax(scale * S) row by row: S fp32 rows x cols with row stride lds, P of
// element type out_dt (DT_F32 / DT_F16 / DT_BF16) with row stride ldp.
hipError_t launch_softmax_rows(const float* S, int64_t rows, int64_t cols, int64_t lds,
                               float scale, void* P, int64_t ldp, int out_dt, hipStream_t s);

}  // namespace g15
