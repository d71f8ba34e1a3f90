// attention.hpp -- the attention probabilities P = softmax(scale * Q K^T) in one
// kernel (kernel_attention.hip): the scores never leave the registers.
#pragma once

#include "kernels.hpp"

namespace g15 {

// a: M query rows, N <= 512 keys, K <= 64 head dimension, batch items; A = Q
// [M x K], B = K^T [K x N] (b_rowmajor) or K [N x K]; C = P [M x N] of
// a.epi.out_dtype; a.epi.scale the score scale, a.epi.flags 0; a.split the
// workgroups to launch (attention_workgroups). hipErrorInvalidValue for shapes past
// those limits.
hipError_t launch_attention_probs(const LaunchArgs& a, bool bf16, bool b_rowmajor, hipStream_t s);

// Workgroups that stay resident on a device of cu_count CUs (two per CU), a
// multiple of 8.
int attention_workgroups(int cu_count);

}  // namespace g15
