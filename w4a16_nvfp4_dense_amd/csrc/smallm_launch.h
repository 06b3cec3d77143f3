// smallm_launch.h -- host interface of the small-batch matrix-core arm
// (9 <= M <= 16 token rows).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "kernels.h"

namespace ffn {

constexpr int kSmallMaxM = 16;

// Whether the small-batch arm covers the dual GEMM (rows = N, cols = K) and
// the down GEMM (rows = K, cols = N) of an M-row batch.
bool smallm_supported(int M, int K, int N);

// fp32 floats of the down GEMM's partial sums (0 when it needs none).
size_t smallm_partial_floats(int M, int K, int N);

// Dual GEMM (gate and up; out = OUT_F32_PAIR or OUT_H_*), no workspace.
hipError_t launch_smallm_dual(int M, OutKind out, const void *x, const WeightArg &w0, const WeightArg &w1,
                              void *out0, void *out1, int N, int K, hipStream_t stream);
// Down GEMM: out[M, K] bf16 from h[M, N] bf16; `partials` holds
// smallm_partial_floats(M, K, N) floats.
hipError_t launch_smallm_down(int M, const void *h, const WeightArg &w, void *out, float *partials, int K, int N,
                              hipStream_t stream);

}  // namespace ffn
