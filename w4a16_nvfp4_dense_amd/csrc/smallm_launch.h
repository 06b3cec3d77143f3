// smallm_launch.h -- host interface of the small-batch matrix-core arm
// (9 <= M <= 40 token rows).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "kernels.h"

namespace ffn {

constexpr int kSmallMaxM = 40;

// Whether the small-batch arm covers the dual GEMM (rows = N, cols = K) and
// the down GEMM (rows = K, cols = N) of an M-row batch.
bool smallm_supported(int M, int K, int N);

// Whether the dual GEMM's reduction is split in parts (it then needs
// smallm_dual_partial_floats(M, K, N) floats of workspace).
bool smallm_dual_split(int M, int K, int N);

// fp32 floats of the down GEMM's partial sums (0 when it needs none).
size_t smallm_partial_floats(int M, int K, int N);

// fp32 floats of the dual GEMM's partial sums (0 when it needs none).
size_t smallm_dual_partial_floats(int M, int K, int N);

// 64-bit ready words that a split reduction of either GEMM uses (0 when
// neither is split): one per workgroup, set to a per-launch tag by the
// workgroups of the lower parts and cleared by the one that finishes their
// tiles, so they need no initialisation; the two GEMMs of a forward may share
// them (stream-ordered).
size_t smallm_flag_words(int M, int K, int N);

// Dual GEMM (gate and up; out = OUT_F32_PAIR or OUT_H_*); `partials` holds
// smallm_dual_partial_floats(M, K, N) floats and `flags` smallm_flag_words()
// words (both may be null when the reduction is not split).
hipError_t launch_smallm_dual(int M, OutKind out, const void *x, const WeightArg &w0, const WeightArg &w1,
                              void *out0, void *out1, float *partials, unsigned long long *flags, int N, int K,
                              hipStream_t stream);
// Down GEMM: out[M, K] bf16 from h[M, N] bf16; `partials` holds
// smallm_partial_floats(M, K, N) floats, `flags` as above.
hipError_t launch_smallm_down(int M, const void *h, const WeightArg &w, void *out, float *partials,
                              unsigned long long *flags, int K, int N, hipStream_t stream);

}  // namespace ffn
