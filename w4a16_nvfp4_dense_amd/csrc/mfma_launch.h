// mfma_launch.h -- host interface of the prefill GEMMs (matrix-core arm).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "kernels.h"

namespace ffn {

constexpr int kMfmaMaxM = 128;     // token rows per launch (larger batches are cut into blocks)
constexpr int kMfmaMaxGrid = 256;  // workgroups of a stream-K launch

// Stream-K scratch: the partial-tile slots and, for the dual GEMM's in-kernel
// finishing, one 64-bit ready word per slot and wave (set to a per-launch tag
// by the writer, cleared by the reader; contents need no initialisation).
struct MfmaScratch {
    float *partials;             // mfma_partials_floats() floats
    unsigned long long *flags;   // mfma_flag_words() words
};

size_t mfma_partials_floats();
size_t mfma_flag_words();
// Bytes of the scratch at `base` (partials, then flags), and the scratch there.
size_t mfma_scratch_bytes();
MfmaScratch mfma_scratch(void *base);

// Dual GEMM (gate and up, rows = N, cols = K) and down GEMM (rows = K,
// cols = N) for 1 <= M <= kMfmaMaxM token rows; cols must be a multiple of 64.
// With ws == nullptr every workgroup computes whole tiles (no scratch);
// otherwise the work is balanced over the compute units with stream-K.
hipError_t launch_mfma_dual(int M, OutKind out, const void *x, const WeightArg &w0, const WeightArg &w1,
                            void *out0, void *out1, int rows, int cols, const MfmaScratch *ws,
                            hipStream_t stream);
hipError_t launch_mfma_down(int M, InKind in, const void *in0, const float *in1, const WeightArg &w, void *out,
                            int rows, int cols, const MfmaScratch *ws, hipStream_t stream);

}  // namespace ffn
