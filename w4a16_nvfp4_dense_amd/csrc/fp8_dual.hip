// fp8_dual.hip -- host launch of the FP8 dual gate+up GEMV (one launch per
// batch of 1 <= M <= 8 rows) and the instantiations with fp32 gate and up out;
// those with h in the epilogue are in fp8_dual_silu.hip and fp8_dual_gelu.hip.
#include <hip/hip_runtime.h>

#include "fp8_gemv.h"

namespace ffn {

hipError_t fp8_dual_pair(int M, const Fp8Params &p, hipStream_t stream)
{
    return fp8_launch_batch<2, IN_BF16, OUT_F32_PAIR>(M, p, stream);
}

hipError_t launch_fp8_dual(int M, OutKind out, const void *x, const Fp8WeightArg &w0, const Fp8WeightArg &w1,
                           void *out0, void *out1, int rows, int cols, hipStream_t stream)
{
    if (M < 1 || M > 8 || rows < 1 || cols < 16 || cols % 16 != 0)
        return hipErrorNotSupported;
    const Fp8Params p = fp8_params(x, nullptr, w0, w1, out0, out1, rows, cols);
    switch (out) {
    case OUT_F32_PAIR: return fp8_dual_pair(M, p, stream);
    case OUT_H_SILU: return fp8_dual_h_silu(M, p, stream);
    case OUT_H_GELU: return fp8_dual_h_gelu(M, p, stream);
    default: return hipErrorNotSupported;
    }
}

}  // namespace ffn
