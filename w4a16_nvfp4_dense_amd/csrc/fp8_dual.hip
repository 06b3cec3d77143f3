// fp8_dual.hip -- host launch of the FP8 dual gate+up GEMV and its
// instantiations (the down GEMV's are in fp8_down.hip, so the two compile in
// parallel).
#include <hip/hip_runtime.h>

#include "fp8_gemv.h"

namespace ffn {

hipError_t launch_fp8_dual(int M, OutKind out, const void *x, const Fp8WeightArg &w0, const Fp8WeightArg &w1,
                           void *out0, void *out1, int rows, int cols, hipStream_t stream)
{
    if (M < 1 || M > 8 || rows < 1 || cols < 16 || cols % 16 != 0)
        return hipErrorNotSupported;
    Fp8Params p{};
    p.in0 = x;
    p.codes0 = w0.codes;
    p.bs0 = w0.block_scale;
    p.codes1 = w1.codes;
    p.bs1 = w1.block_scale;
    p.out0 = out0;
    p.out1 = out1;
    p.rows = rows;
    p.cols = cols;
    p.cpr = cols / 16;
    p.bcols = (cols + 127) / 128;
    switch (out) {
    case OUT_F32_PAIR: return fp8_launch_groups<2, IN_BF16, OUT_F32_PAIR>(M, p, 2, 4, stream);
    case OUT_H_SILU: return fp8_launch_groups<2, IN_BF16, OUT_H_SILU>(M, p, 2, 2, stream);
    case OUT_H_GELU: return fp8_launch_groups<2, IN_BF16, OUT_H_GELU>(M, p, 2, 2, stream);
    default: return hipErrorNotSupported;
    }
}

}  // namespace ffn
