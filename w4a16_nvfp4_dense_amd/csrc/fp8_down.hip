// fp8_down.hip -- host launch of the FP8 down GEMV (bf16 h, or gate and up
// with the activation fused into the staging) and its instantiations.
#include <hip/hip_runtime.h>

#include "fp8_gemv.h"

namespace ffn {

hipError_t launch_fp8_down(int M, InKind in, const void *in0, const float *in1, const Fp8WeightArg &w, void *out,
                           int rows, int cols, hipStream_t stream)
{
    if (M < 1 || M > 8 || rows < 1 || cols < 16 || cols % 16 != 0)
        return hipErrorNotSupported;
    Fp8Params p{};
    p.in0 = in0;
    p.in1 = in1;
    p.codes0 = w.codes;
    p.bs0 = w.block_scale;
    p.codes1 = w.codes;
    p.bs1 = w.block_scale;
    p.out0 = out;
    p.rows = rows;
    p.cols = cols;
    p.cpr = cols / 16;
    p.bcols = (cols + 127) / 128;
    switch (in) {
    case IN_BF16: return fp8_launch_groups<1, IN_BF16, OUT_BF16>(M, p, 2, 2, stream);
    case IN_GATEUP_SILU: return fp8_launch_groups<1, IN_GATEUP_SILU, OUT_BF16>(M, p, 4, 2, stream);
    case IN_GATEUP_GELU: return fp8_launch_groups<1, IN_GATEUP_GELU, OUT_BF16>(M, p, 4, 2, stream);
    default: return hipErrorNotSupported;
    }
}

}  // namespace ffn
