// fp8_down.hip -- host launch of the FP8 down GEMV (one launch per batch of
// 1 <= M <= 8 rows) and the instantiations that read h in bf16; those with
// the activation fused into the staging are in fp8_down_silu.hip and
// fp8_down_gelu.hip.
#include <hip/hip_runtime.h>

#include "fp8_gemv.h"

namespace ffn {

hipError_t fp8_down_h(int M, const Fp8Params &p, hipStream_t stream)
{
    return fp8_launch_batch<1, IN_BF16, OUT_BF16>(M, p, stream);
}

hipError_t launch_fp8_down(int M, InKind in, const void *in0, const float *in1, const Fp8WeightArg &w, void *out,
                           int rows, int cols, hipStream_t stream)
{
    if (M < 1 || M > 8 || rows < 1 || cols < 16 || cols % 16 != 0)
        return hipErrorNotSupported;
    const Fp8Params p = fp8_params(in0, in1, w, w, out, nullptr, rows, cols);
    switch (in) {
    case IN_BF16: return fp8_down_h(M, p, stream);
    case IN_GATEUP_SILU: return fp8_down_act_silu(M, p, stream);
    case IN_GATEUP_GELU: return fp8_down_act_gelu(M, p, stream);
    default: return hipErrorNotSupported;
    }
}

}  // namespace ffn
