// fp8_down_gelu.hip -- instantiations of the FP8 down GEMV that stage
// h = bf16(GELU-tanh(gate) * up) from fp32 gate and up.
#include <hip/hip_runtime.h>

#include "fp8_gemv.h"

namespace ffn {

hipError_t fp8_down_act_gelu(int M, const Fp8Params &p, hipStream_t stream)
{
    return fp8_launch_batch<1, IN_GATEUP_GELU, OUT_BF16>(M, p, stream);
}

}  // namespace ffn
