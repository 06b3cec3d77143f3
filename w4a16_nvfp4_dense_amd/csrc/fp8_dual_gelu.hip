// fp8_dual_gelu.hip -- instantiations of the FP8 dual GEMV that write
// h = bf16(GELU-tanh(gate) * up) in their epilogue.
#include <hip/hip_runtime.h>

#include "fp8_gemv.h"

namespace ffn {

hipError_t fp8_dual_h_gelu(int M, const Fp8Params &p, hipStream_t stream)
{
    return fp8_launch_batch<2, IN_BF16, OUT_H_GELU>(M, p, stream);
}

}  // namespace ffn
