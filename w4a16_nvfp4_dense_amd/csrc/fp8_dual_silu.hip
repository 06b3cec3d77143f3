// fp8_dual_silu.hip -- instantiations of the FP8 dual GEMV that write
// h = bf16(SiLU(gate) * up) in their epilogue.
#include <hip/hip_runtime.h>

#include "fp8_gemv.h"

namespace ffn {

hipError_t fp8_dual_h_silu(int M, const Fp8Params &p, hipStream_t stream)
{
    return fp8_launch_batch<2, IN_BF16, OUT_H_SILU>(M, p, stream);
}

}  // namespace ffn
