// stream_dual.hip -- instantiations of the row-streaming dual gate+up GEMV
// (gate/up in fp32, or h = act(gate) * up in bf16 from the epilogue).
#include "stream_launch.h"

namespace ffn {

hipError_t launch_stream_dual(int M, OutKind out, const void *x, const WeightArg &w0, const WeightArg &w1,
                              void *out0, void *out1, int rows, int cols, hipStream_t stream)
{
    const int it = stream_iters(cols);
    if (M < 1 || M > 2 || it < 1 || it > kStreamMaxIt)
        return hipErrorNotSupported;
    const StreamParams p = stream_params(x, nullptr, w0, w1, out0, out1, rows, cols);
    switch (out) {
    case OUT_F32_PAIR: return launch_stream_it<2, IN_BF16, OUT_F32_PAIR>(M, it, p, stream);
    case OUT_H_SILU: return launch_stream_it<2, IN_BF16, OUT_H_SILU>(M, it, p, stream);
    case OUT_H_GELU: return launch_stream_it<2, IN_BF16, OUT_H_GELU>(M, it, p, stream);
    default: return hipErrorNotSupported;
    }
}

}  // namespace ffn
