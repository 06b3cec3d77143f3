// wave_dual.hip -- host launch of the many-wave dual gate+up GEMV
// (1 <= M <= 8, one launch per batch) and its instantiations; the down GEMV's
// are in wave_down.hip, so the two compile in parallel.
#include "wave_launch.h"

namespace ffn {

hipError_t launch_wave_dual(int M, OutKind out, const void *x, const WeightArg &w0, const WeightArg &w1, void *out0,
                            void *out1, int rows, int cols, hipStream_t stream)
{
    const int it = wave::wave_iters(cols);
    if (M < 1 || M > 8 || it < 1 || it > wave::kWaveMaxIt)
        return hipErrorNotSupported;
    const WaveParams p = wave::wave_params(x, nullptr, w0, w1, out0, out1, rows, cols);
    switch (out) {
    case OUT_F32_PAIR: return wave::launch_batch<2, IN_BF16, OUT_F32_PAIR>(M, it, p, stream);
    case OUT_H_SILU: return wave::launch_batch<2, IN_BF16, OUT_H_SILU>(M, it, p, stream);
    case OUT_H_GELU: return wave::launch_batch<2, IN_BF16, OUT_H_GELU>(M, it, p, stream);
    default: return hipErrorNotSupported;
    }
}

}  // namespace ffn
