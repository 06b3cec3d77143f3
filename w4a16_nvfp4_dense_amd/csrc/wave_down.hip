// wave_down.hip -- host launch of the many-wave down GEMV (1 <= M <= 8, one
// launch per batch; the input is h in bf16, or gate and up in fp32 with the
// activation fused into the staging) and its instantiations.
#include "wave_launch.h"

namespace ffn {

hipError_t launch_wave_down(int M, InKind in, const void *in0, const float *in1, const WeightArg &w, void *out,
                            int rows, int cols, hipStream_t stream)
{
    const int it = wave::wave_iters(cols);
    if (M < 1 || M > 8 || it < 1 || it > wave::kWaveMaxIt)
        return hipErrorNotSupported;
    const WaveParams p = wave::wave_params(in0, in1, w, w, out, nullptr, rows, cols);
    switch (in) {
    case IN_BF16: return wave::launch_batch<1, IN_BF16, OUT_BF16>(M, it, p, stream);
    case IN_GATEUP_SILU: return wave::launch_batch<1, IN_GATEUP_SILU, OUT_BF16>(M, it, p, stream);
    case IN_GATEUP_GELU: return wave::launch_batch<1, IN_GATEUP_GELU, OUT_BF16>(M, it, p, stream);
    default: return hipErrorNotSupported;
    }
}

}  // namespace ffn
