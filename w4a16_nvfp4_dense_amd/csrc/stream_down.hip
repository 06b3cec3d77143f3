// stream_down.hip -- instantiations of the row-streaming down GEMV (input h in
// bf16, or fp32 gate/up with the activation fused into the input load).
#include "stream_launch.h"

namespace ffn {

int device_cu_count()
{
    static int counts[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = __atomic_load_n(&counts[dev], __ATOMIC_RELAXED);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        __atomic_store_n(&counts[dev], n, __ATOMIC_RELAXED);
    }
    return n;
}

hipError_t launch_stream_down(int M, InKind in, const void *in0, const float *in1, const WeightArg &w,
                              void *out, int rows, int cols, hipStream_t stream)
{
    const int it = stream_iters(cols);
    if (M < 1 || M > 2 || it < 1 || it > kStreamMaxIt)
        return hipErrorNotSupported;
    const StreamParams p = stream_params(in0, in1, w, w, out, nullptr, rows, cols);
    switch (in) {
    case IN_BF16: return launch_stream_it<1, IN_BF16, OUT_BF16>(M, it, p, stream);
    case IN_GATEUP_SILU: return launch_stream_it<1, IN_GATEUP_SILU, OUT_BF16>(M, it, p, stream);
    case IN_GATEUP_GELU: return launch_stream_it<1, IN_GATEUP_GELU, OUT_BF16>(M, it, p, stream);
    default: return hipErrorNotSupported;
    }
}

}  // namespace ffn
