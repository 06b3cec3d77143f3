// wave_launch.hip -- host-side launch of the many-wave GEMV (M = 1, 2) and
// its instantiations.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "wave_gemv.h"

namespace ffn {

namespace {

constexpr int kWaveMaxIt = 12;  // chunks per lane: reduction length up to 24576

// Waves per workgroup and workgroups per compute unit (measured on MI355X at
// the decode shapes): the dual GEMV runs 2 x 8 waves per CU, the down GEMV
// 16 waves in one workgroup per CU.
template <int NMAT>
constexpr int wave_w()
{
    return NMAT == 2 ? 8 : 16;
}
template <int NMAT>
constexpr int wave_blocks_per_cu()
{
    return NMAT == 2 ? 2 : 1;
}

template <int M, int IT, int NMAT, int IN, int OUT>
hipError_t launch_one(const WaveParams &p, hipStream_t stream)
{
    constexpr int W = wave_w<NMAT>();
    auto kern = wave_gemv_kernel<M, IT, NMAT, IN, OUT, W>;
    const int lds = M * IT * 4096;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess)
            return e;
    }
    const int want = device_cu_count() * wave_blocks_per_cu<NMAT>();
    const int blocks = std::max(1, std::min(want, (p.rows + W - 1) / W));
    WaveParams q = p;
    void *args[] = {&q};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), dim3(blocks), dim3(W * 64), args, lds, stream);
}

template <int NMAT, int IN, int OUT>
hipError_t launch_it(int M, int it, const WaveParams &p, hipStream_t stream)
{
#define FFN_WAVE_CASE(IT_)                                                   \
    case IT_:                                                                \
        return M == 1 ? launch_one<1, IT_, NMAT, IN, OUT>(p, stream)         \
                      : launch_one<2, IT_, NMAT, IN, OUT>(p, stream);
    switch (it) {
        FFN_WAVE_CASE(1)
        FFN_WAVE_CASE(2)
        FFN_WAVE_CASE(3)
        FFN_WAVE_CASE(4)
        FFN_WAVE_CASE(5)
        FFN_WAVE_CASE(6)
        FFN_WAVE_CASE(7)
        FFN_WAVE_CASE(8)
        FFN_WAVE_CASE(9)
        FFN_WAVE_CASE(10)
        FFN_WAVE_CASE(11)
        FFN_WAVE_CASE(12)
    default:
        return hipErrorNotSupported;
    }
#undef FFN_WAVE_CASE
}

WaveParams wave_params(const void *in0, const float *in1, const WeightArg &w0, const WeightArg &w1, void *out0,
                       void *out1, int rows, int cols)
{
    WaveParams p{};
    p.in0 = in0;
    p.in1 = in1;
    p.codes0 = w0.codes;
    p.scales0 = w0.scales;
    p.s2_0 = w0.scale2;
    p.codes1 = w1.codes;
    p.scales1 = w1.scales;
    p.s2_1 = w1.scale2;
    p.out0 = out0;
    p.out1 = out1;
    p.rows = rows;
    p.cols = cols;
    p.cpr = cols / 32;
    return p;
}

// Chunks per lane when a whole wave takes one row (the canonical lane count
// for this reduction length is 64), else 0.
int wave_iters(int cols)
{
    const int cpr = cols / 32;
    if (lanes_per_row(cpr) != 64)
        return 0;
    return (cpr + 63) / 64;
}

}  // namespace

hipError_t launch_wave_dual(int M, OutKind out, const void *x, const WeightArg &w0, const WeightArg &w1, void *out0,
                            void *out1, int rows, int cols, hipStream_t stream)
{
    const int it = wave_iters(cols);
    if (M < 1 || M > 2 || it < 1 || it > kWaveMaxIt)
        return hipErrorNotSupported;
    const WaveParams p = wave_params(x, nullptr, w0, w1, out0, out1, rows, cols);
    switch (out) {
    case OUT_F32_PAIR: return launch_it<2, IN_BF16, OUT_F32_PAIR>(M, it, p, stream);
    case OUT_H_SILU: return launch_it<2, IN_BF16, OUT_H_SILU>(M, it, p, stream);
    case OUT_H_GELU: return launch_it<2, IN_BF16, OUT_H_GELU>(M, it, p, stream);
    default: return hipErrorNotSupported;
    }
}

hipError_t launch_wave_down(int M, InKind in, const void *in0, const float *in1, const WeightArg &w, void *out,
                            int rows, int cols, hipStream_t stream)
{
    const int it = wave_iters(cols);
    if (M < 1 || M > 2 || it < 1 || it > kWaveMaxIt)
        return hipErrorNotSupported;
    const WaveParams p = wave_params(in0, in1, w, w, out, nullptr, rows, cols);
    switch (in) {
    case IN_BF16: return launch_it<1, IN_BF16, OUT_BF16>(M, it, p, stream);
    case IN_GATEUP_SILU: return launch_it<1, IN_GATEUP_SILU, OUT_BF16>(M, it, p, stream);
    case IN_GATEUP_GELU: return launch_it<1, IN_GATEUP_GELU, OUT_BF16>(M, it, p, stream);
    default: return hipErrorNotSupported;
    }
}

}  // namespace ffn
