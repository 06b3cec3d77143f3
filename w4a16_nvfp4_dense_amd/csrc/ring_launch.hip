// ring_launch.hip -- host-side launch of the LDS-ring GEMV kernels (M = 1, 2)
// and their instantiations.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "ring_gemv.h"

namespace ffn {

namespace {

constexpr size_t kLdsMax = 160 * 1024;
constexpr int kRingWaves = 4;  // one wave per SIMD: each wave keeps its activations in registers

template <int M, int IT>
constexpr bool ring_fits_regs()
{
    return M * IT <= 12;  // at most 192 VGPRs of activations per lane
}

// Slots per wave: two for the dual GEMV (short rows), one for long rows;
// bounded by LDS and by the vmcnt range.
template <int NMAT, int IT, int ITS>
constexpr int ring_slots(size_t stage_bytes)
{
    constexpr int slot = NMAT * ring_mat_bytes<NMAT, IT>(ITS);
    constexpr int L = NMAT * (IT + ITS);
    int s = NMAT == 2 ? 2 : 1;
    while (s > 1 && (static_cast<size_t>(kRingWaves) * s * slot + stage_bytes > kLdsMax || (s - 1) * L >= 64))
        --s;
    return s;
}

template <int M, int IT, int NMAT, int IN, int OUT, int S>
hipError_t launch_ring_s(RingParams p, size_t lds, hipStream_t stream)
{
    constexpr int ITS = (IT + 1) / 2;
    auto kern = ring_gemv_kernel<M, IT, NMAT, IN, OUT, S, kRingWaves, ITS>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess)
        return e;
    const int cus = device_cu_count();
    const int blocks = std::max(1, std::min(cus, (p.rows + kRingWaves - 1) / kRingWaves));
    void *args[] = {&p};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), dim3(blocks), dim3(kRingWaves * 64), args, lds,
                           stream);
}

template <int M, int IT, int NMAT, int IN, int OUT>
hipError_t launch_ring_one(RingParams p, hipStream_t stream)
{
    constexpr int ITS = (IT + 1) / 2;
    if (p.cpr > 64 * IT || p.cpr <= 64 * (IT - 1) || (p.cpr & 1))
        return hipErrorNotSupported;
    size_t stage = 0;
    if constexpr (IN != IN_BF16) {
        p.pitch = p.cpr + 1;
        stage = static_cast<size_t>(M) * 4 * p.pitch * 16;
    }
    constexpr int slot = NMAT * ring_mat_bytes<NMAT, IT>(ITS);
    // Largest slot count the staging area leaves room for (compile-time cap).
    constexpr int S2 = ring_slots<NMAT, IT, ITS>(0);
    const size_t ring1 = static_cast<size_t>(kRingWaves) * slot;
    const int s_fit = static_cast<int>((kLdsMax - std::min(stage, kLdsMax)) / ring1);
    const int S = std::min(S2, s_fit);
    if (S < 1)
        return hipErrorNotSupported;
    p.stage_off = static_cast<int>(ring1 * S);
    const size_t lds = ring1 * S + stage;
    if (S >= 2)
        return launch_ring_s<M, IT, NMAT, IN, OUT, (S2 >= 2 ? 2 : 1)>(p, lds, stream);
    return launch_ring_s<M, IT, NMAT, IN, OUT, 1>(p, lds, stream);
}

template <int NMAT, int IN, int OUT>
hipError_t launch_ring_it(int M, int it, const RingParams &p, hipStream_t stream)
{
#define FFN_RING_CASE(IT_)                                                                  \
    case IT_:                                                                               \
        if (M == 1)                                                                         \
            return launch_ring_one<1, IT_, NMAT, IN, OUT>(p, stream);                      \
        if constexpr (ring_fits_regs<2, IT_>())                                             \
            return launch_ring_one<2, IT_, NMAT, IN, OUT>(p, stream);                      \
        return hipErrorNotSupported;
    switch (it) {
        FFN_RING_CASE(1)
        FFN_RING_CASE(2)
        FFN_RING_CASE(3)
        FFN_RING_CASE(4)
        FFN_RING_CASE(5)
        FFN_RING_CASE(6)
        FFN_RING_CASE(7)
        FFN_RING_CASE(8)
        FFN_RING_CASE(9)
        FFN_RING_CASE(10)
        FFN_RING_CASE(11)
        FFN_RING_CASE(12)
    default:
        return hipErrorNotSupported;
    }
#undef FFN_RING_CASE
}

RingParams ring_params(const void *in0, const float *in1, const WeightArg &w0, const WeightArg &w1, void *out0,
                       void *out1, int rows, int cols)
{
    RingParams p{};
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

// Chunks per lane when a whole wave takes one row, or 0 when the row is too
// short for that (those rows go to the general kernel).
int ring_iters(int cols)
{
    const int cpr = cols / 32;
    if (lanes_per_row(cpr) != 64 || (cpr & 1))
        return 0;
    return (cpr + 63) / 64;
}

}  // namespace

hipError_t launch_ring_dual(int M, OutKind out, const void *x, const WeightArg &w0, const WeightArg &w1, void *out0,
                            void *out1, int rows, int cols, hipStream_t stream)
{
    const int it = ring_iters(cols);
    if (M < 1 || M > 2 || it < 1 || it > kStreamMaxIt)
        return hipErrorNotSupported;
    const RingParams p = ring_params(x, nullptr, w0, w1, out0, out1, rows, cols);
    switch (out) {
    case OUT_F32_PAIR: return launch_ring_it<2, IN_BF16, OUT_F32_PAIR>(M, it, p, stream);
    case OUT_H_SILU: return launch_ring_it<2, IN_BF16, OUT_H_SILU>(M, it, p, stream);
    case OUT_H_GELU: return launch_ring_it<2, IN_BF16, OUT_H_GELU>(M, it, p, stream);
    default: return hipErrorNotSupported;
    }
}

hipError_t launch_ring_down(int M, InKind in, const void *in0, const float *in1, const WeightArg &w, void *out,
                            int rows, int cols, hipStream_t stream)
{
    const int it = ring_iters(cols);
    if (M < 1 || M > 2 || it < 1 || it > kStreamMaxIt)
        return hipErrorNotSupported;
    const RingParams p = ring_params(in0, in1, w, w, out, nullptr, rows, cols);
    switch (in) {
    case IN_BF16: return launch_ring_it<1, IN_BF16, OUT_BF16>(M, it, p, stream);
    case IN_GATEUP_SILU: return launch_ring_it<1, IN_GATEUP_SILU, OUT_BF16>(M, it, p, stream);
    case IN_GATEUP_GELU: return launch_ring_it<1, IN_GATEUP_GELU, OUT_BF16>(M, it, p, stream);
    default: return hipErrorNotSupported;
    }
}

}  // namespace ffn
