// stream_launch.h -- host-side launch of the row-streaming GEMV kernels:
// picks waves per workgroup and rows per wave so every compute unit gets the
// same number of rows.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>

#include "stream_gemv.h"

namespace ffn {

// Waves per workgroup of the row-streaming kernels (two per SIMD).
constexpr int kStreamWaves = 8;

struct StreamPlan {
    int blocks;
    int rows_per_block;
};

// One workgroup per compute unit, the same number of rows for each (at most
// 64 per wave; more workgroups when the matrix is larger than that).
inline StreamPlan plan_stream(int rows, int waves)
{
    const int cus = device_cu_count();
    int blocks = std::min(cus, rows);
    int rpb = (rows + blocks - 1) / blocks;
    if (rpb > kStreamMaxRowsPerWave * waves)
        rpb = kStreamMaxRowsPerWave * waves;
    blocks = (rows + rpb - 1) / rpb;
    return StreamPlan{blocks, rpb};
}

template <int M, int IT, int NMAT, int IN, int OUT>
hipError_t launch_stream_one(StreamParams p, hipStream_t stream)
{
    constexpr int D = stream_depth<M, NMAT, IT>();
    auto kern = stream_gemv_kernel<M, IT, NMAT, IN, OUT, D, kStreamWaves>;
    size_t lds = 0;
    if constexpr (IN != IN_BF16 || !stream_act_in_regs<M, IT>()) {
        p.pitch = p.cpr + 1;
        lds = static_cast<size_t>(M) * 4 * p.pitch * 16;
        if (lds > 64 * 1024) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
            if (e != hipSuccess)
                return e;
        }
    }
    const StreamPlan plan = plan_stream(p.rows, kStreamWaves);
    p.rows_per_block = plan.rows_per_block;
    void *args[] = {&p};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), dim3(plan.blocks), dim3(kStreamWaves * 64), args,
                           lds, stream);
}

template <int NMAT, int IN, int OUT>
hipError_t launch_stream_it(int M, int it, const StreamParams &p, hipStream_t stream)
{
#define FFN_STREAM_CASE(IT_)                                                        \
    case IT_:                                                                       \
        return M == 1 ? launch_stream_one<1, IT_, NMAT, IN, OUT>(p, stream)         \
                      : launch_stream_one<2, IT_, NMAT, IN, OUT>(p, stream);
    switch (it) {
        FFN_STREAM_CASE(1)
        FFN_STREAM_CASE(2)
        FFN_STREAM_CASE(3)
        FFN_STREAM_CASE(4)
        FFN_STREAM_CASE(5)
        FFN_STREAM_CASE(6)
        FFN_STREAM_CASE(7)
        FFN_STREAM_CASE(8)
        FFN_STREAM_CASE(9)
        FFN_STREAM_CASE(10)
        FFN_STREAM_CASE(11)
        FFN_STREAM_CASE(12)
    default:
        return hipErrorNotSupported;
    }
#undef FFN_STREAM_CASE
}

inline StreamParams stream_params(const void *in0, const float *in1, const WeightArg &w0, const WeightArg &w1,
                                  void *out0, void *out1, int rows, int cols)
{
    StreamParams p{};
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

// Chunks per lane of the row-streaming kernels, or 0 when the row is too
// short for a full wave per row (those rows go to the general kernel).
inline int stream_iters(int cols)
{
    const int cpr = cols / 32;
    if (lanes_per_row(cpr) != 64)
        return 0;
    return (cpr + 63) / 64;
}

}  // namespace ffn
