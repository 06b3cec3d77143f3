// wave_launch.h -- host-side launch templates of the many-wave GEMV
// (1 <= M <= 8), shared by the dual (wave_dual.hip) and down (wave_down.hip)
// translation units, which compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>

#include "wave_gemv.h"

namespace ffn {

namespace wave {

constexpr int kWaveMaxIt = 12;        // chunks per lane: reduction length up to 24576
constexpr int kWaveLdsMax = 144 * 1024;  // of the 160 KB per compute unit

// Pieces the activations are staged in: the fewest whose steps
// (M x ceil(IT / P) x 4 KB) fit the LDS budget.
template <int M, int IT>
constexpr int wave_pieces()
{
    int pc = 1;
    while (M * ((IT + pc - 1) / pc) * 4096 > kWaveLdsMax)
        ++pc;
    return pc;
}

// Steps staged at a time.
template <int M, int IT>
constexpr int wave_piece_steps()
{
    return (IT + wave_pieces<M, IT>() - 1) / wave_pieces<M, IT>();
}

// Waves per workgroup: 16 (at most 128 registers per lane) while the
// weight registers of one row (5 per chunk and matrix), the converted chunk
// (16 per matrix) and the accumulators fit in that with room to spare,
// otherwise 8 (up to 256 registers).
// (With the activations in pieces the weight registers hold one piece of a
// row, and the accumulators of two rows.)
template <int M, int IT, int NMAT>
constexpr int wave_w_regs()
{
    constexpr int IS = wave_piece_steps<M, IT>();
    constexpr int acc = (wave_pieces<M, IT>() > 1 ? kPieceMaxRows : 1) * M * NMAT;
    return (NMAT * IS * 5 + NMAT * 16 + acc + 30 <= 120) ? 16 : 8;
}

// Measured on MI355X at the decode shapes: the dual GEMV runs best as 2 x 8
// waves per compute unit while two workgroups' activations fit in LDS; the
// down GEMV as 16 waves in one workgroup.
template <int M, int IT, int NMAT>
constexpr int wave_w()
{
    return (NMAT == 2 && wave_pieces<M, IT>() == 1 && 2 * M * IT * 4096 <= kWaveLdsMax) ? 8
                                                                                       : wave_w_regs<M, IT, NMAT>();
}

template <int M, int IT, int NMAT>
constexpr int wave_blocks_per_cu()
{
    return (wave_w<M, IT, NMAT>() == 8 && 2 * M * wave_piece_steps<M, IT>() * 4096 <= kWaveLdsMax) ? 2 : 1;
}

template <int M, int IT, int NMAT, int IN, int OUT>
hipError_t launch_one(const WaveParams &p, hipStream_t stream)
{
    constexpr int W = wave_w<M, IT, NMAT>();
    constexpr int P = wave_pieces<M, IT>();
    auto kern = wave_gemv_kernel<M, IT, NMAT, IN, OUT, W, P>;
    const int lds = M * wave_piece_steps<M, IT>() * 4096;
    if (lds > 64 * 1024) {
        static std::atomic<uint64_t> lds_done{0};
        hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), lds, lds_done);
        if (e != hipSuccess)
            return e;
    }
    const int want = device_cu_count() * wave_blocks_per_cu<M, IT, NMAT>();
    int blocks = std::max(1, std::min(want, (p.rows + W - 1) / W));
    if constexpr (P > 1) {
        // every wave holds at most kPieceMaxRows rows
        const int rows_per_block = W * kPieceMaxRows;
        blocks = std::max(blocks, (p.rows + rows_per_block - 1) / rows_per_block);
    }
    WaveParams q = p;
    void *args[] = {&q};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), dim3(blocks), dim3(W * 64), args, lds, stream);
}

template <int IT, int NMAT, int IN, int OUT>
hipError_t launch_m(int M, const WaveParams &p, hipStream_t stream)
{
    switch (M) {
    case 1: return launch_one<1, IT, NMAT, IN, OUT>(p, stream);
    case 2: return launch_one<2, IT, NMAT, IN, OUT>(p, stream);
    case 3: return launch_one<3, IT, NMAT, IN, OUT>(p, stream);
    case 4: return launch_one<4, IT, NMAT, IN, OUT>(p, stream);
    case 5: return launch_one<5, IT, NMAT, IN, OUT>(p, stream);
    case 6: return launch_one<6, IT, NMAT, IN, OUT>(p, stream);
    case 7: return launch_one<7, IT, NMAT, IN, OUT>(p, stream);
    case 8: return launch_one<8, IT, NMAT, IN, OUT>(p, stream);
    default: return hipErrorNotSupported;
    }
}

// One launch for the whole batch (1 <= M <= 8): every weight byte is read
// once for all M activation rows.
template <int NMAT, int IN, int OUT>
hipError_t launch_batch(int M, int it, const WaveParams &p, hipStream_t stream)
{
    switch (it) {
#define FFN_WAVE_CASE(IT_) \
    case IT_: return launch_m<IT_, NMAT, IN, OUT>(M, p, stream);
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
#undef FFN_WAVE_CASE
    default: return hipErrorNotSupported;
    }
}

inline WaveParams wave_params(const void *in0, const float *in1, const WeightArg &w0, const WeightArg &w1, void *out0,
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
inline int wave_iters(int cols)
{
    const int cpr = cols / 32;
    if (lanes_per_row(cpr) != 64)
        return 0;
    return (cpr + 63) / 64;
}

}  // namespace wave

}  // namespace ffn
