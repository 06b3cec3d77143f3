// mfma_launch.hip -- host-side launch of the prefill GEMMs (9 <= M tokens,
// up to 128 per launch) and their instantiations.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "mfma_gemm.h"
#include "mfma_launch.h"

namespace ffn {

namespace {

// Ring stages: 4 (three units in flight), or fewer if they do not fit in
// ~150 KB of LDS. Measured on MI355X at 5120/17408 with 48 to 128 tokens:
// 4 stages beat 3 (slower at 128 tokens) and 5 to 8 (the most that fit) by
// 2 to 5 us per forward.
template <int MT>
constexpr int stages()
{
    constexpr int s = (150 * 1024) / mfma_stage_bytes<MT>();
    return s > 4 ? 4 : s;
}

template <int MT, int NMAT, int IN, int OUT, bool FIX = false>
hipError_t launch_t(MfmaParams p, int G, hipStream_t stream)
{
    constexpr int S = stages<MT>();
    auto kern = mfma_gemm_kernel<MT, NMAT, IN, OUT, S, FIX>;
    const int lds = S * mfma_stage_bytes<MT>();
    static std::atomic<uint64_t> lds_done{0};
    hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), lds, lds_done);
    if (e != hipSuccess)
        return e;
    void *args[] = {&p};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), dim3(G), dim3(kMfmaWaves * 64), args, lds, stream);
}

// The GEMM, then (stream-K) the reduction of the split tiles. The dual GEMM
// finishes its split tiles in the kernel when the scratch has ready words:
// the workgroup holding a tile's last unit adds the lower workgroups' pieces
// once their ready words carry this launch's tag.
template <int MT, int NMAT, int IN, int OUT>
hipError_t launch_gemm_reduce(const MfmaParams &p, int G, hipStream_t stream)
{
    if constexpr (NMAT == 2) {
        if (p.partials != nullptr && p.flags != nullptr)
            return launch_t<MT, NMAT, IN, OUT, true>(p, G, stream);
    }
    hipError_t e = launch_t<MT, NMAT, IN, OUT>(p, G, stream);
    if (e != hipSuccess || p.partials == nullptr)
        return e;
    hipLaunchKernelGGL((mfma_reduce_kernel<MT, NMAT, OUT>), dim3(p.tiles, mfma_reduce_blocks<MT>()), dim3(256), 0,
                       stream, p, G);
    return hipGetLastError();
}

template <int NMAT, int IN, int OUT>
hipError_t launch_mt(const MfmaParams &p, int G, hipStream_t stream)
{
    switch ((p.M + 31) / 32) {
    case 1: return launch_gemm_reduce<1, NMAT, IN, OUT>(p, G, stream);
    case 2: return launch_gemm_reduce<2, NMAT, IN, OUT>(p, G, stream);
    case 3: return launch_gemm_reduce<3, NMAT, IN, OUT>(p, G, stream);
    case 4: return launch_gemm_reduce<4, NMAT, IN, OUT>(p, G, stream);
    default: return hipErrorNotSupported;
    }
}

// Grid and stream-K bookkeeping for one GEMM. With a workspace the grid is
// one workgroup per compute unit (capped at kMfmaMaxGrid) and a reduction
// launch finishes the split tiles; without one it is one workgroup per tile.
void plan(MfmaParams &p, int nmat, const MfmaScratch *ws, int &G)
{
    const int rows_tile = nmat == 2 ? mfma_rows_per_tile<2>() : mfma_rows_per_tile<1>();
    p.tiles = (p.rows + rows_tile - 1) / rows_tile;
    p.units_per_tile = p.cols / kUnitCols;
    p.units = p.tiles * p.units_per_tile;
    p.partials = nullptr;
    if (ws == nullptr) {
        G = p.tiles;
        return;
    }
    G = std::max(1, std::min({device_cu_count(), kMfmaMaxGrid, p.units}));
    if (G <= p.tiles && p.units % G == 0 && (p.units / G) % p.units_per_tile == 0)
        return;  // every workgroup owns whole tiles
    p.partials = ws->partials;
    p.flags = ws->flags;
    p.tag = launch_tag();
}

MfmaParams params(int M, const void *in0, const float *in1, const WeightArg &w0, const WeightArg &w1, void *out0,
                  void *out1, int rows, int cols)
{
    MfmaParams p{};
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
    p.M = M;
    p.rows = rows;
    p.cols = cols;
    return p;
}

}  // namespace

size_t mfma_partials_floats()
{
    return static_cast<size_t>(2) * kMfmaMaxGrid * mfma_slot_floats<4>();
}

size_t mfma_flag_words()
{
    return static_cast<size_t>(2) * kMfmaMaxGrid * kMfmaWaves;
}

size_t mfma_scratch_bytes()
{
    return mfma_partials_floats() * sizeof(float) + mfma_flag_words() * sizeof(unsigned long long);
}

MfmaScratch mfma_scratch(void *base)
{
    float *partials = static_cast<float *>(base);
    return MfmaScratch{partials, reinterpret_cast<unsigned long long *>(partials + mfma_partials_floats())};
}

hipError_t launch_mfma_dual(int M, OutKind out, const void *x, const WeightArg &w0, const WeightArg &w1,
                            void *out0, void *out1, int rows, int cols, const MfmaScratch *ws,
                            hipStream_t stream)
{
    if (M < 1 || M > kMfmaMaxM || cols % kUnitCols != 0)
        return hipErrorNotSupported;
    MfmaParams p = params(M, x, nullptr, w0, w1, out0, out1, rows, cols);
    int G = 0;
    plan(p, 2, ws, G);
    switch (out) {
    case OUT_F32_PAIR: return launch_mt<2, IN_BF16, OUT_F32_PAIR>(p, G, stream);
    case OUT_H_SILU: return launch_mt<2, IN_BF16, OUT_H_SILU>(p, G, stream);
    case OUT_H_GELU: return launch_mt<2, IN_BF16, OUT_H_GELU>(p, G, stream);
    default: return hipErrorNotSupported;
    }
}

hipError_t launch_mfma_down(int M, InKind in, const void *in0, const float *in1, const WeightArg &w, void *out,
                            int rows, int cols, const MfmaScratch *ws, hipStream_t stream)
{
    if (M < 1 || M > kMfmaMaxM || cols % kUnitCols != 0)
        return hipErrorNotSupported;
    MfmaParams p = params(M, in0, in1, w, w, out, nullptr, rows, cols);
    int G = 0;
    plan(p, 1, ws, G);
    switch (in) {
    case IN_BF16: return launch_mt<1, IN_BF16, OUT_BF16>(p, G, stream);
    case IN_GATEUP_SILU: return launch_mt<1, IN_GATEUP_SILU, OUT_BF16>(p, G, stream);
    case IN_GATEUP_GELU: return launch_mt<1, IN_GATEUP_GELU, OUT_BF16>(p, G, stream);
    default: return hipErrorNotSupported;
    }
}

}  // namespace ffn
