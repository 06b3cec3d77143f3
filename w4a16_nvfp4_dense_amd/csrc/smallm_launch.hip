// smallm_launch.hip -- host-side launch of the small-batch GEMMs and their
// instantiations.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "smallm_gemm.h"
#include "smallm_launch.h"

namespace ffn {

namespace {

// Split of one GEMM: P parts of the reduction (each at most kSmMaxRounds
// rounds, so a wave's activations fit in registers) and G row-tile groups,
// about one workgroup per compute unit in all.
struct SmallPlan {
    int parts, groups, rounds;
};

SmallPlan plan(int rows, int cols)
{
    const int nb = cols / 256;  // 256-column blocks (4 units)
    const int tiles = rows / kSmRows;
    constexpr int max_blocks = kSmWaves * kSmMaxRounds / 4;  // per part
    SmallPlan s{};
    s.parts = std::max(1, (nb + max_blocks - 1) / max_blocks);
    const int max_units = 4 * ((nb + s.parts - 1) / s.parts);
    s.rounds = (max_units + kSmWaves - 1) / kSmWaves;
    s.groups = std::max(1, std::min(tiles, device_cu_count() / s.parts));
    return s;
}

// Rows in whole tiles; the reduction in whole 256-column blocks, so that every
// 16-byte piece of a row's scales lies wholly inside the row (a round's pieces
// past the end of its part are clamped to the row's last piece and never
// used; a piece straddling the end would be loaded shifted).
bool shape_ok(int rows, int cols)
{
    return rows > 0 && rows % kSmRows == 0 && cols > 0 && cols % 256 == 0;
}

template <int NMAT, int OUT>
hipError_t launch_t(const SmallParams &p, int rounds, hipStream_t stream)
{
    const void *kern = nullptr;
    switch (rounds) {
    case 1: kern = reinterpret_cast<const void *>(smallm_gemm_kernel<NMAT, OUT, 1>); break;
    case 2: kern = reinterpret_cast<const void *>(smallm_gemm_kernel<NMAT, OUT, 2>); break;
    case 3: kern = reinterpret_cast<const void *>(smallm_gemm_kernel<NMAT, OUT, 3>); break;
    case 4: kern = reinterpret_cast<const void *>(smallm_gemm_kernel<NMAT, OUT, 4>); break;
    case 5: kern = reinterpret_cast<const void *>(smallm_gemm_kernel<NMAT, OUT, 5>); break;
    default: return hipErrorNotSupported;
    }
    constexpr int lds = sm_lds_bytes<NMAT>();
    static std::atomic<uint64_t> lds_done[5];  // per rounds instantiation
    hipError_t e = allow_lds(kern, lds, lds_done[rounds - 1]);
    if (e != hipSuccess)
        return e;
    void *args[] = {const_cast<SmallParams *>(&p)};
    return hipLaunchKernel(kern, dim3(p.parts * p.groups), dim3(kSmWaves * 64), args, lds, stream);
}

SmallParams params(int M, const void *in0, const WeightArg &w0, const WeightArg &w1, void *out0, void *out1,
                   int rows, int cols, const SmallPlan &s)
{
    SmallParams p{};
    p.in0 = in0;
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
    p.parts = s.parts;
    p.groups = s.groups;
    return p;
}

}  // namespace

bool smallm_supported(int M, int K, int N)
{
    // the dual GEMM keeps its whole reduction in one part
    return M >= 1 && M <= kSmallMaxM && shape_ok(N, K) && shape_ok(K, N) && plan(N, K).parts == 1;
}

size_t smallm_partial_floats(int M, int K, int N)
{
    const SmallPlan s = plan(K, N);
    return s.parts > 1 ? static_cast<size_t>(s.parts) * M * K : 0;
}

hipError_t launch_smallm_dual(int M, OutKind out, const void *x, const WeightArg &w0, const WeightArg &w1,
                              void *out0, void *out1, int N, int K, hipStream_t stream)
{
    if (!smallm_supported(M, K, N))
        return hipErrorNotSupported;
    const SmallPlan s = plan(N, K);
    const SmallParams p = params(M, x, w0, w1, out0, out1, N, K, s);
    switch (out) {
    case OUT_F32_PAIR: return launch_t<2, OUT_F32_PAIR>(p, s.rounds, stream);
    case OUT_H_SILU: return launch_t<2, OUT_H_SILU>(p, s.rounds, stream);
    case OUT_H_GELU: return launch_t<2, OUT_H_GELU>(p, s.rounds, stream);
    default: return hipErrorNotSupported;
    }
}

hipError_t launch_smallm_down(int M, const void *h, const WeightArg &w, void *out, float *partials, int K, int N,
                              hipStream_t stream)
{
    if (!smallm_supported(M, K, N))
        return hipErrorNotSupported;
    const SmallPlan s = plan(K, N);
    if (s.parts == 1) {
        const SmallParams p = params(M, h, w, w, out, nullptr, K, N, s);
        return launch_t<1, OUT_BF16>(p, s.rounds, stream);
    }
    const SmallParams p = params(M, h, w, w, partials, nullptr, K, N, s);
    hipError_t e = launch_t<1, OUT_PART_F32>(p, s.rounds, stream);
    if (e != hipSuccess)
        return e;
    const size_t n = static_cast<size_t>(M) * K;
    hipLaunchKernelGGL(smallm_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                       partials, s.parts, n, w.scale2, static_cast<uint16_t *>(out));
    return hipGetLastError();
}

}  // namespace ffn
