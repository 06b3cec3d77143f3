// smallm_launch.hip -- host-side launch of the small-batch GEMMs and their
// instantiations.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "smallm_gemm.h"
#include "smallm_launch.h"

namespace ffn {

namespace {

// Token groups of 16 for M rows.
int token_groups(int M)
{
    return (M + 15) / 16;
}

// Rounds a wave may take per tile and part: its activations (8 registers per
// round and token group) and accumulators must fit the 128 registers a lane
// has with 16 waves per compute unit. Compiled: two groups, the dual GEMM
// needs 124-128 at 4 rounds (16 bytes per lane spilled without PARTIAL) and the
// down GEMM 127-128 at 5 (8 bytes spilled without PARTIAL; 4 rounds, which fit,
// measured slower: 61.5 vs 59.9 us at 17 rows, 67.2 vs 66.9 us at 32); three
// groups, the dual GEMM 120-122 at 2 rounds and the down GEMM 127-128 at 3.
constexpr int max_rounds(int tg, int nmat)
{
    return tg == 1 ? kSmMaxRounds : tg == 2 ? (nmat == 1 ? kSmMaxRounds : kSmMaxRoundsTwoGroups) : (nmat == 1 ? 3 : 2);
}

// Split of one GEMM: P parts of the reduction (each at most max_rounds(tg)
// rounds) and G row-tile groups, about one workgroup per compute unit in all.
struct SmallPlan {
    int parts, groups, rounds, tg;
};

SmallPlan plan(int rows, int cols, int M, int nmat)
{
    const int nb = cols / 256;  // 256-column blocks (4 units)
    const int tiles = rows / kSmRows;
    SmallPlan s{};
    s.tg = token_groups(M);
    const int max_blocks = kSmWaves * max_rounds(s.tg, nmat) / 4;  // per part
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

template <int NMAT, int OUT, int TG, bool SPLIT, bool PARTIAL>
hipError_t launch_tg(const SmallParams &p, int rounds, hipStream_t stream)
{
    const void *kern = nullptr;
    if (rounds > max_rounds(TG, NMAT))
        return hipErrorNotSupported;
    switch (rounds) {
    case 1: kern = reinterpret_cast<const void *>(smallm_gemm_kernel<NMAT, OUT, 1, TG, SPLIT, PARTIAL>); break;
    case 2: kern = reinterpret_cast<const void *>(smallm_gemm_kernel<NMAT, OUT, 2, TG, SPLIT, PARTIAL>); break;
    case 3:
        if constexpr (max_rounds(TG, NMAT) >= 3) {
            kern = reinterpret_cast<const void *>(smallm_gemm_kernel<NMAT, OUT, 3, TG, SPLIT, PARTIAL>);
            break;
        }
        return hipErrorNotSupported;
    case 4:
        if constexpr (max_rounds(TG, NMAT) >= 4) {
            kern = reinterpret_cast<const void *>(smallm_gemm_kernel<NMAT, OUT, 4, TG, SPLIT, PARTIAL>);
            break;
        }
        return hipErrorNotSupported;
    case 5:
        if constexpr (max_rounds(TG, NMAT) >= 5) {
            kern = reinterpret_cast<const void *>(smallm_gemm_kernel<NMAT, OUT, 5, TG, SPLIT, PARTIAL>);
            break;
        }
        return hipErrorNotSupported;
    default: return hipErrorNotSupported;
    }
    constexpr int lds = sm_lds_bytes<NMAT, TG>();
    static std::atomic<uint64_t> lds_done[kSmMaxRounds];  // per rounds instantiation
    hipError_t e = allow_lds(kern, lds, lds_done[rounds - 1]);
    if (e != hipSuccess)
        return e;
    void *args[] = {const_cast<SmallParams *>(&p)};
    return hipLaunchKernel(kern, dim3(p.parts * p.groups), dim3(kSmWaves * 64), args, lds, stream);
}

template <int NMAT, int OUT, int TG, bool SPLIT>
hipError_t launch_split(const SmallParams &p, int rounds, hipStream_t stream)
{
    return p.M < 16 * TG ? launch_tg<NMAT, OUT, TG, SPLIT, true>(p, rounds, stream)
                         : launch_tg<NMAT, OUT, TG, SPLIT, false>(p, rounds, stream);
}

template <int NMAT, int OUT>
hipError_t launch_t(const SmallParams &p, const SmallPlan &s, hipStream_t stream)
{
    const bool split = s.parts > 1;
    switch (s.tg) {
    case 1: return split ? launch_split<NMAT, OUT, 1, true>(p, s.rounds, stream) : launch_split<NMAT, OUT, 1, false>(p, s.rounds, stream);
    case 2: return split ? launch_split<NMAT, OUT, 2, true>(p, s.rounds, stream) : launch_split<NMAT, OUT, 2, false>(p, s.rounds, stream);
    case 3: return split ? launch_split<NMAT, OUT, 3, true>(p, s.rounds, stream) : launch_split<NMAT, OUT, 3, false>(p, s.rounds, stream);
    default: return hipErrorNotSupported;
    }
}

SmallParams params(int M, const void *in0, const WeightArg &w0, const WeightArg &w1, void *out0, void *out1,
                   int rows, int cols, const SmallPlan &s, float *part0, float *part1,
                   unsigned long long *flags)
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
    p.part0 = part0;
    p.part1 = part1;
    p.flags = flags;
    p.tag = s.parts > 1 ? launch_tag() : 0;
    return p;
}

}  // namespace

bool smallm_supported(int M, int K, int N)
{
    return M >= 1 && M <= kSmallMaxM && shape_ok(N, K) && shape_ok(K, N);
}

bool smallm_dual_split(int M, int K, int N)
{
    return plan(N, K, M, 2).parts > 1;
}

size_t smallm_partial_floats(int M, int K, int N)
{
    const SmallPlan s = plan(K, N, M, 1);
    return s.parts > 1 ? static_cast<size_t>(s.parts) * M * K : 0;
}

size_t smallm_dual_partial_floats(int M, int K, int N)
{
    const SmallPlan s = plan(N, K, M, 2);
    return s.parts > 1 ? static_cast<size_t>(2) * s.parts * M * N : 0;
}

size_t smallm_flag_words(int M, int K, int N)
{
    const SmallPlan d = plan(N, K, M, 2), w = plan(K, N, M, 1);
    const int grid = std::max(d.parts > 1 ? d.parts * d.groups : 0, w.parts > 1 ? w.parts * w.groups : 0);
    return static_cast<size_t>(grid);
}

hipError_t launch_smallm_dual(int M, OutKind out, const void *x, const WeightArg &w0, const WeightArg &w1,
                              void *out0, void *out1, float *partials, unsigned long long *flags, int N, int K,
                              hipStream_t stream)
{
    if (!smallm_supported(M, K, N))
        return hipErrorNotSupported;
    const SmallPlan s = plan(N, K, M, 2);
    // A reduction split in parts: both projections' pieces, finished by the
    // last part's workgroup of each tile group.
    float *gpart = nullptr, *upart = nullptr;
    if (s.parts > 1) {
        if (partials == nullptr || flags == nullptr)
            return hipErrorNotSupported;
        gpart = partials;
        upart = partials + static_cast<size_t>(s.parts) * M * N;
    }
    const SmallParams p = params(M, x, w0, w1, out0, out1, N, K, s, gpart, upart, flags);
    switch (out) {
    case OUT_F32_PAIR: return launch_t<2, OUT_F32_PAIR>(p, s, stream);
    case OUT_H_SILU: return launch_t<2, OUT_H_SILU>(p, s, stream);
    case OUT_H_GELU: return launch_t<2, OUT_H_GELU>(p, s, stream);
    default: return hipErrorNotSupported;
    }
}

hipError_t launch_smallm_down(int M, const void *h, const WeightArg &w, void *out, float *partials,
                              unsigned long long *flags, int K, int N, hipStream_t stream)
{
    if (!smallm_supported(M, K, N))
        return hipErrorNotSupported;
    const SmallPlan s = plan(K, N, M, 1);
    if (s.parts > 1 && (partials == nullptr || flags == nullptr))
        return hipErrorNotSupported;
    const SmallParams p = params(M, h, w, w, out, nullptr, K, N, s, partials, partials, flags);
    return launch_t<1, OUT_BF16>(p, s, stream);
}

}  // namespace ffn
