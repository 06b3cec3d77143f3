// abi.cpp -- the C entry points of libffn_nvfp4: host-side validation and
// dispatch to the kernels. Every check runs before anything is enqueued, and
// no HIP call is made when a check fails.
#include "ffn_nvfp4.h"

#include <cmath>
#include <cstdint>

#include "kernels.h"
#include "mfma_launch.h"
#include "quantize.h"
#include "smallm_launch.h"

namespace {

constexpr int kMaxDim = 65536;
constexpr int kMaxGemvM = 8;
constexpr int kMaxM = 65536;

bool aligned(const void *p, uintptr_t a)
{
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

bool dim_ok(int d)
{
    return d > 0 && d <= kMaxDim && d % 32 == 0;
}

int check_weight(const ffn_nvfp4_weight *w)
{
    if (!w || !w->codes || !w->scales)
        return FFN_NVFP4_ERR_NULL;
    if (!aligned(w->codes, 16) || !aligned(w->scales, 2))
        return FFN_NVFP4_ERR_ALIGN;
    if (!std::isfinite(w->scale2))
        return FFN_NVFP4_ERR_SCALE2;
    return FFN_NVFP4_OK;
}

int check_batch(int M)
{
    return (M >= 0 && M <= kMaxM) ? FFN_NVFP4_OK : FFN_NVFP4_ERR_BATCH;
}

// Batches above kMaxGemvM rows run on the matrix-core arm, which needs K and
// N in multiples of 64.
int check_prefill_shape(int M, int K, int N)
{
    if (M > kMaxGemvM && (K % 64 != 0 || N % 64 != 0))
        return FFN_NVFP4_ERR_SHAPE;
    return FFN_NVFP4_OK;
}

// ... and scales aligned to 8 bytes (the small-batch arm loads a row's 8
// scale bytes of a 128-column unit at once).
int check_prefill_scales(int M, const ffn_nvfp4_weight *a, const ffn_nvfp4_weight *b = nullptr,
                         const ffn_nvfp4_weight *c = nullptr)
{
    if (M <= kMaxGemvM)
        return FFN_NVFP4_OK;
    for (const ffn_nvfp4_weight *w : {a, b, c})
        if (w && !aligned(w->scales, 8))
            return FFN_NVFP4_ERR_ALIGN;
    return FFN_NVFP4_OK;
}

size_t round256(size_t b)
{
    return (b + 255) & ~static_cast<size_t>(255);
}

// Workspace of the matrix-core arm: h for one block of up to kMfmaMaxM rows
// and the stream-K partial slots.
struct PrefillLayout {
    size_t h, partials, total;
};

// Batches of 9 to 40 rows take the small-batch arm when it covers the shape;
// its workspace is h, the down projection's partial sums and, when the dual
// projection's reduction is split in parts, its partial sums, then the ready
// words of the split reductions.
bool small_arm(int M, int K, int N)
{
    return M > kMaxGemvM && ffn::smallm_supported(M, K, N);
}

struct SmallLayout {
    size_t down_partials, dual_partials, flags, total;
};

SmallLayout small_layout(int M, int K, int N)
{
    SmallLayout l{};
    l.down_partials = round256(static_cast<size_t>(M) * static_cast<size_t>(N) * 2);
    l.dual_partials = l.down_partials + round256(ffn::smallm_partial_floats(M, K, N) * sizeof(float));
    l.flags = l.dual_partials + round256(ffn::smallm_dual_partial_floats(M, K, N) * sizeof(float));
    l.total = l.flags + round256(ffn::smallm_flag_words(M, K, N) * sizeof(unsigned long long));
    return l;
}

PrefillLayout prefill_layout(int M, int N)
{
    PrefillLayout l{};
    const int mb = M < ffn::kMfmaMaxM ? M : ffn::kMfmaMaxM;
    l.h = 0;
    l.partials = round256(static_cast<size_t>(mb) * N * 2);
    l.total = l.partials + round256(ffn::mfma_scratch_bytes());
    return l;
}

ffn::WeightArg warg(const ffn_nvfp4_weight *w)
{
    return ffn::WeightArg{w->codes, w->scales, w->scale2};
}

int launch_status(hipError_t e)
{
    return e == hipSuccess ? FFN_NVFP4_OK : FFN_NVFP4_ERR_LAUNCH;
}

// 1 <= M <= 8: the many-wave GEMV for rows of 33 chunks or more, else the
// general LDS-staged kernel. Both share one per-row arithmetic, so a row's
// result does not depend on which one ran.
hipError_t run_dual(int M, ffn::OutKind out, const void *x, const ffn::WeightArg &g, const ffn::WeightArg &u,
                    void *out0, void *out1, int N, int K, hipStream_t stream)
{
    hipError_t e = ffn::launch_wave_dual(M, out, x, g, u, out0, out1, N, K, stream);
    if (e != hipErrorNotSupported)
        return e;
    return ffn::launch_gemv(M, 2, ffn::IN_BF16, out, x, nullptr, g, u, out0, out1, N, K, stream);
}

hipError_t run_down(int M, ffn::InKind in, const void *in0, const float *in1, const ffn::WeightArg &d,
                    void *out, int K, int N, hipStream_t stream)
{
    hipError_t e = ffn::launch_wave_down(M, in, in0, in1, d, out, K, N, stream);
    if (e != hipErrorNotSupported)
        return e;
    return ffn::launch_gemv(M, 1, in, ffn::OUT_BF16, in0, in1, d, d, out, nullptr, K, N, stream);
}

// Matrix-core arm, in blocks of up to kMfmaMaxM rows.
hipError_t run_prefill_dual(int M, const void *x, const ffn::WeightArg &g, const ffn::WeightArg &u, float *gate_out,
                            float *up_out, int N, int K, hipStream_t stream)
{
    // The dual entry has no workspace: the small-batch arm only when its
    // reduction is not split.
    if (small_arm(M, K, N) && !ffn::smallm_dual_split(M, K, N))
        return ffn::launch_smallm_dual(M, ffn::OUT_F32_PAIR, x, g, u, gate_out, up_out, nullptr, nullptr, N, K,
                                       stream);
    for (int m0 = 0; m0 < M; m0 += ffn::kMfmaMaxM) {
        const int mb = M - m0 < ffn::kMfmaMaxM ? M - m0 : ffn::kMfmaMaxM;
        const size_t xo = static_cast<size_t>(m0) * K, oo = static_cast<size_t>(m0) * N;
        hipError_t e = ffn::launch_mfma_dual(mb, ffn::OUT_F32_PAIR, static_cast<const uint16_t *>(x) + xo, g, u,
                                             gate_out + oo, up_out + oo, N, K, nullptr, stream);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t run_prefill_down(int M, ffn::InKind in, const float *gate_in, const float *up_in,
                            const ffn::WeightArg &d, void *out, int K, int N, hipStream_t stream)
{
    for (int m0 = 0; m0 < M; m0 += ffn::kMfmaMaxM) {
        const int mb = M - m0 < ffn::kMfmaMaxM ? M - m0 : ffn::kMfmaMaxM;
        const size_t io = static_cast<size_t>(m0) * N, oo = static_cast<size_t>(m0) * K;
        hipError_t e = ffn::launch_mfma_down(mb, in, gate_in + io, up_in + io, d,
                                             static_cast<uint16_t *>(out) + oo, K, N, nullptr, stream);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t run_prefill_forward(int M, ffn::OutKind epi, const void *x, const ffn::WeightArg &g,
                               const ffn::WeightArg &u, const ffn::WeightArg &d, void *workspace, void *out, int K,
                               int N, hipStream_t stream)
{
    if (small_arm(M, K, N)) {
        const SmallLayout l = small_layout(M, K, N);
        uint8_t *ws = static_cast<uint8_t *>(workspace);
        unsigned long long *flags = reinterpret_cast<unsigned long long *>(ws + l.flags);
        hipError_t e = ffn::launch_smallm_dual(M, epi, x, g, u, workspace, nullptr,
                                               reinterpret_cast<float *>(ws + l.dual_partials), flags, N, K, stream);
        if (e != hipSuccess)
            return e;
        return ffn::launch_smallm_down(M, workspace, d, out, reinterpret_cast<float *>(ws + l.down_partials), flags,
                                       K, N, stream);
    }
    const PrefillLayout l = prefill_layout(M, N);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    ffn::MfmaScratch scratch = ffn::mfma_scratch(ws + l.partials);
    void *h = ws + l.h;
    for (int m0 = 0; m0 < M; m0 += ffn::kMfmaMaxM) {
        const int mb = M - m0 < ffn::kMfmaMaxM ? M - m0 : ffn::kMfmaMaxM;
        hipError_t e = ffn::launch_mfma_dual(mb, epi, static_cast<const uint16_t *>(x) + static_cast<size_t>(m0) * K,
                                             g, u, h, nullptr, N, K, &scratch, stream);
        if (e != hipSuccess)
            return e;
        e = ffn::launch_mfma_down(mb, ffn::IN_BF16, h, nullptr, d,
                                  static_cast<uint16_t *>(out) + static_cast<size_t>(m0) * K, K, N, &scratch, stream);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace

extern "C" {

int ffn_nvfp4_version(void)
{
    return 100;  // 0.1.0
}

const char *ffn_nvfp4_strerror(int status)
{
    switch (status) {
    case FFN_NVFP4_OK: return "ok";
    case FFN_NVFP4_ERR_NULL: return "a required pointer is NULL";
    case FFN_NVFP4_ERR_ALIGN:
        return "pointer misaligned (codes/x/out/workspace need 16 bytes, scales 2, or 8 when M > 8)";
    case FFN_NVFP4_ERR_SHAPE:
        return "K and N must be positive multiples of 32 (of 64 when M > 8), at most 65536";
    case FFN_NVFP4_ERR_BATCH: return "unsupported batch size M";
    case FFN_NVFP4_ERR_ACT: return "unknown activation";
    case FFN_NVFP4_ERR_WORKSPACE: return "workspace too small";
    case FFN_NVFP4_ERR_LAUNCH: return "kernel launch failed";
    case FFN_NVFP4_ERR_SCALE2: return "scale2 is not finite";
    default: return "unknown status";
    }
}

size_t ffn_nvfp4_workspace_bytes(int M, int K, int N)
{
    if (check_batch(M) != FFN_NVFP4_OK || !dim_ok(K) || !dim_ok(N))
        return 0;
    if (M == 0 || check_prefill_shape(M, K, N) != FFN_NVFP4_OK)
        return 0;
    if (small_arm(M, K, N))
        return small_layout(M, K, N).total;
    if (M > kMaxGemvM)
        return prefill_layout(M, N).total;
    // h = act(gate) * up in bf16, [M, N]
    return round256(static_cast<size_t>(M) * static_cast<size_t>(N) * 2);
}

int ffn_nvfp4_dual_gemv(const void *x, int M, int K, int N, const ffn_nvfp4_weight *gate,
                        const ffn_nvfp4_weight *up, float *gate_out, float *up_out, hipStream_t stream)
{
    int rc;
    if ((rc = check_weight(gate)) || (rc = check_weight(up)))
        return rc;
    if (!dim_ok(K) || !dim_ok(N))
        return FFN_NVFP4_ERR_SHAPE;
    if ((rc = check_batch(M)) || (rc = check_prefill_shape(M, K, N)))
        return rc;
    if (M == 0)
        return FFN_NVFP4_OK;
    if (!x || !gate_out || !up_out)
        return FFN_NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(gate_out, 16) || !aligned(up_out, 16))
        return FFN_NVFP4_ERR_ALIGN;
    if ((rc = check_prefill_scales(M, gate, up)))
        return rc;
    if (M > kMaxGemvM)
        return launch_status(run_prefill_dual(M, x, warg(gate), warg(up), gate_out, up_out, N, K, stream));
    return launch_status(run_dual(M, ffn::OUT_F32_PAIR, x, warg(gate), warg(up), gate_out, up_out, N, K, stream));
}

int ffn_nvfp4_down_gemv(const float *gate_in, const float *up_in, int M, int N, int K,
                        const ffn_nvfp4_weight *down, int act, void *out, hipStream_t stream)
{
    int rc;
    if ((rc = check_weight(down)))
        return rc;
    if (!dim_ok(K) || !dim_ok(N))
        return FFN_NVFP4_ERR_SHAPE;
    if ((rc = check_batch(M)) || (rc = check_prefill_shape(M, K, N)))
        return rc;
    if (act != FFN_NVFP4_ACT_SILU && act != FFN_NVFP4_ACT_GELU_TANH)
        return FFN_NVFP4_ERR_ACT;
    if (M == 0)
        return FFN_NVFP4_OK;
    if (!gate_in || !up_in || !out)
        return FFN_NVFP4_ERR_NULL;
    if (!aligned(gate_in, 16) || !aligned(up_in, 16) || !aligned(out, 16))
        return FFN_NVFP4_ERR_ALIGN;
    if ((rc = check_prefill_scales(M, down)))
        return rc;
    const ffn::InKind in = act == FFN_NVFP4_ACT_SILU ? ffn::IN_GATEUP_SILU : ffn::IN_GATEUP_GELU;
    if (M > kMaxGemvM)
        return launch_status(run_prefill_down(M, in, gate_in, up_in, warg(down), out, K, N, stream));
    return launch_status(run_down(M, in, gate_in, up_in, warg(down), out, K, N, stream));
}

int ffn_nvfp4_forward(const void *x, int M, int K, int N, const ffn_nvfp4_weight *gate,
                      const ffn_nvfp4_weight *up, const ffn_nvfp4_weight *down, int act, void *workspace,
                      size_t workspace_bytes, void *out, hipStream_t stream)
{
    int rc;
    if ((rc = check_weight(gate)) || (rc = check_weight(up)) || (rc = check_weight(down)))
        return rc;
    if (!dim_ok(K) || !dim_ok(N))
        return FFN_NVFP4_ERR_SHAPE;
    if ((rc = check_batch(M)) || (rc = check_prefill_shape(M, K, N)))
        return rc;
    if (act != FFN_NVFP4_ACT_SILU && act != FFN_NVFP4_ACT_GELU_TANH)
        return FFN_NVFP4_ERR_ACT;
    if (M == 0)
        return FFN_NVFP4_OK;
    if (!x || !out || !workspace)
        return FFN_NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(workspace, 16))
        return FFN_NVFP4_ERR_ALIGN;
    if ((rc = check_prefill_scales(M, gate, up, down)))
        return rc;
    if (workspace_bytes < ffn_nvfp4_workspace_bytes(M, K, N))
        return FFN_NVFP4_ERR_WORKSPACE;
    // The dual GEMV's epilogue computes h = bf16(act(s2_g gate) * (s2_u up))
    // once per element (64 rows per instruction); the down GEMV streams W_d
    // against h staged in LDS or registers. Bit-identical to the dual GEMV
    // followed by the down GEMV with the activation in its input load.
    const ffn::OutKind epi = act == FFN_NVFP4_ACT_SILU ? ffn::OUT_H_SILU : ffn::OUT_H_GELU;
    if (M > kMaxGemvM)
        return launch_status(run_prefill_forward(M, epi, x, warg(gate), warg(up), warg(down), workspace, out, K, N,
                                                 stream));
    hipError_t e = run_dual(M, epi, x, warg(gate), warg(up), workspace, nullptr, N, K, stream);
    if (e != hipSuccess)
        return FFN_NVFP4_ERR_LAUNCH;
    return launch_status(run_down(M, ffn::IN_BF16, workspace, nullptr, warg(down), out, K, N, stream));
}

size_t ffn_nvfp4_quantize_workspace_bytes(int rows, int cols)
{
    if (rows <= 0 || rows > kMaxDim || !dim_ok(cols))
        return 0;
    return static_cast<size_t>(ffn::kQuantizeMaxPartials) * sizeof(uint32_t);
}

int ffn_nvfp4_quantize(const void *w, int rows, int cols, uint8_t *codes, uint8_t *scales, float *scale2,
                       void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (rows <= 0 || rows > kMaxDim || !dim_ok(cols))
        return FFN_NVFP4_ERR_SHAPE;
    if (!w || !codes || !scales || !scale2 || !workspace)
        return FFN_NVFP4_ERR_NULL;
    if (!aligned(w, 16) || !aligned(codes, 8) || !aligned(scale2, 4) || !aligned(workspace, 4))
        return FFN_NVFP4_ERR_ALIGN;
    if (workspace_bytes < ffn_nvfp4_quantize_workspace_bytes(rows, cols))
        return FFN_NVFP4_ERR_WORKSPACE;
    return launch_status(ffn::launch_quantize(w, rows, cols, codes, scales, scale2, static_cast<uint32_t *>(workspace),
                                              stream));
}

}  // extern "C"
