// abi_w4a4.cpp -- the C entry points of the W4A4 prefill arm: host-side
// validation, workspace layout and dispatch. Every check runs before anything
// is enqueued.
#include "ffn_w4a4.h"

#include <cmath>
#include <cstdint>

#include "kernels.h"
#include "mfma_launch.h"

namespace {

constexpr int kMaxDim = 65536;
constexpr int kMaxM = 65536;

bool aligned(const void *p, uintptr_t a)
{
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

size_t round256(size_t b)
{
    return (b + 255) & ~static_cast<size_t>(255);
}

int check_shape(int M, int K, int N)
{
    if (K <= 0 || K > kMaxDim || K % 256 != 0 || N <= 0 || N > kMaxDim || N % 64 != 0)
        return FFN_NVFP4_ERR_SHAPE;
    if (M < 0 || M > kMaxM)
        return FFN_NVFP4_ERR_BATCH;
    return FFN_NVFP4_OK;
}

int check_mx(const ffn_mxfp4_weight *w)
{
    if (!w || !w->codes || !w->scales)
        return FFN_NVFP4_ERR_NULL;
    if (!aligned(w->codes, 16) || !aligned(w->scales, 8))
        return FFN_NVFP4_ERR_ALIGN;
    if (!std::isfinite(w->scale2))
        return FFN_NVFP4_ERR_SCALE2;
    return FFN_NVFP4_OK;
}

// Workspace: [mx(x) codes][mx(x) exponents][h][down partial slots].
struct W4Layout {
    size_t xe, h, partials, dual_total, total;
};

W4Layout layout(int M, int K, int N)
{
    W4Layout l{};
    l.xe = round256(static_cast<size_t>(M) * static_cast<size_t>(K / 2));
    l.h = l.xe + round256(static_cast<size_t>(M) * static_cast<size_t>(K / 32));
    l.dual_total = l.h;
    l.partials = l.h + round256(static_cast<size_t>(M) * static_cast<size_t>(N) * 2);
    l.total = l.partials + round256(ffn::mfma_scratch_bytes());
    return l;
}

// Workspace of the all-FP4 entries: [mx(x) codes][mx(x) exponents][h]
// [mx(h) codes][mx(h) exponents][down partial sums][ready words] (the down
// entry uses the parts from mx(h) on).
struct Fp4Layout {
    size_t xe, h, hc, he, part, flags, total;
};

Fp4Layout fp4_layout(int M, int K, int N)
{
    Fp4Layout l{};
    l.xe = round256(static_cast<size_t>(M) * static_cast<size_t>(K / 2));
    l.h = l.xe + round256(static_cast<size_t>(M) * static_cast<size_t>(K / 32));
    l.hc = l.h + round256(static_cast<size_t>(M) * static_cast<size_t>(N) * 2);
    l.he = l.hc + round256(static_cast<size_t>(M) * static_cast<size_t>(N / 2));
    l.part = l.he + round256(static_cast<size_t>(M) * static_cast<size_t>(N / 32));
    l.flags = l.part + round256(ffn::w4a4_down_partial_floats(K, N) * sizeof(float));
    l.total = l.flags + round256(ffn::w4a4_down_flag_words(K, N) * sizeof(unsigned long long));
    return l;
}

int check_fp4_shape(int M, int K, int N)
{
    int rc = check_shape(M, K, N);
    if (rc == FFN_NVFP4_OK && N % 256 != 0)
        rc = FFN_NVFP4_ERR_SHAPE;  // the down reduction runs in 256-column pieces
    return rc;
}

ffn::MxWeightArg marg(const ffn_mxfp4_weight *w)
{
    return ffn::MxWeightArg{w->codes, w->scales, w->scale2};
}

int launch_status(hipError_t e)
{
    return e == hipSuccess ? FFN_NVFP4_OK : FFN_NVFP4_ERR_LAUNCH;
}

// h [M, N] bf16 -> MXFP4 in the workspace, then the down GEMM in blocks of
// 128 token rows (one launch each; the blocks share the partial sums and
// ready words, in stream order).
hipError_t run_fp4_down(const void *h, int M, int K, int N, const ffn_mxfp4_weight *down, uint8_t *ws,
                        const Fp4Layout &l, void *out, hipStream_t stream)
{
    hipError_t e = ffn::launch_mx_quant_bf16(h, M, N, ws + l.hc, ws + l.he, stream);
    constexpr int kBlock = 128;
    for (int m0 = 0; m0 < M && e == hipSuccess; m0 += kBlock) {
        const int mb = M - m0 < kBlock ? M - m0 : kBlock;
        e = ffn::launch_w4a4_down(mb, ws + l.hc + static_cast<size_t>(m0) * (N / 2),
                                  ws + l.he + static_cast<size_t>(m0) * (N / 32), marg(down),
                                  static_cast<uint16_t *>(out) + static_cast<size_t>(m0) * K, K, N,
                                  reinterpret_cast<float *>(ws + l.part),
                                  reinterpret_cast<unsigned long long *>(ws + l.flags), stream);
    }
    return e;
}

}  // namespace

extern "C" {

int ffn_w4a4_prepare_weight(const ffn_nvfp4_weight *w, int rows, int cols, uint8_t *mx_codes, uint8_t *mx_scales,
                            hipStream_t stream)
{
    if (!w || !w->codes || !w->scales || !mx_codes || !mx_scales)
        return FFN_NVFP4_ERR_NULL;
    if (rows <= 0 || rows > kMaxDim || cols <= 0 || cols > kMaxDim || cols % 32 != 0)
        return FFN_NVFP4_ERR_SHAPE;
    if (!aligned(w->codes, 16) || !aligned(w->scales, 2) || !aligned(mx_codes, 16))
        return FFN_NVFP4_ERR_ALIGN;
    return launch_status(ffn::launch_mx_requant(w->codes, w->scales, rows, cols, mx_codes, mx_scales, stream));
}

size_t ffn_w4a4_workspace_bytes(int M, int K, int N)
{
    if (M == 0 || check_shape(M, K, N) != FFN_NVFP4_OK)
        return 0;
    return layout(M, K, N).total;
}

int ffn_w4a4_dual_gemm(const void *x, int M, int K, int N, const ffn_mxfp4_weight *gate,
                       const ffn_mxfp4_weight *up, float *gate_out, float *up_out, void *workspace,
                       size_t workspace_bytes, hipStream_t stream)
{
    int rc;
    if ((rc = check_mx(gate)) || (rc = check_mx(up)) || (rc = check_shape(M, K, N)))
        return rc;
    if (M == 0)
        return FFN_NVFP4_OK;
    if (!x || !gate_out || !up_out || !workspace)
        return FFN_NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(gate_out, 16) || !aligned(up_out, 16) || !aligned(workspace, 16))
        return FFN_NVFP4_ERR_ALIGN;
    const W4Layout l = layout(M, K, N);
    if (workspace_bytes < l.dual_total)
        return FFN_NVFP4_ERR_WORKSPACE;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    hipError_t e = ffn::launch_mx_quant_bf16(x, M, K, ws, ws + l.xe, stream);
    if (e != hipSuccess)
        return FFN_NVFP4_ERR_LAUNCH;
    return launch_status(ffn::launch_w4a4_dual(M, ffn::OUT_F32_PAIR, ws, ws + l.xe, marg(gate), marg(up), gate_out,
                                               up_out, N, K, stream));
}

int ffn_w4a4_forward(const void *x, int M, int K, int N, const ffn_mxfp4_weight *gate,
                     const ffn_mxfp4_weight *up, const ffn_nvfp4_weight *down, int act, void *workspace,
                     size_t workspace_bytes, void *out, hipStream_t stream)
{
    int rc;
    if ((rc = check_mx(gate)) || (rc = check_mx(up)) || (rc = check_shape(M, K, N)))
        return rc;
    if (!down || !down->codes || !down->scales)
        return FFN_NVFP4_ERR_NULL;
    if (!aligned(down->codes, 16) || !aligned(down->scales, 8))
        return FFN_NVFP4_ERR_ALIGN;
    if (!std::isfinite(down->scale2))
        return FFN_NVFP4_ERR_SCALE2;
    if (act != FFN_NVFP4_ACT_SILU && act != FFN_NVFP4_ACT_GELU_TANH)
        return FFN_NVFP4_ERR_ACT;
    if (M == 0)
        return FFN_NVFP4_OK;
    if (!x || !out || !workspace)
        return FFN_NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(workspace, 16))
        return FFN_NVFP4_ERR_ALIGN;
    if (workspace_bytes < ffn_w4a4_workspace_bytes(M, K, N))
        return FFN_NVFP4_ERR_WORKSPACE;
    const W4Layout l = layout(M, K, N);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    uint16_t *h = reinterpret_cast<uint16_t *>(ws + l.h);
    hipError_t e = ffn::launch_mx_quant_bf16(x, M, K, ws, ws + l.xe, stream);
    if (e != hipSuccess)
        return FFN_NVFP4_ERR_LAUNCH;
    const ffn::OutKind epi = act == FFN_NVFP4_ACT_SILU ? ffn::OUT_H_SILU : ffn::OUT_H_GELU;
    e = ffn::launch_w4a4_dual(M, epi, ws, ws + l.xe, marg(gate), marg(up), h, nullptr, N, K, stream);
    if (e != hipSuccess)
        return FFN_NVFP4_ERR_LAUNCH;
    // The down projection on the W4A16 matrix-core arm, in blocks of up to
    // 128 token rows (stream-K partial slots in the workspace).
    ffn::MfmaScratch scratch = ffn::mfma_scratch(ws + l.partials);
    const ffn::WeightArg d{down->codes, down->scales, down->scale2};
    for (int m0 = 0; m0 < M; m0 += ffn::kMfmaMaxM) {
        const int mb = M - m0 < ffn::kMfmaMaxM ? M - m0 : ffn::kMfmaMaxM;
        e = ffn::launch_mfma_down(mb, ffn::IN_BF16, h + static_cast<size_t>(m0) * N, nullptr, d,
                                  static_cast<uint16_t *>(out) + static_cast<size_t>(m0) * K, K, N, &scratch,
                                  stream);
        if (e != hipSuccess)
            return FFN_NVFP4_ERR_LAUNCH;
    }
    return FFN_NVFP4_OK;
}

size_t ffn_w4a4_fp4_workspace_bytes(int M, int K, int N)
{
    if (M == 0 || check_fp4_shape(M, K, N) != FFN_NVFP4_OK)
        return 0;
    return fp4_layout(M, K, N).total;
}

int ffn_w4a4_down_gemm(const void *h, int M, int N, int K, const ffn_mxfp4_weight *down, void *out,
                       void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    int rc;
    if ((rc = check_mx(down)) || (rc = check_fp4_shape(M, K, N)))
        return rc;
    if (M == 0)
        return FFN_NVFP4_OK;
    if (!h || !out || !workspace)
        return FFN_NVFP4_ERR_NULL;
    if (!aligned(h, 16) || !aligned(out, 16) || !aligned(workspace, 16))
        return FFN_NVFP4_ERR_ALIGN;
    if (workspace_bytes < ffn_w4a4_fp4_workspace_bytes(M, K, N))
        return FFN_NVFP4_ERR_WORKSPACE;
    return launch_status(run_fp4_down(h, M, K, N, down, static_cast<uint8_t *>(workspace),
                                      fp4_layout(M, K, N), out, stream));
}

int ffn_w4a4_forward_fp4(const void *x, int M, int K, int N, const ffn_mxfp4_weight *gate,
                         const ffn_mxfp4_weight *up, const ffn_mxfp4_weight *down, int act, void *workspace,
                         size_t workspace_bytes, void *out, hipStream_t stream)
{
    int rc;
    if ((rc = check_mx(gate)) || (rc = check_mx(up)) || (rc = check_mx(down)) || (rc = check_fp4_shape(M, K, N)))
        return rc;
    if (act != FFN_NVFP4_ACT_SILU && act != FFN_NVFP4_ACT_GELU_TANH)
        return FFN_NVFP4_ERR_ACT;
    if (M == 0)
        return FFN_NVFP4_OK;
    if (!x || !out || !workspace)
        return FFN_NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(workspace, 16))
        return FFN_NVFP4_ERR_ALIGN;
    if (workspace_bytes < ffn_w4a4_fp4_workspace_bytes(M, K, N))
        return FFN_NVFP4_ERR_WORKSPACE;
    const Fp4Layout l = fp4_layout(M, K, N);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    uint16_t *h = reinterpret_cast<uint16_t *>(ws + l.h);
    hipError_t e = ffn::launch_mx_quant_bf16(x, M, K, ws, ws + l.xe, stream);
    if (e != hipSuccess)
        return FFN_NVFP4_ERR_LAUNCH;
    const ffn::OutKind epi = act == FFN_NVFP4_ACT_SILU ? ffn::OUT_H_SILU : ffn::OUT_H_GELU;
    e = ffn::launch_w4a4_dual(M, epi, ws, ws + l.xe, marg(gate), marg(up), h, nullptr, N, K, stream);
    if (e != hipSuccess)
        return FFN_NVFP4_ERR_LAUNCH;
    return launch_status(run_fp4_down(h, M, K, N, down, ws, l, out, stream));
}

}  // extern "C"
