// abi_fp8.cpp -- the C entry points of the block-scaled FP8 FFN: host-side
// validation and dispatch to the FP8 GEMV kernels. Every check runs before
// anything is enqueued, and no HIP call is made when a check fails.
#include "ffn_fp8.h"

#include <cstdint>

#include "kernels.h"

namespace {

constexpr int kFp8MaxDim = 24576;  // 64 lanes x 24 chunks of 16 columns
constexpr int kFp8MaxM = 8;

bool aligned(const void *p, uintptr_t a)
{
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

bool dim_ok(int d)
{
    return d > 0 && d <= kFp8MaxDim && d % 16 == 0;
}

int check_weight(const ffn_fp8_weight *w)
{
    if (!w || !w->codes || !w->block_scale)
        return FFN_NVFP4_ERR_NULL;
    if (!aligned(w->codes, 16) || !aligned(w->block_scale, 4))
        return FFN_NVFP4_ERR_ALIGN;
    return FFN_NVFP4_OK;
}

int check_common(int M, int K, int N)
{
    if (!dim_ok(K) || !dim_ok(N))
        return FFN_NVFP4_ERR_SHAPE;
    if (M < 0 || M > kFp8MaxM)
        return FFN_NVFP4_ERR_BATCH;
    return FFN_NVFP4_OK;
}

bool act_ok(int act)
{
    return act == FFN_NVFP4_ACT_SILU || act == FFN_NVFP4_ACT_GELU_TANH;
}

ffn::Fp8WeightArg warg(const ffn_fp8_weight *w)
{
    return ffn::Fp8WeightArg{w->codes, w->block_scale};
}

int launch_status(hipError_t e)
{
    return e == hipSuccess ? FFN_NVFP4_OK : FFN_NVFP4_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t ffn_fp8_workspace_bytes(int M, int K, int N)
{
    if (M == 0 || check_common(M, K, N) != FFN_NVFP4_OK)
        return 0;
    const size_t h = static_cast<size_t>(M) * static_cast<size_t>(N) * 2;  // bf16 [M, N]
    return (h + 255) & ~static_cast<size_t>(255);
}

int ffn_fp8_dual_gemv(const void *x, int M, int K, int N, const ffn_fp8_weight *gate, const ffn_fp8_weight *up,
                      float *gate_out, float *up_out, hipStream_t stream)
{
    int rc;
    if ((rc = check_weight(gate)) || (rc = check_weight(up)) || (rc = check_common(M, K, N)))
        return rc;
    if (M == 0)
        return FFN_NVFP4_OK;
    if (!x || !gate_out || !up_out)
        return FFN_NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(gate_out, 16) || !aligned(up_out, 16))
        return FFN_NVFP4_ERR_ALIGN;
    return launch_status(
        ffn::launch_fp8_dual(M, ffn::OUT_F32_PAIR, x, warg(gate), warg(up), gate_out, up_out, N, K, stream));
}

int ffn_fp8_down_gemv(const float *gate_in, const float *up_in, int M, int N, int K, const ffn_fp8_weight *down,
                      int act, void *out, hipStream_t stream)
{
    int rc;
    if ((rc = check_weight(down)) || (rc = check_common(M, K, N)))
        return rc;
    if (!act_ok(act))
        return FFN_NVFP4_ERR_ACT;
    if (M == 0)
        return FFN_NVFP4_OK;
    if (!gate_in || !up_in || !out)
        return FFN_NVFP4_ERR_NULL;
    if (!aligned(gate_in, 16) || !aligned(up_in, 16) || !aligned(out, 16))
        return FFN_NVFP4_ERR_ALIGN;
    const ffn::InKind in = act == FFN_NVFP4_ACT_SILU ? ffn::IN_GATEUP_SILU : ffn::IN_GATEUP_GELU;
    return launch_status(ffn::launch_fp8_down(M, in, gate_in, up_in, warg(down), out, K, N, stream));
}

int ffn_fp8_forward(const void *x, int M, int K, int N, const ffn_fp8_weight *gate, const ffn_fp8_weight *up,
                    const ffn_fp8_weight *down, int act, void *workspace, size_t workspace_bytes, void *out,
                    hipStream_t stream)
{
    int rc;
    if ((rc = check_weight(gate)) || (rc = check_weight(up)) || (rc = check_weight(down)) ||
        (rc = check_common(M, K, N)))
        return rc;
    if (!act_ok(act))
        return FFN_NVFP4_ERR_ACT;
    if (M == 0)
        return FFN_NVFP4_OK;
    if (!x || !out || !workspace)
        return FFN_NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(workspace, 16))
        return FFN_NVFP4_ERR_ALIGN;
    if (workspace_bytes < ffn_fp8_workspace_bytes(M, K, N))
        return FFN_NVFP4_ERR_WORKSPACE;
    // h = bf16(act(gate) * up) from the dual GEMV's epilogue, then the down
    // GEMV against h: bit-identical to the dual entry followed by the down
    // entry (the same fp32 gate and up, the same one rounding of h).
    const ffn::OutKind epi = act == FFN_NVFP4_ACT_SILU ? ffn::OUT_H_SILU : ffn::OUT_H_GELU;
    hipError_t e = ffn::launch_fp8_dual(M, epi, x, warg(gate), warg(up), workspace, nullptr, N, K, stream);
    if (e != hipSuccess)
        return FFN_NVFP4_ERR_LAUNCH;
    return launch_status(ffn::launch_fp8_down(M, ffn::IN_BF16, workspace, nullptr, warg(down), out, K, N, stream));
}

}  // extern "C"
