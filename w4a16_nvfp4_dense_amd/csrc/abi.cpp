// abi.cpp -- the C entry points of libffn_nvfp4: host-side validation and
// dispatch to the kernels. Every check runs before anything is enqueued, and
// no HIP call is made when a check fails.
#include "ffn_nvfp4.h"

#include <cmath>
#include <cstdint>

#include "kernels.h"

namespace {

constexpr int kMaxDim = 65536;
constexpr int kMaxGemvM = 8;

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
    return (M >= 0 && M <= kMaxGemvM) ? FFN_NVFP4_OK : FFN_NVFP4_ERR_BATCH;
}

ffn::WeightArg warg(const ffn_nvfp4_weight *w)
{
    return ffn::WeightArg{w->codes, w->scales, w->scale2};
}

int launch_status(hipError_t e)
{
    return e == hipSuccess ? FFN_NVFP4_OK : FFN_NVFP4_ERR_LAUNCH;
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
    case FFN_NVFP4_ERR_ALIGN: return "pointer misaligned (codes/x/out/workspace need 16 bytes, scales 2)";
    case FFN_NVFP4_ERR_SHAPE: return "K and N must be positive multiples of 32, at most 65536";
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
    if (M == 0)
        return 0;
    // gate and up in fp32, [M, N] each, one after the other
    size_t bytes = 2 * static_cast<size_t>(M) * static_cast<size_t>(N) * 4;
    return (bytes + 255) & ~static_cast<size_t>(255);
}

int ffn_nvfp4_dual_gemv(const void *x, int M, int K, int N, const ffn_nvfp4_weight *gate,
                        const ffn_nvfp4_weight *up, float *gate_out, float *up_out, hipStream_t stream)
{
    int rc;
    if ((rc = check_weight(gate)) || (rc = check_weight(up)))
        return rc;
    if (!dim_ok(K) || !dim_ok(N))
        return FFN_NVFP4_ERR_SHAPE;
    if ((rc = check_batch(M)))
        return rc;
    if (M == 0)
        return FFN_NVFP4_OK;
    if (!x || !gate_out || !up_out)
        return FFN_NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(gate_out, 16) || !aligned(up_out, 16))
        return FFN_NVFP4_ERR_ALIGN;
    return launch_status(ffn::launch_gemv(M, 2, ffn::IN_BF16, ffn::OUT_F32_PAIR, x, nullptr, warg(gate),
                                          warg(up), gate_out, up_out, N, K, stream));
}

int ffn_nvfp4_down_gemv(const float *gate_in, const float *up_in, int M, int N, int K,
                        const ffn_nvfp4_weight *down, int act, void *out, hipStream_t stream)
{
    int rc;
    if ((rc = check_weight(down)))
        return rc;
    if (!dim_ok(K) || !dim_ok(N))
        return FFN_NVFP4_ERR_SHAPE;
    if ((rc = check_batch(M)))
        return rc;
    if (act != FFN_NVFP4_ACT_SILU && act != FFN_NVFP4_ACT_GELU_TANH)
        return FFN_NVFP4_ERR_ACT;
    if (M == 0)
        return FFN_NVFP4_OK;
    if (!gate_in || !up_in || !out)
        return FFN_NVFP4_ERR_NULL;
    if (!aligned(gate_in, 16) || !aligned(up_in, 16) || !aligned(out, 16))
        return FFN_NVFP4_ERR_ALIGN;
    const ffn::InKind in = act == FFN_NVFP4_ACT_SILU ? ffn::IN_GATEUP_SILU : ffn::IN_GATEUP_GELU;
    return launch_status(ffn::launch_gemv(M, 1, in, ffn::OUT_BF16, gate_in, up_in, warg(down), warg(down), out,
                                          nullptr, K, N, stream));
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
    if ((rc = check_batch(M)))
        return rc;
    if (act != FFN_NVFP4_ACT_SILU && act != FFN_NVFP4_ACT_GELU_TANH)
        return FFN_NVFP4_ERR_ACT;
    if (M == 0)
        return FFN_NVFP4_OK;
    if (!x || !out || !workspace)
        return FFN_NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(workspace, 16))
        return FFN_NVFP4_ERR_ALIGN;
    if (workspace_bytes < ffn_nvfp4_workspace_bytes(M, K, N))
        return FFN_NVFP4_ERR_WORKSPACE;
    // Dual GEMV writes gate and up (fp32) to the workspace; the down GEMV
    // stages bf16(act(gate) * up) into LDS as it loads them.
    float *gate_ws = static_cast<float *>(workspace);
    float *up_ws = gate_ws + static_cast<size_t>(M) * N;
    hipError_t e = ffn::launch_gemv(M, 2, ffn::IN_BF16, ffn::OUT_F32_PAIR, x, nullptr, warg(gate), warg(up),
                                    gate_ws, up_ws, N, K, stream);
    if (e != hipSuccess)
        return FFN_NVFP4_ERR_LAUNCH;
    const ffn::InKind in = act == FFN_NVFP4_ACT_SILU ? ffn::IN_GATEUP_SILU : ffn::IN_GATEUP_GELU;
    return launch_status(ffn::launch_gemv(M, 1, in, ffn::OUT_BF16, gate_ws, up_ws, warg(down), warg(down), out,
                                          nullptr, K, N, stream));
}

}  // extern "C"
