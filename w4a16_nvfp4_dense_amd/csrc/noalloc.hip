// noalloc.hip -- ffn_nvfp4_forward_noalloc: the FFN forward for callers that
// cannot allocate device memory (code under stream capture, serving loops,
// harnesses that forbid hipMalloc). The forward's workspace (h between the
// two projections, and the partial sums of the matrix-core arms) lives in one
// file-scope device array instead, of kNoallocScratchBytes per device.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "ffn_nvfp4.h"

constexpr size_t kNoallocScratchBytes = size_t{4} << 20;  // 4 MiB

// Each device that runs the entry point holds its own copy until the process
// ends. In host code `scratch` names a host-side stand-in, never the device
// memory: only the address hipGetSymbolAddress returns is passed on.
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch`, per device

// The address of this device's copy of `scratch`, looked up once per device
// with that device current. The stream must belong to the current device.
int device_scratch(hipStream_t stream, void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return FFN_NVFP4_ERR_LAUNCH;
    if (stream != nullptr) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev)
            return FFN_NVFP4_ERR_LAUNCH;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return FFN_NVFP4_ERR_LAUNCH;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return FFN_NVFP4_OK;
}

}  // namespace

extern "C" int ffn_nvfp4_forward_noalloc(const void *x, int M, int K, int N, const ffn_nvfp4_weight *gate,
                                         const ffn_nvfp4_weight *up, const ffn_nvfp4_weight *down, int act,
                                         void *out, hipStream_t stream)
{
    // ffn_nvfp4_workspace_bytes is 0 for shapes the forward rejects; the
    // forward then reports why.
    if (ffn_nvfp4_workspace_bytes(M, K, N) > kNoallocScratchBytes)
        return FFN_NVFP4_ERR_WORKSPACE;
    void *ws = nullptr;
    const int rc = device_scratch(stream, &ws);
    if (rc != FFN_NVFP4_OK)
        return rc;
    return ffn_nvfp4_forward(x, M, K, N, gate, up, down, act, ws, kNoallocScratchBytes, out, stream);
}
