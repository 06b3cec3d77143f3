// stream_read.hip -- ffn_diag_read: a plain streaming read of the weight
// buffers, the bandwidth ceiling the decode GEMVs are measured against.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ffn_diag.h"
#include "ffn_nvfp4.h"
#include "kernels.h"
#include "nvfp4_device.h"

namespace ffn {

namespace {

constexpr int kReadMaxBufs = 8;
constexpr int kReadThreads = 512;
constexpr int kReadInFlight = 8;  // 16-byte loads per thread per round

struct ReadParams {
    const u32x4_t *buf[kReadMaxBufs];
    uint64_t units[kReadMaxBufs];  // sizes in 16-byte units
    int n;
    uint32_t *sink;
};

// The buffers one after the other (the loop over them is uniform, so the
// pointer stays in scalar registers); each is read grid-stride, every thread
// with kReadInFlight independent 16-byte loads in flight.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const ReadParams p)
{
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kReadThreads;
    const uint64_t t0 = static_cast<uint64_t>(blockIdx.x) * kReadThreads + threadIdx.x;
    uint32_t acc = 0;
    for (int b = 0; b < p.n; ++b) {
        const u32x4_t *src = p.buf[b];
        const uint64_t total = p.units[b];
        for (uint64_t u0 = t0; u0 < total; u0 += kReadInFlight * stride) {
            u32x4_t v[kReadInFlight];
#pragma unroll
            for (int k = 0; k < kReadInFlight; ++k) {
                const uint64_t u = u0 + k * stride;
                v[k] = __builtin_nontemporal_load(src + (u < total ? u : u0));
            }
#pragma unroll
            for (int k = 0; k < kReadInFlight; ++k)
                acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
        }
    }
    if (acc == 0x9E3779B9u)
        *p.sink = acc;
}

}  // namespace

}  // namespace ffn

extern "C" int ffn_diag_read(const void *const *bufs, const size_t *bytes, int n, uint32_t *sink,
                             hipStream_t stream)
{
    using namespace ffn;
    if (n < 1 || n > kReadMaxBufs)
        return FFN_NVFP4_ERR_SHAPE;
    if (!bufs || !bytes || !sink)
        return FFN_NVFP4_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(sink) & 3) != 0)
        return FFN_NVFP4_ERR_ALIGN;
    ReadParams p{};
    p.sink = sink;
    p.n = 0;
    uint64_t at = 0;
    for (int i = 0; i < n; ++i) {
        if (bytes[i] % 16 != 0)
            return FFN_NVFP4_ERR_SHAPE;
        if (bytes[i] == 0)
            continue;
        if (!bufs[i])
            return FFN_NVFP4_ERR_NULL;
        if ((reinterpret_cast<uintptr_t>(bufs[i]) & 15) != 0)
            return FFN_NVFP4_ERR_ALIGN;
        p.buf[p.n] = static_cast<const u32x4_t *>(bufs[i]);
        p.units[p.n] = bytes[i] / 16;
        ++p.n;
        at += bytes[i] / 16;
    }
    if (at == 0)
        return FFN_NVFP4_OK;
    const int blocks = device_cu_count();
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kReadThreads), 0, stream, p);
    return hipGetLastError() == hipSuccess ? FFN_NVFP4_OK : FFN_NVFP4_ERR_LAUNCH;
}
