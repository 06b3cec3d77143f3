// quantize.hip -- BF16 -> NVFP4 weight quantiser: the step that produces the
// weights the FFN streams (qwen35_dense.rs page, weight loader: a dense BF16
// weight is turned into NVFP4 on the GPU by a global-absmax pass, then a pass
// that writes packed E2M1 codes, per-16 E4M3 scales and the per-tensor
// weight_scale_2).
//
// The pages give no scale rule. The one used fills both formats:
//   scale2     = amax / (6 * 448)     (largest E2M1 value x largest E4M3 value)
//   block byte = E4M3(bmax / (6 * scale2)), nearest, ties to even, at most 448
//   code       = E2M1(w * (1 / (E4M3 value * scale2))), nearest, ties to even, at most 6
// with everything zero when amax = 0, and code 0 where E4M3 value * scale2 is
// zero. Each step is one correctly rounded fp32 division or multiplication (no
// fused multiply-add), so the integers it decides are reproducible; the codes
// of a block take one reciprocal and 16 multiplications. Inputs must be
// finite.
//
// Two launches, both memory-bound streams over the weight:
//   absmax_kernel:   per-workgroup maxima of |w| (taken on the bf16 bit
//                    patterns: for finite values the magnitude order is the
//                    unsigned order of the low 15 bits), written to the
//                    workspace;
//   quantize_kernel: every workgroup reduces those maxima (a few KB from L2),
//                    then each thread encodes one 16-element block at a time:
//                    32 bytes in (two 16-byte loads), 8 code bytes and 1 scale
//                    byte out, so a wave reads 2 KB and writes 512 + 64 bytes
//                    contiguously.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kernels.h"
#include "nvfp4_device.h"
#include "quantize.h"

namespace ffn {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits)
{
    return __uint_as_float(bits << 16);
}

// Maximum over the workgroup of a per-thread value (exact: max has no rounding).
__device__ __forceinline__ uint32_t workgroup_max(uint32_t m, uint32_t *sh)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), o)));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
        sh[wave] = m;
    __syncthreads();
    m = sh[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w)
        m = max(m, sh[w]);
    return m;
}

// E4M3FN byte nearest to s (finite, s >= 0), ties to the even mantissa,
// saturating at 448 (0x7E). Normals round the fp32 mantissa to 3 bits; below
// 2^-6 the value is a multiple of 2^-9 (s * 512 is exact, then rounded to an
// integer, ties to even), and 8 * 2^-9 = 2^-6 is byte 0x08.
__device__ __forceinline__ uint32_t e4m3_encode(float s)
{
    if (s >= 448.0f)
        return 0x7E;
    const uint32_t bits = __float_as_uint(s);
    const int e = static_cast<int>((bits >> 23) & 0xFF) - 127;
    if (e < -6)
        return static_cast<uint32_t>(__builtin_rintf(s * 512.0f));
    uint32_t m3 = (bits >> 20) & 7;
    const uint32_t rem = bits & 0xFFFFF;
    if (rem > 0x80000 || (rem == 0x80000 && (m3 & 1)))
        ++m3;
    uint32_t E = static_cast<uint32_t>(e + 7);
    if (m3 == 8) {
        m3 = 0;
        ++E;
    }
    if (E > 15 || (E == 15 && m3 == 7))
        return 0x7E;
    return (E << 3) | m3;
}

// Value of a non-negative E4M3FN byte (0x00 .. 0x7E).
__device__ __forceinline__ float e4m3_decode(uint32_t b)
{
    const uint32_t E = b >> 3, m = b & 7;
    return E == 0 ? static_cast<float>(m) * 0.001953125f  // m * 2^-9
                  : __uint_as_float(((E + 120) << 23) | (m << 20));
}

// E2M1 code nearest to q (finite), ties to the even code, saturating at 6;
// a zero result is code 0 whatever the sign. The grid is 0, .5, 1, 1.5, 2,
// 3, 4, 6, and each midpoint goes to its even neighbour.
__device__ __forceinline__ uint32_t e2m1_encode(float q)
{
    const float a = fabsf(q);
    const uint32_t k = a <= 0.25f ? 0
                     : a < 0.75f  ? 1
                     : a <= 1.25f ? 2
                     : a < 1.75f  ? 3
                     : a <= 2.5f  ? 4
                     : a < 3.5f   ? 5
                     : a <= 5.0f  ? 6
                                  : 7;
    return (q < 0.0f && k != 0) ? (k | 8) : k;
}

__global__ __launch_bounds__(kThreads) void absmax_kernel(const u32x4_t *w, size_t n16, uint32_t *partial)
{
    __shared__ uint32_t sh[kThreads / 64];
    uint32_t m = 0;
    for (size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; i < n16;
         i += static_cast<size_t>(gridDim.x) * kThreads) {
        const u32x4_t v = w[i];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            m = max(m, max(v[q] & 0x7FFFu, (v[q] >> 16) & 0x7FFFu));
    }
    m = workgroup_max(m, sh);
    if (threadIdx.x == 0)
        partial[blockIdx.x] = m;
}

__global__ __launch_bounds__(kThreads) void quantize_kernel(const u32x4_t *w, size_t nblocks, const uint32_t *partial,
                                                            int npartial, uint2 *codes, uint8_t *scales,
                                                            float *scale2_out)
{
    __shared__ uint32_t sh[kThreads / 64];
    uint32_t m = 0;
    for (int i = threadIdx.x; i < npartial; i += kThreads)
        m = max(m, partial[i]);
    m = workgroup_max(m, sh);
    const float amax = bf16_bits_to_float(m);
    const float scale2 = amax / 2688.0f;  // 6 * 448
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *scale2_out = amax == 0.0f ? 0.0f : scale2;
    const float d = scale2 * 6.0f;
    for (size_t b = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; b < nblocks;
         b += static_cast<size_t>(gridDim.x) * kThreads) {
        const u32x4_t v0 = w[2 * b];
        const u32x4_t v1 = w[2 * b + 1];
        uint32_t bits[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            bits[2 * q] = v0[q] & 0xFFFF;
            bits[2 * q + 1] = v0[q] >> 16;
            bits[8 + 2 * q] = v1[q] & 0xFFFF;
            bits[8 + 2 * q + 1] = v1[q] >> 16;
        }
        uint32_t bm = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j)
            bm = max(bm, bits[j] & 0x7FFFu);
        uint32_t sb = 0;
        float denom = 0.0f;
        if (amax != 0.0f) {
            sb = e4m3_encode(bf16_bits_to_float(bm) / d);
            denom = e4m3_decode(sb) * scale2;
        }
        uint2 packed = {0u, 0u};
        if (denom != 0.0f) {
            const float inv = 1.0f / denom;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const uint32_t code = e2m1_encode(bf16_bits_to_float(bits[j]) * inv);
                if (j < 8)
                    packed.x |= code << (4 * j);
                else
                    packed.y |= code << (4 * (j - 8));
            }
        }
        codes[b] = packed;
        scales[b] = static_cast<uint8_t>(sb);
    }
}

int absmax_blocks(size_t n16)
{
    // about 8 loads of 16 bytes per thread, at most kQuantizeMaxPartials workgroups
    const size_t want = (n16 + static_cast<size_t>(kThreads) * 8 - 1) / (static_cast<size_t>(kThreads) * 8);
    return static_cast<int>(std::max<size_t>(1, std::min<size_t>(want, kQuantizeMaxPartials)));
}

}  // namespace

hipError_t launch_quantize(const void *w, int rows, int cols, uint8_t *codes, uint8_t *scales, float *scale2,
                           uint32_t *partial, hipStream_t stream)
{
    const size_t n = static_cast<size_t>(rows) * static_cast<size_t>(cols);
    const size_t n16 = n / 8;      // 16-byte pieces of 8 bf16
    const size_t nblocks = n / 16;  // 16-element scale blocks
    const int g1 = absmax_blocks(n16);
    hipLaunchKernelGGL(absmax_kernel, dim3(g1), dim3(kThreads), 0, stream, static_cast<const u32x4_t *>(w), n16,
                       partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    // a few workgroups per compute unit: each first re-reduces the g1 maxima
    const size_t want = (nblocks + kThreads - 1) / kThreads;
    const int g2 = static_cast<int>(std::max<size_t>(1, std::min<size_t>(want, static_cast<size_t>(device_cu_count()) * 8)));
    hipLaunchKernelGGL(quantize_kernel, dim3(g2), dim3(kThreads), 0, stream, static_cast<const u32x4_t *>(w), nblocks,
                       partial, g1, reinterpret_cast<uint2 *>(codes), scales, scale2);
    return hipGetLastError();
}

}  // namespace ffn
