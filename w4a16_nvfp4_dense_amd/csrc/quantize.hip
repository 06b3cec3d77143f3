// quantize.hip -- BF16 -> NVFP4 weight quantiser: the step that produces the
// weights the FFN streams (qwen35_dense.rs page, weight loader: a dense BF16
// weight is turned into NVFP4 on the GPU by a global-absmax pass, then a pass
// that writes packed E2M1 codes, per-16 E4M3 scales and the per-tensor
// weight_scale_2).
//
// The pages give no scale rule. The one used fills both formats:
//   scale2     = amax / (6 * 448)     (largest E2M1 value x largest E4M3 value)
//   block byte = E4M3(bmax / (6 * scale2)), nearest, ties to even, at most 448
//   code       = E2M1(w * (1 / (E4M3 value * scale2))), nearest, ties to even, at most 6,
//                with the sign of w (negatives that round to zero give -0)
// with everything zero when amax = 0, and code 0 where E4M3 value * scale2 is
// zero. Each step is one correctly rounded fp32 division or multiplication (no
// fused multiply-add), so the integers it decides are reproducible; the codes
// of a block take one reciprocal and 16 multiplications. Inputs must be
// finite. The two roundings are gfx950's conversions: v_cvt_pk_fp8_f32 (E4M3
// nearest-even, the input clamped to 448 first) and v_cvt_scalef32_pk_fp4_f32
// with unit scale (E2M1 nearest-even, saturating, sign kept); both were
// checked to round exactly so on every E4M3 and E2M1 value, midpoint and
// neighbour of a midpoint, and 400k random values.
//
// Two launches, both memory-bound streams over the weight:
//   quantize_absmax_kernel: per-workgroup maxima of |w| (taken on the bf16 bit
//                    patterns: for finite values the magnitude order is the
//                    unsigned order of the low 15 bits), written to the
//                    workspace; two workgroups per compute unit, each thread
//                    with four 16-element blocks (eight 16-byte loads) in
//                    flight per step;
//   quantize_kernel: every workgroup reduces those maxima (2 KB from L2, one
//                    per absmax workgroup; fewer of them shorten this prologue
//                    that delays every workgroup's stream), then each thread
//                    encodes one 16-element block at a time: 32 bytes in (two
//                    16-byte loads, issued one block ahead so the first ones
//                    overlap the prologue), 8 code bytes and 1 scale byte out
//                    (non-temporal stores), so a wave reads 2 KB and writes
//                    512 + 64 bytes contiguously.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kernels.h"
#include "nvfp4_device.h"
#include "quantize.h"

namespace ffn {

namespace {

constexpr int kThreads = 256;

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));  // a block's 8 code bytes
constexpr int kAbsmaxInFlight = 4;  // 16-element blocks per thread and step of the absmax pass
constexpr int kAbsmaxGroupsPerCu = 2;

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
// saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_encode(float s)
{
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(fminf(s, 448.0f), 0.0f, 0, false)) & 0xFF;
}

// Value of a non-negative E4M3FN byte (0x00 .. 0x7E).
__device__ __forceinline__ float e4m3_decode(uint32_t b)
{
    const uint32_t E = b >> 3, m = b & 7;
    return E == 0 ? static_cast<float>(m) * 0.001953125f  // m * 2^-9
                  : __uint_as_float(((E + 120) << 23) | (m << 20));
}

// Four E2M1 codes of (a0, a1, a2, a3) * inv, nearest with ties to the even
// code, saturating at 6, sign kept: code i in nibble i of the result.
__device__ __forceinline__ uint32_t e2m1_encode4(float a0, float a1, float a2, float a3, float inv)
{
    uint32_t p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a0 * inv, a1 * inv, 1.0f, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, a2 * inv, a3 * inv, 1.0f, 1);
    return p & 0xFFFF;
}

}  // namespace

__global__ __launch_bounds__(kThreads) void quantize_absmax_kernel(const u32x4_t *w, size_t nblocks,
                                                                   uint32_t *partial)
{
    __shared__ uint32_t sh[kThreads / 64];
    uint32_t m = 0;
    const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
    for (size_t b0 = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; b0 < nblocks;
         b0 += kAbsmaxInFlight * stride) {
        u32x4_t v[2 * kAbsmaxInFlight];
#pragma unroll
        for (int k = 0; k < kAbsmaxInFlight; ++k) {
            // past the end, block b0 again (the maximum is unchanged by a repeat)
            const size_t b = b0 + k * stride < nblocks ? b0 + k * stride : b0;
            v[2 * k] = w[2 * b];
            v[2 * k + 1] = w[2 * b + 1];
        }
#pragma unroll
        for (int k = 0; k < 2 * kAbsmaxInFlight; ++k)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                m = max(m, max(v[k][q] & 0x7FFFu, (v[k][q] >> 16) & 0x7FFFu));
    }
    m = workgroup_max(m, sh);
    if (threadIdx.x == 0)
        partial[blockIdx.x] = m;
}

__global__ __launch_bounds__(kThreads) void quantize_kernel(const u32x4_t *w, size_t nblocks, const uint32_t *partial,
                                                            int npartial, u32x2_t *codes, uint8_t *scales,
                                                            float *scale2_out)
{
    __shared__ uint32_t sh[kThreads / 64];
    const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
    size_t b = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
    u32x4_t n0 = {0u, 0u, 0u, 0u}, n1 = {0u, 0u, 0u, 0u};  // the next block's 32 bytes
    if (b < nblocks) {
        n0 = w[2 * b];
        n1 = w[2 * b + 1];
    }
    uint32_t m = 0;
    for (int i = threadIdx.x; i < npartial; i += kThreads)
        m = max(m, partial[i]);
    m = workgroup_max(m, sh);
    const float amax = bf16_bits_to_float(m);
    const float scale2 = amax / 2688.0f;  // 6 * 448
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *scale2_out = amax == 0.0f ? 0.0f : scale2;
    const float d = scale2 * 6.0f;
    for (; b < nblocks; b += stride) {
        const u32x4_t v0 = n0;
        const u32x4_t v1 = n1;
        if (b + stride < nblocks) {
            n0 = w[2 * (b + stride)];
            n1 = w[2 * (b + stride) + 1];
        }
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
        u32x2_t packed = {0u, 0u};
        if (denom != 0.0f) {
            const float inv = 1.0f / denom;
            float f[16];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                f[j] = bf16_bits_to_float(bits[j]);
            packed.x = e2m1_encode4(f[0], f[1], f[2], f[3], inv) | (e2m1_encode4(f[4], f[5], f[6], f[7], inv) << 16);
            packed.y = e2m1_encode4(f[8], f[9], f[10], f[11], inv) | (e2m1_encode4(f[12], f[13], f[14], f[15], inv) << 16);
        }
        // non-temporal: the 50 MB of codes and scales are not read back here,
        // and stores that stream out at once leave less to write back while
        // the next quantise reads (73.4 -> 67.1 us per 17408 x 5120 weight)
        __builtin_nontemporal_store(packed, codes + b);
        __builtin_nontemporal_store(static_cast<uint8_t>(sb), scales + b);
    }
}

namespace {

// Workgroups of the quantise pass: a few per compute unit, at most
// kQuantizeMaxPartials.
int quantize_blocks(size_t nblocks)
{
    const size_t want = (nblocks + kThreads - 1) / kThreads;
    const size_t cap = std::min<size_t>(kQuantizeMaxPartials, static_cast<size_t>(device_cu_count()) * 8);
    return static_cast<int>(std::max<size_t>(1, std::min(want, cap)));
}

// Workgroups of the absmax pass, one partial maximum each: kAbsmaxGroupsPerCu
// per compute unit, at most kQuantizeMaxPartials.
int absmax_blocks(size_t nblocks)
{
    const size_t want = (nblocks + kThreads - 1) / kThreads;
    const size_t cap =
        std::min<size_t>(kQuantizeMaxPartials, static_cast<size_t>(device_cu_count()) * kAbsmaxGroupsPerCu);
    return static_cast<int>(std::max<size_t>(1, std::min(want, cap)));
}

}  // namespace

hipError_t launch_quantize(const void *w, int rows, int cols, uint8_t *codes, uint8_t *scales, float *scale2,
                           uint32_t *partial, hipStream_t stream)
{
    const size_t nblocks = static_cast<size_t>(rows) * static_cast<size_t>(cols) / 16;  // 16-element blocks
    const int ga = absmax_blocks(nblocks);
    const int g = quantize_blocks(nblocks);
    hipLaunchKernelGGL(quantize_absmax_kernel, dim3(ga), dim3(kThreads), 0, stream, static_cast<const u32x4_t *>(w),
                       nblocks, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(quantize_kernel, dim3(g), dim3(kThreads), 0, stream, static_cast<const u32x4_t *>(w), nblocks,
                       partial, ga, reinterpret_cast<u32x2_t *>(codes), scales, scale2);
    return hipGetLastError();
}

}  // namespace ffn
