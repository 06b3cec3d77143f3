// w4a4.hip -- the W4A4 prefill arm on gfx950's FP4 matrix cores: gate and up
// from 4-bit weights against activations quantised to 4 bits on every call,
// the down projection left on the W4A16 arm (dense_ffn.rs page, the W4A4
// native-FP4 prefill and the NVFP4 W4A4 MMQ arm of forward_prefill, which
// keeps the heavy-tailed down projection at higher precision).
//
// Scale format. v_mfma_scale_f32_32x32x64_f8f6f4 multiplies E2M1 operands
// with one E8M0 (power-of-two) scale per 32 consecutive elements of each
// operand row, so both operands are MXFP4 (OCP MX v1.0): per row and 32-element
// block, se = floor(log2(amax)) - 2 clamped to [-127, 127] (E8M0 byte
// se + 127; 0 for a block of zeros) and each element E2M1(v * 2^-se), nearest
// with ties to even, saturating at 6, sign kept. NVFP4 weights (E4M3 per 16)
// are requantised to this form once (mx_requant_kernel); the per-tensor
// scale2 stays an fp32 factor of the epilogue.
//
// Operand layout of the 32x32x64 FP4 product (checked on the GPU): lane l
// holds row l % 32 of its operand and the 32 elements of block l / 32 of the
// 64-column step in the low 4 registers (element 2 j in the low nibble of
// byte j, i.e. the storage layout, so 16 contiguous code bytes load straight
// into the operand), its E8M0 scale applies to that (row, block), and
// accumulator v of lane l is D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].
#include <hip/hip_runtime.h>

#include "kernels.h"
#include "nvfp4_device.h"

namespace ffn {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float w4_f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_w4_t __attribute__((ext_vector_type(2)));

constexpr int kMxBlock = 32;
constexpr int kW4Threads = 256;  // 4 waves
constexpr int kW4TokensPerWave = 32;
constexpr int kW4RowsPerTile = 32;
constexpr int kW4TokensPerGroup = 4 * kW4TokensPerWave;

// Shared exponent of a block with maximum magnitude amax (finite, >= 0).
// Subnormal maxima have floor(log2) <= -127, so they clamp to -127 like the
// smallest normals.
__device__ __forceinline__ int mx_exponent(float amax)
{
    const uint32_t bits = __float_as_uint(amax);
    if (bits == 0)
        return 0;
    const int ex = static_cast<int>((bits >> 23) & 0xFF);
    const int se = (ex == 0 ? -127 : ex - 127) - 2;
    return se < -127 ? -127 : (se > 127 ? 127 : se);
}

// 2^-se as an fp32 (se in [-127, 125] for finite inputs: a normal number).
__device__ __forceinline__ float mx_inverse_scale(int se)
{
    return __uint_as_float(static_cast<uint32_t>(127 - se) << 23);
}

// Eight values times inv as E2M1 codes, element 2 j in the low nibble of
// byte j (gfx950's conversion with unit scale: nearest-even, saturating,
// sign kept).
__device__ __forceinline__ uint32_t e2m1_pack8(const float *v, float inv)
{
    uint32_t p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0] * inv, v[1] * inv, 1.0f, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[2] * inv, v[3] * inv, 1.0f, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[4] * inv, v[5] * inv, 1.0f, 2);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[6] * inv, v[7] * inv, 1.0f, 3);
    return p;
}

// Quantises the 32 values of one block and stores its 16 code bytes and
// E8M0 byte.
__device__ __forceinline__ void mx_store_block(const float (&v)[kMxBlock], uint8_t *codes, uint8_t *e8m0)
{
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kMxBlock; ++j)
        amax = fmaxf(amax, fabsf(v[j]));
    const int se = mx_exponent(amax);
    const float inv = mx_inverse_scale(se);
    u32x4_t c;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        c[q] = e2m1_pack8(v + 8 * q, inv);
    *reinterpret_cast<u32x4_t *>(codes) = c;
    *e8m0 = static_cast<uint8_t>(se + 127);
}

// bf16 [rows, cols] -> MXFP4: one thread per 32-element block (64 bytes in,
// 17 bytes out; neighbouring threads take neighbouring blocks).
__global__ __launch_bounds__(256) void mx_quant_bf16_kernel(const uint16_t *x, int rows, int cols, uint8_t *codes,
                                                           uint8_t *e8m0)
{
    const int nb = cols / kMxBlock;
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= static_cast<long>(rows) * nb)
        return;
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(x + t * kMxBlock);
    float v[kMxBlock];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const u32x4_t w = src[q];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[8 * q + 2 * k] = __uint_as_float(w[k] << 16);
            v[8 * q + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
    }
    mx_store_block(v, codes + t * (kMxBlock / 2), e8m0 + t);
}

// NVFP4 [rows, cols] (codes, scales; scale2 left out) -> MXFP4: one thread per
// 32-element block; the NVFP4 values e2m1 * e4m3 are exact in fp32.
__global__ __launch_bounds__(256) void mx_requant_kernel(const uint8_t *codes, const uint8_t *scales, int rows,
                                                        int cols, uint8_t *mx_codes, uint8_t *mx_e8m0)
{
    const int nb = cols / kMxBlock;
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= static_cast<long>(rows) * nb)
        return;
    const u32x4_t c = *reinterpret_cast<const u32x4_t *>(codes + t * (kMxBlock / 2));
    const uint32_t sw = *reinterpret_cast<const uint16_t *>(scales + t * 2);
    const float s0 = e4m3_to_f32<0>(sw), s1 = e4m3_to_f32<1>(sw);
    float v[kMxBlock];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float s = q < 2 ? s0 : s1;
        const f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[q], 1.0f, 0);
        const f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[q], 1.0f, 1);
        const f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[q], 1.0f, 2);
        const f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[q], 1.0f, 3);
        v[8 * q + 0] = p0[0] * s;
        v[8 * q + 1] = p0[1] * s;
        v[8 * q + 2] = p1[0] * s;
        v[8 * q + 3] = p1[1] * s;
        v[8 * q + 4] = p2[0] * s;
        v[8 * q + 5] = p2[1] * s;
        v[8 * q + 6] = p3[0] * s;
        v[8 * q + 7] = p3[1] * s;
    }
    mx_store_block(v, mx_codes + t * (kMxBlock / 2), mx_e8m0 + t);
}

struct W4a4Params {
    const uint8_t *xc;  // MXFP4 activations [M, K/2], [M, K/32]
    const uint8_t *xe;
    const uint8_t *gc;  // MXFP4 gate, up [N, K/2], [N, K/32]
    const uint8_t *ge;
    const uint8_t *uc;
    const uint8_t *ue;
    float s2g, s2u;
    void *out0;  // fp32 gate [M, N], or bf16 h [M, N]
    float *out1;  // fp32 up [M, N]
    int M, N, K;
};

// One 256-column piece (4 steps of 64) of a lane's operand row: 4 x 16 code
// bytes and the 8 E8M0 bytes of blocks 8 q .. 8 q + 7, shifted down by one
// byte in the upper lane half so that step t's scale is byte 2 (t % 2) of
// word t / 2 in every lane.
struct W4Piece {
    u32x4_t c[4];
    uint32_t s[2];
};

__device__ __forceinline__ void w4_load(W4Piece &p, const uint8_t *codes_row, const uint8_t *e8m0_row, int q,
                                        int half)
{
#pragma unroll
    for (int t = 0; t < 4; ++t)
        p.c[t] = *reinterpret_cast<const u32x4_t *>(codes_row + (4 * q + t) * 32 + 16 * half);
    const u32x2_w4_t s = *reinterpret_cast<const u32x2_w4_t *>(e8m0_row + 8 * q);
    const uint64_t s64 = (static_cast<uint64_t>(s[1]) << 32 | s[0]) >> (8 * half);
    p.s[0] = static_cast<uint32_t>(s64);
    p.s[1] = static_cast<uint32_t>(s64 >> 32);
}

__device__ __forceinline__ i32x8_t w4_operand(const u32x4_t &c)
{
    return i32x8_t{static_cast<int>(c[0]), static_cast<int>(c[1]), static_cast<int>(c[2]), static_cast<int>(c[3]),
                   0, 0, 0, 0};
}

// Step t of a piece for both projections (format 4 = E2M1 for both operands;
// the byte select of each scale register is 2 (t % 2)).
template <int T>
__device__ __forceinline__ void w4_step(w4_f32x16_t &cg, w4_f32x16_t &cu, const W4Piece &a, const W4Piece &g,
                                        const W4Piece &u)
{
    constexpr int OPSEL = 2 * (T % 2);
    const i32x8_t A = w4_operand(a.c[T]);
    cg = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, w4_operand(g.c[T]), cg, 4, 4, OPSEL,
                                                         static_cast<int>(a.s[T / 2]), OPSEL,
                                                         static_cast<int>(g.s[T / 2]));
    cu = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, w4_operand(u.c[T]), cu, 4, 4, OPSEL,
                                                         static_cast<int>(a.s[T / 2]), OPSEL,
                                                         static_cast<int>(u.s[T / 2]));
}

// Dual GEMM: workgroup (x, y) takes weight rows 32 x .. 32 x + 31 of both
// projections and tokens 128 y .. 128 y + 127, one wave per 32 tokens. A lane
// loads its own operand rows straight from global memory (16 contiguous code
// bytes per step), one 256-column piece ahead of the products. Tokens past M
// re-read row M - 1 and are not stored.
template <int OUT>
__global__ __launch_bounds__(kW4Threads) void w4a4_dual_kernel(const W4a4Params p)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t0 = blockIdx.y * kW4TokensPerGroup + wave * kW4TokensPerWave;
    if (t0 >= p.M)
        return;
    const int n0 = blockIdx.x * kW4RowsPerTile;
    const int half = lane >> 5;
    const int tok = min(t0 + (lane & 31), p.M - 1);
    const int n = n0 + (lane & 31);
    const size_t kc = static_cast<size_t>(p.K) / 2, ke = static_cast<size_t>(p.K) / 32;
    const uint8_t *xr = p.xc + tok * kc, *xs = p.xe + tok * ke;
    const uint8_t *gr = p.gc + n * kc, *gs = p.ge + n * ke;
    const uint8_t *ur = p.uc + n * kc, *us = p.ue + n * ke;
    const int pieces = p.K / 256;
    w4_f32x16_t cg = {}, cu = {};
    W4Piece a, g, u;
    w4_load(a, xr, xs, 0, half);
    w4_load(g, gr, gs, 0, half);
    w4_load(u, ur, us, 0, half);
    for (int q = 0; q < pieces; ++q) {
        W4Piece an, gn, un;
        const int qn = q + 1 < pieces ? q + 1 : q;  // the last piece re-reads itself (unused)
        w4_load(an, xr, xs, qn, half);
        w4_load(gn, gr, gs, qn, half);
        w4_load(un, ur, us, qn, half);
        w4_step<0>(cg, cu, a, g, u);
        w4_step<1>(cg, cu, a, g, u);
        w4_step<2>(cg, cu, a, g, u);
        w4_step<3>(cg, cu, a, g, u);
        a = an;
        g = gn;
        u = un;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int row = t0 + 8 * (v / 4) + 4 * half + (v % 4);
        if (row < p.M) {
            const size_t o = static_cast<size_t>(row) * p.N + n;
            if constexpr (OUT == OUT_F32_PAIR) {
                static_cast<float *>(p.out0)[o] = p.s2g * cg[v];
                p.out1[o] = p.s2u * cu[v];
            } else {
                constexpr int A = (OUT == OUT_H_SILU) ? ACT_SILU : ACT_GELU_TANH;
                static_cast<uint16_t *>(p.out0)[o] = to_bf16_bits(gate_act<A>(p.s2g * cg[v]) * (p.s2u * cu[v]));
            }
        }
    }
}

}  // namespace

hipError_t launch_mx_quant_bf16(const void *x, int rows, int cols, uint8_t *codes, uint8_t *e8m0,
                                hipStream_t stream)
{
    if (rows < 1 || cols < kMxBlock || cols % kMxBlock != 0)
        return hipErrorNotSupported;
    const long blocks = static_cast<long>(rows) * (cols / kMxBlock);
    const int grid = static_cast<int>((blocks + 255) / 256);
    hipLaunchKernelGGL(mx_quant_bf16_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const uint16_t *>(x), rows,
                       cols, codes, e8m0);
    return hipGetLastError();
}

hipError_t launch_mx_requant(const uint8_t *codes, const uint8_t *scales, int rows, int cols, uint8_t *mx_codes,
                             uint8_t *mx_e8m0, hipStream_t stream)
{
    if (rows < 1 || cols < kMxBlock || cols % kMxBlock != 0)
        return hipErrorNotSupported;
    const long blocks = static_cast<long>(rows) * (cols / kMxBlock);
    const int grid = static_cast<int>((blocks + 255) / 256);
    hipLaunchKernelGGL(mx_requant_kernel, dim3(grid), dim3(256), 0, stream, codes, scales, rows, cols, mx_codes,
                       mx_e8m0);
    return hipGetLastError();
}

hipError_t launch_w4a4_dual(int M, OutKind out, const uint8_t *xc, const uint8_t *xe, const MxWeightArg &g,
                            const MxWeightArg &u, void *out0, float *out1, int N, int K, hipStream_t stream)
{
    if (M < 1 || N < kW4RowsPerTile || N % kW4RowsPerTile != 0 || K < 256 || K % 256 != 0)
        return hipErrorNotSupported;
    W4a4Params p{xc, xe, g.codes, g.e8m0, u.codes, u.e8m0, g.scale2, u.scale2, out0, out1, M, N, K};
    const dim3 grid(N / kW4RowsPerTile, (M + kW4TokensPerGroup - 1) / kW4TokensPerGroup);
    switch (out) {
    case OUT_F32_PAIR:
        hipLaunchKernelGGL(w4a4_dual_kernel<OUT_F32_PAIR>, grid, dim3(kW4Threads), 0, stream, p);
        break;
    case OUT_H_SILU:
        hipLaunchKernelGGL(w4a4_dual_kernel<OUT_H_SILU>, grid, dim3(kW4Threads), 0, stream, p);
        break;
    case OUT_H_GELU:
        hipLaunchKernelGGL(w4a4_dual_kernel<OUT_H_GELU>, grid, dim3(kW4Threads), 0, stream, p);
        break;
    default: return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace ffn
