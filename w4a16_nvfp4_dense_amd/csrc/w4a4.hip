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


// LDS stage of one 256-column piece: A codes (128 token rows x 128 B), B codes
// (32 gate rows, then 32 up rows, x 128 B), A scales (128 rows x 8 B), B
// scales (64 rows x 8 B). In a row's 128 code bytes the 16-byte chunk c sits
// at slot c ^ ((row / 2) % 8), so that the 16 lanes of a ds_read_b128 phase
// (16 consecutive rows, one chunk) hit 16 distinct 16-byte bank groups.
constexpr int kW4Stages = 3;
constexpr int kW4ACodes = 0;
constexpr int kW4BCodes = 128 * 128;
constexpr int kW4AScales = kW4BCodes + 64 * 128;
constexpr int kW4BScales = kW4AScales + 128 * 8;
constexpr int kW4Stage = kW4BScales + 64 * 8;                 // 26112 B
constexpr int kW4Dummy = kW4Stages * kW4Stage;                 // 256 B never read
constexpr int kW4LdsBytes = kW4Dummy + 256;                    // 78592 B: two workgroups per CU

__device__ __forceinline__ int w4_slot(int row, int chunk)
{
    return chunk ^ ((row >> 1) & 7);
}

__device__ __forceinline__ i32x8_t w4_operand(const u32x4_t &c)
{
    return i32x8_t{static_cast<int>(c[0]), static_cast<int>(c[1]), static_cast<int>(c[2]), static_cast<int>(c[3]),
                   0, 0, 0, 0};
}

// The 8 E8M0 bytes of a row's piece, shifted down by one byte in the upper
// lane half: step t's scale is then byte 2 (t % 2) of word t / 2.
__device__ __forceinline__ void w4_scales(uint32_t (&s)[2], const FFN_LDS uint8_t *row8, int half)
{
    const u32x2_w4_t v = *reinterpret_cast<const FFN_LDS u32x2_w4_t *>(row8);
    const uint64_t s64 = (static_cast<uint64_t>(v[1]) << 32 | v[0]) >> (8 * half);
    s[0] = static_cast<uint32_t>(s64);
    s[1] = static_cast<uint32_t>(s64 >> 32);
}

// Dual GEMM: workgroup (x, y) takes weight rows 32 x .. 32 x + 31 of both
// projections and tokens 128 y .. 128 y + 127, wave w the token tile
// 32 w .. 32 w + 31 for the whole reduction. Per 256-column piece the
// workgroup stages the activation codes and scales and both projections'
// codes and scales into a 3-stage LDS ring with direct global-to-LDS loads
// (every load instruction reads 8 rows x 128 contiguous bytes; every wave
// issues the same 8 loads per stage, one of them into a dummy area), one
// piece ahead of the products; each wave then reads its operands in the
// MFMA layout (ds_read_b128) and runs 8 products. Tokens past M re-read row
// M - 1 and are not stored.
template <int OUT>
__global__ __launch_bounds__(kW4Threads) void w4a4_dual_kernel(const W4a4Params p)
{
    extern __shared__ u32x4_t lds_raw[];
    FFN_LDS uint8_t *lds = (FFN_LDS uint8_t *)lds_raw;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tg0 = blockIdx.y * kW4TokensPerGroup;
    const int n0 = blockIdx.x * kW4RowsPerTile;
    const int half = lane >> 5;
    const size_t kc = static_cast<size_t>(p.K) / 2, ke = static_cast<size_t>(p.K) / 32;
    const int pieces = p.K / 256;

    // Load sources of this lane (piece 0; piece q adds 128 q code bytes, 8 q
    // scale bytes). A codes: loads j = 0..3 cover rows 32 w + 8 j + lane / 8.
    const uint8_t *asrc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int R = 32 * wave + 8 * j + (lane >> 3);
        const int tok = min(tg0 + R, p.M - 1);
        asrc[j] = p.xc + tok * kc + 16 * w4_slot(R, lane & 7);
    }
    // B codes: loads j = 0, 1 cover rows 16 w + 8 j + lane / 8 (gate rows
    // 0..31, up rows 32..63).
    const uint8_t *bsrc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int Rb = 16 * wave + 8 * j + (lane >> 3);
        const uint8_t *base = Rb < 32 ? p.gc : p.uc;
        bsrc[j] = base + (n0 + (Rb & 31)) * kc + 16 * w4_slot(Rb, lane & 7);
    }
    // Scales: one dword per lane, rows 32 w + lane / 2 (A), and for waves 0
    // and 1 the gate or up rows (B; waves 2 and 3 load a dummy).
    const int atok = min(tg0 + 32 * wave + (lane >> 1), p.M - 1);
    const uint8_t *assrc = p.xe + atok * ke + 4 * (lane & 1);
    const uint8_t *bsbase = wave == 1 ? p.ue : p.ge;
    const uint8_t *bssrc = bsbase + (n0 + (lane >> 1)) * ke + 4 * (lane & 1);
    const bool bscale_wave = wave < 2;

    auto issue = [&](int q, int st) {
        FFN_LDS uint8_t *base = lds + st * kW4Stage;
        const size_t co = static_cast<size_t>(q) * 128, so = static_cast<size_t>(q) * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(asrc[j] + co),
                                             reinterpret_cast<FFN_LDS void *>(base + kW4ACodes +
                                                                              (32 * wave + 8 * j) * 128),
                                             16, 0, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(bsrc[j] + co),
                                             reinterpret_cast<FFN_LDS void *>(base + kW4BCodes +
                                                                              (16 * wave + 8 * j) * 128),
                                             16, 0, 0);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(assrc + so),
                                         reinterpret_cast<FFN_LDS void *>(base + kW4AScales + 32 * wave * 8), 4, 0,
                                         0);
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void *>(bssrc + so),
            reinterpret_cast<FFN_LDS void *>(bscale_wave ? base + kW4BScales + 32 * wave * 8 : lds + kW4Dummy), 4,
            0, 0);
    };

    // prologue: pieces 0 .. S - 2 (a piece past the end loads the last one
    // again, so every wait below has the same number of loads in flight)
#pragma unroll
    for (int k = 0; k < kW4Stages - 1; ++k)
        issue(min(k, pieces - 1), k);

    w4_f32x16_t cg = {}, cu = {};
    const int ar = 32 * wave + (lane & 31);  // this lane's A row in a stage
    const int br = lane & 31;                // its B row (gate; up is 32 rows on)
    for (int q = 0; q < pieces; ++q) {
        const int st = q % kW4Stages;
        wait_vmcnt<8 * (kW4Stages - 2)>();
        lds_barrier();
        issue(min(q + kW4Stages - 1, pieces - 1), (q + kW4Stages - 1) % kW4Stages);
        const FFN_LDS uint8_t *base = lds + st * kW4Stage;
        uint32_t sa[2], sg[2], su[2];
        w4_scales(sa, base + kW4AScales + ar * 8, half);
        w4_scales(sg, base + kW4BScales + br * 8, half);
        w4_scales(su, base + kW4BScales + (32 + br) * 8, half);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int c = 2 * t + half;
            const u32x4_t a = *reinterpret_cast<const FFN_LDS u32x4_t *>(base + kW4ACodes + ar * 128 +
                                                                          16 * w4_slot(ar, c));
            const u32x4_t g = *reinterpret_cast<const FFN_LDS u32x4_t *>(base + kW4BCodes + br * 128 +
                                                                          16 * w4_slot(br, c));
            const u32x4_t u = *reinterpret_cast<const FFN_LDS u32x4_t *>(base + kW4BCodes + (32 + br) * 128 +
                                                                          16 * w4_slot(32 + br, c));
            const i32x8_t A = w4_operand(a);
            if (t % 2 == 0) {
                cg = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, w4_operand(g), cg, 4, 4, 0,
                                                                     static_cast<int>(sa[t / 2]), 0,
                                                                     static_cast<int>(sg[t / 2]));
                cu = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, w4_operand(u), cu, 4, 4, 0,
                                                                     static_cast<int>(sa[t / 2]), 0,
                                                                     static_cast<int>(su[t / 2]));
            } else {
                cg = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, w4_operand(g), cg, 4, 4, 2,
                                                                     static_cast<int>(sa[t / 2]), 2,
                                                                     static_cast<int>(sg[t / 2]));
                cu = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, w4_operand(u), cu, 4, 4, 2,
                                                                     static_cast<int>(sa[t / 2]), 2,
                                                                     static_cast<int>(su[t / 2]));
            }
        }
    }
    wait_vmcnt<0>();  // the trailing re-loads land before the workgroup ends
    const int n = n0 + (lane & 31);
    const int t0 = tg0 + 32 * wave;
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

template <int OUT>
hipError_t launch_dual_t(const W4a4Params &p, dim3 grid, hipStream_t stream)
{
    auto kern = w4a4_dual_kernel<OUT>;
    static std::atomic<uint64_t> lds_done{0};
    hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), kW4LdsBytes, lds_done);
    if (e != hipSuccess)
        return e;
    W4a4Params q = p;
    void *args[] = {&q};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), grid, dim3(kW4Threads), args, kW4LdsBytes, stream);
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
    case OUT_F32_PAIR: return launch_dual_t<OUT_F32_PAIR>(p, grid, stream);
    case OUT_H_SILU: return launch_dual_t<OUT_H_SILU>(p, grid, stream);
    case OUT_H_GELU: return launch_dual_t<OUT_H_GELU>(p, grid, stream);
    default: return hipErrorNotSupported;
    }
}

}  // namespace ffn
