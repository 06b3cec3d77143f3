// w4a4.hip -- the W4A4 prefill arm on gfx950's FP4 matrix cores: gate and up
// from 4-bit weights against activations quantised to 4 bits on every call,
// and the down projection either left on the W4A16 arm (the NVFP4 W4A4 MMQ
// arm of forward_prefill keeps the heavy-tailed down projection at higher
// precision) or run here too against h quantised to 4 bits (the W4A4
// native-FP4 prefill quantises the down input and runs all three GEMMs on FP4
// products) (dense_ffn.rs page, forward_prefill).
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

// bf16 [rows, cols] -> MXFP4: four threads per 32-element block, each with 8
// consecutive elements (one 16-byte load; a wave reads 1 KB contiguously and
// writes 256 code bytes), the block maximum taken over the quad with DPP (max
// is exact in any order, so every code and exponent equals that of one thread
// per block). rows * cols / 8 threads; cols is a multiple of 32, so a quad is
// wholly inside or past the end.
__global__ __launch_bounds__(256) void mx_quant_bf16_kernel(const uint16_t *x, long pieces, uint8_t *codes,
                                                           uint8_t *e8m0)
{
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;  // 8-element piece
    if (t >= pieces)
        return;
    const u32x4_t w = *reinterpret_cast<const u32x4_t *>(x + t * 8);
    float v[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float(w[k] << 16);
        v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        amax = fmaxf(amax, fabsf(v[j]));
    amax = fmaxf(amax, dpp_move<0xB1>(amax));  // quad_perm [1,0,3,2]
    amax = fmaxf(amax, dpp_move<0x4E>(amax));  // quad_perm [2,3,0,1]
    const int se = mx_exponent(amax);
    reinterpret_cast<uint32_t *>(codes)[t] = e2m1_pack8(v, mx_inverse_scale(se));
    if ((t & 3) == 0)
        e8m0[t >> 2] = static_cast<uint8_t>(se + 127);
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

// N: weight rows (outputs per token), K: reduction length. The down GEMM
// (DOWN) uses the gate fields for its one weight and out0 for bf16 out.
struct W4a4Params {
    const uint8_t *xc;  // MXFP4 activations [M, K/2], [M, K/32]
    const uint8_t *xe;
    const uint8_t *gc;  // MXFP4 gate, up [N, K/2], [N, K/32]
    const uint8_t *ge;
    const uint8_t *uc;
    const uint8_t *ue;
    float s2g, s2u;
    void *out0;  // fp32 gate [M, N], or bf16 h [M, N], or (DOWN) bf16 out [M, N]
    float *out1;  // fp32 up [M, N]
    int M, N, K;
    int R;  // weight rows of each projection per workgroup
    int P;  // DOWN: parts of the reduction (consecutive workgroups of a row block)
    float *part;                // DOWN, P > 1: P x [M, N] fp32 pieces (unscaled)
    unsigned long long *flags;  // DOWN, P > 1: one ready word per workgroup
    unsigned long long tag;     // this launch's ready value (nonzero)
};

// LDS stage of one 256-column piece for a workgroup with NF weight fragments
// of 32 rows: A codes (128 token rows x 128 B), B codes (32 NF rows x 128 B),
// A scales (128 rows x 8 B), B scales (32 NF rows x 8 B). B row b holds weight
// row n0 + b / 2 of the gate (b even) or the up (b odd) projection, so the
// gate and up outputs of one row land in neighbouring lanes. In a row's 128
// code bytes the 16-byte chunk c sits at slot c ^ ((row / 2) % 8), so that
// the 16 lanes of a ds_read_b128 phase (16 consecutive rows, one chunk) hit
// 16 distinct 16-byte bank groups.
template <int NF>
struct W4Stage {
    static constexpr int kACodes = 0;
    static constexpr int kBCodes = 128 * 128;
    static constexpr int kAScales = kBCodes + 32 * NF * 128;
    static constexpr int kBScales = kAScales + 128 * 8;
    static constexpr int kBytes = kBScales + 32 * NF * 8;
};
constexpr int kW4MaxFrags = 6;
constexpr int kW4LdsMax = 160 * 1024;

// Ring stages: 4 (three pieces in flight), or as many as fit.
template <int NF>
constexpr int w4_stages()
{
    constexpr int s = (kW4LdsMax - 256) / W4Stage<NF>::kBytes;
    return s > 4 ? 4 : s;
}

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

// The value of lane l ^ 1 (DPP quad permutation 1, 0, 3, 2).
__device__ __forceinline__ float w4_pair_swap(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF,
                                                                 false));
}

// Dual GEMM: workgroup (x, y) takes weight rows n0 = R x .. n0 + R - 1 of both
// projections (2 R B rows, in NF fragments of 32) and tokens 128 y ..
// 128 y + 127, wave w the token tile 32 w .. 32 w + 31 against all of the
// workgroup's B rows, for the whole reduction. The host picks R so that the
// grid has about one workgroup per compute unit: every workgroup then does the
// same work in one round (with fixed 32-row tiles, 17408 rows made 544 tiles
// for 512 resident slots, and the last 32 ran as a second round). Per
// 256-column piece the workgroup stages the activation codes and scales and
// the B rows' codes and scales into an S-stage LDS ring with direct
// global-to-LDS loads (every code load reads 8 rows x 128 contiguous bytes;
// every wave issues the same loads per piece, the spare scale loads into a
// dummy area), S - 1 pieces ahead of the products; each wave then reads its
// operands in the MFMA layout (ds_read_b128) and runs 4 NF products. Tokens
// past M re-read row M - 1, B rows past the workgroup's rows re-read its last
// row, and neither is stored.
//
// DOWN: one weight, B row b is row n0 + b of it, and workgroup x takes row
// block x / P and part x % P of the reduction (256-column pieces q0 .. q1 - 1
// with q0 = part pieces / P); one token group (M <= 128). With P > 1 the
// lower parts store their fp32 sums with device-coherent stores and set a
// ready word; the last part (the highest id of the block, so it waits only
// for workgroups dispatched before it) adds them in part order and its own
// sums last, then writes bf16 s2 * sum.
template <bool DOWN, int OUT, int NF, int S, bool SPLIT>
__global__ __launch_bounds__(kW4Threads) void w4a4_gemm_kernel(const W4a4Params p)
{
    using St = W4Stage<NF>;
    constexpr int SB = (NF + 3) / 4;     // B scale loads per wave
    constexpr int LPP = 5 + NF + SB;     // loads per wave and piece
    constexpr int kDummy = S * St::kBytes;
    extern __shared__ u32x4_t lds_raw[];
    FFN_LDS uint8_t *lds = (FFN_LDS uint8_t *)lds_raw;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tg0 = blockIdx.y * kW4TokensPerGroup;
    const int P = DOWN ? p.P : 1;
    const int rb = DOWN ? static_cast<int>(blockIdx.x) / P : static_cast<int>(blockIdx.x);
    const int part = DOWN ? static_cast<int>(blockIdx.x) - rb * P : 0;
    const int n0 = rb * p.R;
    const int nlast = min(n0 + p.R, p.N) - 1;  // last weight row of this workgroup
    const int half = lane >> 5;
    const size_t kc = static_cast<size_t>(p.K) / 2, ke = static_cast<size_t>(p.K) / 32;
    const int q0 = part * (p.K / 256) / P;               // first piece of this part
    const int pieces = (part + 1) * (p.K / 256) / P - q0;  // >= 1 (P <= K / 256)
    auto brow = [&](int b) { return DOWN ? min(n0 + b, nlast) : min(n0 + (b >> 1), nlast); };

    // Load sources of this lane (piece 0; piece q adds 128 q code bytes, 8 q
    // scale bytes). A codes: loads j = 0..3 cover rows 32 w + 8 j + lane / 8.
    const uint8_t *asrc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int R = 32 * wave + 8 * j + (lane >> 3);
        const int tok = min(tg0 + R, p.M - 1);
        asrc[j] = p.xc + tok * kc + 16 * w4_slot(R, lane & 7) + 128 * q0;
    }
    // B codes: load i covers B rows 8 (NF w + i) + lane / 8.
    const uint8_t *bsrc[NF];
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        const int b = 8 * (NF * wave + i) + (lane >> 3);
        bsrc[i] = ((!DOWN && (b & 1)) ? p.uc : p.gc) + brow(b) * kc + 16 * w4_slot(b, lane & 7) + 128 * q0;
    }
    // Scales: one dword per lane. A: rows 32 w + lane / 2. B: load j takes
    // fragment f = w + 4 j, rows 32 f + lane / 2 (past NF: a dummy load).
    const int atok = min(tg0 + 32 * wave + (lane >> 1), p.M - 1);
    const uint8_t *assrc = p.xe + atok * ke + 4 * (lane & 1) + 8 * q0;
    const uint8_t *bssrc[SB];
#pragma unroll
    for (int j = 0; j < SB; ++j) {
        const int f = min(wave + 4 * j, NF - 1);
        const int b = 32 * f + (lane >> 1);
        bssrc[j] = ((!DOWN && (b & 1)) ? p.ue : p.ge) + brow(b) * ke + 4 * (lane & 1) + 8 * q0;
    }

    auto issue = [&](int q, int st) {
        FFN_LDS uint8_t *base = lds + st * St::kBytes;
        const size_t co = static_cast<size_t>(q) * 128, so = static_cast<size_t>(q) * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(asrc[j] + co),
                                             reinterpret_cast<FFN_LDS void *>(base + St::kACodes +
                                                                              (32 * wave + 8 * j) * 128),
                                             16, 0, 0);
#pragma unroll
        for (int i = 0; i < NF; ++i)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(bsrc[i] + co),
                                             reinterpret_cast<FFN_LDS void *>(base + St::kBCodes +
                                                                              8 * (NF * wave + i) * 128),
                                             16, 0, 0);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(assrc + so),
                                         reinterpret_cast<FFN_LDS void *>(base + St::kAScales + 32 * wave * 8), 4, 0,
                                         0);
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int f = wave + 4 * j;
            __builtin_amdgcn_global_load_lds(
                reinterpret_cast<const void *>(bssrc[j] + so),
                reinterpret_cast<FFN_LDS void *>(f < NF ? base + St::kBScales + 32 * f * 8 : lds + kDummy), 4, 0, 0);
        }
    };

    // prologue: pieces 0 .. S - 2 (a piece past the end loads the last one
    // again, so every wait below has the same number of loads in flight)
#pragma unroll
    for (int k = 0; k < S - 1; ++k)
        issue(min(k, pieces - 1), k);

    w4_f32x16_t acc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f)
        acc[f] = w4_f32x16_t{};
    const int ar = 32 * wave + (lane & 31);  // this lane's A row in a stage
    const int br = lane & 31;                // its B row in every fragment
    for (int q = 0; q < pieces; ++q) {
        const int st = q % S;
        wait_vmcnt<LPP * (S - 2)>();
        lds_barrier();
        issue(min(q + S - 1, pieces - 1), (q + S - 1) % S);
        const FFN_LDS uint8_t *base = lds + st * St::kBytes;
        uint32_t sa[2], sb[NF][2];
        w4_scales(sa, base + St::kAScales + ar * 8, half);
#pragma unroll
        for (int f = 0; f < NF; ++f)
            w4_scales(sb[f], base + St::kBScales + (32 * f + br) * 8, half);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int c = 2 * t + half;
            const u32x4_t a = *reinterpret_cast<const FFN_LDS u32x4_t *>(base + St::kACodes + ar * 128 +
                                                                          16 * w4_slot(ar, c));
            const i32x8_t A = w4_operand(a);
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const int b = 32 * f + br;
                const u32x4_t w = *reinterpret_cast<const FFN_LDS u32x4_t *>(base + St::kBCodes + b * 128 +
                                                                              16 * w4_slot(b, c));
                if (t % 2 == 0)
                    acc[f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        A, w4_operand(w), acc[f], 4, 4, 0, static_cast<int>(sa[t / 2]), 0,
                        static_cast<int>(sb[f][t / 2]));
                else
                    acc[f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        A, w4_operand(w), acc[f], 4, 4, 2, static_cast<int>(sa[t / 2]), 2,
                        static_cast<int>(sb[f][t / 2]));
            }
        }
    }
    wait_vmcnt<0>();  // the trailing re-loads land before the workgroup ends
    const int t0 = tg0 + 32 * wave;
    if constexpr (DOWN) {
        // accumulator v of fragment f: token t0 + 8 (v / 4) + 4 half + v % 4,
        // output row n0 + 32 f + br; its offset in an [M, N] array (0, a
        // valid and unused one, past the rows or the tokens)
        auto elem = [&](int f, int v) {
            const int n = n0 + 32 * f + br;
            const int tok = t0 + 8 * (v / 4) + 4 * half + (v % 4);
            return (n <= nlast && tok < p.M) ? tok * p.N + n : -1;
        };
        if constexpr (SPLIT) {
            const int part_bytes = p.M * p.N * 4;  // <= 128 x 65536 x 4
            if (part != P - 1) {
                const __amdgpu_buffer_rsrc_t rs = raw_buffer(p.part + static_cast<size_t>(part) * p.M * p.N,
                                                             part_bytes);
#pragma unroll
                for (int f = 0; f < NF; ++f)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int e = elem(f, v);
                        if (e >= 0)
                            store_device_coherent(rs, 4 * e, acc[f][v]);
                    }
                wait_vmcnt<0>();
                __syncthreads();
                if (threadIdx.x == 0)
                    __hip_atomic_store(p.flags + blockIdx.x, p.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return;
            }
            const int g0 = static_cast<int>(blockIdx.x) - part;
            for (int pp = 0; pp < P - 1; ++pp)
                wait_ready([&](int) { return p.flags + g0 + pp; }, 1, p.tag);
            __syncthreads();  // every wave has seen the words: clear them
            if (threadIdx.x == 0)
                for (int pp = 0; pp < P - 1; ++pp)
                    __hip_atomic_store(p.flags + g0 + pp, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            constexpr int PC = 2;  // parts per batch (all loads of a batch in flight before its additions)
            float sum[NF][16];
            for (int p0 = 0; p0 < P - 1; p0 += PC) {
                float v_[PC][NF][16];
#pragma unroll
                for (int c = 0; c < PC; ++c) {
                    if (p0 + c >= P - 1)
                        continue;
                    const __amdgpu_buffer_rsrc_t rs =
                        raw_buffer(p.part + static_cast<size_t>(p0 + c) * p.M * p.N, part_bytes);
#pragma unroll
                    for (int f = 0; f < NF; ++f)
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            v_[c][f][v] = load_device_coherent_f32(rs, 4 * max(elem(f, v), 0));
                }
#pragma unroll
                for (int c = 0; c < PC; ++c)
#pragma unroll
                    for (int f = 0; f < NF; ++f)
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            if (p0 + c < P - 1)
                                sum[f][v] = (p0 + c == 0) ? v_[c][f][v] : sum[f][v] + v_[c][f][v];
            }
#pragma unroll
            for (int f = 0; f < NF; ++f)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[f][v] = sum[f][v] + acc[f][v];  // this workgroup's part last
        }
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int e = elem(f, v);
                if (e >= 0)
                    static_cast<uint16_t *>(p.out0)[e] = to_bf16_bits(p.s2g * acc[f][v]);
            }
        return;
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const int b = 32 * f + br;
        const int n = n0 + (b >> 1);
        const bool row_ok = n <= nlast;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int tok = t0 + 8 * (v / 4) + 4 * half + (v % 4);
            const size_t o = static_cast<size_t>(tok) * p.N + n;
            if constexpr (OUT == OUT_F32_PAIR) {
                if (row_ok && tok < p.M) {
                    if (b & 1)
                        p.out1[o] = p.s2u * acc[f][v];
                    else
                        static_cast<float *>(p.out0)[o] = p.s2g * acc[f][v];
                }
            } else {
                constexpr int A = (OUT == OUT_H_SILU) ? ACT_SILU : ACT_GELU_TANH;
                const float u = w4_pair_swap(acc[f][v]);  // the up value of row n
                if (!(b & 1) && row_ok && tok < p.M)
                    static_cast<uint16_t *>(p.out0)[o] = to_bf16_bits(gate_act<A>(p.s2g * acc[f][v]) * (p.s2u * u));
            }
        }
    }
}

template <bool DOWN, int OUT, int NF, bool SPLIT>
hipError_t launch_gemm_t(const W4a4Params &p, dim3 grid, hipStream_t stream)
{
    constexpr int S = w4_stages<NF>();
    constexpr int lds = S * W4Stage<NF>::kBytes + 256;
    static_assert(S >= 2 && lds <= kW4LdsMax, "LDS ring");
    auto kern = w4a4_gemm_kernel<DOWN, OUT, NF, S, SPLIT>;
    static std::atomic<uint64_t> lds_done{0};
    hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), lds, lds_done);
    if (e != hipSuccess)
        return e;
    W4a4Params q = p;
    void *args[] = {&q};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), grid, dim3(kW4Threads), args, lds, stream);
}

template <int OUT>
hipError_t launch_dual_nf(const W4a4Params &p, int nf, dim3 grid, hipStream_t stream)
{
    switch (nf) {
    case 1: return launch_gemm_t<false, OUT, 1, false>(p, grid, stream);
    case 2: return launch_gemm_t<false, OUT, 2, false>(p, grid, stream);
    case 3: return launch_gemm_t<false, OUT, 3, false>(p, grid, stream);
    case 4: return launch_gemm_t<false, OUT, 4, false>(p, grid, stream);
    case 5: return launch_gemm_t<false, OUT, 5, false>(p, grid, stream);
    case 6: return launch_gemm_t<false, OUT, 6, false>(p, grid, stream);
    default: return hipErrorNotSupported;
    }
}

// Down GEMM split: row blocks of kW4DownRows rows, and as many parts of the
// reduction as fill about one workgroup per compute unit (at most
// kW4MaxParts, at most one per 256-column piece).
constexpr int kW4DownFrags = 2;
constexpr int kW4DownRows = 32 * kW4DownFrags;
constexpr int kW4MaxParts = 8;

int w4_down_parts(int rows, int cols)
{
    const int blocks = (rows + kW4DownRows - 1) / kW4DownRows;
    int P = device_cu_count() / blocks;
    P = P < 1 ? 1 : (P > kW4MaxParts ? kW4MaxParts : P);
    return P > cols / 256 ? cols / 256 : P;
}

}  // namespace

hipError_t launch_mx_quant_bf16(const void *x, int rows, int cols, uint8_t *codes, uint8_t *e8m0,
                                hipStream_t stream)
{
    if (rows < 1 || cols < kMxBlock || cols % kMxBlock != 0)
        return hipErrorNotSupported;
    const long pieces = static_cast<long>(rows) * (cols / 8);
    const int grid = static_cast<int>((pieces + 255) / 256);
    hipLaunchKernelGGL(mx_quant_bf16_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const uint16_t *>(x), pieces,
                       codes, e8m0);
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
    if (M < 1 || N < 1 || K < 256 || K % 256 != 0)
        return hipErrorNotSupported;
    // Rows per workgroup: N over the compute units (at least one fragment's
    // worth, at most kW4MaxFrags fragments), so one round of about one
    // workgroup per compute unit covers every row of a token group.
    const int cus = device_cu_count();
    int R = (N + cus - 1) / cus;
    R = R < 16 ? 16 : (R > 16 * kW4MaxFrags ? 16 * kW4MaxFrags : R);
    const int nf = (R + 15) / 16;
    W4a4Params p{xc, xe, g.codes, g.e8m0, u.codes, u.e8m0, g.scale2, u.scale2, out0, out1, M, N, K, R, 1, nullptr,
                 nullptr, 0};
    const dim3 grid((N + R - 1) / R, (M + kW4TokensPerGroup - 1) / kW4TokensPerGroup);
    switch (out) {
    case OUT_F32_PAIR: return launch_dual_nf<OUT_F32_PAIR>(p, nf, grid, stream);
    case OUT_H_SILU: return launch_dual_nf<OUT_H_SILU>(p, nf, grid, stream);
    case OUT_H_GELU: return launch_dual_nf<OUT_H_GELU>(p, nf, grid, stream);
    default: return hipErrorNotSupported;
    }
}

size_t w4a4_down_partial_floats(int rows, int cols)
{
    const int P = w4_down_parts(rows, cols);
    return P > 1 ? static_cast<size_t>(P) * kW4TokensPerGroup * rows : 0;
}

size_t w4a4_down_flag_words(int rows, int cols)
{
    const int P = w4_down_parts(rows, cols);
    return P > 1 ? static_cast<size_t>(P) * ((rows + kW4DownRows - 1) / kW4DownRows) : 0;
}

hipError_t launch_w4a4_down(int M, const uint8_t *hc, const uint8_t *he, const MxWeightArg &d, uint16_t *out,
                            int rows, int cols, float *part, unsigned long long *flags, hipStream_t stream)
{
    if (M < 1 || M > kW4TokensPerGroup || rows < 1 || cols < 256 || cols % 256 != 0)
        return hipErrorNotSupported;
    const int P = w4_down_parts(rows, cols);
    if (P > 1 && (part == nullptr || flags == nullptr))
        return hipErrorNotSupported;
    W4a4Params p{hc, he, d.codes, d.e8m0, nullptr, nullptr, d.scale2, 0.0f, out, nullptr, M, rows, cols,
                 kW4DownRows, P, part, flags, P > 1 ? launch_tag() : 0};
    const dim3 grid(((rows + kW4DownRows - 1) / kW4DownRows) * P, 1);
    return P > 1 ? launch_gemm_t<true, OUT_BF16, kW4DownFrags, true>(p, grid, stream)
                 : launch_gemm_t<true, OUT_BF16, kW4DownFrags, false>(p, grid, stream);
}

}  // namespace ffn
