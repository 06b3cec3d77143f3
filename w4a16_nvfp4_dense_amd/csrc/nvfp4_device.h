// nvfp4_device.h -- gfx950 device helpers for NVFP4 (E2M1 codes + E4M3 scales)
// dequantisation, bf16 dot products, wave-level reductions and the gate
// activations of the gated FFN.
//
// Format (dense_ffn.rs page, DenseFfnLayer::ensure_int8_weight doc comment):
// packed E2M1 codes [rows, cols/2], one E4M3 scale per 16 columns
// [rows, cols/16], one fp32 per-tensor scale2. The even column of a byte is its
// low nibble.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ffn {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Byte SEL of `word` holds two E2M1 codes; returns them as a bf16 pair with
// element 0 = low nibble. The hardware conversion takes an fp32 scale of which
// it only uses the power-of-two exponent, so it is called with 1.0 and the
// E4M3 block scale is applied separately. E2M1 values are exact in bf16.
template <int SEL>
__device__ __forceinline__ bf16x2_t fp4x2_to_bf16x2(uint32_t word)
{
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, SEL);
}

// Byte SEL of `word` as an OCP E4M3FN value (gfx950 decodes the OCP variant:
// bias 7, no infinities, S.1111.111 = NaN). Exact in fp32.
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t word)
{
    return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), SEL);
}

// Eight codes (one dword) times one block scale, as eight bf16 (exact).
__device__ __forceinline__ bf16x8_t dequant8(uint32_t d, float sc)
{
    const f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
    const f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
    const f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
    const f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
    bf16x8_t w;
    w[0] = static_cast<__bf16>(p0[0] * sc);
    w[1] = static_cast<__bf16>(p0[1] * sc);
    w[2] = static_cast<__bf16>(p1[0] * sc);
    w[3] = static_cast<__bf16>(p1[1] * sc);
    w[4] = static_cast<__bf16>(p2[0] * sc);
    w[5] = static_cast<__bf16>(p2[1] * sc);
    w[6] = static_cast<__bf16>(p3[0] * sc);
    w[7] = static_cast<__bf16>(p3[1] * sc);
    return w;
}

// c + a.x*b.x + a.y*b.y with bf16 pairs and an fp32 accumulator.
__device__ __forceinline__ float dot2_bf16(bf16x2_t a, bf16x2_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

// The first link of a chain, 0 + a.x*b.x + a.y*b.y (the same operation as
// dot2_bf16(a, b, 0.0f)). Written as the three-operand form with an inline
// zero: the builtin selects the accumulating two-operand form, which needs a
// register cleared to zero first (one extra move per chain).
__device__ __forceinline__ float dot2_bf16_first(bf16x2_t a, bf16x2_t b)
{
    float d;
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
    return d;
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u)
{
    return __builtin_bit_cast(bf16x2_t, u);
}

// Round two fp32 values to bf16 (nearest even) and pack lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16)
{
    return __builtin_bit_cast(float, bits16 << 16);
}

// LDS address space (a C-style cast is the only way to spell a pointer into it).
#define FFN_LDS __attribute__((address_space(3)))

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt low bits [3:0], high bits [15:14]; expcnt [6:4] = 7; lgkmcnt [11:8] = 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Exchange between the workgroups of one launch, without a fence. Data moves
// with stores and loads that carry the device-scope cache policy (sc1, as
// agent-scope atomics use): a store is written through the XCD's L2 to
// memory, a load is not served by a line another XCD may have changed. A
// writer publishes with an agent-scope atomic store of the launch's tag to a
// ready word once its own stores have completed (s_waitcnt vmcnt(0)); the
// reader waits for the tag. (A release fence instead writes back the XCD's
// whole L2, which holds what the GEMMs keep resident: 21 us slower per
// prefill forward; 8-byte atomic stores for the data, which leave half lines
// to merge below the L2, 9 us slower.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void *base, int bytes)
{
    // word 3: the raw-buffer format bits of gfx9 devices
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void store_device_coherent(__amdgpu_buffer_rsrc_t r, int byte_off, const f32x4_t &v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, byte_off, 0, 16 /* sc1 */);
}
__device__ __forceinline__ f32x4_t load_device_coherent(__amdgpu_buffer_rsrc_t r, int byte_off)
{
    return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16 /* sc1 */));
}
__device__ __forceinline__ void store_device_coherent(__amdgpu_buffer_rsrc_t r, int byte_off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, byte_off, 0, 16 /* sc1 */);
}
__device__ __forceinline__ float load_device_coherent_f32(__amdgpu_buffer_rsrc_t r, int byte_off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 16 /* sc1 */));
}

// Waits (bounded: a correct launch never reaches the limit) until the n ready
// words word(0) .. word(n - 1) all hold `tag`. A poll has the loads of up to
// 8 words in flight together. Every lane reads the same words and the first
// lane's result decides, so the exit is uniform. (Both callers wait for one
// word at a time: for the pieces of one tile, polling all words at once
// measured 0.2-1.2 us slower per forward.)
template <typename WordAt>
__device__ __forceinline__ void wait_ready(WordAt word, int n, unsigned long long tag)
{
    for (int spin = 0; spin < (1 << 22); ++spin) {
        bool ready = true;
        for (int k0 = 0; k0 < n; k0 += 8) {
            unsigned long long v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (k0 + k < n)
                    v[k] = __hip_atomic_load(word(k0 + k), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (k0 + k < n)
                    ready = ready && v[k] == tag;
        }
        if (__builtin_amdgcn_readfirstlane(static_cast<int>(ready)))
            break;
        __builtin_amdgcn_s_sleep(1);
    }
}

// Workgroup barrier for LDS only: waits for this wave's LDS traffic and meets
// the other waves, without the vector-memory drain of __syncthreads() (which
// would also wait for global loads still in flight for later use).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt untouched
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------- activations
// SiLU(g) = g / (1 + e^-g). GELU with the tanh approximation,
// 0.5 g (1 + tanh(s (g + 0.044715 g^3))), s = sqrt(2/pi), is written in the
// equivalent form g / (1 + e^(-2 s (g + 0.044715 g^3))) so both gates cost one
// exponential and one reciprocal. Large |g| saturate to g or -0 without NaN.
enum Act : int { ACT_SILU = 0, ACT_GELU_TANH = 1 };

template <int ACT>
__device__ __forceinline__ float gate_act(float g)
{
    float z;
    if constexpr (ACT == ACT_SILU) {
        z = -g;
    } else {
        constexpr float two_s = 1.5957691216057308f;  // 2 * sqrt(2/pi)
        z = -two_s * (g + 0.044715f * g * g * g);
    }
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(z));
}

// ------------------------------------------------------ wave-level reductions
// DPP lane moves (GFX9 encodings): quad_perm, row (16-lane) mirrors and row
// broadcasts. `update_dpp(old, src, ...)` writes `old` in lanes whose row is
// masked off, so masked rows add zero.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_move(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Sum of v over each aligned segment of LPR lanes (LPR = 8, 16, 32 or 64),
// in a fixed tree order; the total is valid in the segment's last lane
// (lane % LPR == LPR - 1). Every lane of the wave must execute this.
template <int LPR>
__device__ __forceinline__ float segment_sum(float v)
{
    static_assert(LPR == 8 || LPR == 16 || LPR == 32 || LPR == 64, "segment width");
    v += dpp_move<0xB1>(v);   // quad_perm [1,0,3,2]: pairs
    v += dpp_move<0x4E>(v);   // quad_perm [2,3,0,1]: quads
    v += dpp_move<0x141>(v);  // row_half_mirror: 8 lanes
    if constexpr (LPR >= 16)
        v += dpp_move<0x140>(v);  // row_mirror: 16 lanes
    if constexpr (LPR >= 32)
        v += dpp_move<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3: 32 lanes in rows 1, 3
    if constexpr (LPR >= 64)
        v += dpp_move<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3: 64 lanes in row 3
    return v;
}

}  // namespace ffn
