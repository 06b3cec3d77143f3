// ring_gemv.h -- LDS-ring NVFP4 GEMV for decode batches (M = 1, 2): the dual
// gate+up GEMV and the down GEMV (dense_ffn.rs page, DenseFfnLayer::forward
// and forward_k2), streamed through LDS with the gfx950 direct global->LDS
// loads.
//
// Why LDS. Streaming HBM near its peak needs a lot of loads in flight per CU
// (on MI355X, well over 100 KB per CU measured with plain read kernels). Load
// buffers in registers cap that well below, because the same registers hold
// the activations and the math. Here each wave owns S slots of a ring in LDS,
// each slot one weight row (codes and scales of one row, or of the same row
// of W_g and W_u); global_load_lds_dwordx4 / _dword write straight into the
// slots without touching registers, so a CU keeps up to ~120 KB of weight
// rows in flight while its registers hold the activation and the arithmetic.
//
// Layout of the work. A whole wave works on one row at a time; lane l owns
// the 32-column chunks l, l + 64, ... (IT chunks), i.e. bytes [16 (l + 64 i),
// +16) of the row's codes, which is exactly where the direct load of
// instruction i, lane l, puts them in the slot. Scales are moved 4 bytes per
// lane. Lanes past the row end load a clamped in-range address and write into
// the slot's padding; their chunk is zeroed through its scale and activation.
// One workgroup per CU; rows are dealt out to the waves of the grid round-robin.
//
// The direct loads complete in order on the vector memory counter, which the
// compiler does not associate with the LDS they write: before reading slot s
// the kernel waits explicitly until only the loads issued after that slot's
// row are outstanding; before refilling a slot, the LDS reads of it must be
// done (the compiler orders those). The activations (x, or h) sit in
// registers for the whole kernel: loaded directly for bf16 input, or for fp32
// gate/up input computed once per workgroup as bf16(act(gate) * up) into an
// LDS staging area above the ring, then copied to registers.
//
// Per chunk the arithmetic is the same as the other GEMV kernels of the
// library (16 FP4 -> bf16 pair conversions, two 8-term dot2 chains per
// activation row folded in with the E4M3 block scales, fixed DPP tree over the
// 64 lanes), so results are bit-identical to them.
#pragma once

#include "kernels.h"
#include "nvfp4_device.h"

namespace ffn {

struct RingParams {
    const void *in0;
    const float *in1;
    const uint8_t *codes0;
    const uint8_t *scales0;
    const uint8_t *codes1;
    const uint8_t *scales1;
    float s2_0;
    float s2_1;
    void *out0;
    void *out1;
    int rows;
    int cols;
    int cpr;             // 32-column chunks per row (even)
    int stage_off;       // byte offset of the activation staging area in LDS (gate/up input)
    int pitch;           // staging pitch in 16-byte units (cpr + 1)
};

#define FFN_LDS __attribute__((address_space(3)))

// Bytes of one ring slot: per weight IT KB of code padding-included, then the
// scales rounded up to 256 bytes (64 lanes x 4 bytes per load).
template <int NMAT, int IT>
constexpr int ring_mat_bytes(int its)
{
    return IT * 1024 + its * 256;
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt low bits [3:0], high bits [15:14]; expcnt [6:4] = 7; lgkmcnt [11:8] = 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most `ahead` rows (of L loads each) issued after this one are
// outstanding; `ahead` is wave-uniform and in [0, S - 1].
template <int S, int L>
__device__ __forceinline__ void wait_rows_ahead(int ahead)
{
    if constexpr (S >= 5) { if (ahead >= 4) { wait_vmcnt<4 * L>(); return; } }
    if constexpr (S >= 4) { if (ahead >= 3) { wait_vmcnt<3 * L>(); return; } }
    if constexpr (S >= 3) { if (ahead >= 2) { wait_vmcnt<2 * L>(); return; } }
    if constexpr (S >= 2) { if (ahead >= 1) { wait_vmcnt<1 * L>(); return; } }
    wait_vmcnt<0>();
}

template <int M, int IT, int NMAT, int IN, int OUT, int S, int W, int ITS>
__global__ __launch_bounds__(64 * W) void ring_gemv_kernel(const RingParams p)
{
    static_assert(S >= 1 && S <= 5, "slots per wave");
    constexpr int MATB = ring_mat_bytes<NMAT, IT>(ITS);
    constexpr int SLOT = NMAT * MATB;
    constexpr int L = NMAT * (IT + ITS);  // direct loads per row
    static_assert((S - 1) * L < 64, "outstanding loads must fit the vmcnt counter");

    extern __shared__ u32x4_t lds_raw[];
    // generic -> LDS address space (a C-style cast is the only way to spell it)
    FFN_LDS uint8_t *lds = (FFN_LDS uint8_t *)lds_raw;
    const int lane = threadIdx.x & 63;
    // The wave index is uniform across the wave; saying so keeps row
    // addresses in scalar registers (scalar base + per-lane offset loads).
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Rows are interleaved over all waves of the grid (wave g takes rows g,
    // g + G, g + 2G, ...), so at any moment the whole GPU streams one window
    // of consecutive rows, which HBM serves far better than scattered blocks.
    const int G = gridDim.x * W;
    const int r0 = blockIdx.x * W + wave;
    const int nrows = r0 < p.rows ? (p.rows - r0 + G - 1) / G : 0;
    const int cpr = p.cpr;
    FFN_LDS uint8_t *ring = lds + wave * (S * SLOT);

    // This lane's chunks; lanes past the row end are clamped and zeroed.
    int coff[IT];
    bool cok[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int c = lane + 64 * i;
        cok[i] = c < cpr;
        coff[i] = cok[i] ? c : cpr - 1;
    }
    const int sdw = cpr / 2;  // dwords of scales per row
    int soff[ITS];
#pragma unroll
    for (int i = 0; i < ITS; ++i)
        soff[i] = min(lane + 64 * i, sdw - 1);

    const size_t row_codes = static_cast<size_t>(cpr) * 16;
    const size_t row_scales = static_cast<size_t>(cpr) * 2;
    auto load_row = [&](int slot, int r) {
        FFN_LDS uint8_t *dst = ring + slot * SLOT;
#pragma unroll
        for (int t = 0; t < NMAT; ++t) {
            const uint8_t *cb = (t == 0 ? p.codes0 : p.codes1) + static_cast<size_t>(r) * row_codes;
            const uint8_t *sb = (t == 0 ? p.scales0 : p.scales1) + static_cast<size_t>(r) * row_scales;
#pragma unroll
            for (int i = 0; i < IT; ++i)
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(cb + coff[i] * 16),
                                                 reinterpret_cast<FFN_LDS void *>(dst + t * MATB + i * 1024),
                                                 16, 0, 0);
#pragma unroll
            for (int i = 0; i < ITS; ++i)
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(sb + soff[i] * 4),
                                                 reinterpret_cast<FFN_LDS void *>(dst + t * MATB + IT * 1024 + i * 256),
                                                 4, 0, 0);
        }
    };

    // Activations into registers. bf16 input: loaded directly, before the
    // ring prefetch (in-order completion: waiting for them does not wait for
    // the weights).
    u32x4_t a[M][IT][4];
    if constexpr (IN == IN_BF16) {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int i = 0; i < IT; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    a[m][i][q] = *reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(p.in0) +
                                                                     static_cast<size_t>(m) * p.cols +
                                                                     coff[i] * 32 + q * 8);
    }
    const int npre = min(nrows, S);
    for (int s = 0; s < npre; ++s)
        load_row(s, r0 + s * G);
    if constexpr (IN != IN_BF16) {
        // h = bf16(act(gate) * up), once per workgroup, into the staging area.
        constexpr int A = (IN == IN_GATEUP_SILU) ? ACT_SILU : ACT_GELU_TANH;
        FFN_LDS u32x4_t *stage = reinterpret_cast<FFN_LDS u32x4_t *>(lds + p.stage_off);
        const int total = M * cpr * 4;
        for (int s = threadIdx.x; s < total; s += 64 * W) {
            const int m = s / (cpr * 4);
            const int rem = s - m * cpr * 4;
            const size_t off = static_cast<size_t>(m) * p.cols + static_cast<size_t>(rem) * 8;
            const f32x4_t *g = reinterpret_cast<const f32x4_t *>(static_cast<const float *>(p.in0) + off);
            const f32x4_t *u = reinterpret_cast<const f32x4_t *>(p.in1 + off);
            const f32x4_t g0 = g[0], g1 = g[1], u0 = u[0], u1 = u[1];
            u32x4_t v;
            v[0] = pack_bf16x2(gate_act<A>(g0[0]) * u0[0], gate_act<A>(g0[1]) * u0[1]);
            v[1] = pack_bf16x2(gate_act<A>(g0[2]) * u0[2], gate_act<A>(g0[3]) * u0[3]);
            v[2] = pack_bf16x2(gate_act<A>(g1[0]) * u1[0], gate_act<A>(g1[1]) * u1[1]);
            v[3] = pack_bf16x2(gate_act<A>(g1[2]) * u1[2], gate_act<A>(g1[3]) * u1[3]);
            stage[(m * 4 + (rem & 3)) * p.pitch + (rem >> 2)] = v;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int i = 0; i < IT; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    a[m][i][q] = stage[(m * 4 + q) * p.pitch + coff[i]];
    }
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int i = 0; i < IT; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                a[m][i][q] = cok[i] ? a[m][i][q] : u32x4_t{0, 0, 0, 0};

    // outv[t][m] holds, in lane j, the result for row r0 + j.
    float outv[NMAT][M];
#pragma unroll
    for (int t = 0; t < NMAT; ++t)
#pragma unroll
        for (int m = 0; m < M; ++m)
            outv[t][m] = 0.0f;

    for (int jb = 0; jb < nrows; jb += S) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int j = jb + s;
            if (j < nrows) {
                wait_rows_ahead<S, L>(min(S - 1, nrows - 1 - j));
                const FFN_LDS uint8_t *slot = ring + s * SLOT;
                float acc[NMAT][M];
#pragma unroll
                for (int t = 0; t < NMAT; ++t)
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        acc[t][m] = 0.0f;
#pragma unroll
                for (int i = 0; i < IT; ++i) {
#pragma unroll
                    for (int t = 0; t < NMAT; ++t) {
                        const u32x4_t w =
                            *reinterpret_cast<const FFN_LDS u32x4_t *>(slot + t * MATB + i * 1024 + lane * 16);
                        const uint32_t sraw = *reinterpret_cast<const FFN_LDS uint16_t *>(
                            slot + t * MATB + IT * 1024 + coff[i] * 2);
                        const uint32_t sw = cok[i] ? sraw : 0u;
                        bf16x2_t wp[16];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            wp[4 * q + 0] = fp4x2_to_bf16x2<0>(w[q]);
                            wp[4 * q + 1] = fp4x2_to_bf16x2<1>(w[q]);
                            wp[4 * q + 2] = fp4x2_to_bf16x2<2>(w[q]);
                            wp[4 * q + 3] = fp4x2_to_bf16x2<3>(w[q]);
                        }
                        const float s0 = e4m3_to_f32<0>(sw);
                        const float s1 = e4m3_to_f32<1>(sw);
#pragma unroll
                        for (int m = 0; m < M; ++m) {
                            float t0 = 0.0f, t1 = 0.0f;
#pragma unroll
                            for (int b = 0; b < 4; ++b) {
                                t0 = dot2_bf16(wp[b], as_bf16x2(a[m][i][0][b]), t0);
                                t1 = dot2_bf16(wp[8 + b], as_bf16x2(a[m][i][2][b]), t1);
                            }
#pragma unroll
                            for (int b = 0; b < 4; ++b) {
                                t0 = dot2_bf16(wp[4 + b], as_bf16x2(a[m][i][1][b]), t0);
                                t1 = dot2_bf16(wp[12 + b], as_bf16x2(a[m][i][3][b]), t1);
                            }
                            acc[t][m] = __builtin_fmaf(t0, s0, acc[t][m]);
                            acc[t][m] = __builtin_fmaf(t1, s1, acc[t][m]);
                        }
                    }
                }
                // Refill the slot with the row S ahead once its LDS reads are
                // done (the compiler waits for them before the direct loads).
                if (j + S < nrows)
                    load_row(s, r0 + (j + S) * G);
#pragma unroll
                for (int t = 0; t < NMAT; ++t)
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        const float v = segment_sum<64>(acc[t][m]);
                        const float total = __builtin_bit_cast(
                            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
                        outv[t][m] = (lane == j) ? total : outv[t][m];
                    }
            }
        }
    }

    // One store per output row of the wave, from lane j.
    if (lane < nrows) {
        const int r = r0 + lane * G;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const size_t o = static_cast<size_t>(m) * p.rows + r;
            if constexpr (OUT == OUT_F32_PAIR) {
                static_cast<float *>(p.out0)[o] = p.s2_0 * outv[0][m];
                static_cast<float *>(p.out1)[o] = p.s2_1 * outv[1][m];
            } else if constexpr (OUT == OUT_BF16) {
                static_cast<uint16_t *>(p.out0)[o] = to_bf16_bits(p.s2_0 * outv[0][m]);
            } else {
                constexpr int A = (OUT == OUT_H_SILU) ? ACT_SILU : ACT_GELU_TANH;
                const float h = gate_act<A>(p.s2_0 * outv[0][m]) * (p.s2_1 * outv[1][m]);
                static_cast<uint16_t *>(p.out0)[o] = to_bf16_bits(h);
            }
        }
    }
}

}  // namespace ffn
