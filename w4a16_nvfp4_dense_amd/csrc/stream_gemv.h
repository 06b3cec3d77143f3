// stream_gemv.h -- row-streaming NVFP4 GEMV for small batches (M = 1, 2):
// the decode-time dual gate+up GEMV and down GEMV (dense_ffn.rs page,
// DenseFfnLayer::forward and forward_k2).
//
// Layout of the work. A whole wave (64 lanes) works on one weight row at a
// time; lane l owns the 32-column chunks l, l + 64, l + 128, ... of the
// reduction dimension (IT chunks), so each 128-bit load instruction of the
// wave reads 1 KB of contiguous codes. The lane's activation chunks never
// change from row to row: for short rows (M * IT <= 4) they are loaded once
// into registers and reused for every row the wave processes; for long rows
// they are staged once per workgroup in LDS, laid out [m][quarter][chunk] so
// the 64 lanes read 64 consecutive 16-byte units.
//
// The host sizes the grid to one workgroup per compute unit and gives every
// workgroup the same number of rows (17408 = 256 * 68 rows for the
// 5120 x 17408 gate/up projections), split over its waves in contiguous
// ranges that differ by at most one row (at most 64 rows per wave): no tail of
// a grid of many small workgroups. Streaming HBM at full rate needs on the
// order of 128 KB of loads in flight per CU (measured), so each wave keeps D
// rows of loads in flight and a CU runs 8 waves (2 per SIMD).
//
// Within a wave the weight loads are software-pipelined D rows ahead and
// marked non-temporal (each weight byte is used exactly once). The loop body
// has no branches: rows past the block are computed from a dummy row (row 0
// of the matrix, which stays cached) and discarded, so the compiler can count
// outstanding loads statically and never drains the pipeline. Row results
// are gathered into lane j of a register (row j of the block) and written
// with one coalesced store at the end; the gate activation of the dual GEMV's
// epilogue then runs once per row, 64 rows per instruction.
//
// For the down GEMV fed with fp32 gate/up (activation fused into the input
// load), the workgroup issues its weight prefetch, then computes
// bf16(act(gate) * up) once per workgroup into LDS while those loads are in
// flight.
//
// Per chunk: 16 hardware FP4 -> bf16 pair conversions, two 8-term dot2 chains
// per activation row (one per 16-column scale block), each folded into the
// fp32 accumulator with its E4M3 block scale; at the end of a row a fixed DPP
// tree sums the 64 lanes. Deterministic, no atomics, no cross-wave reduction.
#pragma once

#include "kernels.h"
#include "nvfp4_device.h"

namespace ffn {

struct StreamParams {
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
    int cpr;             // 32-column chunks per row
    int rows_per_block;  // rows of one workgroup, split evenly over its waves (<= 64 per wave)
    int pitch;           // LDS pitch in 16-byte units (cpr + 1) when activations are staged
};

constexpr int kStreamMaxRowsPerWave = 64;

// Rows prefetched ahead: as many as fit in about 160 VGPRs of load buffers
// (200 when the activations live in LDS, 96 for two activation rows), capped
// so the outstanding-load count stays within the 6-bit vmcnt counter.
template <int M, int NMAT, int IT>
constexpr int stream_depth()
{
    constexpr int per_row = NMAT * IT * 5;  // 4 VGPRs of codes + 1 of scales per chunk
    constexpr int loads_per_row = NMAT * IT * 2;
    int d = (M == 1 ? (M * IT <= 4 ? 160 : 200) : 96) / per_row;
    while (d > 1 && (d - 1) * loads_per_row > 60)
        --d;
    return d < 1 ? 1 : (d > 8 ? 8 : d);
}

template <int M, int IT>
constexpr bool stream_act_in_regs()
{
    return M * IT <= 4;
}

template <int NMAT, int IT>
struct RowBuf {
    u32x4_t c[NMAT][IT];
    uint32_t s[NMAT][IT];
};

// D: rows in flight per wave; MAXW: most waves per workgroup the kernel is
// compiled for (1..16; 4 gives each wave a whole SIMD's register file).
template <int M, int IT, int NMAT, int IN, int OUT, int D, int MAXW>
__global__ __launch_bounds__(64 * MAXW) void stream_gemv_kernel(const StreamParams p)
{
    constexpr bool AREG = stream_act_in_regs<M, IT>();
    extern __shared__ u32x4_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int b0 = blockIdx.x * p.rows_per_block;
    const int nb = max(min(b0 + p.rows_per_block, p.rows) - b0, 0);
    const int r0 = b0 + (nb * wave) / nwaves;
    const int r1 = b0 + (nb * (wave + 1)) / nwaves;
    const int nrows = r1 - r0;
    const int cpr = p.cpr;

    // Chunk offsets of this lane; chunks past the row end are clamped to a
    // valid address and contribute nothing (zero activation, zero scale).
    int coff[IT];
    bool cok[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int c = lane + 64 * i;
        cok[i] = c < cpr;
        coff[i] = cok[i] ? c : cpr - 1;
    }
    const size_t row_codes = static_cast<size_t>(cpr) * 16;
    const size_t row_scales = static_cast<size_t>(cpr) * 2;

    RowBuf<NMAT, IT> buf[D];
    // Row r of the block (r >= r1: dummy row 0, never used).
    auto load_row = [&](RowBuf<NMAT, IT> &b, int r) {
        const size_t rr = r < r1 ? static_cast<size_t>(r) : 0;
        const uint8_t *cb0 = p.codes0 + rr * row_codes;
        const uint8_t *sb0 = p.scales0 + rr * row_scales;
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            b.c[0][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(cb0) + coff[i]);
            b.s[0][i] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(sb0) + coff[i]);
        }
        if constexpr (NMAT == 2) {
            const uint8_t *cb1 = p.codes1 + rr * row_codes;
            const uint8_t *sb1 = p.scales1 + rr * row_scales;
#pragma unroll
            for (int i = 0; i < IT; ++i) {
                b.c[1][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(cb1) + coff[i]);
                b.s[1][i] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(sb1) + coff[i]);
            }
        }
    };

    // Activations. Their loads are issued before the weight prefetch, so
    // waiting for them does not wait for the weights (loads complete in order).
    u32x4_t a[AREG ? M : 1][AREG ? IT : 1][4];
    if constexpr (AREG && IN == IN_BF16) {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int i = 0; i < IT; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    a[m][i][q] = *reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(p.in0) +
                                                                     static_cast<size_t>(m) * p.cols +
                                                                     coff[i] * 32 + q * 8);
        if (nrows > 0) {
#pragma unroll
            for (int d = 0; d < D; ++d)
                load_row(buf[d], r0 + d);
        }
    } else {
        // Stage the activation rows into LDS once per workgroup (computing
        // bf16(act(gate) * up) for fp32 gate/up input). Each thread takes SU
        // 16-byte units per batch and issues a batch's loads together; the
        // first batch goes out before the weight prefetch.
        constexpr int SU = (IN == IN_BF16) ? 8 : 4;
        const int total = M * cpr * 4;
        const int nthr = static_cast<int>(blockDim.x);
        bool first = true;
        for (int base = 0; base < total; base += SU * nthr) {
            u32x4_t v[SU];
            f32x4_t g0[SU], g1[SU], u0[SU], u1[SU];
#pragma unroll
            for (int k = 0; k < SU; ++k) {
                const int s = min(base + k * nthr + static_cast<int>(threadIdx.x), total - 1);
                const int m = s / (cpr * 4);
                const int rem = s - m * cpr * 4;
                const size_t off = static_cast<size_t>(m) * p.cols + static_cast<size_t>(rem) * 8;
                if constexpr (IN == IN_BF16) {
                    v[k] = *reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(p.in0) + off);
                } else {
                    const f32x4_t *g = reinterpret_cast<const f32x4_t *>(static_cast<const float *>(p.in0) + off);
                    const f32x4_t *u = reinterpret_cast<const f32x4_t *>(p.in1 + off);
                    g0[k] = g[0];
                    g1[k] = g[1];
                    u0[k] = u[0];
                    u1[k] = u[1];
                }
            }
            if (first && nrows > 0) {
#pragma unroll
                for (int d = 0; d < D; ++d)
                    load_row(buf[d], r0 + d);
            }
            first = false;
#pragma unroll
            for (int k = 0; k < SU; ++k) {
                const int s = base + k * nthr + static_cast<int>(threadIdx.x);
                if (s < total) {
                    if constexpr (IN != IN_BF16) {
                        constexpr int A = (IN == IN_GATEUP_SILU) ? ACT_SILU : ACT_GELU_TANH;
                        v[k][0] = pack_bf16x2(gate_act<A>(g0[k][0]) * u0[k][0], gate_act<A>(g0[k][1]) * u0[k][1]);
                        v[k][1] = pack_bf16x2(gate_act<A>(g0[k][2]) * u0[k][2], gate_act<A>(g0[k][3]) * u0[k][3]);
                        v[k][2] = pack_bf16x2(gate_act<A>(g1[k][0]) * u1[k][0], gate_act<A>(g1[k][1]) * u1[k][1]);
                        v[k][3] = pack_bf16x2(gate_act<A>(g1[k][2]) * u1[k][2], gate_act<A>(g1[k][3]) * u1[k][3]);
                    }
                    const int m = s / (cpr * 4);
                    const int rem = s - m * cpr * 4;
                    lds[(m * 4 + (rem & 3)) * p.pitch + (rem >> 2)] = v[k];
                }
            }
        }
        __syncthreads();
        if constexpr (AREG) {
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int i = 0; i < IT; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        a[m][i][q] = lds[(m * 4 + q) * p.pitch + coff[i]];
        }
    }
    if constexpr (AREG) {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int i = 0; i < IT; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    a[m][i][q] = cok[i] ? a[m][i][q] : u32x4_t{0, 0, 0, 0};
    }

    // outv[t][m] holds, in lane j, the result for row r0 + j.
    float outv[NMAT][M];
#pragma unroll
    for (int t = 0; t < NMAT; ++t)
#pragma unroll
        for (int m = 0; m < M; ++m)
            outv[t][m] = 0.0f;

    const int nsteps = (nrows + D - 1) / D;
    for (int k = 0; k < nsteps; ++k) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int j = k * D + d;  // row index within the block
            // An opaque zero added to the LDS index: the activation reads are
            // the same for every row, and without it the compiler hoists them
            // out of the row loop into registers (IT * 16 VGPRs per row of x).
            int lz = 0;
            if constexpr (!AREG)
                asm volatile("s_mov_b32 %0, 0" : "=s"(lz));
            float acc[NMAT][M];
#pragma unroll
            for (int t = 0; t < NMAT; ++t)
#pragma unroll
                for (int m = 0; m < M; ++m)
                    acc[t][m] = 0.0f;
#pragma unroll
            for (int i = 0; i < IT; ++i) {
                u32x4_t av[M][4];
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if constexpr (AREG) {
                            av[m][q] = a[m][i][q];
                        } else {
                            // unconditional read (coff is in range), masked without a branch
                            const uint32_t keep = cok[i] ? 0xFFFFFFFFu : 0u;
                            av[m][q] = lds[(m * 4 + q) * p.pitch + coff[i] + lz] & keep;
                        }
                    }
#pragma unroll
                for (int t = 0; t < NMAT; ++t) {
                    const u32x4_t w = buf[d].c[t][i];
                    const uint32_t sw = cok[i] ? buf[d].s[t][i] : 0u;
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
                            t0 = dot2_bf16(wp[b], as_bf16x2(av[m][0][b]), t0);
                            t1 = dot2_bf16(wp[8 + b], as_bf16x2(av[m][2][b]), t1);
                        }
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            t0 = dot2_bf16(wp[4 + b], as_bf16x2(av[m][1][b]), t0);
                            t1 = dot2_bf16(wp[12 + b], as_bf16x2(av[m][3][b]), t1);
                        }
                        acc[t][m] = __builtin_fmaf(t0, s0, acc[t][m]);
                        acc[t][m] = __builtin_fmaf(t1, s1, acc[t][m]);
                    }
                }
                // Keep one chunk's temporaries live at a time when the
                // activations come from LDS (long rows).
                if constexpr (!AREG)
                    __builtin_amdgcn_sched_barrier(0);
            }
            // Refill this buffer with the row D ahead (dummy past the block).
            // The scheduling barriers keep the refill after this row's compute
            // and before the next row's, so D rows stay in flight.
            __builtin_amdgcn_sched_barrier(0);
            load_row(buf[d], r0 + j + D);
            __builtin_amdgcn_sched_barrier(0);
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

    // One store per output row of the block, from lane j.
    if (lane < nrows) {
        const int r = r0 + lane;
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
