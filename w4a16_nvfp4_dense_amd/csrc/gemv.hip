// gemv.hip -- weight-streaming NVFP4 x bf16 GEMV for 1 <= M <= 8 rows on
// gfx950: the dual gate+up GEMV and the down GEMV of the gated FFN
// (dense_ffn.rs page: DenseFfnLayer::forward for M = 1; forward_k2,
// forward_k3 and forward_km for the speculative-verify batches, where every
// weight byte is read once for all M rows).
//
// Work decomposition. The reduction dimension of a weight row (cols) is cut
// into 32-column chunks: 16 bytes of E2M1 codes (one 128-bit load) plus two
// E4M3 scale bytes. A row is owned by a "slot" of LPR lanes (LPR = 8..64,
// picked so LPR divides the chunk count when possible); lane i of the slot
// takes chunks i, i + LPR, i + 2 LPR, ... so each 128-bit load instruction of
// a slot covers LPR * 16 contiguous bytes of the row. A wave holds 64 / LPR
// slots; for the dual GEMV a slot owns the same row of both W_g and W_u, so
// the activation it reads is used twice.
//
// The activation rows a[m, :] (bf16) are staged in LDS once per workgroup,
// laid out [m][q][chunk] in 16-byte units (q = which 8-column quarter of the
// chunk) so that the lanes of a slot, reading consecutive chunks, hit
// consecutive LDS addresses. For the down GEMV the staging computes
// h = bf16(act(gate) * up) from the fp32 dual outputs: the activation is fused
// into the load of the down GEMV's input. When M * cols does not fit the LDS
// budget, the reduction dimension is staged in pieces; a lane still visits its
// chunks in increasing order, so results do not depend on the piece size.
//
// Per chunk a lane converts the 32 codes to 16 bf16 pairs once (hardware
// FP4 -> bf16 conversion), then for every activation row takes two 8-term
// dot2 chains (one per 16-column scale block) and folds each into its fp32
// accumulator with the block's E4M3 scale. The slot's partial sums are
// combined by a fixed DPP tree within the wave; there is no cross-wave
// shared-memory reduction and no atomics, so results are bit-reproducible,
// and a row's result does not depend on M.
#include <atomic>
#include <cstdint>

#include "kernels.h"
#include "nvfp4_device.h"

namespace ffn {
namespace {

constexpr int kThreads = 256;               // 4 waves per workgroup
constexpr int kWaves = kThreads / 64;
constexpr size_t kLdsBudget = 64 * 1024;    // bytes of staged activations per workgroup
constexpr int kGroup = 4;                   // chunks loaded per lane before computing

struct GemvParams {
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
    int rows;       // output rows of each weight
    int cols;       // reduction length
    int cpr;        // 32-column chunks per row (cols / 32)
    int piece;      // chunks staged per LDS piece (multiple of LPR unless single piece)
    int npieces;
    int pitch;      // LDS row pitch in 16-byte units (piece + 1)
};

// Stage chunks [c0, c0 + n) of every activation row into LDS.
template <int M, int IN>
__device__ __forceinline__ void stage_piece(const GemvParams &p, u32x4_t *lds, int c0, int n)
{
    const int total = M * n * 4;
    for (int s = threadIdx.x; s < total; s += blockDim.x) {
        const int m = s / (n * 4);
        const int rem = s - m * n * 4;
        const int cl = rem >> 2;
        const int q = rem & 3;
        const size_t col = static_cast<size_t>(c0 + cl) * 32 + q * 8;
        const size_t off = static_cast<size_t>(m) * p.cols + col;
        u32x4_t v;
        if constexpr (IN == IN_BF16) {
            v = *reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(p.in0) + off);
        } else {
            const f32x4_t *g = reinterpret_cast<const f32x4_t *>(static_cast<const float *>(p.in0) + off);
            const f32x4_t *u = reinterpret_cast<const f32x4_t *>(p.in1 + off);
            const f32x4_t g0 = g[0], g1 = g[1], u0 = u[0], u1 = u[1];
            constexpr int A = (IN == IN_GATEUP_SILU) ? ACT_SILU : ACT_GELU_TANH;
            v[0] = pack_bf16x2(gate_act<A>(g0[0]) * u0[0], gate_act<A>(g0[1]) * u0[1]);
            v[1] = pack_bf16x2(gate_act<A>(g0[2]) * u0[2], gate_act<A>(g0[3]) * u0[3]);
            v[2] = pack_bf16x2(gate_act<A>(g1[0]) * u1[0], gate_act<A>(g1[1]) * u1[1]);
            v[3] = pack_bf16x2(gate_act<A>(g1[2]) * u1[2], gate_act<A>(g1[3]) * u1[3]);
        }
        lds[(m * 4 + q) * p.pitch + cl] = v;
    }
}

// acc[m] += sum over the chunk's 32 columns of w * a[m], for one weight.
template <int M>
__device__ __forceinline__ void chunk_dot(const u32x4_t w, uint32_t sc, const u32x4_t *lds, int pitch,
                                          int cl, float (&acc)[M])
{
    bf16x2_t wp[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        wp[4 * q + 0] = fp4x2_to_bf16x2<0>(w[q]);
        wp[4 * q + 1] = fp4x2_to_bf16x2<1>(w[q]);
        wp[4 * q + 2] = fp4x2_to_bf16x2<2>(w[q]);
        wp[4 * q + 3] = fp4x2_to_bf16x2<3>(w[q]);
    }
    const float s0 = e4m3_to_f32<0>(sc);
    const float s1 = e4m3_to_f32<1>(sc);
#pragma unroll
    for (int m = 0; m < M; ++m) {
        u32x4_t a[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            a[q] = lds[(m * 4 + q) * pitch + cl];
        float t0 = dot2_bf16_first(wp[0], as_bf16x2(a[0][0]));
        float t1 = dot2_bf16_first(wp[8], as_bf16x2(a[2][0]));
#pragma unroll
        for (int b = 1; b < 4; ++b) {
            t0 = dot2_bf16(wp[b], as_bf16x2(a[0][b]), t0);
            t1 = dot2_bf16(wp[8 + b], as_bf16x2(a[2][b]), t1);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            t0 = dot2_bf16(wp[4 + b], as_bf16x2(a[1][b]), t0);
            t1 = dot2_bf16(wp[12 + b], as_bf16x2(a[3][b]), t1);
        }
        acc[m] = __builtin_fmaf(t0, s0, acc[m]);
        acc[m] = __builtin_fmaf(t1, s1, acc[m]);
    }
}

template <int M, int LPR, int NMAT, int IN, int OUT>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const GemvParams p)
{
    extern __shared__ u32x4_t lds[];
    constexpr int SLOTS = 64 / LPR;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int slot = lane / LPR;
    const int li = lane % LPR;
    const int row = (blockIdx.x * kWaves + wave) * SLOTS + slot;
    const bool row_ok = row < p.rows;
    const int srow = row_ok ? row : 0;

    const uint8_t *cb0 = p.codes0 + static_cast<size_t>(srow) * p.cpr * 16;
    const uint8_t *sb0 = p.scales0 + static_cast<size_t>(srow) * p.cpr * 2;
    const uint8_t *cb1 = nullptr;
    const uint8_t *sb1 = nullptr;
    if constexpr (NMAT == 2) {
        cb1 = p.codes1 + static_cast<size_t>(srow) * p.cpr * 16;
        sb1 = p.scales1 + static_cast<size_t>(srow) * p.cpr * 2;
    }

    float acc0[M], acc1[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        acc0[m] = 0.0f;
        acc1[m] = 0.0f;
    }

    for (int pc = 0; pc < p.npieces; ++pc) {
        const int c0 = pc * p.piece;
        const int n = min(p.piece, p.cpr - c0);
        if (pc)
            __syncthreads();
        stage_piece<M, IN>(p, lds, c0, n);
        __syncthreads();
        if (!row_ok)
            continue;
        const int iters = (n + LPR - 1) / LPR;
        for (int ib = 0; ib < iters; ib += kGroup) {
            u32x4_t cw0[kGroup], cw1[kGroup];
            uint32_t sw0[kGroup], sw1[kGroup];
#pragma unroll
            for (int g = 0; g < kGroup; ++g) {
                const int cl = li + LPR * (ib + g);
                const bool ok = cl < n;  // also false past the last iteration
                const int c = c0 + cl;
                cw0[g] = ok ? *reinterpret_cast<const u32x4_t *>(cb0 + static_cast<size_t>(c) * 16) : u32x4_t{0, 0, 0, 0};
                sw0[g] = ok ? *reinterpret_cast<const uint16_t *>(sb0 + static_cast<size_t>(c) * 2) : 0u;
                if constexpr (NMAT == 2) {
                    cw1[g] = ok ? *reinterpret_cast<const u32x4_t *>(cb1 + static_cast<size_t>(c) * 16) : u32x4_t{0, 0, 0, 0};
                    sw1[g] = ok ? *reinterpret_cast<const uint16_t *>(sb1 + static_cast<size_t>(c) * 2) : 0u;
                }
            }
#pragma unroll
            for (int g = 0; g < kGroup; ++g) {
                const int cl = li + LPR * (ib + g);
                if (cl < n) {
                    chunk_dot<M>(cw0[g], sw0[g], lds, p.pitch, cl, acc0);
                    if constexpr (NMAT == 2)
                        chunk_dot<M>(cw1[g], sw1[g], lds, p.pitch, cl, acc1);
                }
            }
        }
    }

    // Combine the slot's lanes (every lane of the wave takes part).
#pragma unroll
    for (int m = 0; m < M; ++m) {
        acc0[m] = segment_sum<LPR>(acc0[m]);
        if constexpr (NMAT == 2)
            acc1[m] = segment_sum<LPR>(acc1[m]);
    }
    if (!row_ok || li != LPR - 1)
        return;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const size_t o = static_cast<size_t>(m) * p.rows + row;
        if constexpr (OUT == OUT_F32_PAIR) {
            static_cast<float *>(p.out0)[o] = p.s2_0 * acc0[m];
            static_cast<float *>(p.out1)[o] = p.s2_1 * acc1[m];
        } else if constexpr (OUT == OUT_BF16) {
            static_cast<uint16_t *>(p.out0)[o] = to_bf16_bits(p.s2_0 * acc0[m]);
        } else {
            constexpr int A = (OUT == OUT_H_SILU) ? ACT_SILU : ACT_GELU_TANH;
            const float h = gate_act<A>(p.s2_0 * acc0[m]) * (p.s2_1 * acc1[m]);
            static_cast<uint16_t *>(p.out0)[o] = to_bf16_bits(h);
        }
    }
}

template <int M, int LPR, int NMAT, int IN, int OUT>
hipError_t launch_one(const GemvParams &p, size_t lds_bytes, hipStream_t stream)
{
    constexpr int SLOTS = 64 / LPR;
    const int rows_per_block = kWaves * SLOTS;
    const int blocks = (p.rows + rows_per_block - 1) / rows_per_block;
    auto kern = gemv_kernel<M, LPR, NMAT, IN, OUT>;
    if (lds_bytes > 64 * 1024) {
        // the staged size depends on the shape: allow the whole LDS once
        static std::atomic<uint64_t> lds_done{0};
        hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), 160 * 1024, lds_done);
        if (e != hipSuccess)
            return e;
    }
    GemvParams arg = p;
    void *args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), dim3(blocks), dim3(kThreads), args,
                           lds_bytes, stream);
}

template <int M, int NMAT, int IN, int OUT>
hipError_t launch_lpr(int lpr, const GemvParams &p, size_t lds_bytes, hipStream_t stream)
{
    switch (lpr) {
    case 8: return launch_one<M, 8, NMAT, IN, OUT>(p, lds_bytes, stream);
    case 16: return launch_one<M, 16, NMAT, IN, OUT>(p, lds_bytes, stream);
    case 32: return launch_one<M, 32, NMAT, IN, OUT>(p, lds_bytes, stream);
    default: return launch_one<M, 64, NMAT, IN, OUT>(p, lds_bytes, stream);
    }
}

template <int NMAT, int IN, int OUT>
hipError_t launch_m(int M, int lpr, const GemvParams &p, size_t lds_bytes, hipStream_t stream)
{
    switch (M) {
    case 1: return launch_lpr<1, NMAT, IN, OUT>(lpr, p, lds_bytes, stream);
    case 2: return launch_lpr<2, NMAT, IN, OUT>(lpr, p, lds_bytes, stream);
    case 3: return launch_lpr<3, NMAT, IN, OUT>(lpr, p, lds_bytes, stream);
    case 4: return launch_lpr<4, NMAT, IN, OUT>(lpr, p, lds_bytes, stream);
    case 5: return launch_lpr<5, NMAT, IN, OUT>(lpr, p, lds_bytes, stream);
    case 6: return launch_lpr<6, NMAT, IN, OUT>(lpr, p, lds_bytes, stream);
    case 7: return launch_lpr<7, NMAT, IN, OUT>(lpr, p, lds_bytes, stream);
    case 8: return launch_lpr<8, NMAT, IN, OUT>(lpr, p, lds_bytes, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Compute units of the current device, cached per device.
int device_cu_count()
{
    static int counts[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = __atomic_load_n(&counts[dev], __ATOMIC_RELAXED);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        __atomic_store_n(&counts[dev], n, __ATOMIC_RELAXED);
    }
    return n;
}

unsigned long long launch_tag()
{
    static std::atomic<unsigned long long> counter{0};
    unsigned long long z = counter.fetch_add(1, std::memory_order_relaxed) +
                           reinterpret_cast<uintptr_t>(&counter) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;  // splitmix64 finaliser
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z != 0 ? z : 1;
}

// Lanes per row as a function of the reduction length only: the smallest of
// 8/16/32/64 covering the row's chunks, 64 for rows of 33 chunks or more. Every
// kernel that computes a row with a given reduction length uses this split and
// the same per-lane order, so a row's result does not depend on M or on which
// kernel ran it.
int lanes_per_row(int cpr)
{
    int l = 8;
    while (l < 64 && l < cpr)
        l *= 2;
    return l;
}

namespace {

}  // namespace

hipError_t launch_gemv(int M, int nmat, InKind in, OutKind out, const void *in0, const float *in1,
                       const WeightArg &w0, const WeightArg &w1, void *out0, void *out1, int rows,
                       int cols, hipStream_t stream)
{
    GemvParams p{};
    p.in0 = in0;
    p.in1 = in1;
    p.codes0 = w0.codes;
    p.scales0 = w0.scales;
    p.s2_0 = w0.scale2;
    p.codes1 = w1.codes;
    p.scales1 = w1.scales;
    p.s2_1 = w1.scale2;
    p.out0 = out0;
    p.out1 = out1;
    p.rows = rows;
    p.cols = cols;
    p.cpr = cols / 32;
    const int lpr = lanes_per_row(p.cpr);
    // Largest piece (in chunks) whose staged copy fits the budget.
    const size_t unit = static_cast<size_t>(M) * 4 * 16;
    int piece = static_cast<int>(kLdsBudget / unit) - 1;
    if (piece >= p.cpr) {
        piece = p.cpr;
    } else {
        piece = (piece / lpr) * lpr;
        if (piece <= 0)
            return hipErrorInvalidValue;
    }
    p.piece = piece;
    p.npieces = (p.cpr + piece - 1) / piece;
    p.pitch = piece + 1;
    const size_t lds_bytes = unit * static_cast<size_t>(p.pitch);

    if (nmat == 2 && in == IN_BF16 && out == OUT_F32_PAIR)
        return launch_m<2, IN_BF16, OUT_F32_PAIR>(M, lpr, p, lds_bytes, stream);
    if (nmat == 2 && in == IN_BF16 && out == OUT_H_SILU)
        return launch_m<2, IN_BF16, OUT_H_SILU>(M, lpr, p, lds_bytes, stream);
    if (nmat == 2 && in == IN_BF16 && out == OUT_H_GELU)
        return launch_m<2, IN_BF16, OUT_H_GELU>(M, lpr, p, lds_bytes, stream);
    if (nmat == 1 && in == IN_BF16 && out == OUT_BF16)
        return launch_m<1, IN_BF16, OUT_BF16>(M, lpr, p, lds_bytes, stream);
    if (nmat == 1 && in == IN_GATEUP_SILU && out == OUT_BF16)
        return launch_m<1, IN_GATEUP_SILU, OUT_BF16>(M, lpr, p, lds_bytes, stream);
    if (nmat == 1 && in == IN_GATEUP_GELU && out == OUT_BF16)
        return launch_m<1, IN_GATEUP_GELU, OUT_BF16>(M, lpr, p, lds_bytes, stream);
    return hipErrorInvalidValue;
}

}  // namespace ffn
