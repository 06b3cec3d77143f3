// fp8_gemv.h -- many-wave GEMV over block-scaled FP8 weights for decode and
// verify batches (1 <= M <= 8 activation rows): the dual gate+up GEMV with the
// gated activation in its epilogue, and the down GEMV with bf16 h or with the
// activation fused into its activation staging.
//
// Weight format (qwen35_dense.rs page, the doc comment on which FP8 scale
// layouts the native path accepts): E4M3FN bytes, row-major [rows, cols], and
// an fp32 block-scale grid [ceil(rows/128), ceil(cols/128)], row-major;
// element (r, c) = e4m3(w[r, c]) * block_scale[r/128, c/128]. The pages run
// these weights through a fused gate+up launch and an activation-fused down
// launch (dense_ffn.rs page, DenseFfnLayer::forward, the FP8 dispatch).
//
// The structure is that of the NVFP4 many-wave GEMV (one whole weight row per
// wave at a time, many waves per compute unit, activations staged once per
// workgroup in LDS, the next row's loads issued as soon as a row's arithmetic
// is done), with a 16-column chunk: lane l owns chunks l, l + 64, ... of a
// row, 16 bytes of codes each. Per chunk a lane converts its 16 codes to
// eight bf16 pairs (exact: E4M3 values have 4 significant bits and fit
// bf16's range), runs one 8-term dot2 chain per activation row, and folds the
// chain into its accumulator with the chunk's block scale (a chunk lies in
// one 128-column block: 128 is a multiple of 16). In step i lane l's chunk
// lies in block 8 i + l / 8 of its row's grid row, so the 8 lanes of a group
// share one scale: lane l loads grid entries l, l + 64, ... once per row (one
// register per 8 steps instead of one per step, which lets the long down
// rows run 16 waves per compute unit), and each step fetches its scale from
// lane 8 (i % 8) + l / 8 with ds_bpermute. The grid (0.1% of the codes) stays
// in cache. The wave reduction and the epilogues are those of the NVFP4
// kernel (a fixed DPP tree), with unit per-tensor scales.
#pragma once

#include "kernels.h"
#include "nvfp4_device.h"
#include "wave_gemv.h"

namespace ffn {

struct Fp8Params {
    const void *in0;
    const float *in1;
    const uint8_t *codes0;
    const float *bs0;
    const uint8_t *codes1;
    const float *bs1;
    void *out0;
    void *out1;
    int rows;
    int cols;
    int cpr;    // 16-column chunks per row
    int bcols;  // block-scale grid columns, ceil(cols / 128)
};

// Two E4M3FN codes (bytes 2 SEL and 2 SEL + 1 of `word`) as a bf16 pair,
// element 0 from the lower byte. The conversion's scale operand only carries
// a power-of-two exponent, so it is 1.0 and the block scale is applied to the
// chunk's dot product instead. Exact.
template <bool SEL>
__device__ __forceinline__ bf16x2_t fp8x2_to_bf16x2(uint32_t word)
{
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, SEL);
}

// Scale registers of steps I0 .. I0 + IS - 1: step i's blocks 8 i .. 8 i + 7
// sit in register i / 8 (entry 8 (i % 8) + l / 8 of grid blocks
// 64 (i / 8) ..).
template <int I0, int IS>
constexpr int fp8_scale_reg0()
{
    return I0 / 8;
}

template <int I0, int IS>
constexpr int fp8_scale_regs()
{
    return (I0 + IS - 1) / 8 - I0 / 8 + 1;
}

// One row of NMAT weights in registers: 16 code bytes per lane and step, and
// NB block-scale registers (grid entries lane + 64 k).
template <int IS, int NMAT, int NB>
struct Fp8Row {
    u32x4_t wc[NMAT][IS];
    float bs[NMAT][NB];
};

// Issues the loads of steps I0 .. I0 + IS - 1 of row r (the row has IT
// steps); NT marks the code loads non-temporal. In the last step a lane past
// the row end re-reads the row's last chunk (row_geom), whose result
// fp8_row_dot drops. Scale entries past the grid row's end are clamped to its
// last entry (no step reads them).
template <bool NT, int IT, int NMAT, int I0 = 0, int IS = IT>
__device__ __forceinline__ void fp8_load_row(Fp8Row<IS, NMAT, fp8_scale_regs<I0, IS>()> &w, const Fp8Params &p, int r,
                                             const RowGeom &rg)
{
    static_assert(I0 >= 0 && IS >= 1 && I0 + IS <= IT, "piece of the row");
    constexpr int K0 = fp8_scale_reg0<I0, IS>();
    constexpr int NB = fp8_scale_regs<I0, IS>();
#pragma unroll
    for (int t = 0; t < NMAT; ++t) {
        const u32x4_t *cb = reinterpret_cast<const u32x4_t *>((t == 0 ? p.codes0 : p.codes1) +
                                                              static_cast<size_t>(r) * static_cast<size_t>(p.cols));
        const float *sb = (t == 0 ? p.bs0 : p.bs1) + static_cast<size_t>(r >> 7) * static_cast<size_t>(p.bcols);
#pragma unroll
        for (int j = 0; j < IS; ++j) {
            const int i = I0 + j;
            const int c = (i == IT - 1) ? rg.clast : rg.lane + 64 * i;
            if constexpr (NT)
                w.wc[t][j] = __builtin_nontemporal_load(cb + c);
            else
                w.wc[t][j] = cb[c];
        }
#pragma unroll
        for (int k = 0; k < NB; ++k)
            w.bs[t][k] = sb[min(rg.lane + 64 * (K0 + k), p.bcols - 1)];
    }
}

// Steps A .. B - 1 of row r into a whole row's registers (and, with SC, the
// row's block scales).
template <bool NT, int IT, int NMAT, int A, int B, bool SC>
__device__ __forceinline__ void fp8_load_steps(Fp8Row<IT, NMAT, fp8_scale_regs<0, IT>()> &w, const Fp8Params &p,
                                               int r, const RowGeom &rg)
{
    constexpr int NB = fp8_scale_regs<0, IT>();
#pragma unroll
    for (int t = 0; t < NMAT; ++t) {
        const u32x4_t *cb = reinterpret_cast<const u32x4_t *>((t == 0 ? p.codes0 : p.codes1) +
                                                              static_cast<size_t>(r) * static_cast<size_t>(p.cols));
        const float *sb = (t == 0 ? p.bs0 : p.bs1) + static_cast<size_t>(r >> 7) * static_cast<size_t>(p.bcols);
        if constexpr (SC) {
#pragma unroll
            for (int k = 0; k < NB; ++k)
                w.bs[t][k] = sb[min(rg.lane + 64 * k, p.bcols - 1)];
        }
#pragma unroll
        for (int i = A; i < B; ++i) {
            const int c = (i == IT - 1) ? rg.clast : rg.lane + 64 * i;
            if constexpr (NT)
                w.wc[t][i] = __builtin_nontemporal_load(cb + c);
            else
                w.wc[t][i] = cb[c];
        }
    }
}

// The block scale of step i for this lane: grid block 8 i + lane / 8, held by
// lane 8 (i % 8) + lane / 8 in register i / 8 - K0.
template <int I0, int IS, int NB>
__device__ __forceinline__ float fp8_step_scale(const float (&bs)[NB], int i, int lane)
{
    constexpr int K0 = fp8_scale_reg0<I0, IS>();
    const int src = 8 * (i % 8) + (lane >> 3);
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_ds_bpermute(src * 4, __builtin_bit_cast(int, bs[i / 8 - K0])));
}

// Per-lane partial sums of one row over steps I0 .. I0 + IS - 1 (activations
// staged for those steps, two 16-byte units per chunk): acc[t][m] += bs *
// (8-term dot2 chain over the chunk), starting from zero (INIT) or adding.
template <int M, int IT, int NMAT, int I0 = 0, int IS = IT, bool INIT = true>
__device__ __forceinline__ void fp8_row_dot(float (&acc)[NMAT][M], const Fp8Row<IS, NMAT, fp8_scale_regs<I0, IS>()> &w,
                                            const u32x4_t *act, const RowGeom &rg)
{
    constexpr int NB = fp8_scale_regs<I0, IS>();
    // An opaque zero keeps the activation reads inside the row loop (see
    // row_dot).
    int lz;
    asm volatile("s_mov_b32 %0, 0" : "=s"(lz));
    const u32x4_t *ar = act + lz + rg.lane;
    if constexpr (INIT) {
#pragma unroll
        for (int t = 0; t < NMAT; ++t)
#pragma unroll
            for (int m = 0; m < M; ++m)
                acc[t][m] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < IS; ++j) {
        const int i = I0 + j;
        // past the row end the re-read chunk's result is dropped by a select
        // (its codes may hold NaN, which a zero factor would not remove)
        const bool live = (i < IT - 1) || rg.oklast;
        bf16x2_t wp[NMAT][8];
        float sc[NMAT];
#pragma unroll
        for (int t = 0; t < NMAT; ++t) {
            sc[t] = fp8_step_scale<I0, IS, NB>(w.bs[t], i, rg.lane);
            const u32x4_t c = w.wc[t][j];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                wp[t][2 * q + 0] = fp8x2_to_bf16x2<false>(c[q]);
                wp[t][2 * q + 1] = fp8x2_to_bf16x2<true>(c[q]);
            }
        }
        u32x4_t an[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            an[h] = ar[(j * 2 + h) * 64];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            u32x4_t a[2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
                a[h] = an[h];
            if (m + 1 < M) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    an[h] = ar[(((m + 1) * IS + j) * 2 + h) * 64];
            }
#pragma unroll
            for (int t = 0; t < NMAT; ++t) {
                // columns 2b, 2b + 1 of the chunk: codes pair wp[b],
                // activations unit b / 4, pair b % 4
                float d = dot2_bf16_first(wp[t][0], as_bf16x2(a[0][0]));
#pragma unroll
                for (int b = 1; b < 8; ++b)
                    d = dot2_bf16(wp[t][b], as_bf16x2(a[b >> 2][b & 3]), d);
                const float nv = __builtin_fmaf(d, sc[t], acc[t][m]);
                acc[t][m] = live ? nv : acc[t][m];
            }
#pragma unroll
            for (int t = 0; t < NMAT; ++t)
                asm volatile("" : "+v"(acc[t][m])::"memory");
        }
    }
}

// Row registers of piece p of an IT-step row cut into P pieces.
template <int IT, int NMAT, int P, int p>
using Fp8PieceRow = Fp8Row<piece_steps<IT, P, p>(), NMAT,
                           fp8_scale_regs<p * ((IT + P - 1) / P), piece_steps<IT, P, p>()>()>;

// One piece of the staged kernel (steps I0 .. I0 + IS - 1 of every row), then
// the next; as wave_pieces of the NVFP4 kernel (the next piece's first row
// goes out at the end of a piece, ahead of the barrier and the restaging).
template <int M, int IT, int NMAT, int IN, int W, int P, int p>
__device__ __forceinline__ void fp8_pieces(const Fp8Params &fp, u32x4_t *act, float (&acc)[kPieceMaxRows][NMAT][M],
                                           int g, int G, const RowGeom &rg, Fp8PieceRow<IT, NMAT, P, p> &w)
{
    constexpr int IP = (IT + P - 1) / P;
    constexpr int I0 = p * IP;
    constexpr int IS = piece_steps<IT, P, p>();
    constexpr bool kNt = NMAT == 2;
    if constexpr (p > 0)
        lds_barrier();
    stage_act<M, IS, IN, W, I0, 2>(act, fp.in0, fp.in1, fp.cols, fp.cpr, [&] {
        if (p == 0 && g < fp.rows)
            fp8_load_row<kNt, IT, NMAT, I0, IS>(w, fp, g, rg);
    });
    lds_barrier();
#pragma unroll
    for (int k = 0; k < kPieceMaxRows; ++k) {
        const int r = g + k * G;
        if (r >= fp.rows)
            break;
        fp8_row_dot<M, IT, NMAT, I0, IS, p == 0>(acc[k], w, act, rg);
        if (k + 1 < kPieceMaxRows && r + G < fp.rows)
            fp8_load_row<kNt, IT, NMAT, I0, IS>(w, fp, r + G, rg);
    }
    if constexpr (p + 1 < P) {
        Fp8PieceRow<IT, NMAT, P, p + 1> wn;
        if (g < fp.rows)
            fp8_load_row<kNt, IT, NMAT, I0 + IP, piece_steps<IT, P, p + 1>()>(wn, fp, g, rg);
        fp8_pieces<M, IT, NMAT, IN, W, P, p + 1>(fp, act, acc, g, G, rg, wn);
    }
}

// The down GEMV issues only the first kFp8FirstSteps steps of its first
// weight row (and the row's block scales) with its activation loads, and the
// rest once the activations have arrived: at the decode shape the 17 KB rows
// of the whole grid would otherwise queue ahead of them (17.8 vs 18.7 us with
// the whole row issued after the activations; with 2 of 17 steps issued
// early the forward measures 44.22 vs 44.57 us at M = 1 and 46.05 vs
// 46.74 us at M = 2). Rows of fewer than kFp8SplitMinSteps steps issue the
// whole row after the activations.
//
// W waves per workgroup; wave g = wave * gridDim.x + blockIdx.x takes rows
// g, g + G, ... (G = all waves of the grid). Dynamic LDS: M * IT * 2 KB, or
// M * ceil(IT / P) * 2 KB with the activations staged in P pieces (each wave
// then holds at most kPieceMaxRows rows). The dual GEMV (NMAT = 2) issues its
// first weight row before staging and streams codes non-temporally; the down
// GEMV stages first (with the activation fused into the staging when its
// input is gate and up) and uses cached loads, as the NVFP4 kernels do.
constexpr int kFp8FirstSteps = 2;
constexpr int kFp8SplitMinSteps = 6;

template <int M, int IT, int NMAT, int IN, int OUT, int W, int P = 1>
__global__ __launch_bounds__(64 * W) void fp8_gemv_kernel(const Fp8Params p)
{
    extern __shared__ u32x4_t act[];
    constexpr bool kNt = NMAT == 2;
    constexpr bool kWeightsFirst = NMAT == 2;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = gridDim.x * W;
    const int g = wave * static_cast<int>(gridDim.x) + static_cast<int>(blockIdx.x);
    const RowGeom rg = row_geom<IT>(p.cpr);
    if constexpr (P > 1) {
        float acc[kPieceMaxRows][NMAT][M];
        Fp8PieceRow<IT, NMAT, P, 0> w0;
        fp8_pieces<M, IT, NMAT, IN, W, P, 0>(p, act, acc, g, G, rg, w0);
#pragma unroll
        for (int k = 0; k < kPieceMaxRows; ++k) {
            const int r = g + k * G;
            if (r >= p.rows)
                break;
            row_store<M, NMAT, OUT>(acc[k], r, p.rows, 1.0f, 1.0f, p.out0, p.out1, rg.lane);
        }
        return;
    }
    Fp8Row<IT, NMAT, fp8_scale_regs<0, IT>()> w;
    if (kWeightsFirst && g < p.rows)
        fp8_load_row<kNt, IT, NMAT>(w, p, g, rg);
    if constexpr (kWeightsFirst || IT < kFp8SplitMinSteps) {
        stage_act<M, IT, IN, W, 0, 2, !kWeightsFirst>(act, p.in0, p.in1, p.cols, p.cpr, [&] {
            if (!kWeightsFirst && g < p.rows)
                fp8_load_row<kNt, IT, NMAT>(w, p, g, rg);
        });
        lds_barrier();
    } else {
        stage_act<M, IT, IN, W, 0, 2, false>(act, p.in0, p.in1, p.cols, p.cpr, [&] {
            if (g < p.rows)
                fp8_load_steps<kNt, IT, NMAT, 0, kFp8FirstSteps, true>(w, p, g, rg);
        });
        lds_barrier();
        if (g < p.rows)
            fp8_load_steps<kNt, IT, NMAT, kFp8FirstSteps, IT, false>(w, p, g, rg);
    }
    for (int r = g; r < p.rows; r += G) {
        float acc[NMAT][M];
        fp8_row_dot<M, IT, NMAT>(acc, w, act, rg);
        if (r + G < p.rows)
            fp8_load_row<kNt, IT, NMAT>(w, p, r + G, rg);
        row_store<M, NMAT, OUT>(acc, r, p.rows, 1.0f, 1.0f, p.out0, p.out1, rg.lane);
    }
}

// ------------------------------------------------------------------ launch
// (host side; included by the FP8 launch sources)

constexpr int kFp8MaxIt = 24;            // chunks per lane: reduction length up to 24576
constexpr int kFp8LdsMax = 144 * 1024;   // of the 160 KB per compute unit

// Pieces the steps of a row are processed in: the fewest whose activations
// (M x ceil(IT / P) x 2 KB) fit the LDS budget and whose code registers
// (4 per step and matrix) stay within 160, so that long rows of the dual
// GEMV do not spill.
template <int M, int IT, int NMAT>
constexpr int fp8_pieces_count()
{
    int pc = 1;
    while (M * ((IT + pc - 1) / pc) * 2048 > kFp8LdsMax || NMAT * ((IT + pc - 1) / pc) * 4 > 160)
        ++pc;
    return pc;
}

template <int M, int IT, int NMAT>
constexpr int fp8_piece_steps()
{
    return (IT + fp8_pieces_count<M, IT, NMAT>() - 1) / fp8_pieces_count<M, IT, NMAT>();
}

// Waves per workgroup: 16 (at most 128 registers per lane) while one row's
// weight registers (4 per step and matrix, plus the scale registers), the
// converted chunk (8 per matrix) and the accumulators fit with room to
// spare, otherwise 8.
template <int M, int IT, int NMAT>
constexpr int fp8_w_regs()
{
    constexpr int IS = fp8_piece_steps<M, IT, NMAT>();
    constexpr int acc = (fp8_pieces_count<M, IT, NMAT>() > 1 ? kPieceMaxRows : 1) * M * NMAT;
    return (NMAT * (IS * 4 + (IS + 7) / 8 + 1) + NMAT * 8 + acc + 30 <= 120) ? 16 : 8;
}

// The dual GEMV as 2 x 8 waves per compute unit while two workgroups'
// activations fit in LDS (as for NVFP4), else by registers.
template <int M, int IT, int NMAT>
constexpr int fp8_w()
{
    return (NMAT == 2 && fp8_pieces_count<M, IT, NMAT>() == 1 && 2 * M * IT * 2048 <= kFp8LdsMax)
               ? 8
               : fp8_w_regs<M, IT, NMAT>();
}

template <int M, int IT, int NMAT>
constexpr int fp8_blocks_per_cu()
{
    return (fp8_w<M, IT, NMAT>() == 8 && 2 * M * fp8_piece_steps<M, IT, NMAT>() * 2048 <= kFp8LdsMax) ? 2 : 1;
}

template <int M, int IT, int NMAT, int IN, int OUT>
hipError_t fp8_launch_one(const Fp8Params &p, hipStream_t stream)
{
    constexpr int W = fp8_w<M, IT, NMAT>();
    constexpr int P = fp8_pieces_count<M, IT, NMAT>();
    auto kern = fp8_gemv_kernel<M, IT, NMAT, IN, OUT, W, P>;
    const int lds = M * fp8_piece_steps<M, IT, NMAT>() * 2048;
    if (lds > 64 * 1024) {
        static std::atomic<uint64_t> lds_done{0};
        hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), lds, lds_done);
        if (e != hipSuccess)
            return e;
    }
    const int want = device_cu_count() * fp8_blocks_per_cu<M, IT, NMAT>();
    int blocks = want < (p.rows + W - 1) / W ? want : (p.rows + W - 1) / W;
    if (blocks < 1)
        blocks = 1;
    if constexpr (P > 1) {
        const int rows_per_block = W * kPieceMaxRows;
        const int need = (p.rows + rows_per_block - 1) / rows_per_block;
        if (blocks < need)
            blocks = need;
    }
    Fp8Params q = p;
    void *args[] = {&q};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), dim3(blocks), dim3(W * 64), args, lds, stream);
}

template <int IT, int NMAT, int IN, int OUT>
hipError_t fp8_launch_m(int M, const Fp8Params &p, hipStream_t stream)
{
    switch (M) {
    case 1: return fp8_launch_one<1, IT, NMAT, IN, OUT>(p, stream);
    case 2: return fp8_launch_one<2, IT, NMAT, IN, OUT>(p, stream);
    case 3: return fp8_launch_one<3, IT, NMAT, IN, OUT>(p, stream);
    case 4: return fp8_launch_one<4, IT, NMAT, IN, OUT>(p, stream);
    case 5: return fp8_launch_one<5, IT, NMAT, IN, OUT>(p, stream);
    case 6: return fp8_launch_one<6, IT, NMAT, IN, OUT>(p, stream);
    case 7: return fp8_launch_one<7, IT, NMAT, IN, OUT>(p, stream);
    case 8: return fp8_launch_one<8, IT, NMAT, IN, OUT>(p, stream);
    default: return hipErrorNotSupported;
    }
}

// One launch for the whole batch (1 <= M <= 8): every weight byte is read
// once for all M activation rows.
template <int NMAT, int IN, int OUT>
hipError_t fp8_launch_batch(int M, const Fp8Params &p, hipStream_t stream)
{
    const int it = (p.cpr + 63) / 64;
    if (M < 1 || M > 8 || it < 1 || it > kFp8MaxIt)
        return hipErrorNotSupported;
    switch (it) {
#define FFN_FP8_CASE(IT_) \
    case IT_: return fp8_launch_m<IT_, NMAT, IN, OUT>(M, p, stream);
    FFN_FP8_CASE(1)
    FFN_FP8_CASE(2)
    FFN_FP8_CASE(3)
    FFN_FP8_CASE(4)
    FFN_FP8_CASE(5)
    FFN_FP8_CASE(6)
    FFN_FP8_CASE(7)
    FFN_FP8_CASE(8)
    FFN_FP8_CASE(9)
    FFN_FP8_CASE(10)
    FFN_FP8_CASE(11)
    FFN_FP8_CASE(12)
    FFN_FP8_CASE(13)
    FFN_FP8_CASE(14)
    FFN_FP8_CASE(15)
    FFN_FP8_CASE(16)
    FFN_FP8_CASE(17)
    FFN_FP8_CASE(18)
    FFN_FP8_CASE(19)
    FFN_FP8_CASE(20)
    FFN_FP8_CASE(21)
    FFN_FP8_CASE(22)
    FFN_FP8_CASE(23)
    FFN_FP8_CASE(24)
#undef FFN_FP8_CASE
    default: return hipErrorNotSupported;
    }
}

// Parameters of a launch over one weight (down) or two (dual).
inline Fp8Params fp8_params(const void *in0, const float *in1, const Fp8WeightArg &w0, const Fp8WeightArg &w1,
                            void *out0, void *out1, int rows, int cols)
{
    Fp8Params p{};
    p.in0 = in0;
    p.in1 = in1;
    p.codes0 = w0.codes;
    p.bs0 = w0.block_scale;
    p.codes1 = w1.codes;
    p.bs1 = w1.block_scale;
    p.out0 = out0;
    p.out1 = out1;
    p.rows = rows;
    p.cols = cols;
    p.cpr = cols / 16;
    p.bcols = (cols + 127) / 128;
    return p;
}

// The instantiations are spread over translation units that compile in
// parallel: fp8_dual.hip (fp32 gate and up), fp8_dual_silu.hip and
// fp8_dual_gelu.hip (h in the epilogue), fp8_down.hip (h in bf16),
// fp8_down_silu.hip and fp8_down_gelu.hip (the activation fused into the
// staging).
hipError_t fp8_dual_pair(int M, const Fp8Params &p, hipStream_t stream);
hipError_t fp8_dual_h_silu(int M, const Fp8Params &p, hipStream_t stream);
hipError_t fp8_dual_h_gelu(int M, const Fp8Params &p, hipStream_t stream);
hipError_t fp8_down_h(int M, const Fp8Params &p, hipStream_t stream);
hipError_t fp8_down_act_silu(int M, const Fp8Params &p, hipStream_t stream);
hipError_t fp8_down_act_gelu(int M, const Fp8Params &p, hipStream_t stream);

}  // namespace ffn
