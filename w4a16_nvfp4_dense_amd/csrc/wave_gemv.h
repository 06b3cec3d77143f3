// wave_gemv.h -- many-wave NVFP4 GEMV for decode and verify batches
// (1 <= M <= 8 activation rows in one launch, so every weight byte is read
// once for the whole batch; activations staged in LDS, in pieces of the
// reduction when they do not fit): the dual gate+up GEMV and the down GEMV (dense_ffn.rs page,
// DenseFfnLayer::forward, forward_k2 / forward_k3 / forward_km) for rows of
// 33 chunks (1056 columns) or more.
//
// Why. One wave per SIMD issues a VALU instruction at best every ~7.5 cycles,
// and the FP4 conversions are slow instructions, so a GEMV that keeps one
// wave per SIMD (its activations in registers) spends most of its time
// issuing arithmetic, not streaming. Here a compute unit runs many waves
// (up to 5 per SIMD), each with a small register footprint: a wave takes one
// whole weight row at a time, issues all of that row's loads at once (16
// bytes of codes per lane per 32-column chunk), and the activations sit in
// LDS, staged once per workgroup. The next row's loads go out as soon as a
// row's arithmetic is done. Measured on MI355X at the 5120/17408 decode
// shapes, the dual GEMV beat a one-wave-per-SIMD ring 17.1 to 19.6 us with
// 2 x 8 waves per compute unit, the down GEMV 11.1 to 13.8 us with 16.
//
// The arithmetic per chunk and the reduction are those of the other GEMV
// kernels of the library (lane l owns chunks l, l + 64, ...; 16 FP4 -> bf16
// pair conversions, two 8-term dot2 chains per activation row folded in with
// the E4M3 block scales, a fixed DPP tree over the 64 lanes), so results are
// bit-identical to them.
#pragma once

#include "kernels.h"
#include "nvfp4_device.h"

namespace ffn {

struct WaveParams {
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
    int cpr;  // 32-column chunks per row
};

// Geometry of one weight row as seen by one lane: lane l owns chunks
// l, l + 64, ..., l + 64 (IT - 1); only the last step can run past the row end
// (64 (IT - 1) < cpr <= 64 IT), where the lane re-reads the row's last chunk
// and its result is dropped.
struct RowGeom {
    int lane;
    int clast;    // chunk the lane reads in the last step
    bool oklast;  // whether that chunk is really the lane's
    size_t row_codes, row_scales;
};

template <int IT>
__device__ __forceinline__ RowGeom row_geom(int cpr)
{
    RowGeom rg;
    rg.lane = threadIdx.x & 63;
    rg.clast = min(rg.lane + 64 * (IT - 1), cpr - 1);
    rg.oklast = rg.lane + 64 * (IT - 1) < cpr;
    rg.row_codes = static_cast<size_t>(cpr) * 16;
    rg.row_scales = static_cast<size_t>(cpr) * 2;
    return rg;
}

// Bytes 0 and 1 of `word` as OCP E4M3FN values (a chunk's two block scales),
// in one conversion. Exact in fp32.
__device__ __forceinline__ f32x2_t e4m3x2_to_f32x2(uint32_t word)
{
    return __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(word), false);
}

// One row of NMAT weights in registers: 16 bytes of codes and 2 bytes of
// scales per lane and step.
template <int IT, int NMAT>
struct WaveRow {
    u32x4_t wc[NMAT][IT];
    uint32_t ws[NMAT][IT];
};

// Issues all loads of steps I0 .. I0 + IS - 1 of row r (a row has IT steps;
// the whole row by default); NT marks them non-temporal.
template <bool NT, int IT, int NMAT, int I0 = 0, int IS = IT>
__device__ __forceinline__ void load_row(WaveRow<IS, NMAT> &w, const uint8_t *codes0, const uint8_t *scales0,
                                         const uint8_t *codes1, const uint8_t *scales1, int r, const RowGeom &rg)
{
    static_assert(I0 >= 0 && IS >= 1 && I0 + IS <= IT, "piece of the row");
#pragma unroll
    for (int t = 0; t < NMAT; ++t) {
        const u32x4_t *cb =
            reinterpret_cast<const u32x4_t *>((t == 0 ? codes0 : codes1) + static_cast<size_t>(r) * rg.row_codes);
        const uint16_t *sb =
            reinterpret_cast<const uint16_t *>((t == 0 ? scales0 : scales1) + static_cast<size_t>(r) * rg.row_scales);
#pragma unroll
        for (int j = 0; j < IS; ++j) {
            const int i = I0 + j;
            const int c = (i == IT - 1) ? rg.clast : rg.lane + 64 * i;
            if constexpr (NT) {
                w.wc[t][j] = __builtin_nontemporal_load(cb + c);
                w.ws[t][j] = __builtin_nontemporal_load(sb + c);
            } else {
                w.wc[t][j] = cb[c];
                w.ws[t][j] = sb[c];
            }
        }
    }
}

// Issues the loads of steps A .. B - 1 of row r into a whole row's registers.
template <bool NT, int IT, int NMAT, int A, int B>
__device__ __forceinline__ void load_steps(WaveRow<IT, NMAT> &w, const uint8_t *codes0, const uint8_t *scales0,
                                           const uint8_t *codes1, const uint8_t *scales1, int r, const RowGeom &rg)
{
#pragma unroll
    for (int t = 0; t < NMAT; ++t) {
        const u32x4_t *cb =
            reinterpret_cast<const u32x4_t *>((t == 0 ? codes0 : codes1) + static_cast<size_t>(r) * rg.row_codes);
        const uint16_t *sb =
            reinterpret_cast<const uint16_t *>((t == 0 ? scales0 : scales1) + static_cast<size_t>(r) * rg.row_scales);
#pragma unroll
        for (int i = A; i < B; ++i) {
            const int c = (i == IT - 1) ? rg.clast : rg.lane + 64 * i;
            if constexpr (NT) {
                w.wc[t][i] = __builtin_nontemporal_load(cb + c);
                w.ws[t][i] = __builtin_nontemporal_load(sb + c);
            } else {
                w.wc[t][i] = cb[c];
                w.ws[t][i] = sb[c];
            }
        }
    }
}

// Steps of the first weight row that a down-GEMV wave issues together with
// its activation loads; the rest go out once the activations have landed, so
// that they do not wait behind the whole grid's first rows. Measured on
// MI355X against issuing the whole row first (forward, median of 12 x 1000):
// 9-step rows (N = 17408) 28.88 -> 28.10 us at M = 1 and 34.79 -> 33.55 us
// at M = 2 with 5 steps (6 or 7 gain less, or lose at M = 2); 11-step rows
// (N = 21504) 36.49 -> 35.64 us with 1 step (5 or 6 steps gain 0.4 us).
template <int IT>
constexpr int first_row_split()
{
    return IT >= 10 ? 1 : (IT >= 6 ? (IT + 1) / 2 : IT);
}

// Stages the columns of steps I0 .. I0 + IS - 1 of M activation rows of
// `cols` (= 8 CQ cpr) columns into LDS as 16-byte units
// ((m * IS + j) * CQ + q) * 64 + l: unit q of the chunk lane l reads in step
// I0 + j (chunk l + 64 (I0 + j); zero past the row end), so every read is
// conflict-free and its address is the lane's offset plus a constant. A chunk
// is CQ = 4 units (32 columns: 16 bytes of FP4 codes) or CQ = 2 (16 columns:
// 16 bytes of FP8 codes). Uses M * IS * CQ KB. The W waves of the workgroup load in batches of SU units per
// thread; `issue()` runs right after the last batch's global loads (the
// first weight row goes out there: waiting for the activations then does not
// wait for the weights, as loads complete in order, and the weight registers
// are not live while earlier batches are in flight). With LATE, `issue()`
// runs after the last batch's LDS stores instead, i.e. once the activations
// have arrived, so that they are not queued behind the weight rows of the
// whole grid (measured faster for the FP8 down GEMV's 17 KB rows, slightly
// slower for the NVFP4 one). The caller synchronises the workgroup before
// reading.
template <int M, int IS, int IN, int W, int I0 = 0, int CQ = 4, bool LATE = false, class F>
__device__ __forceinline__ void stage_act(u32x4_t *act, const void *in0, const float *in1, int cols, int cpr,
                                          F &&issue)
{
    static_assert(CQ == 2 || CQ == 4, "16-byte units per chunk");
    constexpr int kQs = CQ == 4 ? 2 : 1;  // log2 CQ
    constexpr int IT = IS;  // steps staged
    constexpr int total = M * IT * 64 * CQ;
    constexpr int nthr = 64 * W;
    constexpr int need = (total + nthr - 1) / nthr;
    constexpr int SU = (IN == IN_BF16) ? (need < 8 ? need : 8) : 2;
    constexpr int nbatch = (total + SU * nthr - 1) / (SU * nthr);
#pragma unroll
    for (int bi = 0; bi < nbatch; ++bi) {
        const int base = bi * SU * nthr;
        u32x4_t v[SU];
#pragma unroll
        for (int k = 0; k < SU; ++k) {
            // global piece u: row m, chunk c, quarter q (q fastest)
            const int u = base + k * nthr + static_cast<int>(threadIdx.x);
            const int m = min(u / (IT * 64 * CQ), M - 1);
            const int rem = u - m * IT * 64 * CQ;
            const int c = min(64 * I0 + (rem >> kQs), cpr - 1);
            const size_t off = static_cast<size_t>(m) * cols + static_cast<size_t>(c) * (8 * CQ) + (rem & (CQ - 1)) * 8;
            if constexpr (IN == IN_BF16) {
                v[k] = *reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(in0) + off);
            } else {
                constexpr int A = (IN == IN_GATEUP_SILU) ? ACT_SILU : ACT_GELU_TANH;
                const f32x4_t *gp = reinterpret_cast<const f32x4_t *>(static_cast<const float *>(in0) + off);
                const f32x4_t *up = reinterpret_cast<const f32x4_t *>(in1 + off);
                const f32x4_t g0 = gp[0], g1 = gp[1], u0 = up[0], u1 = up[1];
                v[k][0] = pack_bf16x2(gate_act<A>(g0[0]) * u0[0], gate_act<A>(g0[1]) * u0[1]);
                v[k][1] = pack_bf16x2(gate_act<A>(g0[2]) * u0[2], gate_act<A>(g0[3]) * u0[3]);
                v[k][2] = pack_bf16x2(gate_act<A>(g1[0]) * u1[0], gate_act<A>(g1[1]) * u1[1]);
                v[k][3] = pack_bf16x2(gate_act<A>(g1[2]) * u1[2], gate_act<A>(g1[3]) * u1[3]);
            }
        }
        if (!LATE && bi == nbatch - 1)
            issue();
#pragma unroll
        for (int k = 0; k < SU; ++k) {
            const int u = base + k * nthr + static_cast<int>(threadIdx.x);
            if (u < total) {
                const int m = u / (IT * 64 * CQ);
                const int rem = u - m * IT * 64 * CQ;
                const int c = rem >> kQs;  // chunk l + 64 (I0 + j), c = 64 j + l
                act[((m * IT + (c >> 6)) * CQ + (rem & (CQ - 1))) * 64 + (c & 63)] =
                    64 * I0 + c < cpr ? v[k] : u32x4_t{0, 0, 0, 0};
            }
        }
        if (LATE && bi == nbatch - 1)
            issue();
    }
}

// Per-lane partial sums of one row: acc[t][m] = sum over the lane's chunks of
// (two 8-term dot2 chains of 16 columns each) times their E4M3 block scales,
// over steps I0 .. I0 + IS - 1 of the row's IT steps (activations staged for
// those steps), starting from zero (INIT) or adding to acc.
template <int M, int IT, int NMAT, int I0 = 0, int IS = IT, bool INIT = true>
__device__ __forceinline__ void row_dot(float (&acc)[NMAT][M], const WaveRow<IS, NMAT> &w, const u32x4_t *act,
                                        const RowGeom &rg)
{
    // The activation reads are the same for every row; an opaque zero keeps
    // them inside the row loop (hoisted, they would pin M * IT * 16 registers
    // for the whole kernel).
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
        const int i = I0 + j;  // step of the row
        // this chunk's weights of every matrix as bf16 pairs, and scales
        bf16x2_t wp[NMAT][16];
        float s0[NMAT], s1[NMAT];
#pragma unroll
        for (int t = 0; t < NMAT; ++t) {
            const u32x4_t c = w.wc[t][j];
            // past the row end: zero activations, and a zero scale so that a
            // NaN scale of the re-read chunk cannot leak in
            const uint32_t sw = (i < IT - 1 || rg.oklast) ? w.ws[t][j] : 0u;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                wp[t][4 * q + 0] = fp4x2_to_bf16x2<0>(c[q]);
                wp[t][4 * q + 1] = fp4x2_to_bf16x2<1>(c[q]);
                wp[t][4 * q + 2] = fp4x2_to_bf16x2<2>(c[q]);
                wp[t][4 * q + 3] = fp4x2_to_bf16x2<3>(c[q]);
            }
            const f32x2_t sp = e4m3x2_to_f32x2(sw);  // one conversion for both blocks
            s0[t] = sp[0];
            s1[t] = sp[1];
        }
        // Activation row m + 1 is read from LDS while row m's products run
        // (two rows of registers at most).
        u32x4_t an[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            an[q] = ar[(j * 4 + q) * 64];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            u32x4_t a[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                a[q] = an[q];
            if (m + 1 < M) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    an[q] = ar[(((m + 1) * IS + j) * 4 + q) * 64];
            }
#pragma unroll
            for (int t = 0; t < NMAT; ++t) {
                float t0 = dot2_bf16_first(wp[t][0], as_bf16x2(a[0][0]));
                float t1 = dot2_bf16_first(wp[t][8], as_bf16x2(a[2][0]));
#pragma unroll
                for (int b = 1; b < 4; ++b) {
                    t0 = dot2_bf16(wp[t][b], as_bf16x2(a[0][b]), t0);
                    t1 = dot2_bf16(wp[t][8 + b], as_bf16x2(a[2][b]), t1);
                }
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    t0 = dot2_bf16(wp[t][4 + b], as_bf16x2(a[1][b]), t0);
                    t1 = dot2_bf16(wp[t][12 + b], as_bf16x2(a[3][b]), t1);
                }
                acc[t][m] = __builtin_fmaf(t0, s0[t], acc[t][m]);
                acc[t][m] = __builtin_fmaf(t1, s1[t], acc[t][m]);
            }
            // One activation row at a time: its accumulators pass through an
            // empty asm that also orders memory, so its arithmetic is done
            // before the activation reads of the row after next (otherwise
            // all of them are issued first and pinned in registers).
#pragma unroll
            for (int t = 0; t < NMAT; ++t)
                asm volatile("" : "+v"(acc[t][m])::"memory");
        }
    }
}

// The wave sums of P values per lane (P = 2, 4 or 8), transposed: at each of
// the first log2 P levels of segment_sum<64>'s tree a lane keeps half of its
// values and adds the partner's copies of them, so P values cost about 3 P
// instructions instead of 8 P. Every sum combines the same lanes in the same
// tree as segment_sum<64> (pairs, quads, mirrored halves of rows, rows, 32
// lanes, 64 lanes; only the operand order of an addition can differ, and
// addition commutes), so the totals are bit-identical to it. Which half a
// lane keeps is chosen from parities of its lane bits that the mirror
// partners of the later levels share. The total returned in a lane is that
// of value wave_sum_index<P>(lane), in every row of the wave.
template <int P>
__device__ __forceinline__ int wave_sum_index(int lane)
{
    const int p = lane & 15;
    const int c1 = (p ^ (p >> 2)) & 1;         // kept half at the pairs level
    const int c2 = ((p >> 1) ^ (p >> 2)) & 1;  // ... at the quads level
    const int c3 = ((p >> 2) ^ (p >> 3)) & 1;  // ... at the half-row level
    if constexpr (P == 2)
        return c1;
    else if constexpr (P == 4)
        return 2 * c1 + c2;
    else
        return 4 * c1 + 2 * c2 + c3;
}

// One level: partner lanes (DPP control CTRL) hold the same N values; the
// lane keeps the upper half when c is set and adds the partner's copy.
template <int N, int CTRL>
__device__ __forceinline__ void wave_sum_split(float *v, bool c)
{
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
        const float keep = c ? v[j + N / 2] : v[j];
        const float send = c ? v[j] : v[j + N / 2];
        v[j] = keep + dpp_move<CTRL>(send);
    }
}

template <int P>
__device__ __forceinline__ float wave_sums(float (&v)[P], int lane)
{
    static_assert(P == 2 || P == 4 || P == 8, "values per lane");
    const int p = lane & 15;
    wave_sum_split<P, 0xB1>(v, ((p ^ (p >> 2)) & 1) != 0);  // quad_perm [1,0,3,2]: pairs
    if constexpr (P >= 4)
        wave_sum_split<P / 2, 0x4E>(v, (((p >> 1) ^ (p >> 2)) & 1) != 0);  // quad_perm [2,3,0,1]: quads
    else
        v[0] += dpp_move<0x4E>(v[0]);
    if constexpr (P >= 8)
        wave_sum_split<2, 0x141>(v, (((p >> 2) ^ (p >> 3)) & 1) != 0);  // row_half_mirror: 8 lanes
    else
        v[0] += dpp_move<0x141>(v[0]);
    float t = v[0];
    t += dpp_move<0x140>(t);  // row_mirror: 16 lanes
    t += __shfl_xor(t, 16);   // rows 0 + 1, rows 2 + 3
    t += __shfl_xor(t, 32);   // all four rows
    return t;
}

// Sums the lanes' partials of row r over the wave (the fixed tree of
// segment_sum<64>) and writes the row's outputs for the M activation rows
// (outputs [M, rows]): from lane 63 for one row, else from lanes 0 .. M - 1
// (lane l holds activation row wave_sum_index(l)).
template <int M, int NMAT, int OUT>
__device__ __forceinline__ void row_store(float (&acc)[NMAT][M], int r, int rows, float s2_0, float s2_1, void *out0,
                                          void *out1, int lane)
{
    constexpr int P = M == 1 ? 1 : M == 2 ? 2 : M <= 4 ? 4 : 8;
    static_assert(M <= 8, "activation rows");
    float tot[NMAT];
    int m = 0;
    bool mine;
    if constexpr (P == 1) {
#pragma unroll
        for (int t = 0; t < NMAT; ++t)
            tot[t] = segment_sum<64>(acc[t][0]);
        mine = lane == 63;
    } else {
#pragma unroll
        for (int t = 0; t < NMAT; ++t) {
            float v[P];
#pragma unroll
            for (int i = 0; i < P; ++i)
                v[i] = i < M ? acc[t][i < M ? i : 0] : 0.0f;
            tot[t] = wave_sums<P>(v, lane);
        }
        m = wave_sum_index<P>(lane);
        mine = lane < P && m < M;
    }
    if (mine) {
        const size_t o = static_cast<size_t>(m) * rows + r;
        if constexpr (OUT == OUT_F32_PAIR) {
            static_cast<float *>(out0)[o] = s2_0 * tot[0];
            static_cast<float *>(out1)[o] = s2_1 * tot[NMAT - 1];
        } else if constexpr (OUT == OUT_BF16) {
            static_cast<uint16_t *>(out0)[o] = to_bf16_bits(s2_0 * tot[0]);
        } else {
            constexpr int A = (OUT == OUT_H_SILU) ? ACT_SILU : ACT_GELU_TANH;
            const float h = gate_act<A>(s2_0 * tot[0]) * (s2_1 * tot[NMAT - 1]);
            static_cast<uint16_t *>(out0)[o] = to_bf16_bits(h);
        }
    }
}

// Rows a wave holds accumulators for when the activations are staged in
// pieces (the launcher sizes the grid so that no wave has more).
constexpr int kPieceMaxRows = 2;

// Steps of piece p of an IT-step row cut into P pieces.
template <int IT, int P, int p>
constexpr int piece_steps()
{
    constexpr int IP = (IT + P - 1) / P;
    return (IT - p * IP < IP) ? IT - p * IP : IP;
}

// One piece of the staged kernel (steps I0 .. I0 + IS - 1 of every row), then
// the next: the workgroup stages the piece's activations (for the first piece
// the first row's weights go out behind them; for later pieces they went out
// at the end of the previous piece), and each wave adds the piece's products
// of its rows g, g + G to their accumulators. A barrier before each
// restaging keeps the previous piece in LDS until every wave is done with it.
// (Issuing the next piece's first row at the end of a piece rather than after
// the restaging: 54.63 -> 53.75 us at M = 5, 71.51 -> 70.60 us at M = 8,
// bit-identical.)
template <int M, int IT, int NMAT, int IN, int W, int P, int p>
__device__ __forceinline__ void wave_pieces(const WaveParams &wp, u32x4_t *act, float (&acc)[kPieceMaxRows][NMAT][M],
                                            int g, int G, const RowGeom &rg,
                                            WaveRow<piece_steps<IT, P, p>(), NMAT> &w)
{
    constexpr int IP = (IT + P - 1) / P;
    constexpr int I0 = p * IP;
    constexpr int IS = piece_steps<IT, P, p>();
    constexpr bool kNt = NMAT == 2;
    if constexpr (p > 0)
        lds_barrier();
    stage_act<M, IS, IN, W, I0>(act, wp.in0, wp.in1, wp.cols, wp.cpr, [&] {
        if (p == 0 && g < wp.rows)
            load_row<kNt, IT, NMAT, I0, IS>(w, wp.codes0, wp.scales0, wp.codes1, wp.scales1, g, rg);
    });
    lds_barrier();
#pragma unroll
    for (int k = 0; k < kPieceMaxRows; ++k) {
        const int r = g + k * G;
        if (r >= wp.rows)
            break;
        row_dot<M, IT, NMAT, I0, IS, p == 0>(acc[k], w, act, rg);
        if (k + 1 < kPieceMaxRows && r + G < wp.rows)
            load_row<kNt, IT, NMAT, I0, IS>(w, wp.codes0, wp.scales0, wp.codes1, wp.scales1, r + G, rg);
    }
    if constexpr (p + 1 < P) {
        // the next piece's first row goes out now, ahead of the barrier and
        // the next activation staging
        constexpr int ISn = piece_steps<IT, P, p + 1>();
        WaveRow<ISn, NMAT> wn;
        if (g < wp.rows)
            load_row<kNt, IT, NMAT, I0 + IP, ISn>(wn, wp.codes0, wp.scales0, wp.codes1, wp.scales1, g, rg);
        wave_pieces<M, IT, NMAT, IN, W, P, p + 1>(wp, act, acc, g, G, rg, wn);
    }
}

// W waves per workgroup; each wave takes rows g, g + G, ... (G = all waves of
// the grid), with g = wave * gridDim.x + blockIdx.x: when the rows do not
// divide evenly, the waves that get one more row are the low waves of every
// workgroup, one per SIMD, so every compute unit and SIMD gets the same
// share. Each wave issues its next row's loads as soon as a row's arithmetic
// is done; a down-GEMV wave issues only the first first_row_split<IT>() steps
// of its first row with its activation loads, and the rest once they have
// landed. Dynamic LDS: M * IT * 4 KB.
//
// When that exceeds the LDS budget (long rows and up to 8 activation rows:
// the down GEMV of a verify batch), the activations are staged in P pieces of
// steps instead (M * ceil(IT / P) * 4 KB), every weight row is still read once
// for all M rows, and each wave keeps its rows' accumulators across pieces
// (at most kPieceMaxRows rows per wave). A lane still visits its chunks in
// increasing order, so the results are those of the one-piece kernel.
//
// Measured on MI355X at the decode shapes (each change alone, same run):
// issuing the first weight row before the activation loads and meeting at an
// LDS-only barrier takes the dual GEMV from 18.4 to 17.2 us; plain (cached)
// weight loads take the down GEMV from 11.4 to 10.75 us, while they slow the
// dual GEMV (19.2 us), which keeps non-temporal loads; reading the next
// activation row from LDS while the current one's products run takes the
// dual GEMV from 19.3 to 18.6 us at M = 1 and from 50.5 to 48.8 us at M = 8;
// converting a chunk's two E4M3 scales with one packed conversion instead of
// two takes it from 18.63 to 18.39 us (and the GELU-tanh shape's from 23.22
// to 22.98 us).
template <int M, int IT, int NMAT, int IN, int OUT, int W, int P = 1>
__global__ __launch_bounds__(64 * W) void wave_gemv_kernel(const WaveParams p)
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
        WaveRow<piece_steps<IT, P, 0>(), NMAT> w0;
        wave_pieces<M, IT, NMAT, IN, W, P, 0>(p, act, acc, g, G, rg, w0);
#pragma unroll
        for (int k = 0; k < kPieceMaxRows; ++k) {
            const int r = g + k * G;
            if (r >= p.rows)
                break;
            row_store<M, NMAT, OUT>(acc[k], r, p.rows, p.s2_0, p.s2_1, p.out0, p.out1, rg.lane);
        }
        return;
    }
    WaveRow<IT, NMAT> w;
    if (kWeightsFirst && g < p.rows)
        load_row<kNt, IT, NMAT>(w, p.codes0, p.scales0, p.codes1, p.scales1, g, rg);
    constexpr int kSplit = kWeightsFirst ? IT : first_row_split<IT>();
    stage_act<M, IT, IN, W>(act, p.in0, p.in1, p.cols, p.cpr, [&] {
        if (!kWeightsFirst && g < p.rows)
            load_steps<kNt, IT, NMAT, 0, kSplit>(w, p.codes0, p.scales0, p.codes1, p.scales1, g, rg);
    });
    lds_barrier();
    if constexpr (kSplit < IT) {
        if (g < p.rows)
            load_steps<kNt, IT, NMAT, kSplit, IT>(w, p.codes0, p.scales0, p.codes1, p.scales1, g, rg);
    }
    for (int r = g; r < p.rows; r += G) {
        float acc[NMAT][M];
        row_dot<M, IT, NMAT>(acc, w, act, rg);
        // the next row's loads go out before this row's reduction and store
        if (r + G < p.rows)
            load_row<kNt, IT, NMAT>(w, p.codes0, p.scales0, p.codes1, p.scales1, r + G, rg);
        row_store<M, NMAT, OUT>(acc, r, p.rows, p.s2_0, p.s2_1, p.out0, p.out1, rg.lane);
    }
}

}  // namespace ffn
