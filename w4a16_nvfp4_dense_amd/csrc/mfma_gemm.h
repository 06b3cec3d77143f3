// mfma_gemm.h -- the prefill arm of the NVFP4 gated FFN (dense_ffn.rs page,
// DenseFfnLayer::forward_prefill / forward_prefill_inner): the two projections
// and the down projection as GEMMs over up to 128 token rows, on bf16 matrix
// cores (v_mfma_f32_32x32x16_bf16) with the weights dequantised on the fly.
//
// Product. For a weight W [rows, cols] (NVFP4) and an activation block
// A [M, cols] (bf16, M <= 32 * MT), every wave computes
//     D[m, r] = sum_c A[m, c] * W[r, c]
// for all M token rows and 32 (two projections) or 64 (one projection) weight
// rows. The activation fragment is the MFMA's A operand (rows = tokens), the
// dequantised weight fragment its B operand (columns = weight rows), so a
// lane's accumulators cover 16 tokens of one weight row and output rows are
// written 32 consecutive elements at a time.
//
// Dequantisation. Each weight element is dequantised exactly once per launch,
// in registers, by the one wave that owns its row: FP4 pair -> fp32 pair
// (v_cvt_scalef32_pk_f32_fp4 with unit scale), times the E4M3 block scale,
// rounded to bf16. E2M1 x E4M3 has at most 6 significant bits, so the bf16
// weight is exact and the only rounding in the product is the fp32
// accumulation inside the matrix core. scale2 multiplies in the epilogue.
//
// K order. The reduction runs over units of 64 columns. In a unit, lane half
// h (lane / 32) of a wave holds columns [32 h, 32 h + 32) of its row (16 code
// bytes), and MFMA step s (of 4) takes columns 32 h + 8 s .. + 7 from each
// half; the activation fragment is read with the same column map.
//
// Data movement. Per unit, a workgroup (4 waves, one per SIMD) stages into
// one LDS ring stage: the activation block [32 MT rows, 64 cols] bf16, with
// its 16-byte pieces XOR-swizzled by row pair (conflict-free ds_read_b128 of
// 32 rows at one column), and each wave's raw codes (1 KB per 32 rows) and
// scales. All of it moves with gfx950 direct global->LDS loads (no
// registers), S - 1 units ahead of the math. The loads complete in order on
// the vector memory counter, which the compiler does not tie to the LDS they
// fill: each iteration waits explicitly for its unit and then meets the other
// waves at a barrier, after which the stage of the previous unit is free.
//
// Work split (stream-K). The reduction of every 128- (or 256-) row tile is cut
// into units; the T x KU units of the launch are dealt out to the G
// workgroups as G contiguous, equal ranges (workgroup g takes
// [floor(g U / G), floor((g + 1) U / G))), so all compute units finish
// together whatever the tile count. A workgroup that holds a whole tile runs
// the epilogue itself; the pieces of a tile split between workgroups go to
// fp32 slots of the workspace. With G = T every workgroup owns exactly one
// whole tile and no slot is touched. Split tiles are finished in one of two
// ways:
//  - the down GEMM (a tile shared by ~13 workgroups at 128 tokens): by
//    mfma_reduce_kernel, launched next, which adds the pieces in k order and
//    runs the same epilogue;
//  - the dual GEMM (a tile shared by 2-3 workgroups; FIX): inside the launch.
//    Each workgroup walks its range downwards, so a lower workgroup reaches
//    its piece of a shared tile (the top of its range) first and the highest
//    one (whose range starts inside the tile) reaches it last. The lower ones
//    store their pieces with device-coherent 16-byte stores (sc1: written
//    through to memory, past the XCD's L2) and then set one ready word per
//    wave to the launch's tag; the highest waits for those words, reads the
//    pieces with device-coherent loads, adds them nearest first and runs the
//    epilogue. A workgroup only ever waits for lower-numbered ones, which
//    were dispatched first and wait only for lower ones still, so the waits
//    end even when not all workgroups are resident at once. No fence is
//    used: a release fence writes back the XCD's whole L2, which holds the
//    activation block.
#pragma once

#include "kernels.h"
#include "nvfp4_device.h"

namespace ffn {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kMfmaWaves = 4;
constexpr int kUnitCols = 64;  // reduction columns per unit

struct MfmaParams {
    const void *in0;   // bf16 [M, cols], or fp32 gate [M, cols] (gate/up input)
    const float *in1;  // fp32 up [M, cols] (gate/up input)
    const uint8_t *codes0;
    const uint8_t *scales0;
    const uint8_t *codes1;
    const uint8_t *scales1;
    float s2_0;
    float s2_1;
    void *out0;
    void *out1;
    float *partials;   // 2 G slots of partial tiles (stream-K only)
    unsigned long long *flags;  // 4 ready words per slot (in-kernel finishing only)
    unsigned long long tag;     // this launch's ready value (nonzero)
    int M;             // token rows, 1 <= M <= 32 * MT
    int rows;          // weight rows (output columns)
    int cols;          // reduction length, a multiple of 64
    int tiles;         // T
    int units_per_tile;  // KU = cols / 64
    int units;           // U = T * KU
};

template <int MT>
constexpr int mfma_stage_bytes()
{
    return MT * 4096 + 8192 + 1024;  // activations, codes (4 waves x 2 x 1 KB), scales (4 x 256 B)
}

// Weight rows per wave / per workgroup tile: two projections share 32 rows,
// one projection takes 64 rows as two 32-row fragments.
template <int NMAT>
constexpr int mfma_rows_per_tile()
{
    return kMfmaWaves * (NMAT == 2 ? 32 : 64);
}

// Floats of one partial slot: 4 waves x 2 x MT accumulator tiles x 16 x 64.
// Within a wave's part, accumulator values q = 4 q4 .. 4 q4 + 3 of tile
// (f, mt) of lane l are 16 contiguous bytes at float
// (((f MT + mt) 4 + q4) 64 + l) 4, so a piece is written and read with
// 16-byte accesses.
template <int MT>
constexpr int mfma_slot_floats()
{
    return kMfmaWaves * 2 * MT * 16 * 64;
}

// First unit of workgroup g, and the workgroup that owns unit u.
__host__ __device__ inline int sk_begin(long long g, long long U, long long G)
{
    return static_cast<int>(g * U / G);
}
__host__ __device__ inline int sk_owner(long long u, long long U, long long G)
{
    // the largest g with floor(g U / G) <= u
    return static_cast<int>(((u + 1) * G + U - 1) / U) - 1;
}

// Wait until at most `ahead` units (of L loads each) issued after the one to
// be consumed are outstanding; `ahead` is wave-uniform and in [0, MAXA].
template <int MAXA, int L>
__device__ __forceinline__ void wait_units(int ahead)
{
    static_assert(MAXA >= 0 && MAXA * L < 64, "vmcnt range");
    if constexpr (MAXA == 0) {
        wait_vmcnt<0>();
    } else {
        if (ahead >= MAXA) {
            wait_vmcnt<MAXA * L>();
            return;
        }
        wait_units<MAXA - 1, L>(ahead);
    }
}

// Hides a wave-uniform value from the optimiser, so that what is derived from
// it inside a rarely taken branch is computed there and not hoisted out of the
// main loop (where it would hold registers for the whole kernel).
__device__ __forceinline__ int opaque_uniform(int x)
{
    asm volatile("" : "+s"(x));
    return x;
}

// The same for a per-lane value.
__device__ __forceinline__ int opaque_lane(int x)
{
    asm volatile("" : "+v"(x));
    return x;
}

// Epilogue of one accumulator position. Accumulator (f, mt, v) of lane
// `lane` of wave `wave` holds D[m, row] with m = 32 mt + 8 (v / 4) + 4 (lane /
// 32) + v % 4 and row = row lane % 32 of fragment f. (y0, y1) are fragments 0
// and 1 at (mt, v): gate and up of one row (two projections, written as the
// fp32 pair or as h = bf16(act(s2_0 y0) * (s2_1 y1))), or two rows 32 apart
// (one projection, bf16(s2_0 y)).
template <int NMAT, int OUT, int ROWS_TILE>
__device__ __forceinline__ void emit_pair(const MfmaParams &p, int rows, int M, int t, int wave, int lane, int mt,
                                          int v, float y0, float y1)
{
    const int m = 32 * mt + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    if (m >= M)
        return;
    if constexpr (NMAT == 2) {
        const int row = t * ROWS_TILE + wave * 32 + (lane & 31);
        if (row >= rows)
            return;
        const float gv = y0 * p.s2_0;
        const float uv = y1 * p.s2_1;
        const size_t o = static_cast<size_t>(m) * rows + row;
        if constexpr (OUT == OUT_F32_PAIR) {
            static_cast<float *>(p.out0)[o] = gv;
            static_cast<float *>(p.out1)[o] = uv;
        } else {
            constexpr int A = (OUT == OUT_H_SILU) ? ACT_SILU : ACT_GELU_TANH;
            static_cast<uint16_t *>(p.out0)[o] = to_bf16_bits(gate_act<A>(gv) * uv);
        }
    } else {
        const int row = t * ROWS_TILE + wave * 64 + (lane & 31);
        uint16_t *out = static_cast<uint16_t *>(p.out0) + static_cast<size_t>(m) * rows;
        if (row < rows)
            out[row] = to_bf16_bits(y0 * p.s2_0);
        if (row + 32 < rows)
            out[row + 32] = to_bf16_bits(y1 * p.s2_0);
    }
}

template <int MT, int NMAT, int IN, int OUT, int S, bool FIX = false>
__global__ __launch_bounds__(kMfmaWaves * 64) void mfma_gemm_kernel(const MfmaParams p)
{
    static_assert(MT >= 1 && MT <= 4, "token tiles");
    static_assert(S <= 16, "ring stages");
    constexpr int STAGE = mfma_stage_bytes<MT>();
    constexpr int XB = MT * 4096;                           // activation bytes per stage
    constexpr int L = (IN == IN_BF16 ? MT : 0) + 3;         // direct loads per unit per wave
    static_assert(S >= 3 && (S - 2) * L < 64, "ring stages / vmcnt range");
    constexpr int ROWS_WAVE = NMAT == 2 ? 32 : 64;
    constexpr int ROWS_TILE = kMfmaWaves * ROWS_WAVE;
    constexpr int SLOT = mfma_slot_floats<MT>();

    extern __shared__ u32x4_t lds_raw[];
    FFN_LDS uint8_t *lds = (FFN_LDS uint8_t *)lds_raw;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5;
    const int r = lane & 31;
    const long long U = p.units;
    const long long G = gridDim.x;
    const int g = blockIdx.x;
    const int u_begin = sk_begin(g, U, G);
    const int n = sk_begin(g + 1, U, G) - u_begin;
    const int KU = p.units_per_tile;
    const int cols = p.cols;
    const int M = p.M;
    const size_t row_codes = static_cast<size_t>(cols) / 2;
    const size_t row_scales = static_cast<size_t>(cols) / 16;

    // Weight row of fragment f, row r of this wave, in tile t (clamped: rows
    // past the end load row rows - 1 and are never stored).
    auto wrow = [&](int t, int f, int rr) {
        const int row = t * ROWS_TILE + wave * ROWS_WAVE + (NMAT == 2 ? 0 : f * 32) + rr;
        return min(row, p.rows - 1);
    };

    // The unit of step j: increasing, or with in-kernel finishing (FIX)
    // decreasing, so that of the workgroups sharing a tile the highest one
    // reaches its piece of it last and the lower ones write theirs earlier.
    auto unit_at = [&](int jj) { return FIX ? u_begin + n - 1 - jj : u_begin + jj; };

    // Activation slot P (16 bytes) of a stage holds row P / 8, 16-byte piece
    // (P % 8) ^ ((row / 2) % 8) of the unit. A row is 128 bytes, so even rows
    // start at bank 0 and odd rows at bank 32; swizzling by the row pair makes
    // the 16 rows one read pass serves (a column piece each) cover all 64
    // banks once (by row % 8, rows r and r + 8 of a pass collided: measured
    // 3.2 conflict cycles per LDS instruction).
    auto issue = [&](int v, int st) {
        const int t = v / KU;
        const int k0 = (v - t * KU) * kUnitCols;
        FFN_LDS uint8_t *base = lds + st * STAGE;
        if constexpr (IN == IN_BF16) {
            const uint16_t *X = static_cast<const uint16_t *>(p.in0);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int P = (wave * MT + i) * 64 + lane;
                const int m = P >> 3;
                const int c = (P & 7) ^ ((m >> 1) & 7);
                const int ms = min(m, M - 1);
                __builtin_amdgcn_global_load_lds(
                    reinterpret_cast<const void *>(X + static_cast<size_t>(ms) * cols + k0 + 8 * c),
                    reinterpret_cast<FFN_LDS void *>(base + (wave * MT + i) * 1024), 16, 0, 0);
            }
        } else {
            // h = bf16(act(gate) * up) computed while staging (gate, up fp32).
            constexpr int A = (IN == IN_GATEUP_SILU) ? ACT_SILU : ACT_GELU_TANH;
            const float *Gp = static_cast<const float *>(p.in0);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int P = (wave * MT + i) * 64 + lane;
                const int m = P >> 3;
                const int c = (P & 7) ^ ((m >> 1) & 7);
                const size_t off = static_cast<size_t>(min(m, M - 1)) * cols + k0 + 8 * c;
                const f32x4_t g0 = *reinterpret_cast<const f32x4_t *>(Gp + off);
                const f32x4_t g1 = *reinterpret_cast<const f32x4_t *>(Gp + off + 4);
                const f32x4_t u0 = *reinterpret_cast<const f32x4_t *>(p.in1 + off);
                const f32x4_t u1 = *reinterpret_cast<const f32x4_t *>(p.in1 + off + 4);
                u32x4_t hv;
                hv[0] = pack_bf16x2(gate_act<A>(g0[0]) * u0[0], gate_act<A>(g0[1]) * u0[1]);
                hv[1] = pack_bf16x2(gate_act<A>(g0[2]) * u0[2], gate_act<A>(g0[3]) * u0[3]);
                hv[2] = pack_bf16x2(gate_act<A>(g1[0]) * u1[0], gate_act<A>(g1[1]) * u1[1]);
                hv[3] = pack_bf16x2(gate_act<A>(g1[2]) * u1[2], gate_act<A>(g1[3]) * u1[3]);
                *reinterpret_cast<FFN_LDS u32x4_t *>(base + P * 16) = hv;
            }
        }
        // codes: lane (r, h) -> row r, bytes [16 h, 16 h + 16) of the unit
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const uint8_t *cb = (f == 0 || NMAT == 1) ? p.codes0 : p.codes1;
            __builtin_amdgcn_global_load_lds(
                reinterpret_cast<const void *>(cb + static_cast<size_t>(wrow(t, f, r)) * row_codes + k0 / 2 + 16 * h),
                reinterpret_cast<FFN_LDS void *>(base + XB + (wave * 2 + f) * 1024), 16, 0, 0);
        }
        // scales: lane (f = h, r) -> the unit's 4 scale bytes of row r of fragment f
        {
            const uint8_t *sb = (h == 0 || NMAT == 1) ? p.scales0 : p.scales1;
            __builtin_amdgcn_global_load_lds(
                reinterpret_cast<const void *>(sb + static_cast<size_t>(wrow(t, h, r)) * row_scales + k0 / 16),
                reinterpret_cast<FFN_LDS void *>(base + XB + 8192 + wave * 256), 4, 0, 0);
        }
    };

    f32x16_t acc[2][MT];

    // The dequantised weight fragments of one unit (register double buffer).
    struct Frags {
        bf16x8_t w[2][4];
    };
    auto load_weights = [&](int st, Frags &F) {
        const FFN_LDS uint8_t *base = lds + st * STAGE;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const u32x4_t cw = *reinterpret_cast<const FFN_LDS u32x4_t *>(base + XB + (wave * 2 + f) * 1024 + lane * 16);
            const uint32_t sw = *reinterpret_cast<const FFN_LDS uint16_t *>(base + XB + 8192 + wave * 256 + f * 128 +
                                                                           r * 4 + h * 2);
            const float sc0 = e4m3_to_f32<0>(sw);
            const float sc1 = e4m3_to_f32<1>(sw);
            F.w[f][0] = dequant8(cw[0], sc0);
            F.w[f][1] = dequant8(cw[1], sc0);
            F.w[f][2] = dequant8(cw[2], sc1);
            F.w[f][3] = dequant8(cw[3], sc1);
        }
    };
    // The unit's products: activation fragments straight from the stage.
    auto mfma_unit = [&](int st, const Frags &F) {
        const FFN_LDS uint8_t *base = lds + st * STAGE;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = 32 * mt + r;
                const bf16x8_t a =
                    *reinterpret_cast<const FFN_LDS bf16x8_t *>(base + m * 128 + (((4 * h + s) ^ ((m >> 1) & 7)) * 16));
                acc[0][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, F.w[0][s], acc[0][mt], 0, 0, 0);
                acc[1][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, F.w[1][s], acc[1][mt], 0, 0, 0);
            }
    };

    auto store_out = [&](int t) {
        const int rows = opaque_uniform(p.rows);
        const int M = opaque_uniform(p.M);
        const int ln = opaque_lane(lane);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                emit_pair<NMAT, OUT, ROWS_TILE>(p, rows, M, t, wave, ln, mt, v, acc[0][mt][v], acc[1][mt][v]);
    };

    auto slot_ptr = [&](int gg, int t) {
        const int slot = 2 * gg + (t == sk_begin(gg, U, G) / KU ? 0 : 1);
        return p.partials + static_cast<size_t>(slot) * SLOT + static_cast<size_t>(wave) * (SLOT / kMfmaWaves);
    };

    // Software pipeline: up to S - 1 units in flight in the LDS ring. In the
    // step for unit j the weights of unit j + 1 are read and dequantised into
    // the other register set while the matrix cores work on unit j (whose
    // activation fragments are read from its stage as they are needed).
    // F0 holds the weights of the next unit to multiply.
    const int npre = min(n, S - 1);
    for (int j = 0; j < npre; ++j)
        issue(unit_at(j), j);
    Frags F0, F1;
    wait_units<S - 2, L>(min(S - 2, n - 1));
    lds_barrier();
    load_weights(0, F0);
    auto step = [&](Frags &cur, Frags &nxt, int j) {
        // unit j + 1 has landed (past the end: nothing outstanding) ...
        wait_units<S - 3, L>(max(0, min(S - 3, n - 2 - j)));
        // ... in every wave, and every wave is done with unit j - 1's stage
        lds_barrier();
        if (j + S - 1 < n)
            issue(unit_at(j + S - 1), (j + S - 1) % S);
        load_weights((j + 1) % S, nxt);  // past the end: a harmless re-read
        mfma_unit(j % S, cur);
        // The compiler interleaves the next unit's dequantisation with these
        // products. (A hand interleave by scheduling-group barriers, fragment
        // by fragment, measured 1.4-2.1 us per forward slower at 96 and 128
        // tokens with the 4-stage ring.)
    };

    // FIX: finish tile t, whose top unit this workgroup's current piece
    // holds (acc): add the lower workgroups' pieces of the tile to it, the
    // nearest first (a fixed order: a tile's sum depends only on the shape),
    // each piece's loads all in flight before its additions.
    auto finish = [&](int t) {
        const int g_lo = sk_owner(static_cast<long long>(t) * KU, U, G);
        for (int gg = g - 1; gg >= g_lo; --gg) {
            unsigned long long *flag = p.flags + 4 * (2 * gg + (t == sk_begin(gg, U, G) / KU ? 0 : 1)) + wave;
            wait_ready([&](int) { return flag; }, 1, p.tag);
            __hip_atomic_store(flag, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const __amdgpu_buffer_rsrc_t rsrc = raw_buffer(slot_ptr(gg, t), SLOT / kMfmaWaves * 4);
            f32x4_t v[2][MT][4];
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        v[f][mt][q4] = load_device_coherent(
                            rsrc, (((f * MT + mt) * 4 + q4) * 64 + opaque_lane(lane)) * 16);
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            acc[f][mt][4 * q4 + c] += v[f][mt][q4][c];
        }
        store_out(t);
    };

    // Pieces: maximal runs of this workgroup's units inside one tile. The
    // ring runs on across pieces; the accumulators only live inside one.
    int j = 0;
    int fin_t = -1;       // FIX: the tile this workgroup finishes after its loop
    int wrote = 0;        // FIX: slots it wrote (bit 0: slot 2 g, bit 1: 2 g + 1), published at the end
    while (j < n) {
        int t, ku0, len;
        if constexpr (FIX) {
            const int top = u_begin + n - 1 - j;
            t = top / KU;
            const int lo = max(u_begin, t * KU);
            ku0 = lo - t * KU;
            len = top - lo + 1;
        } else {
            t = (u_begin + j) / KU;
            ku0 = u_begin + j - t * KU;
            len = min(KU - ku0, n - j);
        }
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[f][mt] = f32x16_t{};
        // Two units per trip so the register sets swap roles without copies;
        // an odd piece ends with one step and a copy of the next unit's set.
        const int jend = j + len;
        for (; j + 1 < jend; j += 2) {
            step(F0, F1, j);
            step(F1, F0, j + 1);
        }
        if (j < jend) {
            step(F0, F1, j);
            F0 = F1;
            ++j;
        }
        if (ku0 == 0 && len == KU) {
            store_out(t);
            continue;
        }
        if constexpr (FIX) {
            // A piece that holds its tile's top unit without being the whole
            // tile starts inside the tile, so at the range's first unit: in
            // decreasing order it is the workgroup's last piece. The tile is
            // finished after the ready words of this workgroup are set.
            if (ku0 + len == KU) {
                fin_t = t;
                break;
            }
        }
        // A piece of a tile shared with other workgroups: to its slot, for
        // mfma_reduce_kernel or (FIX) the workgroup that finishes the tile.
        float *part = slot_ptr(g, t);
        f32x4_t *mine = reinterpret_cast<f32x4_t *>(part) + opaque_lane(lane);
        const __amdgpu_buffer_rsrc_t rsrc = raw_buffer(part, SLOT / kMfmaWaves * 4);
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const f32x4_t v = {acc[f][mt][4 * q4], acc[f][mt][4 * q4 + 1], acc[f][mt][4 * q4 + 2],
                                       acc[f][mt][4 * q4 + 3]};
                    const int idx = ((f * MT + mt) * 4 + q4) * 64;
                    if constexpr (FIX)  // read by another compute unit in this launch
                        store_device_coherent(rsrc, (idx + opaque_lane(lane)) * 16, v);
                    else
                        mine[idx] = v;
                }
        if constexpr (FIX)
            wrote |= (t == sk_begin(g, U, G) / KU) ? 1 : 2;
    }
    if constexpr (FIX) {
        // Publish this wave's part of the slot written above once its
        // device-coherent stores have completed (nothing else is in flight at
        // the end of the range). (A release fence instead, which writes the
        // XCD's L2 back, measured 21 us slower per forward.)
        if (wrote != 0) {
            wait_vmcnt<0>();
#pragma unroll
            for (int b = 0; b < 2; ++b)
                if (wrote & (1 << b))
                    __hip_atomic_store(p.flags + 4 * (2 * g + b) + wave, p.tag, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
        if (fin_t >= 0)
            finish(fin_t);
    }
}

// Finishes the tiles a stream-K launch left as pieces: every element sums its
// pieces in k order (the slot order) and goes through the same epilogue. A
// thread takes accumulator values 4 q4 .. 4 q4 + 3 of one lane and tile of a
// fragment pair (16-byte loads) and issues the loads of up to 16 pieces
// before adding any of them, so a tile split many ways is not read one
// dependent load at a time.
// Grid: (tiles, mfma_reduce_blocks<MT>()), 256 threads.
template <int MT>
constexpr int mfma_reduce_blocks()
{
    return (kMfmaWaves * MT * 16 * 64 / 4 + 255) / 256;
}

template <int MT, int NMAT, int OUT>
__global__ __launch_bounds__(256) void mfma_reduce_kernel(const MfmaParams p, int G)
{
    constexpr int ROWS_TILE = mfma_rows_per_tile<NMAT>();
    constexpr int SLOT = mfma_slot_floats<MT>();
    constexpr int PER_WAVE = MT * 16 * 64;  // positions of one fragment of one wave
    constexpr int B = 16;                   // pieces loaded at once
    const int t = blockIdx.x;
    const int e = (blockIdx.y * 256 + threadIdx.x) * 4;
    if (e >= kMfmaWaves * PER_WAVE)
        return;
    const long long U = p.units;
    const int KU = p.units_per_tile;
    const int g_lo = sk_owner(static_cast<long long>(t) * KU, U, G);
    const int g_hi = sk_owner(static_cast<long long>(t) * KU + KU - 1, U, G);
    if (g_lo == g_hi)
        return;  // one workgroup held the whole tile and stored it
    const int wave = e / PER_WAVE;
    const int rem = e - wave * PER_WAVE;  // float offset of fragment 0's 4 values
    const int lane = (rem >> 2) & 63;
    const int mt = rem >> 10;             // (rem / 4) / 64 = mt * 4 + q4
    const int q4 = (rem >> 8) & 3;
    f32x4_t y0 = {0.0f, 0.0f, 0.0f, 0.0f}, y1 = y0;
    for (int g0 = g_lo; g0 <= g_hi; g0 += B) {
        f32x4_t x0[B], x1[B];
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const int gg = g0 + i;  // uniform over the workgroup (one tile)
            if (gg > g_hi)
                break;
            const int slot = 2 * gg + (t == sk_begin(gg, U, G) / KU ? 0 : 1);
            const float *src = p.partials + static_cast<size_t>(slot) * SLOT + wave * (SLOT / kMfmaWaves) + rem;
            x0[i] = *reinterpret_cast<const f32x4_t *>(src);
            x1[i] = *reinterpret_cast<const f32x4_t *>(src + PER_WAVE);
        }
#pragma unroll
        for (int i = 0; i < B; ++i) {
            if (g0 + i > g_hi)
                break;
            if (g0 + i == g_lo) {
                y0 = x0[i];
                y1 = x1[i];
            } else {
                y0 = y0 + x0[i];
                y1 = y1 + x1[i];
            }
        }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
        emit_pair<NMAT, OUT, ROWS_TILE>(p, p.rows, p.M, t, wave, lane, mt, 4 * q4 + c, y0[c], y1[c]);
}

}  // namespace ffn
