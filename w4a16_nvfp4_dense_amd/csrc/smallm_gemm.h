// smallm_gemm.h -- the small-batch matrix-core arm of the NVFP4 gated FFN
// (9 <= M <= 40 token rows): the dual gate+up projection and the down
// projection as skinny GEMMs on bf16 matrix cores, for the batch sizes between
// the batched GEMV and the 128-row prefill tiles (dense_ffn.rs page, the
// prefill GEMM dispatch by token count, whose small-M tiles exist because
// padding a few tokens to a 64- or 128-row tile wastes most of it).
//
// Product. The weight rows are cut into tiles of 16 and the reduction into
// units of 64 columns. For every tile the workgroup's 16 waves take 16
// consecutive units at a time (a "round" of 1024 columns, wave q the q-th
// unit) and compute D[m, r] = sum_c A[m, c] W[r, c] over them with
// v_mfma_f32_16x16x32_bf16: activations as the A operand (rows = tokens), the
// dequantised weights as the B operand (columns = weight rows). A lane's four
// accumulators hold one weight row (lane % 16) and four tokens
// (4 (lane / 16) + v). At the end of the tile the 16 waves add their
// accumulators through LDS in a fixed order (waves 0-7 and 8-15 in wave
// order, then the two halves). At M <= 16 this MFMA shape reads each
// weight once per 16 cycles, twice the rate of the 32x32x16 shape. Batches
// of 17 to 32 rows run two token groups of 16 (TG = 2), and 33 to 40 rows
// three (TG = 3): each dequantised weight fragment feeds the products of every
// group, so a weight is still read and dequantised once. (Above 40 rows the
// 128-row arm is as fast: measured at 48 rows, 89.7 us with three groups
// against 89.0 us there, while 33 and 40 rows take 81.1 and 84.8 us against
// 88.3 us.)
//
// Dequantisation. As in the prefill arm: FP4 pair -> fp32 pair (unit-scale
// hardware conversion) times the E4M3 block scale, rounded to bf16, which is
// exact (E2M1 x E4M3 has at most 6 significant bits), so the matrix core's fp32
// accumulation is the only rounding of the product. scale2 multiplies in the
// epilogue.
//
// Why this data movement. In the MFMA operand layout the 16 lanes of a quarter
// wave hold 16 different rows, so a load straight into that layout touches 16
// cache lines per quarter wave; measured, such loads (of the activations
// above all) cost several times the whole weight stream. Here every global
// load is coalesced (a quarter wave reads 256 or 64 contiguous bytes of one
// to four rows) and the operand layout is made on chip:
//   - activations: a wave's units are the same in every tile of the
//     workgroup, so it loads its slice of the activations once (16 bytes per
//     lane and load, four tokens per quarter wave) and moves it into operand
//     layout with ds_bpermute; the slice stays in registers for all tiles;
//   - weights: the workgroup streams each round's codes (16 rows x 512 bytes
//     per projection) and scales (16 x 64 bytes) with direct global->LDS
//     loads into a ring of kSmStages stages, kSmStages - 1 rounds ahead, and
//     every wave reads its unit from LDS in operand layout.
// K order inside a unit: MFMA step s (of 2) gives lane group g = lane / 16 the
// columns 16 g + 8 s .. + 7, so a lane's codes of a unit are 8 contiguous
// bytes and both steps use one scale.
//
// Work split. Workgroup w takes part w % P of the reduction (P consecutive
// ranges of 256-column blocks, each at most as many rounds as a wave's
// activations fit in registers: 5 rounds; with two token groups 4 for the
// dual GEMM; with three, 2 for the dual GEMM and 3 for the down GEMM) and
// tiles [g T / G, (g + 1) T / G) with g = w / P, T tiles and G = gridDim / P
// groups. With P = 1 the epilogue writes finished outputs. With P > 1
// (SPLIT) every workgroup stores its part's fp32 sums of its tiles with
// device-coherent stores; the lower parts' workgroups then set their ready
// words, and the last part's workgroup (the highest id of the P, so it waits
// only for workgroups dispatched before it, which wait for nobody) adds the
// parts in order, part 0 first, and runs the epilogue. (A first version that
// let the last workgroup to finish add the parts, behind device-scope
// release/acquire fences, measured slower than a separate reduction launch:
// the fences write back and invalidate the XCD's L2.) The order of every sum
// is fixed, and a token row's result does not depend on the other rows of the
// batch within one token-group count (the count sets the parts, hence the
// order of the sums).
#pragma once

#include "kernels.h"
#include "nvfp4_device.h"

namespace ffn {

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kSmWaves = 16;                  // waves per workgroup
constexpr int kSmRows = 16;                   // weight rows per tile
constexpr int kSmUnit = 64;                   // reduction columns per wave and round
constexpr int kSmRound = kSmWaves * kSmUnit;  // reduction columns per round
constexpr int kSmMaxRounds = 5;               // rounds per tile and part (activations kept in registers)
constexpr int kSmStages = 3;                  // LDS ring stages (deeper measured slower: the arm is bound by its arithmetic, not by load latency)
constexpr int kSmMaxGroups = 3;               // token groups of 16 (M <= 48; the arm takes M <= 40)
constexpr int kSmMaxRoundsTwoGroups = 4;      // rounds per tile and part of the dual GEMM with two token groups

struct SmallParams {
    const void *in0;  // bf16 [M, cols]
    const uint8_t *codes0;
    const uint8_t *scales0;
    const uint8_t *codes1;
    const uint8_t *scales1;
    float s2_0;
    float s2_1;
    void *out0;
    void *out1;
    int M;       // token rows, 1 <= M <= 16 TG
    int rows;    // weight rows (output columns), a multiple of 16
    int cols;    // reduction length, a multiple of 256
    int parts;   // P
    int groups;  // G: workgroups per part
    float *part0;  // P x [M, rows] fp32 pieces of the first projection (split reductions)
    float *part1;  // the same for the second projection
    unsigned long long *flags;  // one ready word per workgroup (split reductions)
    unsigned long long tag;     // this launch's ready value (nonzero)
};

// LDS of one ring stage: codes [NMAT][2 row halves][4 column blocks][8 rows]
// [128 B], then scales [NMAT][16 rows][64 B] (16-byte chunks and dwords
// swizzled by row).
template <int NMAT>
constexpr int sm_stage_bytes()
{
    return NMAT * kSmRows * (kSmRound / 2 + kSmRound / 16);
}

// LDS of the reduction area: [TG token groups][16 waves][NMAT] accumulator
// sets of 64 lanes x 16 B.
template <int NMAT, int TG>
constexpr int sm_red_bytes()
{
    return TG * kSmWaves * NMAT * 1024;
}

// Ring, reduction area (the waves' accumulators and the two half sums), and
// 1280 bytes that the dummy loads write and nothing reads.
template <int NMAT, int TG>
constexpr int sm_lds_bytes()
{
    return kSmStages * sm_stage_bytes<NMAT>() + sm_red_bytes<NMAT, TG>() + 1280;
}

// PARTIAL: the batch leaves tokens of its last group empty (M < 16 TG); the
// reduction then skips their partial sums (a separate instantiation: the
// per-lane tests cost full groups 0.4-0.6 us per forward).
template <int NMAT, int OUT, int NR, int TG, bool SPLIT, bool PARTIAL>
__global__ __launch_bounds__(kSmWaves * 64) void smallm_gemm_kernel(const SmallParams p)
{
    static_assert(NR >= 1 && NR <= kSmMaxRounds, "rounds");
    static_assert(TG >= 1 && TG <= kSmMaxGroups, "token groups");
    constexpr int S = kSmStages;
    constexpr int STAGE = sm_stage_bytes<NMAT>();
    constexpr int CODES = NMAT * kSmRows * (kSmRound / 2);  // code bytes of a stage
    static_assert(S >= 3 && 2 * (S - 2) < 64, "ring stages / vmcnt range");

    extern __shared__ u32x4_t lds_raw[];
    FFN_LDS uint8_t *lds = (FFN_LDS uint8_t *)lds_raw;
    FFN_LDS f32x4_t *red = (FFN_LDS f32x4_t *)(lds + S * STAGE);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int q = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int g = lane >> 4;
    const int cols = p.cols;
    const int M = p.M;
    const int T = p.rows / kSmRows;
    const int P = p.parts;
    const int part = blockIdx.x % P;
    const int grp = blockIdx.x / P;
    const int ta = grp * T / p.groups;
    const int ntiles = (grp + 1) * T / p.groups - ta;
    const int NU = cols / kSmUnit;
    const int NB = NU / 4;                               // 256-column blocks (parts end on them)
    const int ua = 4 * (part * NB / P);
    const int nu = 4 * ((part + 1) * NB / P) - ua;       // units of this part
    const int nrounds = (nu + kSmWaves - 1) / kSmWaves;  // <= NR
    const int total = ntiles * nrounds;                  // rounds of this workgroup
    const size_t row_codes = static_cast<size_t>(cols) / 2;
    const size_t row_scales = static_cast<size_t>(cols) / 16;
    const int piece_bytes = P * M * p.rows * 4;  // one projection's pieces (< 2^31, checked by the launcher)

    // Loads of one round: codes (16 rows x 512 bytes per projection) and
    // scales (16 x 64 bytes per projection). Every wave issues exactly two
    // (so the number of loads in flight is the same in every wave):
    //   codes: wave q < 8 NMAT takes projection q / 8, rows 8 ((q / 4) % 2) ..
    //     + 7 and column block q % 4 (128 bytes of each row); lane l loads
    //     row 8 ((q / 4) % 2) + l / 8, 16-byte chunk (l % 8) ^ ((row / 2) % 8)
    //     of the block into LDS slot l, so a quarter wave reads two whole
    //     cache lines and the 8-byte operand reads below (16 rows x 4 lanes)
    //     fall on all 64 banks once;
    //   scales: wave q < 4 NMAT takes rows 4 (q % 4) .. + 3 of projection
    //     q / 4; lane l loads row 4 (q % 4) + l / 16, dword (l % 16) ^ (q % 4)
    //     of the row's 64 bytes into slot l (again conflict-free to read);
    //   the other waves load dummies (valid addresses) into LDS that is never
    //     read.
    // The per-lane row pointers are advanced a tile at a time, so a round
    // costs the scalar unit (shared by the compute unit's 16 waves) only a few
    // instructions. Addresses past the part (a short last round) are clamped
    // inside the row and never used.
    const bool code_wave = q < 8 * NMAT;
    const bool scale_wave = q < 4 * NMAT;
    const int qc = q & (8 * NMAT - 1);  // dummy code waves load what wave qc loads
    const int fc = NMAT == 2 ? (qc >> 3) : 0;
    const int fs = NMAT == 2 ? ((q >> 2) & 1) : 0;
    const int crow = 8 * ((qc >> 2) & 1) + (lane >> 3);  // row of the tile this lane's code chunk is in
    const uint8_t *csrc = (fc == 0 ? p.codes0 : p.codes1) + static_cast<size_t>(ta * kSmRows + crow) * row_codes;
    const uint8_t *ssrc =
        (fs == 0 ? p.scales0 : p.scales1) + static_cast<size_t>(ta * kSmRows + 4 * (q & 3) + (lane >> 4)) * row_scales;
    const uint32_t cchunk = 128 * (qc & 3) + 16 * ((lane & 7) ^ ((crow >> 1) & 7));
    const uint32_t sdword = scale_wave ? 4 * ((lane & 15) ^ (q & 3)) : 0;
    const uint32_t clast = static_cast<uint32_t>(row_codes) - 16;
    const uint32_t slast = static_cast<uint32_t>(row_scales) - 4;
    constexpr int DUMMY = S * STAGE + sm_red_bytes<NMAT, TG>();  // 1 KB + 256 B never read
    auto issue = [&](const uint8_t *cb, const uint8_t *sb, int i, int st) {
        const uint32_t u0 = static_cast<uint32_t>(ua + kSmWaves * i);  // first unit of the round
        FFN_LDS uint8_t *base = lds + st * STAGE;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(cb + min(u0 * (kSmUnit / 2) + cchunk, clast)),
                                         reinterpret_cast<FFN_LDS void *>(code_wave ? base + q * 1024 : lds + DUMMY),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(sb + min(u0 * (kSmUnit / 16) + sdword, slast)),
                                         reinterpret_cast<FFN_LDS void *>(scale_wave ? base + CODES + q * 256
                                                                                     : lds + DUMMY + 1024),
                                         4, 0, 0);
    };
    // Issue side of the ring: the next round to load (tile pointers, round
    // index, stage). After the last round it loads the last round again into
    // stages nothing reads (from L2), so that every wait below has the same
    // number of rounds in flight.
    const size_t tile_codes = kSmRows * row_codes;
    const size_t tile_scales = kSmRows * row_scales;
    int iss_i = 0, iss_st = 0, issued = 0;
    auto issue_next = [&]() {
        issue(csrc, ssrc, iss_i, iss_st);
        if (++issued < total) {
            if (++iss_i == nrounds) {
                iss_i = 0;
                csrc += tile_codes;
                ssrc += tile_scales;
            }
        }
        if (++iss_st == S)
            iss_st = 0;
    };

    // The wave's activation slice, loaded coalesced (lane l: token l / 4,
    // columns 16 (l % 4) + 8 s .. + 7 of the unit; a quarter wave reads four
    // 128-byte token pieces) and moved to operand layout with ds_bpermute
    // (lane (r, g) takes the piece of lane 4 r + g), for every round i (unit
    // ua + 16 i + q) and step s.
    // Ring prologue, round 0 first: the compiler waits for every load in
    // flight before the ds_bpermute below (it cannot tell that the
    // permutation reads no LDS that a direct load writes), so the later
    // prologue rounds are issued after it; round 0 is needed first anyway.
    issue_next();

    // Token group t holds tokens 16 t .. 16 t + 15.
    u32x4_t xr[NR][TG][2];
    {
        const uint16_t *X = static_cast<const uint16_t *>(p.in0);
#pragma unroll
        for (int t = 0; t < TG; ++t) {
            const int tok = min(16 * t + (lane >> 2), M - 1);  // rows past the batch re-read the last one (never stored)
#pragma unroll
            for (int i = 0; i < NR; ++i)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int u = min(ua + kSmWaves * i + q, NU - 1);
                    xr[i][t][s] = *reinterpret_cast<const u32x4_t *>(X + static_cast<size_t>(tok) * cols +
                                                                     u * kSmUnit + 16 * (lane & 3) + 8 * s);
                }
        }
    }

    {
        const int src = (4 * r + g) * 4;  // byte address of the source lane
#pragma unroll
        for (int i = 0; i < NR; ++i)
#pragma unroll
            for (int t = 0; t < TG; ++t)
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        xr[i][t][s][d] = static_cast<uint32_t>(
                            __builtin_amdgcn_ds_bpermute(src, static_cast<int>(xr[i][t][s][d])));
    }

#pragma unroll
    for (int k = 1; k < S - 1; ++k)
        issue_next();

    f32x4_t acc[NMAT][TG];
#pragma unroll
    for (int f = 0; f < NMAT; ++f)
#pragma unroll
        for (int t = 0; t < TG; ++t)
            acc[f][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const uint32_t scale_shift = 8 * g;  // both steps use scale byte g of the unit's 4
    // this lane's operand bytes: unit q is bytes 32 (q % 4) .. + 31 of column
    // block q / 4; the lane's 8 bytes are chunk 2 (q % 4) + g / 2 (swizzled)
    // and half g % 2 of row r, in the load of rows 8 (r / 8) .. + 7; its scale
    // dword is slot q ^ (r / 4)
    const int code_off = (4 * (r >> 3) + (q >> 2)) * 1024 + (r & 7) * 128 +
                         16 * ((2 * (q & 3) + (g >> 1)) ^ ((r >> 1) & 7)) + 8 * (g & 1);
    const int scale_off = CODES + r * 64 + 4 * (q ^ (r >> 2));
    // Tile tt's sums from the 16 waves' accumulators in the reduction area,
    // and its epilogue. Thread pair (2 j, 2 j + 1) takes output j = (t, o),
    // o = 16 m + rr (accumulator m % 4 of lane 16 (m / 4) + rr of every
    // wave), and j + 512 with three token groups: each thread adds waves
    // 8 h .. 8 h + 7 in order (h = tid % 2), and the even thread adds the two
    // halves, half 0 first.
    const FFN_LDS float *redf = reinterpret_cast<const FFN_LDS float *>(red);
    auto finish_tile = [&](int tt) {
      const int h = tid & 1;
      for (int j = tid >> 1; j < TG * 256; j += kSmWaves * 32) {
        const int t = j >> 8;
        const int o = j & 255;
        const int ml = o >> 4;
        const int rr = o & 15;
        const int m = 16 * t + ml;
        if (PARTIAL && m >= M)  // (the pair of threads skips together)
            continue;
        const int at = (16 * (ml >> 2) + rr) * 4 + (ml & 3);
        float y[NMAT];
#pragma unroll
        for (int f = 0; f < NMAT; ++f) {
            float a = redf[((t * kSmWaves + 8 * h) * NMAT + f) * 256 + at];
#pragma unroll
            for (int w = 1; w < 8; ++w)
                a += redf[((t * kSmWaves + 8 * h + w) * NMAT + f) * 256 + at];
            // the partner thread's half (lanes 2 j and 2 j + 1)
            const float b = __builtin_bit_cast(
                float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, a), 0xB1, 0xF, 0xF, true));
            y[f] = a + b;  // in the even thread: half 0 + half 1
        }
        if (h != 0)
            continue;
        const int row = (ta + tt) * kSmRows + rr;
        const size_t o_out = static_cast<size_t>(m) * p.rows + row;
        if constexpr (SPLIT) {
            // this part's piece, for the last part's workgroup (any XCD)
            const int po = (part * M * p.rows + static_cast<int>(o_out)) * 4;
            store_device_coherent(raw_buffer(p.part0, piece_bytes), po, y[0]);
            if constexpr (NMAT == 2)
                store_device_coherent(raw_buffer(p.part1, piece_bytes), po, y[1]);
        } else if constexpr (OUT == OUT_F32_PAIR) {
            static_cast<float *>(p.out0)[o_out] = y[0] * p.s2_0;
            static_cast<float *>(p.out1)[o_out] = y[NMAT - 1] * p.s2_1;
        } else if constexpr (OUT == OUT_H_SILU || OUT == OUT_H_GELU) {
            constexpr int A = (OUT == OUT_H_SILU) ? ACT_SILU : ACT_GELU_TANH;
            static_cast<uint16_t *>(p.out0)[o_out] =
                to_bf16_bits(gate_act<A>(y[0] * p.s2_0) * (y[NMAT - 1] * p.s2_1));
        } else {
            static_cast<uint16_t *>(p.out0)[o_out] = to_bf16_bits(y[0] * p.s2_0);
        }
      }
    };

    int st = 0;  // ring stage of the round being multiplied
    for (int tt = 0; tt < ntiles; ++tt) {
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            if (i >= nrounds)
                break;
            // round v has landed in every wave (S - 2 later rounds of this
            // wave's loads still in flight); the stage of round v - 1 is free
            wait_vmcnt<2 * (S - 2)>();
            lds_barrier();
            issue_next();
            // the previous tile's partial sums were written before this barrier
            if (i == 0 && tt > 0)
                finish_tile(tt - 1);
            if (kSmWaves * i + q < nu) {
                const FFN_LDS uint8_t *base = lds + st * STAGE;
#pragma unroll
                for (int f = 0; f < NMAT; ++f) {
                    const u32x2_t c = *reinterpret_cast<const FFN_LDS u32x2_t *>(base + f * 8192 + code_off);
                    const float sc = e4m3_to_f32<0>(
                        *reinterpret_cast<const FFN_LDS uint32_t *>(base + f * 1024 + scale_off) >> scale_shift);
                    const bf16x8_t b0 = dequant8(c[0], sc);
                    const bf16x8_t b1 = dequant8(c[1], sc);
                    // one dequantised fragment, every token group
#pragma unroll
                    for (int t = 0; t < TG; ++t) {
                        acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xr[i][t][0]),
                                                                           b0, acc[f][t], 0, 0, 0);
                        acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xr[i][t][1]),
                                                                           b1, acc[f][t], 0, 0, 0);
                    }
                }
            }
            if (++st == S)
                st = 0;
        }

        // Tile done: this wave's accumulators to the reduction area, added up
        // during the next tile's first round (after the loop for the last
        // tile), so that no extra barrier is needed and the epilogue's stores
        // have a round to complete. A tile of one round has no barrier between
        // the previous tile's sums, read in that round, and these writes.
        if (nrounds == 1)
            lds_barrier();
        // (a lane's 4 accumulators are tokens 16 t + 4 (lane / 16) .. + 3:
        // lanes whose tokens all lie past the batch write nothing)
#pragma unroll
        for (int t = 0; t < TG; ++t)
#pragma unroll
            for (int f = 0; f < NMAT; ++f) {
                if (!PARTIAL || 16 * t + 4 * (lane >> 4) < M)
                    red[((t * kSmWaves + q) * NMAT + f) * 64 + lane] = acc[f][t];
                acc[f][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            }
    }
    lds_barrier();
    finish_tile(ntiles - 1);

    if constexpr (SPLIT) {
        // The P workgroups blockIdx.x - part .. + P - 1 hold the parts of the
        // same tiles. Every wave waits for its own piece stores (nothing else
        // it issued matters: the ring's trailing loads only fill LDS); once
        // all have, a lower part's workgroup publishes its pieces.
        wait_vmcnt<0>();
        __syncthreads();
        if (part != P - 1) {
            if (q == 0)
                __hip_atomic_store(p.flags + blockIdx.x, p.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        // The last part's workgroup finishes the tiles: thread (q, lane) takes
        // element (token 16 t + tid2 / 16, row tid2 % 16) with tid2 = 64 (q %
        // 4) + lane of the (tile, token group) items q / 4, q / 4 + 4, ... It
        // waits only for lower-numbered workgroups, which were dispatched
        // first and wait for nobody.
        const int g0 = blockIdx.x - part;
        // (one word at a time: polling all of them at once measured no faster)
        for (int pp = 0; pp < P - 1; ++pp)
            wait_ready([&](int) { return p.flags + g0 + pp; }, 1, p.tag);
        __syncthreads();  // every wave has seen the words: clear them
        if (q == 0)
            for (int pp = 0; pp < P - 1; ++pp)
                __hip_atomic_store(p.flags + g0 + pp, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

        const int tid2 = 64 * (q & 3) + lane;
        const int mo = tid2 >> 4;  // token within its group
        const int rr = tid2 & 15;
        const __amdgpu_buffer_rsrc_t rsrc[2] = {raw_buffer(p.part0, piece_bytes),
                                                raw_buffer(NMAT == 2 ? p.part1 : p.part0, piece_bytes)};
        const int part_bytes = M * p.rows * 4;
        const int items = ntiles * TG;
        // (Measured and not kept: 8 items per batch, which spills the
        // two-group kernel's registers, and the last part's own pieces kept in
        // this XCD's L2 with plain stores and loads: 1-2 us slower each.)
        constexpr int IG = 4;  // items per thread and batch
        constexpr int PC = 4;  // parts per batch (all loads of a batch in flight before its additions)
        for (int k0 = q >> 2; k0 < items; k0 += 4 * IG) {
            int off[IG];
            bool ok[IG];
#pragma unroll
            for (int i = 0; i < IG; ++i) {
                const int k = k0 + 4 * i;
                const int tt = k / TG;
                const int m = 16 * (k - tt * TG) + mo;
                ok[i] = k < items && m < M;
                off[i] = ok[i] ? (m * p.rows + (ta + tt) * kSmRows + rr) * 4 : 0;  // 0: a valid, unused read
            }
            float sum[IG][NMAT];
            for (int p0 = 0; p0 < P; p0 += PC) {
                float v[IG][PC][NMAT];
#pragma unroll
                for (int i = 0; i < IG; ++i)
#pragma unroll
                    for (int c = 0; c < PC; ++c)
#pragma unroll
                        for (int f = 0; f < NMAT; ++f)
                            if (p0 + c < P)
                                v[i][c][f] = load_device_coherent_f32(rsrc[f], off[i] + (p0 + c) * part_bytes);
                // the parts in order, part 0 first
#pragma unroll
                for (int i = 0; i < IG; ++i)
#pragma unroll
                    for (int c = 0; c < PC; ++c)
#pragma unroll
                        for (int f = 0; f < NMAT; ++f)
                            if (p0 + c < P)
                                sum[i][f] = (p0 + c == 0) ? v[i][c][f] : sum[i][f] + v[i][c][f];
            }
#pragma unroll
            for (int i = 0; i < IG; ++i) {
                if (!ok[i])
                    continue;
                const size_t o = static_cast<size_t>(off[i] / 4);
                if constexpr (OUT == OUT_F32_PAIR) {
                    static_cast<float *>(p.out0)[o] = sum[i][0] * p.s2_0;
                    static_cast<float *>(p.out1)[o] = sum[i][NMAT - 1] * p.s2_1;
                } else if constexpr (OUT == OUT_H_SILU || OUT == OUT_H_GELU) {
                    constexpr int A = (OUT == OUT_H_SILU) ? ACT_SILU : ACT_GELU_TANH;
                    static_cast<uint16_t *>(p.out0)[o] =
                        to_bf16_bits(gate_act<A>(sum[i][0] * p.s2_0) * (sum[i][NMAT - 1] * p.s2_1));
                } else {
                    static_cast<uint16_t *>(p.out0)[o] = to_bf16_bits(sum[i][0] * p.s2_0);
                }
            }
        }
    }
}

}  // namespace ffn
