// kernels.h -- internal launchers of the NVFP4 FFN kernels (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace ffn {

// Lets `kern` use up to `lds` bytes of dynamic LDS on the current device.
// hipFuncSetAttribute is a host call; `done` (one per kernel, a static of its
// launcher) records the devices it was made on, so it runs once per kernel
// and device instead of on every launch (and never while a caller captures
// the launches into a graph, once they have run eagerly).
inline hipError_t allow_lds(const void *kern, int lds, std::atomic<uint64_t> &done)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        dev = -1;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
    if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0)
        return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess && bit != 0)
        done.fetch_or(bit, std::memory_order_release);
    return e;
}

struct WeightArg {
    const uint8_t *codes;   // [rows, cols/2]
    const uint8_t *scales;  // [rows, cols/16]
    float scale2;
};

// Kinds of input staged into LDS along the reduction dimension.
enum InKind : int {
    IN_BF16 = 0,         // bf16 [M, cols] (x for the dual GEMV, h for the down GEMV)
    IN_GATEUP_SILU = 1,  // fp32 gate, up [M, cols]; staged h = bf16(SiLU(gate) * up)
    IN_GATEUP_GELU = 2,  // same with GELU-tanh
};

// What the row results are turned into.
enum OutKind : int {
    OUT_F32_PAIR = 0,  // two projections: out0 = s2_0 * y0, out1 = s2_1 * y1 (fp32 [M, rows])
    OUT_BF16 = 1,      // one projection: out0 = bf16(s2_0 * y0) [M, rows]
    OUT_H_SILU = 2,    // two projections: out0 = bf16(SiLU(s2_0 y0) * s2_1 y1) [M, rows]
    OUT_H_GELU = 3,    // same with GELU-tanh
};

// Streaming GEMV over NVFP4 weights for 1 <= M <= 8 activation rows:
// y_t[m, r] = sum_c W_t[r, c] * a[m, c] for one (nmat = 1) or two (nmat = 2)
// weights of shape [rows, cols] sharing the same input a. Returns a HIP error
// code (hipSuccess on launch).
hipError_t launch_gemv(int M, int nmat, InKind in, OutKind out,
                       const void *in0, const float *in1,
                       const WeightArg &w0, const WeightArg &w1,
                       void *out0, void *out1, int rows, int cols, hipStream_t stream);

}  // namespace ffn

namespace ffn {

// Many-wave GEMV (1 <= M <= 8; rows of 33 to 768 chunks): one whole row per
// wave at a time, many waves per compute unit, activations staged in LDS
// (in pieces of the reduction when they do not fit); one launch per batch.
// Returns hipErrorNotSupported for shapes it does not cover.
hipError_t launch_wave_dual(int M, OutKind out, const void *x, const WeightArg &w0, const WeightArg &w1,
                            void *out0, void *out1, int rows, int cols, hipStream_t stream);
hipError_t launch_wave_down(int M, InKind in, const void *in0, const float *in1, const WeightArg &w, void *out,
                            int rows, int cols, hipStream_t stream);

// Number of compute units of the current device (cached per device).
int device_cu_count();

// A nonzero 64-bit tag per launch for the ready words of in-kernel exchanges
// (a counter and this library's address through a 64-bit mix), so that a
// ready word left in a reused workspace by other data or another launch
// almost never equals it.
unsigned long long launch_tag();

// Lanes that share one weight row for a reduction of `cpr` 32-column chunks
// (8, 16, 32 or 64); the row-streaming kernels require 64.
int lanes_per_row(int cpr);

}  // namespace ffn

namespace ffn {

// A block-scaled FP8 weight of shape [rows, cols]: E4M3FN codes [rows, cols]
// and the fp32 block-scale grid [ceil(rows/128), ceil(cols/128)].
struct Fp8WeightArg {
    const uint8_t *codes;
    const float *block_scale;
};

// Many-wave GEMV over FP8 weights, 1 <= M <= 8 (one launch per batch);
// cols a multiple of 16, at most 24576.
// The dual takes OUT_F32_PAIR, OUT_H_SILU or OUT_H_GELU; the down takes
// IN_BF16, IN_GATEUP_SILU or IN_GATEUP_GELU and writes bf16. Returns
// hipErrorNotSupported for anything else.
hipError_t launch_fp8_dual(int M, OutKind out, const void *x, const Fp8WeightArg &w0, const Fp8WeightArg &w1,
                           void *out0, void *out1, int rows, int cols, hipStream_t stream);
hipError_t launch_fp8_down(int M, InKind in, const void *in0, const float *in1, const Fp8WeightArg &w, void *out,
                           int rows, int cols, hipStream_t stream);

}  // namespace ffn

namespace ffn {

// An MXFP4 weight of shape [rows, cols]: E2M1 codes [rows, cols/2], E8M0
// exponent bytes [rows, cols/32], and the per-tensor fp32 scale2.
struct MxWeightArg {
    const uint8_t *codes;
    const uint8_t *e8m0;
    float scale2;
};

// bf16 [rows, cols] -> MXFP4 codes and E8M0 bytes (cols a multiple of 32).
hipError_t launch_mx_quant_bf16(const void *x, int rows, int cols, uint8_t *codes, uint8_t *e8m0,
                                hipStream_t stream);
// NVFP4 codes and scales [rows, cols] -> MXFP4 (scale2 is not folded in).
hipError_t launch_mx_requant(const uint8_t *codes, const uint8_t *scales, int rows, int cols, uint8_t *mx_codes,
                             uint8_t *mx_e8m0, hipStream_t stream);
// W4A4 dual GEMM over MXFP4 activations [M, K] and weights [N, K]: OUT_F32_PAIR
// (out0 = fp32 gate, out1 = fp32 up) or OUT_H_SILU / OUT_H_GELU (out0 = bf16 h).
// N a multiple of 32, K a multiple of 256.
hipError_t launch_w4a4_dual(int M, OutKind out, const uint8_t *xc, const uint8_t *xe, const MxWeightArg &g,
                            const MxWeightArg &u, void *out0, float *out1, int N, int K, hipStream_t stream);

// W4A4 down GEMM for one token group (1 <= M <= 128): out[M, rows] (bf16) =
// scale2 * (mx(h) . mx(W)) for MXFP4 h [M, cols] and W [rows, cols], cols a
// multiple of 256. The reduction is split in parts when that fills the
// device better; `part` then holds w4a4_down_partial_floats(rows, cols)
// floats and `flags` w4a4_down_flag_words(rows, cols) words (no
// initialisation needed; calls on one stream may share them).
size_t w4a4_down_partial_floats(int rows, int cols);
size_t w4a4_down_flag_words(int rows, int cols);
hipError_t launch_w4a4_down(int M, const uint8_t *hc, const uint8_t *he, const MxWeightArg &d, uint16_t *out,
                            int rows, int cols, float *part, unsigned long long *flags, hipStream_t stream);

}  // namespace ffn
