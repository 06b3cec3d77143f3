/*
 * ffn_fp8.h -- C ABI of the block-scaled FP8 (W8A16) gated FFN of
 * libffn_nvfp4, for decode and verify batches (1 <= M <= 8 rows).
 *
 * The same layer as ffn_nvfp4.h,
 *     gate = W_g x,   up = W_u x,   h = act(gate) * up,   out = W_d h,
 * over weights loaded natively from an FP8 checkpoint instead of NVFP4
 * (dense_ffn.rs page: DenseFfnWeightsFp8, and DenseFfnLayer::forward's FP8
 * dispatch, a fused gate+up GEMV and an activation-fused down GEMV).
 *
 * Weight format (qwen35_dense.rs page, the doc comment on which FP8 scale
 * layouts the native path accepts): a weight of logical shape [rows, cols] is
 *   - codes      : uint8 [rows, cols], one E4M3FN byte per element
 *                  (OCP: bias 7, no infinities, 0x7F / 0xFF are NaN, max 448);
 *   - block_scale: fp32 [ceil(rows/128), ceil(cols/128)], row-major; the
 *                  multiplier of the 128 x 128 block (DeepSeek-V3 style
 *                  weight_scale_inv grids; a per-tensor scalar scale is the
 *                  uniform grid).
 * Element (r, c) is e4m3(codes[r][c]) * block_scale[r/128][c/128]. There is
 * no per-tensor multiplier. Block scales must be finite (with a non-finite
 * scale the result is unspecified); NaN codes propagate to the outputs they
 * touch.
 * Shapes: W_g, W_u are [N, K]; W_d is [K, N]; K = hidden, N = intermediate.
 *
 * Conventions are those of ffn_nvfp4.h (device pointers owned by the caller,
 * row-major dense matrices, asynchronous on `stream`, host-side validation
 * before anything is enqueued, deterministic results, row m of a batch
 * bit-identical to an M = 1 call on that row, status codes FFN_NVFP4_*,
 * activations ffn_nvfp4_act). Supported: M = 0 (empty call) and 1 <= M <= 8
 * (else FFN_NVFP4_ERR_BATCH); K and N positive multiples of 16, at most
 * 24576 (else FFN_NVFP4_ERR_SHAPE). Alignment (else FFN_NVFP4_ERR_ALIGN):
 * codes, x, out, gate/up buffers and workspace 16 bytes; block_scale 4 bytes.
 *
 * Precision: each E4M3 code is exact in bf16; per 16 consecutive columns a
 * lane sums code * input products in fp32 (bf16 dot products), multiplies
 * the sum by the block scale and adds it to its fp32 accumulator; the wave
 * sums its lanes in a fixed tree.
 */
#ifndef FFN_FP8_H
#define FFN_FP8_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "ffn_nvfp4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* One block-scaled FP8 weight (see the format above). codes: device,
 * 16-byte aligned; block_scale: device, 4-byte aligned. */
typedef struct ffn_fp8_weight {
    const uint8_t *codes;
    const float *block_scale;
} ffn_fp8_weight;

/* Bytes of device workspace ffn_fp8_forward needs: h [M, N] bf16, rounded up
 * to 256; 0 if M = 0 or the shape or batch is unsupported. Its contents need
 * no initialisation. */
size_t ffn_fp8_workspace_bytes(int M, int K, int N);

/* The whole FFN: out[M, K] (bf16) = W_d (act(W_g x) * (W_u x)), x[M, K] bf16.
 * Two launches: the dual GEMV computes h = bf16(act(gate) * up) in its
 * epilogue (gate and up in fp32 up to there) into the workspace; the down
 * GEMV streams W_d against h.
 *   x          device, bf16 [M, K]
 *   gate, up   host structs describing [N, K] weights
 *   down       host struct describing a [K, N] weight
 *   act        ffn_nvfp4_act
 *   workspace  device, >= ffn_fp8_workspace_bytes(M, K, N) bytes; clobbered;
 *              calls that share it must not overlap
 *   out        device, bf16 [M, K]; may not alias x */
int ffn_fp8_forward(const void *x, int M, int K, int N,
                    const ffn_fp8_weight *gate, const ffn_fp8_weight *up,
                    const ffn_fp8_weight *down, int act,
                    void *workspace, size_t workspace_bytes,
                    void *out, hipStream_t stream);

/* Dual GEMV, one pass over x for both projections (dense_ffn.rs page,
 * DenseFfnLayer::forward, w8a16_gemv_dual):
 *   gate_out[m, n] = sum_k W_g[n, k] x[m, k]
 *   up_out[m, n]   = sum_k W_u[n, k] x[m, k]
 *   x          device, bf16 [M, K]
 *   gate_out   device, fp32 [M, N]
 *   up_out     device, fp32 [M, N] */
int ffn_fp8_dual_gemv(const void *x, int M, int K, int N,
                      const ffn_fp8_weight *gate, const ffn_fp8_weight *up,
                      float *gate_out, float *up_out, hipStream_t stream);

/* Down GEMV with the activation fused into its input load (dense_ffn.rs
 * page, DenseFfnLayer::forward, w8a16_gemv_silu_input; GELU-tanh is served
 * the same way):
 *   out[m, j] = bf16(sum_n W_d[j, n] * bf16(act(gate[m, n]) * up[m, n]))
 *   gate_in, up_in   device, fp32 [M, N] (as written by the dual GEMV)
 *   down             host struct describing a [K, N] weight
 *   out              device, bf16 [M, K] */
int ffn_fp8_down_gemv(const float *gate_in, const float *up_in, int M, int N, int K,
                      const ffn_fp8_weight *down, int act,
                      void *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FFN_FP8_H */
