/*
 * ffn_w4a4.h -- C ABI of the W4A4 prefill arm of libffn_nvfp4 (gfx950 FP4
 * matrix cores).
 *
 * The pages run a lossy W4A4 prefill for the dense FFN: 4-bit weights against
 * bf16 activations quantised to 4 bits on every call, each projection's
 * per-tensor scale2 multiplying its products (dense_ffn.rs page, the W4A4
 * native-FP4 prefill and the NVFP4 W4A4 MMQ arm of forward_prefill). Two
 * forms are offered, as the pages describe both:
 *   - ffn_w4a4_forward: gate and up on 4 bits, the heavy-tailed down
 *     projection kept on the W4A16 path (the MMQ arm's hybrid);
 *   - ffn_w4a4_forward_fp4: all three projections on 4 bits, h quantised like
 *     the activations before the down projection (the native-FP4 prefill,
 *     which quantises the down input too).
 *
 * gfx950's FP4 matrix instruction (v_mfma_scale_f32_32x32x64_f8f6f4) takes one
 * power-of-two (E8M0) scale per 32 consecutive elements of each operand row,
 * not NVFP4's E4M3 scale per 16, so here both operands are MXFP4 (OCP MX
 * v1.0):
 *   - per row and 32-element block, the shared exponent is
 *     se = floor(log2(amax)) - 2, clamped to [-127, 127], stored as the E8M0
 *     byte se + 127 (a block of zeros gets se = 0);
 *   - each element is E2M1(v * 2^-se), nearest with ties to even, saturating
 *     at 6, keeping its sign; codes [rows, cols/2] with element 2j in the low
 *     nibble of byte j (the NVFP4 packing);
 *   - weights are requantised once from NVFP4 (ffn_w4a4_prepare_weight),
 *     v = e2m1 * e4m3 (scale2 stays a separate fp32 factor); activations are
 *     quantised inside every call.
 * This is lossy twice (activations and weights); the products of MXFP4
 * values are exact and accumulate in fp32.
 *
 * Conventions, status codes and activations are those of ffn_nvfp4.h. Inputs
 * must be finite.
 */
#ifndef FFN_W4A4_H
#define FFN_W4A4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "ffn_nvfp4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* One MXFP4 weight [rows, cols]. codes: device, uint8 [rows, cols/2],
 * 16-byte aligned; scales: device, E8M0 bytes [rows, cols/32], 8-byte aligned;
 * scale2: host fp32 multiplier of the projection's products. */
typedef struct ffn_mxfp4_weight {
    const uint8_t *codes;
    const uint8_t *scales;
    float scale2;
} ffn_mxfp4_weight;

/* NVFP4 -> MXFP4 requantisation of one weight (done once, at load):
 *   w          host struct of an NVFP4 weight [rows, cols] (codes 16-byte,
 *              scales 2-byte aligned; its scale2 is not used: copy it into
 *              the ffn_mxfp4_weight)
 *   rows       1 .. 65536; cols a positive multiple of 32, at most 65536
 *   mx_codes   device, uint8 [rows, cols/2], 16-byte aligned (written)
 *   mx_scales  device, uint8 [rows, cols/32] (written)
 * One kernel launch on `stream`. */
int ffn_w4a4_prepare_weight(const ffn_nvfp4_weight *w, int rows, int cols, uint8_t *mx_codes, uint8_t *mx_scales,
                            hipStream_t stream);

/* Bytes of device workspace the W4A4 entry points need for (M, K, N): the
 * quantised activations (M K / 2 code bytes and M K / 32 exponent bytes) and,
 * for the forward, h [M, N] bf16 and the down projection's partial-sum slots
 * (as ffn_nvfp4_forward's 128-row arm); each part rounded up to 256 bytes.
 * 0 if M = 0 or the shape is unsupported. Contents need no initialisation. */
size_t ffn_w4a4_workspace_bytes(int M, int K, int N);

/* W4A4 dual GEMM: gate_out = scale2_g * (mx(x) . mx(W_g)),
 * up_out = scale2_u * (mx(x) . mx(W_u)), fp32 [M, N].
 *   x          device, bf16 [M, K], 16-byte aligned
 *   gate, up   host structs of MXFP4 weights [N, K]
 *   workspace  device, >= ffn_w4a4_workspace_bytes(M, K, N) bytes, 16-byte
 *              aligned; clobbered (holds mx(x))
 * M: 0 .. 65536. K: a positive multiple of 256; N: a positive multiple of 64;
 * both at most 65536 (else FFN_NVFP4_ERR_SHAPE). */
int ffn_w4a4_dual_gemm(const void *x, int M, int K, int N, const ffn_mxfp4_weight *gate,
                       const ffn_mxfp4_weight *up, float *gate_out, float *up_out, void *workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* The hybrid FFN: out[M, K] (bf16) = W_d bf16(act(gate) * up) with gate and
 * up from the W4A4 dual GEMM and the NVFP4 down projection on the W4A16
 * matrix-core arm (as ffn_nvfp4_forward for M > 8). `down` is an NVFP4 weight
 * [K, N] with scales 8-byte aligned. Shapes as ffn_w4a4_dual_gemm. */
int ffn_w4a4_forward(const void *x, int M, int K, int N, const ffn_mxfp4_weight *gate,
                     const ffn_mxfp4_weight *up, const ffn_nvfp4_weight *down, int act, void *workspace,
                     size_t workspace_bytes, void *out, hipStream_t stream);

/* Bytes of device workspace ffn_w4a4_down_gemm and ffn_w4a4_forward_fp4 need
 * for (M, K, N): mx(x), h [M, N] bf16, mx(h), and the down projection's fp32
 * partial sums and ready words when its reduction is split over the compute
 * units (about 8 MB at K = 5120; one block of 128 token rows at a time);
 * each part rounded up to 256 bytes. 0 if M = 0 or the shape is unsupported
 * (as ffn_w4a4_dual_gemm, and N a multiple of 256). Contents need no
 * initialisation. */
size_t ffn_w4a4_fp4_workspace_bytes(int M, int K, int N);

/* W4A4 down GEMM: out[M, K] (bf16) = scale2_d * (mx(h) . mx(W_d)), the
 * products exact and summed in fp32 (dense_ffn.rs page, the native-FP4
 * prefill's down projection on the quantised down input).
 *   h          device, bf16 [M, N], 16-byte aligned
 *   down       host struct of an MXFP4 weight [K, N]
 *   out        device, bf16 [M, K], 16-byte aligned
 *   workspace  device, >= ffn_w4a4_fp4_workspace_bytes(M, K, N) bytes,
 *              16-byte aligned; clobbered (holds mx(h) and partial sums)
 * M: 0 .. 65536; K a positive multiple of 256 and N of 256, both at most
 * 65536 (else FFN_NVFP4_ERR_SHAPE). Calls that share a workspace must not
 * overlap (one stream). */
int ffn_w4a4_down_gemm(const void *h, int M, int N, int K, const ffn_mxfp4_weight *down, void *out,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/* The all-W4A4 FFN: out[M, K] (bf16) = down GEMM of h = bf16(act(gate) * up)
 * with gate and up from the W4A4 dual GEMM (the h epilogue of
 * ffn_w4a4_dual_gemm's products) and the down GEMM as ffn_w4a4_down_gemm.
 * `down` is an MXFP4 weight [K, N] (ffn_w4a4_prepare_weight of the NVFP4
 * down projection). Shapes and workspace as ffn_w4a4_down_gemm. */
int ffn_w4a4_forward_fp4(const void *x, int M, int K, int N, const ffn_mxfp4_weight *gate,
                         const ffn_mxfp4_weight *up, const ffn_mxfp4_weight *down, int act, void *workspace,
                         size_t workspace_bytes, void *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FFN_W4A4_H */
