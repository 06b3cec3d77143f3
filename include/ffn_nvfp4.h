/*
 * ffn_nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 W4A16 gated-FFN library.
 *
 * The library computes the dense gated FFN of a decoding transformer layer,
 *     gate = W_g x,   up = W_u x,   h = act(gate) * up,   out = W_d h,
 * with NVFP4 weights and bf16 activations (dense_ffn.rs page, module doc
 * comment and DenseFfnLayer::forward: a dual gate+up GEMV over one activation
 * row, the activation, then the down GEMV).
 *
 * Weight format (dense_ffn.rs page, DenseFfnLayer::ensure_int8_weight doc
 * comment): a weight of logical shape [rows, cols] is
 *   - codes : uint8 [rows, cols/2], two E2M1 codes per byte; the code of the
 *             even column is the low nibble, the odd column the high nibble;
 *   - scales: uint8 [rows, cols/16], one E4M3FN scale per 16 consecutive
 *             columns of a row;
 *   - scale2: one fp32 per-tensor multiplier applied to the projection's
 *             output (dense_ffn.rs page, forward_prefill_inner FP4-MMQ branch:
 *             for gate and up it is applied before the nonlinearity).
 * Element (r, c) is e2m1(code) * e4m3(scale[r][c/16]) * scale2.
 * Shapes: W_g, W_u are [N, K]; W_d is [K, N]; K = hidden, N = intermediate.
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are device memory owned by the caller; the
 *     library never allocates, frees or keeps them past the call. Host structs
 *     are read during the call only.
 *   - Matrices are row-major and dense (no strides); x, h and out are
 *     [M, width] with row m at offset m*width.
 *   - Every call is asynchronous on `stream` (0 = the null stream): the
 *     library enqueues kernels and returns without synchronising. Inputs must
 *     stay valid and unmodified until the work completes.
 *   - M = 0 is an empty call: the weights, K, N and act are still validated,
 *     x / out / workspace may be NULL, nothing is launched, 0 is returned.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     error nothing is launched and a negative status is returned. Faults
 *     during execution surface at the caller's next synchronisation, as for
 *     any HIP kernel.
 *   - Results are deterministic: the same inputs on the same device give
 *     bit-identical outputs. Row m of a batched call is bit-identical to an
 *     M=1 call on that row for every M <= 8. Within each matrix-core arm (see
 *     the batch sizes below) a row's result does not depend on the other rows
 *     of the batch (in the small-batch arm, among batches with the same
 *     number of 16-row token groups); the arms differ from each other and
 *     from the M <= 8 arm in rounding, and the 128-row arm's forward splits
 *     its reductions by the device's compute-unit count.
 *   - The functions hold no global mutable state and may be called from
 *     several host threads (on distinct output buffers), except
 *     ffn_nvfp4_forward_noalloc, whose per-device scratch array is shared by
 *     all of its calls on that device.
 */
#ifndef FFN_NVFP4_H
#define FFN_NVFP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define FFN_NVFP4_OK 0
#define FFN_NVFP4_ERR_NULL (-1)          /* a required pointer is NULL */
#define FFN_NVFP4_ERR_ALIGN (-2)         /* codes / x / out / workspace not 16-byte aligned;
                                            scales not 2-byte (M > 8: 8-byte) aligned */
#define FFN_NVFP4_ERR_SHAPE (-3)         /* K or N not a positive multiple of 32 (of 64 when
                                            M > 8), or larger than 65536 */
#define FFN_NVFP4_ERR_BATCH (-4)         /* M outside the supported set (see below) */
#define FFN_NVFP4_ERR_ACT (-5)           /* unknown activation */
#define FFN_NVFP4_ERR_WORKSPACE (-6)     /* workspace smaller than ffn_nvfp4_workspace_bytes() */
#define FFN_NVFP4_ERR_LAUNCH (-7)        /* HIP reported an error when launching */
#define FFN_NVFP4_ERR_SCALE2 (-8)        /* scale2 is not finite */

/* Activation of the gate. SiLU(g) = g / (1 + e^-g) (Qwen/Llama);
 * GELU-tanh(g) = 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))) (Gemma).
 * dense_ffn.rs page, FfnActivation enum. */
typedef enum ffn_nvfp4_act {
    FFN_NVFP4_ACT_SILU = 0,
    FFN_NVFP4_ACT_GELU_TANH = 1
} ffn_nvfp4_act;

/* One NVFP4 weight (see the format above). codes: device, 16-byte aligned;
 * scales: device, 2-byte aligned; scale2: host value. */
typedef struct ffn_nvfp4_weight {
    const uint8_t *codes;
    const uint8_t *scales;
    float scale2;
} ffn_nvfp4_weight;

/* Supported batch sizes:
 *   M = 0            empty call;
 *   1 <= M <= 8      the weight-streaming GEMV arm: one launch per projection
 *                    for the whole batch, so each weight byte is read once for
 *                    all M rows (dense_ffn.rs page, forward_k2 / forward_k3 /
 *                    forward_km);
 *   9 <= M <= 65536  the matrix-core arms (dense_ffn.rs page, forward_prefill:
 *                    weights dequantised to bf16 feeding bf16 matrix products
 *                    with fp32 accumulation). They need K and N in multiples
 *                    of 64 (else ERR_SHAPE) and scales 8-byte aligned (else
 *                    ERR_ALIGN).
 *     9 <= M <= 40, K and N multiples of 256: the small-batch arm, weights
 *                    read and dequantised once for all rows (one token group
 *                    of 16 rows up to M = 16, two up to 32, three above); its
 *                    reductions are split in parts where a wave's
 *                    activations do not fit its registers, finished inside
 *                    the same launch;
 *     otherwise      the 128-row arm, in blocks of 128 token rows, each block
 *                    reading the weights once.
 * Other M: ERR_BATCH. K and N: positive multiples of 32, at most 65536. */

/* Bytes of device workspace ffn_nvfp4_forward needs for (M, K, N);
 * 0 if M = 0 or the shape is unsupported. For M <= 8 it holds h [M, N] bf16;
 * for the small-batch arm h, the fp32 partial sums of split reductions and
 * their ready words (about 23 MB at M = 40, K = 5120, N = 17408, mostly the
 * dual projection's partial sums);
 * for the 128-row arm, h for one block of up to 128 rows plus the fp32 slots
 * in which that arm leaves the pieces of split reductions (about 64 MiB,
 * whatever M). Its contents need no initialisation. */
size_t ffn_nvfp4_workspace_bytes(int M, int K, int N);

/* The whole FFN: out[M, K] (bf16) = W_d (act(W_g x) * (W_u x)) for
 * x[M, K] (bf16).
 *   x          device, bf16 [M, K], 16-byte aligned
 *   gate, up   host structs describing [N, K] weights
 *   down       host struct describing a [K, N] weight
 *   act        ffn_nvfp4_act
 *   workspace  device, >= ffn_nvfp4_workspace_bytes(M, K, N) bytes, 16-byte
 *              aligned; holds h = bf16(act(gate) * up) between the two
 *              projections (and, for M > 8, partial sums); clobbered by
 *              the call; calls that share a workspace must not overlap
 *   out        device, bf16 [M, K], 16-byte aligned; may not alias x
 * The intermediate h = act(gate) * up is rounded to bf16 once; gate and up
 * are kept in fp32 up to that point. */
int ffn_nvfp4_forward(const void *x, int M, int K, int N,
                      const ffn_nvfp4_weight *gate, const ffn_nvfp4_weight *up,
                      const ffn_nvfp4_weight *down, int act,
                      void *workspace, size_t workspace_bytes,
                      void *out, hipStream_t stream);

/* ffn_nvfp4_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, serving loops,
 * harnesses that forbid hipMalloc). It computes exactly what
 * ffn_nvfp4_forward computes, bit for bit, with the workspace taken from a
 * static device array of the library: 4 MiB per device, held by every device
 * that runs this entry point until the process ends. The call allocates and
 * frees nothing.
 *   - Shapes whose ffn_nvfp4_workspace_bytes(M, K, N) exceeds 4 MiB return
 *     FFN_NVFP4_ERR_WORKSPACE and launch nothing. M <= 8 always fits
 *     (M * N * 2 bytes); the 128-row matrix-core arm never does.
 *   - `stream` must belong to the current device (else FFN_NVFP4_ERR_LAUNCH).
 *   - Every call on one device shares that device's array: calls that
 *     overlap on one device (other streams, other host threads) race and
 *     must be ordered by the caller. The contents need no initialisation.
 * The other arguments, and every error code, are those of ffn_nvfp4_forward. */
int ffn_nvfp4_forward_noalloc(const void *x, int M, int K, int N,
                              const ffn_nvfp4_weight *gate, const ffn_nvfp4_weight *up,
                              const ffn_nvfp4_weight *down, int act,
                              void *out, hipStream_t stream);

/* Dual GEMV (one pass over x for both projections; dense_ffn.rs page,
 * DenseFfnLayer::forward, w4a16_gemv_dual). For M > 8 it runs the
 * small-batch arm when that arm covers the shape without splitting the
 * reduction, else the 128-row arm with one workgroup per output tile (no
 * workspace either way):
 *   gate_out[m, n] = scale2_g * sum_k W_g[n, k] x[m, k]
 *   up_out[m, n]   = scale2_u * sum_k W_u[n, k] x[m, k]
 *   x          device, bf16 [M, K], 16-byte aligned
 *   gate_out   device, fp32 [M, N], 16-byte aligned
 *   up_out     device, fp32 [M, N], 16-byte aligned */
int ffn_nvfp4_dual_gemv(const void *x, int M, int K, int N,
                        const ffn_nvfp4_weight *gate, const ffn_nvfp4_weight *up,
                        float *gate_out, float *up_out, hipStream_t stream);

/* Down GEMV with the activation fused into its input load (dense_ffn.rs
 * page, DenseFfnLayer::forward, w4a16_gemv_silu_input / gelu_mul). For M > 8
 * it runs the 128-row matrix-core arm with one workgroup per output tile (no
 * workspace, so it is much slower than the forward's down projection):
 *   out[m, j] = bf16(scale2_d * sum_n W_d[j, n] * bf16(act(gate[m, n]) * up[m, n]))
 *   gate_in, up_in   device, fp32 [M, N] (as written by the dual GEMV),
 *                    16-byte aligned
 *   down             host struct describing a [K, N] weight
 *   out              device, bf16 [M, K], 16-byte aligned */
int ffn_nvfp4_down_gemv(const float *gate_in, const float *up_in, int M, int N, int K,
                        const ffn_nvfp4_weight *down, int act,
                        void *out, hipStream_t stream);

/* BF16 -> NVFP4 weight quantiser: produces the codes, scales and scale2 the
 * entry points above take (qwen35_dense.rs page, weight loader: a dense BF16
 * weight is quantised on the GPU by a global-absmax pass, then a pass that
 * writes the packed codes and per-16 scales). The pages give no scale rule;
 * this one fills both formats:
 *   scale2       = amax / (6 * 448)                      (amax = max |w|)
 *   scale byte   = E4M3(bmax / (6 * scale2))   per 16 columns, bmax = the block's max |w|
 *   code         = E2M1(w * (1 / (E4M3 value * scale2)))
 * each rounded to the nearest representable value (ties to the even
 * encoding), E4M3 at most 448 and E2M1 at most 6, a code keeping the sign of
 * its input (negatives that round to zero encode -0); a zero code where
 * E4M3 value * scale2 is zero, and all zeros (scale2 = 0) when amax = 0. Each
 * arithmetic step is one correctly rounded fp32 division or multiplication,
 * so the result is reproducible bit for bit. w must be finite.
 *   w          device, bf16 [rows, cols], 16-byte aligned
 *   rows       1 .. 65536
 *   cols       a positive multiple of 32, at most 65536
 *   codes      device, uint8 [rows, cols/2], 8-byte aligned (written)
 *   scales     device, uint8 [rows, cols/16] (written)
 *   scale2     device, one fp32, 4-byte aligned (written; copy it to the
 *              host for ffn_nvfp4_weight.scale2)
 *   workspace  device, >= ffn_nvfp4_quantize_workspace_bytes(rows, cols)
 *              bytes, 4-byte aligned; clobbered; calls that share it must not
 *              overlap
 * Two kernel launches on `stream`; asynchronous like every entry point. */
size_t ffn_nvfp4_quantize_workspace_bytes(int rows, int cols);
int ffn_nvfp4_quantize(const void *w, int rows, int cols, uint8_t *codes, uint8_t *scales, float *scale2,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Static text for a status code. */
const char *ffn_nvfp4_strerror(int status);

/* Library version as 10000*major + 100*minor + patch. */
int ffn_nvfp4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FFN_NVFP4_H */
