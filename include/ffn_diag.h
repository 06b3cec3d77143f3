/*
 * ffn_diag.h -- measurement aid of libffn_nvfp4: the streaming-read ceiling.
 *
 * The decode GEMVs are bound by HBM bandwidth; their time is compared with
 * the time a kernel with the same load width and almost no arithmetic takes
 * to read the same bytes. ffn_diag_read reads every byte of up to 8 device
 * buffers once, in one launch: 16 bytes per lane per load, non-temporal,
 * four loads in flight per thread, one 512-thread workgroup per compute
 * unit, the buffers taken as one concatenated range. Timing one launch over
 * the three weights of an FFN gives the one-launch ceiling; one over W_g and
 * W_u then one over W_d gives the ceiling of a two-launch forward.
 *
 *   bufs   host array of n device pointers, each 16-byte aligned
 *   bytes  host array of n sizes, each a multiple of 16 (0 allowed)
 *   n      1 .. 8
 *   sink   device, one uint32, 4-byte aligned; written only when the XOR of
 *          everything read equals one fixed value (so that the loads cannot
 *          be optimised away); its contents mean nothing
 * Returns FFN_NVFP4_OK, FFN_NVFP4_ERR_NULL, FFN_NVFP4_ERR_ALIGN,
 * FFN_NVFP4_ERR_SHAPE (n out of range, a size not a multiple of 16) or
 * FFN_NVFP4_ERR_LAUNCH. Asynchronous on `stream`; nothing is allocated.
 */
#ifndef FFN_DIAG_H
#define FFN_DIAG_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int ffn_diag_read(const void *const *bufs, const size_t *bytes, int n, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FFN_DIAG_H */
