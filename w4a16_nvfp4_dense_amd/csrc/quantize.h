// quantize.h -- internal launcher of the BF16 -> NVFP4 quantiser (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ffn {

// Workgroups of either pass at most; the absmax pass leaves one uint32 of
// workspace per workgroup.
constexpr int kQuantizeMaxPartials = 2048;

// w: bf16 [rows, cols] (16-byte aligned, cols a multiple of 16); writes codes
// [rows, cols/2] (8-byte aligned), scales [rows, cols/16] and *scale2 (device
// fp32); partial: kQuantizeMaxPartials uint32 of workspace. Two launches on
// `stream`; returns the first HIP launch error.
hipError_t launch_quantize(const void *w, int rows, int cols, uint8_t *codes, uint8_t *scales, float *scale2,
                           uint32_t *partial, hipStream_t stream);

}  // namespace ffn
