// Host-side launchers of the roofline re-measurement kernels (roofline.hip).
// They compute nothing of the attention method.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// shape 0: 16x16x32 f16 products, shape 1: 32x32x16 f16 products; blocks of
// 256 lanes, 8 products per wavefront per iteration; one float per lane to sink.
hipError_t launch_mfma_rate(int shape, int blocks, int iters, float* sink, hipStream_t stream);
// dst[0, bytes) = src[0, bytes); bytes a multiple of 16, both 16-byte aligned.
hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);
// *sum += wrapping 32-bit sum of src's words; bytes a multiple of 16, src 16-byte aligned.
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sum, hipStream_t stream);

}  // namespace mla
