// Roofline re-measurement kernels (gfx950): the MFMA rate of the two product
// shapes the kernels use, and a plain device copy for HBM bandwidth.  They
// compute nothing of the method; bench.py times them next to the vendor
// figures (HBM 8 TB/s, dense fp16/bf16 MFMA 2.5 PFLOP/s) so that a kernel's
// fraction of the roofline can be read against what the part delivers.
#include "device_common.hpp"
#include "roofline.hpp"

namespace mla {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// kShape 0: v_mfma_f32_16x16x32_f16, 8 independent accumulators;
// kShape 1: v_mfma_f32_32x32x16_f16, 4 independent accumulators.  Operands
// live in registers; one result per lane is stored so that nothing is dead.
// Each iteration is 8 products per wavefront.
template <int kShape>
__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, float seed, float* __restrict__ sink) {
    f16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(seed * (float)(threadIdx.x + i));
        b[i] = (_Float16)(seed - (float)i);
    }
    float r = 0.0f;
    if constexpr (kShape == 0) {
        f32x4 c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) r += c[j][0] + c[j][3];
    } else {
        f32x16 c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = f32x16{};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 8; ++j) c[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[j & 3], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) r += c[j][0] + c[j][15];
    }
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = r;
}

// Plain copy, grid-stride, 16 bytes per lane per access; four loads are issued
// before their stores so that each lane keeps 64 bytes in flight.
__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                          int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
        dst[i] = v0;
        dst[i + stride] = v1;
        dst[i + 2 * stride] = v2;
        dst[i + 3 * stride] = v3;
    }
    for (; i < n16; i += stride) dst[i] = src[i];
}

// Read-only stream: the wrapping 32-bit sum of src's words is added to *sum,
// one atomic per wavefront; four 16-byte loads in flight per lane.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sum) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
        const u32x4 v = (v0 + v1) + (v2 + v3);
        acc += (v[0] + v[1]) + (v[2] + v[3]);
    }
    for (; i < n16; i += stride) {
        const u32x4 v = src[i];
        acc += (v[0] + v[1]) + (v[2] + v[3]);
    }
    for (int off = 32; off > 0; off >>= 1) acc += (uint32_t)__shfl_xor((int)acc, off);
    if ((threadIdx.x & 63) == 0) atomicAdd(sum, acc);
}

}  // namespace

hipError_t launch_mfma_rate(int shape, int blocks, int iters, float* sink, hipStream_t stream) {
    if (shape == 0)
        hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, stream, iters, 0.001f, sink);
    else
        hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, iters, 0.001f, sink);
    return hipGetLastError();
}

hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    const int64_t want = (n16 + 255) / 256;
    const unsigned grid = (unsigned)(want < 8192 ? (want > 0 ? want : 1) : 8192);
    hipLaunchKernelGGL(stream_copy_kernel, dim3(grid), dim3(256), 0, stream, reinterpret_cast<const u32x4*>(src),
                       reinterpret_cast<u32x4*>(dst), n16);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sum, hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    const int64_t want = (n16 + 255) / 256;
    const unsigned grid = (unsigned)(want < 8192 ? (want > 0 ? want : 1) : 8192);
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, stream, reinterpret_cast<const u32x4*>(src), n16,
                       sum);
    return hipGetLastError();
}

}  // namespace mla
