// NVFP4 quantization of fp32 rows with 128x4-swizzled e4m3 scales (gfx950).
//
// [FUSED-OUT], PR description: the stand-alone NVFP4 quantization pass over
// the attention output, which the prefill epilogue replaces; kept here as a
// directly checkable form of the epilogue's arithmetic and layout.  One
// thread per entry of the padded scale matrix: real entries quantize their
// 16 inputs (four 16-byte loads), store 8 code bytes and the scale byte;
// padding entries store a zero scale byte.  The block scale's quotient is
// formed as the prefill's P blocks form it (a multiply by fp32(1 / (6 g)),
// the division redone near e4m3 ties), with the same codes as the division.
#include "device_common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

__global__ __launch_bounds__(256) void quantize_rows_kernel(const float* __restrict__ x, int64_t M,
                                                            int K, float g, float u, float inv_u,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
    const int C = K / 16;
    const int cpad = (C + 3) & ~3;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t mpad = (M + 127) & ~(int64_t)127;
    if (idx >= mpad * cpad) return;
    const int64_t m = idx / cpad;
    const int c = (int)(idx % cpad);
    const int64_t so = swizzled_scale_offset(m, c, cpad);
    if (m >= M || c >= C) {
        scales[so] = 0;
        return;
    }
    const f32x4* src = reinterpret_cast<const f32x4*>(x + m * K + 16 * c);
    float v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x4 q = src[i];
        v[4 * i] = q[0];
        v[4 * i + 1] = q[1];
        v[4 * i + 2] = q[2];
        v[4 * i + 3] = q[3];
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, __builtin_fabsf(v[i]));
    const Nvfp4Scale sc = nvfp4_block_scale_fast(a, g, u, inv_u);
    const u32x2 w = {e2m1_encode8(v, sc.inv), e2m1_encode8(v + 8, sc.inv)};
    *reinterpret_cast<u32x2*>(codes + m * (K / 2) + 8 * c) = w;
    scales[so] = (uint8_t)sc.code;
}

}  // namespace

hipError_t launch_quantize_rows(const float* x, int64_t M, int K, float g, uint8_t* codes,
                                uint8_t* scales, hipStream_t stream) {
    const int C = K / 16;
    const int64_t cpad = (C + 3) & ~3;
    const int64_t n = ((M + 127) & ~(int64_t)127) * cpad;
    if (n == 0) return hipSuccess;
    const float u = 6.0f * g;          // fp32(6 g), as on the device
    const float inv_u = 1.0f / u;      // correctly rounded
    hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, x, M,
                       K, g, u, inv_u, codes, scales);
    return hipGetLastError();
}

}  // namespace mla
