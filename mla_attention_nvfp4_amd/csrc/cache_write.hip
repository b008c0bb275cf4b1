// NVFP4 latent cache write for gfx950.
//
// [MO-MLA], commits 1-2: the latent is quantized once, before the cache
// write; [B12X], PR description: NVFP4 latent with a per-layer fp32 outer
// scale and an optional e4m3 RoPE cell; [B12X], review 1: 432/368-byte
// records.  One wavefront writes one token's record:
//   lane i owns latent elements 8i..8i+7 (half of block i/2): it loads them
//   with one 16-byte load, the block amax is exchanged with lane i^1, and
//   the lane stores its 8 codes as one dword, so the 256 code bytes leave as
//   one coalesced 256-byte store; lanes 0..7 store the 32 scale bytes as
//   dwords; lanes 0..31 move the RoPE part; lanes 0..3 zero the tail.
// HBM-bound: 1152 bytes read and one record written per token.
#include "device_common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int kTokensPerBlock = 4;  // one wavefront per token

template <bool kRopeFp8>
__global__ __launch_bounds__(64 * kTokensPerBlock)
void cache_write_kernel(const uint16_t* __restrict__ kv_c, int64_t kv_stride,
                        const uint16_t* __restrict__ k_pe, int64_t pe_stride,
                        const int64_t* __restrict__ slot_mapping, int64_t T,
                        uint8_t* __restrict__ cache, int64_t num_slots, float g) {
    constexpr int kRec = kRopeFp8 ? 368 : 432;
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kTokensPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) return;
    uint8_t* rec = cache + slot * kRec;

    // latent: 8 bf16 per lane
    const u32x4 raw = *reinterpret_cast<const u32x4*>(kv_c + t * kv_stride + 8 * lane);
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_lo(raw[i]);
        x[2 * i + 1] = bf16_hi(raw[i]);
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, __builtin_fabsf(x[i]));
    a = wave_xor_max(a, 1);

    // two-level NVFP4 rule, one IEEE fp32 operation per step
    const Nvfp4Scale sc = nvfp4_block_scale(a, g);
    const uint32_t s = sc.code;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= e2m1_encode(x[i] * sc.inv) << (4 * i);
    reinterpret_cast<uint32_t*>(rec)[lane] = word;

    // scales: block j is held by lanes 2j and 2j+1; lane k < 8 writes blocks 4k..4k+3
    const uint32_t s0 = __shfl(s, (8 * lane) & 63, 64);
    const uint32_t s1 = __shfl(s, (8 * lane + 2) & 63, 64);
    const uint32_t s2 = __shfl(s, (8 * lane + 4) & 63, 64);
    const uint32_t s3 = __shfl(s, (8 * lane + 6) & 63, 64);
    if (lane < 8)
        reinterpret_cast<uint32_t*>(rec + 256)[lane] = s0 | (s1 << 8) | (s2 << 16) | (s3 << 24);

    // RoPE: two values per lane
    if (lane < 32) {
        const uint32_t pe = *reinterpret_cast<const uint32_t*>(k_pe + t * pe_stride + 2 * lane);
        if (kRopeFp8) {
            const uint32_t c0 = e4m3_encode(bf16_lo(pe));
            const uint32_t c1 = e4m3_encode(bf16_hi(pe));
            reinterpret_cast<uint16_t*>(rec + 288)[lane] = (uint16_t)(c0 | (c1 << 8));
        } else {
            reinterpret_cast<uint32_t*>(rec + 288)[lane] = pe;
        }
    }
    // reserved tail
    if (lane < 4) reinterpret_cast<uint32_t*>(rec + kRec - 16)[lane] = 0u;
}

}  // namespace

hipError_t launch_cache_write(const uint16_t* kv_c, int64_t kv_stride, const uint16_t* k_pe,
                              int64_t pe_stride, const int64_t* slot_mapping, int64_t T,
                              uint8_t* cache, int64_t num_slots, bool rope_fp8, float g,
                              hipStream_t stream) {
    const dim3 grid((unsigned)((T + kTokensPerBlock - 1) / kTokensPerBlock));
    const dim3 block(64 * kTokensPerBlock);
    if (rope_fp8)
        hipLaunchKernelGGL(cache_write_kernel<true>, grid, block, 0, stream, kv_c, kv_stride, k_pe,
                           pe_stride, slot_mapping, T, cache, num_slots, g);
    else
        hipLaunchKernelGGL(cache_write_kernel<false>, grid, block, 0, stream, kv_c, kv_stride, k_pe,
                           pe_stride, slot_mapping, T, cache, num_slots, g);
    return hipGetLastError();
}

}  // namespace mla
