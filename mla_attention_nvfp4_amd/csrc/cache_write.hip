// NVFP4 latent cache write for gfx950.
//
// [MO-MLA], commits 1-2: the latent is quantized once, before the cache
// write; [B12X], PR description: NVFP4 latent with a per-layer fp32 outer
// scale and an optional e4m3 RoPE cell; [B12X], review 1: 432/368-byte
// records.  One wavefront writes the records of 4 consecutive tokens (all
// of their loads issued first; 4 measured faster than 2, 8 or 16); for each
// token:
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

constexpr int kWaves = 4;   // wavefronts per workgroup
constexpr int kTpw = 4;     // tokens per wavefront, all loads issued before any is used

template <bool kRopeFp8>
__global__ __launch_bounds__(64 * kWaves)
void cache_write_kernel(const uint16_t* __restrict__ kv_c, int64_t kv_stride,
                        const uint16_t* __restrict__ k_pe, int64_t pe_stride,
                        const int64_t* __restrict__ slot_mapping, int64_t T,
                        uint8_t* __restrict__ cache, int64_t num_slots, float g) {
    constexpr int kRec = kRopeFp8 ? 368 : 432;
    const int lane = threadIdx.x & 63;
    const int64_t t0 = ((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6)) * kTpw;
    if (t0 >= T) return;

    // every load of the wavefront's tokens first (clamped to the last token),
    // so their latencies overlap
    u32x4 raw[kTpw];
    uint32_t pe[kTpw];
    int64_t slot[kTpw];
#pragma unroll
    for (int j = 0; j < kTpw; ++j) {
        const int64_t t = min(t0 + j, T - 1);
        raw[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kv_c + t * kv_stride + 8 * lane));
        pe[j] = lane < 32 ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(k_pe + t * pe_stride + 2 * lane)) : 0u;
        slot[j] = slot_mapping[t];
    }

#pragma unroll
    for (int j = 0; j < kTpw; ++j) {
        // (the same slot in every lane)
        const int64_t sl = (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)slot[j] >> 32)) << 32) |
                                     (uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)slot[j]));
        if (t0 + j >= T || sl < 0 || sl >= num_slots) continue;
        uint8_t* rec = cache + sl * kRec;

        // latent: 8 bf16 per lane
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo(raw[j][i]);
            x[2 * i + 1] = bf16_hi(raw[j][i]);
        }
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fmaxf(a, __builtin_fabsf(x[i]));
        a = wave_xor_max(a, 1);

        // two-level NVFP4 rule, one IEEE fp32 operation per step
        const Nvfp4Scale sc = nvfp4_block_scale(a, g);
        const uint32_t s = sc.code;
        reinterpret_cast<uint32_t*>(rec)[lane] = e2m1_encode8(x, sc.inv);

        // scales: block k is held by lanes 2k and 2k+1; lane k < 8 writes blocks 4k..4k+3
        const uint32_t s0 = __shfl(s, (8 * lane) & 63, 64);
        const uint32_t s1 = __shfl(s, (8 * lane + 2) & 63, 64);
        const uint32_t s2 = __shfl(s, (8 * lane + 4) & 63, 64);
        const uint32_t s3 = __shfl(s, (8 * lane + 6) & 63, 64);
        if (lane < 8)
            reinterpret_cast<uint32_t*>(rec + 256)[lane] = s0 | (s1 << 8) | (s2 << 16) | (s3 << 24);

        // RoPE: two values per lane
        if (lane < 32) {
            if (kRopeFp8) {
                reinterpret_cast<uint16_t*>(rec + 288)[lane] = (uint16_t)e4m3_encode2_hw(bf16_lo(pe[j]), bf16_hi(pe[j]));
            } else {
                reinterpret_cast<uint32_t*>(rec + 288)[lane] = pe[j];
            }
        }
        // reserved tail
        if (lane < 4) reinterpret_cast<uint32_t*>(rec + kRec - 16)[lane] = 0u;
    }
}

}  // namespace

hipError_t launch_cache_write(const uint16_t* kv_c, int64_t kv_stride, const uint16_t* k_pe,
                              int64_t pe_stride, const int64_t* slot_mapping, int64_t T,
                              uint8_t* cache, int64_t num_slots, bool rope_fp8, float g,
                              hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    const int64_t per_block = (int64_t)kWaves * kTpw;
    const dim3 grid((unsigned)((T + per_block - 1) / per_block));
    const dim3 block(64 * kWaves);
    if (rope_fp8)
        hipLaunchKernelGGL(cache_write_kernel<true>, grid, block, 0, stream, kv_c, kv_stride, k_pe,
                           pe_stride, slot_mapping, T, cache, num_slots, g);
    else
        hipLaunchKernelGGL(cache_write_kernel<false>, grid, block, 0, stream, kv_c, kv_stride, k_pe,
                           pe_stride, slot_mapping, T, cache, num_slots, g);
    return hipGetLastError();
}

}  // namespace mla
