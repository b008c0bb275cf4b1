// Cached-context gather from the paged NVFP4 latent cache into bf16 rows
// (gfx950).
//
// [MO-MLA], commit 2: the cached-context chunks of a prefill are gathered
// from the quantized paged cache (and then projected and quantized again as
// prefill operands); [B12X], walkthrough: records are located through the
// block table and the per-layer outer scale is restored on read.
//
// One wavefront per token: lane l dequantizes latent elements 8l .. 8l+7
// (one code word and its block's e4m3 scale) as fp32(g * (s * v)), rounded
// to bf16 (s * v is exact), and stores 16 bytes; lanes 0..7 copy or widen
// the RoPE part (bf16 as stored, e4m3 values exactly in bf16).  A position
// whose page id is outside [0, num_pages), or that lies past the page table,
// gives a zero row.
#include "device_common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

template <bool kRopeFp8>
__global__ __launch_bounds__(256) void cache_gather_kernel(const uint8_t* __restrict__ cache, int64_t num_pages,
                                                           int page_size, uint32_t page_recip,
                                                           const int32_t* __restrict__ page_table, int max_pages,
                                                           const int32_t* __restrict__ cu_ctx,
                                                           const int32_t* __restrict__ ctx_start, float g,
                                                           uint16_t* __restrict__ kv_out, int64_t kv_stride,
                                                           uint16_t* __restrict__ pe_out, int64_t pe_stride) {
    constexpr int kRec = kRopeFp8 ? 368 : 432;
    const int n = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int j = blockIdx.x * 4 + (threadIdx.x >> 6);   // token of this sequence's chunk
    const int r0 = cu_ctx[n];
    if (j >= cu_ctx[n + 1] - r0) return;
    const int64_t r = (int64_t)r0 + j;
    const int pos = (ctx_start ? ctx_start[n] : 0) + j;
    int64_t off = -1;
    if (pos >= 0 && (int64_t)pos < (int64_t)max_pages * page_size) {
        int pi, rem;
        page_divmod(pos, page_size, page_recip, pi, rem);
        const int pg = page_table[(int64_t)n * max_pages + pi];
        if (pg >= 0 && pg < num_pages) off = ((int64_t)pg * page_size + rem) * kRec;
    }
    u32x4 kv = {0u, 0u, 0u, 0u};
    u32x4 pe = {0u, 0u, 0u, 0u};
    if (off >= 0) {
        const uint8_t* rp = cache + off;
        const uint32_t c = *reinterpret_cast<const uint32_t*>(rp + 4 * lane);
        const float s = e4m3_decode(rp[256 + (lane >> 1)]);
        const f32x2 v0 = e2m1_pair<0>(c), v1 = e2m1_pair<1>(c), v2 = e2m1_pair<2>(c), v3 = e2m1_pair<3>(c);
        kv = u32x4{pack_bf16_rne(g * (v0[0] * s), g * (v0[1] * s)), pack_bf16_rne(g * (v1[0] * s), g * (v1[1] * s)),
                   pack_bf16_rne(g * (v2[0] * s), g * (v2[1] * s)), pack_bf16_rne(g * (v3[0] * s), g * (v3[1] * s))};
        if (lane < 8) {
            if constexpr (kRopeFp8) {
                const u32x2 w = *reinterpret_cast<const u32x2*>(rp + 288 + 8 * lane);
                const u32x2 y0 = e4m3x4_to_bf16(w[0]), y1 = e4m3x4_to_bf16(w[1]);
                pe = u32x4{y0[0], y0[1], y1[0], y1[1]};
            } else {
                pe = *reinterpret_cast<const u32x4*>(rp + 288 + 16 * lane);
            }
        }
    }
    *reinterpret_cast<u32x4*>(kv_out + r * kv_stride + 8 * lane) = kv;
    if (lane < 8) *reinterpret_cast<u32x4*>(pe_out + r * pe_stride + 8 * lane) = pe;
}

}  // namespace

hipError_t launch_cache_gather(const uint8_t* cache, int64_t num_pages, bool rope_fp8, int page_size,
                               uint32_t page_recip, const int32_t* page_table, int max_pages,
                               const int32_t* cu_ctx, const int32_t* ctx_start, int N, int max_ctx_len,
                               float g, uint16_t* kv_out, int64_t kv_stride, uint16_t* pe_out,
                               int64_t pe_stride, hipStream_t stream) {
    const dim3 grid((unsigned)((max_ctx_len + 3) / 4), (unsigned)N);
    if (rope_fp8)
        hipLaunchKernelGGL(cache_gather_kernel<true>, grid, dim3(256), 0, stream, cache, num_pages, page_size,
                           page_recip, page_table, max_pages, cu_ctx, ctx_start, g, kv_out, kv_stride, pe_out,
                           pe_stride);
    else
        hipLaunchKernelGGL(cache_gather_kernel<false>, grid, dim3(256), 0, stream, cache, num_pages, page_size,
                           page_recip, page_table, max_pages, cu_ctx, ctx_start, g, kv_out, kv_stride, pe_out,
                           pe_stride);
    return hipGetLastError();
}

}  // namespace mla

// Raw latent cache write: record = the token's 512 bf16 latent values then
// its 64 bf16 RoPE values (1152 bytes), the cache that decode_qdq_kernel
// quantizes on read.  One wavefront per token: 64 lanes x 16 bytes of
// latent, lanes 0..7 x 16 bytes of RoPE.
namespace mla {
namespace {

__global__ __launch_bounds__(256) void raw_cache_write_kernel(const uint16_t* __restrict__ kv, int64_t kv_stride,
                                                              const uint16_t* __restrict__ pe, int64_t pe_stride,
                                                              const int64_t* __restrict__ slots, int64_t T,
                                                              uint8_t* __restrict__ cache, int64_t num_slots) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= T) return;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) return;
    uint8_t* rec = cache + slot * 1152;
    *reinterpret_cast<u32x4*>(rec + 16 * lane) = *reinterpret_cast<const u32x4*>(kv + t * kv_stride + 8 * lane);
    if (lane < 8)
        *reinterpret_cast<u32x4*>(rec + 1024 + 16 * lane) = *reinterpret_cast<const u32x4*>(pe + t * pe_stride + 8 * lane);
}

}  // namespace

hipError_t launch_raw_cache_write(const uint16_t* kv_c, int64_t kv_stride, const uint16_t* k_pe, int64_t pe_stride,
                                  const int64_t* slot_mapping, int64_t T, uint8_t* cache, int64_t num_slots,
                                  hipStream_t stream) {
    hipLaunchKernelGGL(raw_cache_write_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream, kv_c, kv_stride,
                       k_pe, pe_stride, slot_mapping, T, cache, num_slots);
    return hipGetLastError();
}

}  // namespace mla
