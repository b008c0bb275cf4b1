// Internal host-side launchers, one per kernel family.  Arguments have been
// validated by the C ABI layer (abi.hip) before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

hipError_t launch_cache_write(const uint16_t* kv_c, int64_t kv_stride, const uint16_t* k_pe,
                              int64_t pe_stride, const int64_t* slot_mapping, int64_t T,
                              uint8_t* cache, int64_t num_slots, bool rope_fp8, float g,
                              hipStream_t stream);

// Shared by dense and sparse decode.
struct DecodeArgs {
    const uint16_t* q_nope;
    const uint16_t* q_rope;
    int64_t q_stride_b, q_stride_h;
    const uint8_t* cache;
    int64_t num_pages;
    int record_bytes;
    int page_size;
    const int32_t* page_table;
    int max_pages;
    const int32_t* seq_lens;
    const int32_t* indices;   // null for dense
    int topk;
    int B, H;
    float outer_scale, softmax_scale;
    int max_splits;
    float* ws_out;            // [B][max_splits][H][512] fp32, or fp16 in the row's first half (null if max_splits == 1)
    float* ws_lse;            // [B][max_splits][H]
    uint8_t* ws_fmt;          // [B][max_splits][H]: 1 = that partial row is fp16, 0 = fp32
    float* out;               // [B][H][512]
    float* lse;               // [B][H]
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_narrow(const DecodeArgs& a, hipStream_t stream);   // H <= 16

// n = splits_per_seq[b] clamped to [0, S], or S if the pointer is null.
struct MergeArgs {
    const float* part_out;
    const float* part_lse;
    const int32_t* splits_per_seq;
    int B, S, H, D;
    float* out;
    float* lse;
};

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream);

hipError_t launch_quantize_rows(const float* x, int64_t M, int K, float g, uint8_t* codes,
                                uint8_t* scales, hipStream_t stream);

struct PrefillArgs {
    const uint16_t* q; int64_t q_st, q_sh;
    const uint16_t* k; int64_t k_st, k_sh;
    const uint16_t* v; int64_t v_st, v_sh;
    const int32_t* cu_seqlens;
    int N, max_seqlen;
    int64_t T;
    int H;
    float softmax_scale;
    unsigned flags;
    float g_q, g_k, g_v, g_p, g_out;
    void* workspace;
    uint8_t* out_fp4;
    uint8_t* out_scales;
    float* lse;
};

size_t prefill_workspace_bytes(int64_t T, int H, unsigned flags);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// Split policy shared by host and device code.
__host__ __device__ inline int decode_num_splits(int n, int max_splits) {
    if (n <= 0) return 1;
    const int tiles = (n + 63) / 64;
    int want = (n + 255) / 256;
    if (want > max_splits) want = max_splits;
    if (want < 1) want = 1;
    const int chunk = (tiles + want - 1) / want;
    return (tiles + chunk - 1) / chunk;
}

__host__ __device__ inline int decode_chunk_tiles(int n, int max_splits) {
    if (n <= 0) return 1;
    const int tiles = (n + 63) / 64;
    int want = (n + 255) / 256;
    if (want > max_splits) want = max_splits;
    if (want < 1) want = 1;
    return (tiles + want - 1) / want;
}

}  // namespace mla
