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

// Cached-context gather: rows [cu_ctx[n], cu_ctx[n+1]) of the outputs are
// positions ctx_start[n] (0 if null) onward of sequence n, dequantized.
hipError_t launch_cache_gather(const uint8_t* cache, int64_t num_pages, bool rope_fp8, int page_size,
                               uint32_t page_recip, const int32_t* page_table, int max_pages,
                               const int32_t* cu_ctx, const int32_t* ctx_start, int N, int max_ctx_len,
                               float g, uint16_t* kv_out, int64_t kv_stride, uint16_t* pe_out,
                               int64_t pe_stride, hipStream_t stream);

// Shared by dense and sparse decode.
struct DecodeArgs {
    const uint16_t* q_nope;
    const uint16_t* q_rope;
    int64_t q_stride_b, q_stride_h;
    const uint8_t* cache;
    int64_t num_pages;
    int record_bytes;
    int page_size;
    uint32_t page_recip;      // page_recip_of(page_size)
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
    // quantized operands (decode_kernel with P quantized; 0 = plain decode):
    // bit 1 Q quantized (bit 16: as per-tensor FP8), multipliers g_q, g_p
    unsigned qdq_flags;
    float g_q, g_p;
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_narrow(const DecodeArgs& a, hipStream_t stream);   // H <= 16
// Dense decode on NVFP4 records (H > 16) with P quantized (a.qdq_flags bit 4;
// FP8 with bit 64) and Q by bit 1 / 16, a.g_q, a.g_p; then the split merge.
hipError_t launch_decode_pq(const DecodeArgs& a, hipStream_t stream);
// Merge of a decode launch's split partials (after the decode kernel).
hipError_t launch_split_merge(const DecodeArgs& a, hipStream_t stream);
// Decode with quantized operands (dense; record_bytes 432, 368 or 1152 raw).
// flags: 1 Q, 2 K, 4 P, 8 V quantized; 16/32/64/128 the same as per-tensor FP8.
hipError_t launch_decode_qdq(const DecodeArgs& a, unsigned flags, float g_q, float g_k, float g_v, float g_p,
                             hipStream_t stream);
// Raw (bf16) latent cache records: kv_c then k_pe, 1152 bytes.
hipError_t launch_raw_cache_write(const uint16_t* kv_c, int64_t kv_stride, const uint16_t* k_pe, int64_t pe_stride,
                                  const int64_t* slot_mapping, int64_t T, uint8_t* cache, int64_t num_slots,
                                  hipStream_t stream);

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

// Prefill attention.  flags: 1 Q, 2 K, 4 P, 8 V quantized; 16/32/64/128 the
// same operand as per-tensor FP8 instead of NVFP4; 256 2:4 score sparsity.
struct PrefillArgs {
    const uint16_t* q; int64_t q_st, q_sh;
    const uint16_t* k; int64_t k_st, k_sh;
    const uint16_t* v; int64_t v_st, v_sh;
    const int32_t* cu_seqlens;   // query rows of each sequence
    const int32_t* cu_k;         // key rows of each sequence (context attention; unused when causal)
    int N, max_seqlen, max_seqlen_k;
    int64_t T, T_k;              // query rows, key rows (T_k = T when causal)
    int H;
    int causal;                  // keys are the query rows (row i sees keys j <= i)
    float softmax_scale;
    unsigned flags;
    float g_q, g_k, g_v, g_p, g_out;
    void* workspace;
    uint8_t* out_fp4;            // NVFP4 output (codes [T,H,64] + swizzled scales), or null:
    uint8_t* out_scales;
    float* out_f32;              // fp32 rows, (t, h, d) at t*o_st + h*o_sh + d
    int64_t o_st, o_sh;
    float* lse;                  // (t, h) at t*lse_st + h*lse_sh, or null
    int64_t lse_st, lse_sh;
};

size_t prefill_workspace_bytes(int64_t T, int H, unsigned flags);
int prefill_p_tile();   // the attention kernel's key tile (the P schedule)
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// Division of a token position by the page size without an integer
// division sequence: with r = min(floor(2^32 / d), 2^32 - 1) and
// 0 <= n < 2^31, q0 = floor(n r / 2^32) satisfies n/d - 1 < q0 <= n/d
// (n r / 2^32 >= n (2^32/d - 1) / 2^32 > n/d - 1), so one correction step
// gives floor(n / d) and n mod d.
__host__ __device__ inline uint32_t page_recip_of(int d) {
    const uint64_t r = (uint64_t(1) << 32) / (uint64_t)(d < 1 ? 1 : d);
    return r > 0xffffffffull ? 0xffffffffu : (uint32_t)r;
}
__device__ inline void page_divmod(int n, int d, uint32_t r, int& q, int& rem) {
    uint32_t qq = __umulhi((uint32_t)n, r);
    uint32_t rr = (uint32_t)n - qq * (uint32_t)d;
    if (rr >= (uint32_t)d) {
        ++qq;
        rr -= (uint32_t)d;
    }
    q = (int)qq;
    rem = (int)rr;
}

// XCD-aware placement of decode work items.  Workgroups are dispatched
// round-robin over the 8 XCDs (each with its own L2) in linear-id order.
// When the number N of (sequence, head group) units is a multiple of 8, the
// linear id L maps to unit u = x + 8 (k / S) and split s = k % S, with
// x = L % 8 and k = L / 8, so that all S splits of a unit run on XCD u % 8
// and share that L2 for Q and the page table; this is a bijection of
// [0, S N) onto [0, S) x [0, N).  Otherwise u = L / S and s = L % S.
__device__ inline void decode_work_item(int S, int N, int& s, int& u) {
    const int L = (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
    if ((N & 7) == 0) {
        const int k = L >> 3;
        u = (L & 7) + 8 * (k / S);
        s = k % S;
    } else {
        s = L % S;
        u = L / S;
    }
}

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
