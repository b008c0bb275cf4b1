/*
 * mla_nvfp4.h -- C ABI of the NVFP4 MLA attention library for AMD Instinct
 * MI355X (gfx950): libmla_nvfp4.so.
 *
 * DeepSeek-style multi-head latent attention (MLA) whose latent KV cache is
 * stored as NVFP4: 512 e2m1 codes two per byte, one e4m3 scale per 16
 * elements, a per-layer fp32 outer scale, and a 64-d RoPE part in bf16 or
 * e4m3.  The pages this interface follows, cited by title and section:
 *
 *  [FUSED-OUT] vLLM pull request "feat: MLA prefill NVFP4 fused output"
 *  [MO-MLA]    Model-Optimizer pull request "Add NVFP4/FP8 Q/K/P/V + 2:4
 *              attention quantization for MLA (vLLM TRITON_MLA)"
 *  [B12X]      b12x pull request "nvfp4 MLA KV cache + per-layer outer-scale +
 *              fp8-RoPE KV-cell (sm120)"
 *
 * Conventions for every call
 * --------------------------
 *  - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or synchronises; it enqueues its kernels on
 *    `stream` (a hipStream_t; NULL is the null stream) and returns at once.
 *    Results are ordered on that stream.
 *  - bf16 tensors are passed as uint16_t bit patterns.  Strides are in
 *    elements.  All other tensors are dense row-major as stated.
 *  - Return value: MLA_OK (0) or a negative mla_status.  Arguments are
 *    validated on the host before anything is enqueued; on error nothing is
 *    enqueued and mla_last_error() (thread-local) describes the problem.
 *  - Device-side preconditions that are not checked on the host are listed
 *    per call; where a cheap check avoids an out-of-bounds access the kernel
 *    performs it and skips the offending element instead.
 *  - Only gfx950 devices are supported (MLA_ERR_UNSUPPORTED_DEVICE otherwise),
 *    the analogue of [B12X], review 1's point that the NVFP4 kernels need a
 *    guard for the one architecture they were built for.
 *  - A dispatch counts each grid dimension's work-items in 32 bits, so every
 *    launch of a call must fit below 2^32 of them.  A request that would not
 *    is refused with MLA_ERR_UNSUPPORTED, and the caller splits it: more than
 *    268,435,440 tokens in one NVFP4 cache write or 67,108,860 in one raw
 *    cache write, T * H or a sequence length above 268,435,440 in one
 *    prefill (its keys, in the attention call), a context above 67,108,860
 *    tokens in one gather, or more than 2^32 (row, 16-column block) pairs,
 *    rows padded to 128 and blocks to 4, in one row quantization.
 */
#ifndef MLA_NVFP4_H
#define MLA_NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARGUMENT = -1,
    MLA_ERR_RECORD_BYTES = -2,       /* record width not 368 or 432 */
    MLA_ERR_UNSUPPORTED_DEVICE = -3, /* current device is not gfx950 */
    MLA_ERR_WORKSPACE_TOO_SMALL = -4,
    MLA_ERR_HIP = -5,                /* a HIP runtime call failed */
    MLA_ERR_UNSUPPORTED = -6         /* valid request the library does not serve */
} mla_status;

/* Fixed geometry of the latent ([MO-MLA], PR body: absorbed decode over a
 * 512-d latent plus 64-d RoPE; [B12X], review 1: records of 432/368 bytes). */
#define MLA_D_LATENT 512
#define MLA_D_ROPE 64
#define MLA_RECORD_BYTES_BF16_ROPE 432
#define MLA_RECORD_BYTES_FP8_ROPE 368
/* Raw (unquantized) latent record of mla_decode_qdq: 512 + 64 bf16 values. */
#define MLA_RAW_RECORD_BYTES 1152
/* Prefill head dims ([MO-MLA], commit 1: asymmetric 192/128 head dims). */
#define MLA_PREFILL_D_QK 192
#define MLA_PREFILL_D_V 128
/* Key-tile width of the prefill P-quantization schedule (see
 * mla_prefill_nvfp4_out); mla_prefill_p_tile() returns the library's value. */
#define MLA_PREFILL_P_TILE 64
/* Decode splits cover at least this many tokens (see mla_decode_num_splits). */
#define MLA_DECODE_MIN_SPLIT_TOKENS 256

/* qdq_flags bits of mla_prefill_nvfp4_out and mla_prefill_attention.
 * [MO-MLA], commit 1: every prefill matmul operand is fake-quantized once
 * along its own contraction axis, as NVFP4 (1x16 blocks, e4m3 scale) or as
 * per-tensor FP8; and new-token attention may carry token-exact N:M score
 * sparsity.  MLA_QDQ_x switches operand x's quantization on (NVFP4 unless
 * its MLA_QDQ_FP8_x bit is also set; an FP8 bit without its operand's bit is
 * an error).  Per-tensor FP8 of x with multiplier g: code = e4m3(fp32(x *
 * fp32(1/g))) (RNE, satfinite), x_hat = g * value(code); for P every element
 * is quantized so with multiplier g_p (1/448 suits p <= 1). */
#define MLA_QDQ_Q 1u
#define MLA_QDQ_K 2u
#define MLA_QDQ_P 4u
#define MLA_QDQ_V 8u
#define MLA_QDQ_FP8_Q 16u
#define MLA_QDQ_FP8_K 32u
#define MLA_QDQ_FP8_P 64u
#define MLA_QDQ_FP8_V 128u
#define MLA_QDQ_FP8_MASK 240u
/* 2:4 score sparsity: in each group of 4 keys starting at a local key index
 * divisible by 4, a query row keeps its 2 largest scores and masks the other
 * two before the softmax; a key the row cannot see (causal mask, or past the
 * end) ranks as -inf, and of equal scores the lower key index ranks first.
 * The choice compares the fp32-accumulated scores (exact when Q and K are
 * quantized; unquantized bf16 scores within rounding of each other may be
 * chosen either way). */
#define MLA_PREFILL_SPARSE_2_4 256u

/* Thread-local text of the last error raised on this thread ("" if none). */
const char* mla_last_error(void);

/* Record width for a RoPE part in e4m3 (rope_fp8 != 0: 368) or bf16 (432).
 * [B12X], review 1: the record width is the authoritative ABI and decides
 * the RoPE storage type. */
int mla_nvfp4_record_bytes(int rope_fp8);

/* Number of split-K chunks decode uses for a sequence of `seq_len` tokens
 * (or a top-k list of `seq_len` entries) with at most `max_splits` chunks:
 * want = clamp(ceil(seq_len / MLA_DECODE_MIN_SPLIT_TOKENS), 1, max_splits),
 * chunk = ceil(ceil(seq_len/64) / want) tiles of 64 tokens, result =
 * ceil(ceil(seq_len/64) / chunk) (never an empty chunk); 1 for seq_len <= 0.
 * The kernels evaluate the same function on the device. */
int mla_decode_num_splits(int seq_len, int max_splits);

/* Bytes of decode workspace for B sequences, H heads, max_splits chunks:
 * partial outputs [B][max_splits][H][512] (fp32 rows; a row may instead hold
 * fp16 values in its first half), then partial LSE fp32 [B][max_splits][H],
 * then one format byte per partial row [B][max_splits][H] (1 = fp16), each
 * region 256-byte aligned.  0 when max_splits <= 1.  No initial contents are
 * needed; calls that may run concurrently need separate workspaces. */
size_t mla_decode_workspace_bytes(int B, int H, int max_splits);

/* Key-tile width BN_P of the prefill's P-quantization schedule: keys are
 * visited in tiles of BN_P from key 0, and P is quantized against the running
 * max as it stands after each tile.  [MO-MLA], commit 1: its eager oracles
 * follow the kernels' schedules, because P's quantization depends on the max
 * the kernel holds when it quantizes; the tile width is therefore part of the
 * definition of mla_prefill_nvfp4_out with MLA_QDQ_P set.  Returns the value
 * the kernels were compiled with (MLA_PREFILL_P_TILE). */
int mla_prefill_p_tile(void);

/* Bytes of a 128x4-swizzled e4m3 scale buffer for `rows` rows of
 * `scale_cols` scales: ceil(rows/128)*128 * (ceil(scale_cols/4)*4). */
size_t mla_nvfp4_swizzled_scale_bytes(int64_t rows, int64_t scale_cols);

/* Write T tokens into the NVFP4 latent cache.
 * [MO-MLA], commits 1-2 (the latent is quantized once, before the cache
 * write, and decode consumes that representation as is); [B12X], PR
 * description (NVFP4 latent with a per-layer fp32 outer scale; optional fp8
 * RoPE cell).
 *
 *  kv_c          bf16 [T, 512], row stride kv_c_row_stride (multiple of 8),
 *                16-byte aligned
 *  k_pe          bf16 [T, 64], row stride k_pe_row_stride (even), 4-byte
 *                aligned
 *  slot_mapping  int64 [T]: destination slot of token t; a slot < 0 or
 *                >= num_slots skips the token
 *  cache         uint8 [num_slots, record_bytes], 16-byte aligned
 *  record_bytes  432 (bf16 RoPE) or 368 (e4m3 RoPE), else MLA_ERR_RECORD_BYTES
 *  outer_scale   the latent's dequant multiplier g (finite, > 0)
 *
 * Record layout: bytes [0,256) codes, element 2i in the low nibble of byte i;
 * [256,288) 32 e4m3 block scales; then 64 RoPE values (bf16 little-endian, or
 * e4m3 RNE-satfinite of the bf16 value, unscaled); last 16 bytes zero.  Per
 * block of 16: a = max|x|, t = a / (6 g), s = e4m3(t) (RNE, satfinite),
 * d = s * g, code_i = e2m1(x_i * (d == 0 ? 0 : 1/d)) (RNE, satfinite, sign
 * kept), each step one IEEE fp32 operation.  T == 0 is a no-op.
 * Precondition (unchecked): no two tokens share a slot. */
int mla_nvfp4_cache_write(const uint16_t* kv_c, int64_t kv_c_row_stride,
                          const uint16_t* k_pe, int64_t k_pe_row_stride,
                          const int64_t* slot_mapping, int64_t T,
                          uint8_t* cache, int64_t num_slots, int record_bytes,
                          float outer_scale, void* stream);

/* Dense absorbed split-K decode over the paged NVFP4 latent cache.
 * [MO-MLA], commit 1 (split-K absorbed decode over the paged latent with
 * grouped query heads; natural-log LSE for merging) and commit 3 (V is the
 * stored latent itself); [B12X], walkthrough (stage, dequantize, accumulate;
 * outer scale restored on read) and review 2 (Q is bf16, unquantized).
 *
 * For sequence b (L = min(seq_lens[b], max_pages_per_seq * page_size)) and
 * head h, token j < L is record page_table[b][j / page_size] * page_size +
 * j % page_size of the cache.  With k_j = outer_scale * dequant(latent_j),
 * r_j the RoPE part:  z_j = softmax_scale * (q_nope . k_j + q_rope . r_j),
 * out[b][h] = sum_j e^(z_j - m) k_j / sum_j e^(z_j - m), lse[b][h] = m +
 * ln sum_j e^(z_j - m).  L == 0 gives out = 0, lse = -inf.
 *
 *  q_nope, q_rope  bf16 [B, H, 512] and [B, H, 64] with common strides
 *                  q_stride_b, q_stride_h (multiples of 8; 16-byte aligned)
 *  cache           uint8 [num_pages * page_size, record_bytes]
 *  page_table      int32 [B, max_pages_per_seq]
 *  seq_lens        int32 [B]
 *  max_splits      >= 1; sequence b is split into
 *                  mla_decode_num_splits(L, max_splits) chunks whose
 *                  (out, lse) partials are merged as mla_lse_merge does
 *  workspace       >= mla_decode_workspace_bytes(B, H, max_splits) bytes
 *                  (may be NULL when max_splits == 1)
 *  out, lse        fp32 [B, H, 512] and [B, H]
 *
 * Kernel-side checks: a page id outside [0, num_pages) masks that token.
 * Enqueued on `stream`: the decode kernel, which writes single-chunk
 * sequences directly and the partials of split ones to the workspace, then
 * (max_splits > 1) a merge kernel combining each split sequence's partials
 * in chunk order (bitwise deterministic). */
int mla_decode_nvfp4(const uint16_t* q_nope, const uint16_t* q_rope,
                     int64_t q_stride_b, int64_t q_stride_h,
                     const uint8_t* cache, int64_t num_pages, int record_bytes,
                     int page_size, const int32_t* page_table, int max_pages_per_seq,
                     const int32_t* seq_lens, int B, int H,
                     float outer_scale, float softmax_scale, int max_splits,
                     void* workspace, size_t workspace_bytes,
                     float* out, float* lse, void* stream);

/* Allocation-free form of mla_decode_nvfp4, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments and results as mla_decode_nvfp4
 * without the workspace: the split partials go to a scratch array of
 * MLA_DECODE_NOALLOC_SCRATCH_BYTES that the library holds on each device it
 * runs on, from load until the process ends.  A request whose workspace
 * (mla_decode_workspace_bytes(B, H, max_splits)) exceeds that size returns
 * MLA_ERR_WORKSPACE_TOO_SMALL and enqueues nothing.  The call allocates and
 * frees nothing; the scratch needs no initial contents.  Every call on one
 * device shares that device's scratch: calls that may overlap on one device
 * (different streams, or other host threads) race and must be serialised by
 * the caller. */
#define MLA_DECODE_NOALLOC_SCRATCH_BYTES (128u << 20)
int mla_decode_nvfp4_noalloc(const uint16_t* q_nope, const uint16_t* q_rope,
                             int64_t q_stride_b, int64_t q_stride_h,
                             const uint8_t* cache, int64_t num_pages, int record_bytes,
                             int page_size, const int32_t* page_table, int max_pages_per_seq,
                             const int32_t* seq_lens, int B, int H,
                             float outer_scale, float softmax_scale, int max_splits,
                             float* out, float* lse, void* stream);

/* Top-k sparse decode: as mla_decode_nvfp4, but sequence b attends only to
 * the tokens listed in indices[b][0..topk).  [B12X], walkthrough and
 * sequence diagram (sparse MLA decode on the NVFP4 cache with the latent
 * scale).  Entries are logical token positions of sequence b, shared by all
 * heads; an entry < 0 or >= L is masked; a position listed twice counts
 * twice; no valid entry gives out = 0, lse = -inf.  Splits run over the
 * index list: mla_decode_num_splits(topk, max_splits) chunks.
 *
 *  indices    int32 [B, topk] (dense rows), topk >= 1
 *  workspace  >= mla_decode_workspace_bytes(B, H, max_splits) bytes, as for
 *             mla_decode_nvfp4 */
int mla_sparse_decode_nvfp4(const uint16_t* q_nope, const uint16_t* q_rope,
                            int64_t q_stride_b, int64_t q_stride_h,
                            const uint8_t* cache, int64_t num_pages, int record_bytes,
                            int page_size, const int32_t* page_table, int max_pages_per_seq,
                            const int32_t* seq_lens, int B, int H,
                            float outer_scale, float softmax_scale,
                            const int32_t* indices, int topk, int max_splits,
                            void* workspace, size_t workspace_bytes,
                            float* out, float* lse, void* stream);

/* Dense decode with quantized attention operands.  [MO-MLA], PR body and
 * commit 4: every attention matmul operand is fake-quantized once along its
 * own contraction axis; the split-K decode quantizes P after the softmax row
 * sum (the denominator unquantized), takes the caller's Q in an FP32
 * carrier (the dequantized values are used as they are), and, with a raw
 * latent cache, quantizes K along the feature axis and V along the token
 * axis, V in blocks of 16 at absolute token positions.
 *
 * Arguments as mla_decode_nvfp4, plus qdq_flags (the MLA_QDQ_* bits of the
 * prefill: Q, K, P, V and their FP8 format bits) and the multipliers g_q,
 * g_k, g_v, g_p (used for enabled operands; finite, > 0).
 *  record_bytes 432 or 368: NVFP4 records; K and V are the stored latent
 *               (times outer_scale); the K and V flags are refused (the
 *               latent is already quantized once).
 *  record_bytes MLA_RAW_RECORD_BYTES (1152): raw records (mla_raw_cache_write:
 *               512 bf16 latent then 64 bf16 RoPE values); outer_scale unused.
 *               K = [latent, RoPE] quantized along its 576 features (36 NVFP4
 *               blocks of 16, or per-tensor FP8) with g_k when MLA_QDQ_K;
 *               V = latent quantized along tokens with g_v when MLA_QDQ_V:
 *               NVFP4 blocks [16k, 16k+16) of positions < L per dim (the last
 *               one open), or per-tensor FP8.
 * Q (576-d) is quantized along its features like K.  Schedule: the tokens
 * of each split-K chunk (mla_decode_num_splits) are taken in tiles of 32
 * from the chunk start with a running max refreshed per tile; P is quantized
 * against it: NVFP4 16-key blocks aligned to the tile (keys past L count as
 * zeros), or per-tensor FP8.  Chunks merge by LSE in chunk order.
 *  workspace  >= mla_decode_workspace_bytes(B, H, max_splits) (max_splits > 1)
 * Dense only (no top-k form). */
int mla_decode_qdq(const uint16_t* q_nope, const uint16_t* q_rope,
                   int64_t q_stride_b, int64_t q_stride_h,
                   const uint8_t* cache, int64_t num_pages, int record_bytes,
                   int page_size, const int32_t* page_table, int max_pages_per_seq,
                   const int32_t* seq_lens, int B, int H,
                   float outer_scale, float softmax_scale, unsigned qdq_flags,
                   float g_q, float g_k, float g_v, float g_p, int max_splits,
                   void* workspace, size_t workspace_bytes,
                   float* out, float* lse, void* stream);

/* Write T tokens into a raw latent cache (records of MLA_RAW_RECORD_BYTES:
 * the 512 bf16 kv_c values, then the 64 bf16 k_pe values), the cache whose
 * K and V mla_decode_qdq quantizes on read ([MO-MLA], commit 4: the latent
 * cache stays raw in that model).  kv_c, k_pe: bf16 rows with strides
 * (multiples of 8, 16-byte aligned); a slot < 0 or >= num_slots skips the
 * token.  T == 0 is a no-op. */
int mla_raw_cache_write(const uint16_t* kv_c, int64_t kv_c_row_stride,
                        const uint16_t* k_pe, int64_t k_pe_row_stride,
                        const int64_t* slot_mapping, int64_t T,
                        uint8_t* cache, int64_t num_slots, void* stream);

/* Merge S partial attention results over disjoint token sets.  [MO-MLA],
 * commit 1: partials carry a natural-log LSE so that chunks can be merged.  For each (b, h)
 * with n = splits_per_seq[b] (clamped to [0, S]; all S when the pointer is
 * NULL): M = max_{s<n} lse_s; if n == 0 or M == -inf, out = 0 and lse = -inf;
 * else w_s = e^(lse_s - M), out = sum w_s out_s / sum w_s, lse = M + ln sum w_s.
 *
 *  partial_out  fp32 [B, S, H, D];  partial_lse fp32 [B, S, H]
 *  out          fp32 [B, H, D];     lse fp32 [B, H] or NULL
 *  B            0..65535;  H  1..65536
 *  D            multiple of 4, 1..4096 */
int mla_lse_merge(const float* partial_out, const float* partial_lse,
                  const int32_t* splits_per_seq, int B, int S, int H, int D,
                  float* out, float* lse, void* stream);

/* Varlen causal MLA prefill with NVFP4 fake quantization of Q/K/P/V and the
 * output written directly as NVFP4.  [MO-MLA], commit 1 and PR body (varlen
 * prefill, qk 192 / v 128, every matmul operand quantized once along its own
 * contraction axis in 1x16 NVFP4 blocks, P quantized after the softmax row
 * sum with the denominator unquantized, natural-log LSE); [FUSED-OUT], PR
 * description (packed e2m1 output, 128x4-swizzled e4m3 scales, fp32 global
 * scale, the separate quantization pass removed).
 *
 * Sequence n covers rows [cu_seqlens[n], cu_seqlens[n+1]); queries and keys
 * of a sequence coincide; row i attends to keys j <= i.  Flags (MLA_QDQ_*,
 * MLA_PREFILL_SPARSE_2_4): Q and K quantized along the head dim (12 NVFP4
 * blocks of 16, or per-tensor FP8) with multipliers g_q, g_k; V along local
 * token position (NVFP4 blocks [16k,16k+16) from the sequence start, the
 * last one possibly short, per head and dim; or per-tensor FP8) with g_v; P
 * along keys with g_p, in NVFP4 blocks aligned to the local key index (or
 * per-tensor FP8).  Keys are
 * visited in tiles of MLA_PREFILL_P_TILE = 64 from key 0; the running max is
 * refreshed per tile and P is quantized against it (the schedule is part of
 * the definition when MLA_QDQ_P is set).  O = acc / l, LSE = m + ln l, and
 * each 128-d output row (t, h) is quantized in 8 blocks of 16 with
 * multiplier out_global_scale: codes to out_fp4[t][h][0..64) (element 2i low
 * nibble), scales at the swizzled offset of SF[t][8h + blk] with SF having
 * H*8 columns; padding rows of the last 128-row tile are written as zero.
 *
 *  q, k         bf16 [T, H, 192], strides (q_stride_t, q_stride_h) and
 *               (k_stride_t, k_stride_h), multiples of 8, 16-byte aligned
 *  v            bf16 [T, H, 128], strides (v_stride_t, v_stride_h), same rule;
 *               q, k and v hold finite values (non-finite inputs give
 *               unspecified outputs)
 *  cu_seqlens   int32 [N + 1], non-decreasing, cu[0] = 0, cu[N] = T; N <= 65535
 *  max_seqlen   >= every sequence length
 *  g_*          finite, > 0 (ignored when the flag is off)
 *  workspace    >= mla_prefill_workspace_bytes(T, H, qdq_flags) bytes
 *  out_fp4      uint8 [T, H, 64]
 *  out_scales   uint8, mla_nvfp4_swizzled_scale_bytes(T, H * 8) bytes
 *  lse          fp32 [T, H] or NULL
 * Precondition (unchecked): cu_seqlens as stated. */
size_t mla_prefill_workspace_bytes(int64_t T, int H, unsigned qdq_flags);
int mla_prefill_nvfp4_out(const uint16_t* q, int64_t q_stride_t, int64_t q_stride_h,
                          const uint16_t* k, int64_t k_stride_t, int64_t k_stride_h,
                          const uint16_t* v, int64_t v_stride_t, int64_t v_stride_h,
                          const int32_t* cu_seqlens, int N, int max_seqlen,
                          int64_t T, int H, float softmax_scale, unsigned qdq_flags,
                          float g_q, float g_k, float g_v, float g_p,
                          float out_global_scale,
                          void* workspace, size_t workspace_bytes,
                          uint8_t* out_fp4, uint8_t* out_scales, float* lse,
                          void* stream);

/* Varlen prefill attention with fp32 output rows and LSE: the form a chunk of
 * new tokens over cached context needs.  [MO-MLA], commit 1 (varlen prefill,
 * operand quantization as above, natural-log LSE with which chunks of cached
 * context merge) and commit 2 (cached-context chunks are gathered from the
 * quantized paged cache and quantized again as prefill operands); [FUSED-OUT],
 * gate conjuncts (the fused NVFP4 output is for batches without cached
 * context: with context, the chunk outputs are merged first, then quantized).
 *
 * causal != 0: the keys of sequence n are its query rows [cu_seqlens_q[n],
 * cu_seqlens_q[n+1]) of k and v, row i sees keys j <= i (as
 * mla_prefill_nvfp4_out; cu_seqlens_k and T_k are ignored).  causal == 0:
 * the keys of sequence n are rows [cu_seqlens_k[n], cu_seqlens_k[n+1]) of k
 * and v (its cached context) and every query row sees all of them; a
 * sequence without keys gives O = 0 and LSE = -inf.  V's NVFP4 token blocks
 * start at each sequence's first key row; P's tile schedule is that of
 * mla_prefill_nvfp4_out.  O (fp32) = acc / l with the dequant multipliers
 * applied; LSE = m + ln l (natural log).
 *
 *  q            bf16 [T_q, H, 192]; k bf16 [T_k, H, 192]; v bf16 [T_k, H, 128]
 *               (strides as in mla_prefill_nvfp4_out; finite values)
 *  cu_seqlens_q int32 [N + 1], cu_seqlens_k int32 [N + 1] (context only),
 *               non-decreasing from 0 to T_q and T_k; N <= 65535
 *  max_seqlen_q, max_seqlen_k  >= every sequence's query / key count
 *  workspace    >= mla_prefill_workspace_bytes(T_k, H, qdq_flags) bytes
 *               (T_q when causal)
 *  out          fp32, element (t, h, d) at t*out_stride_t + h*out_stride_h + d
 *               (strides multiples of 4, 16-byte aligned)
 *  lse          fp32, (t, h) at t*lse_stride_t + h*lse_stride_h, or NULL
 * A chunked prefill writes both parts into one [T_q, 2, H, 128] buffer
 * (strides 256 H and 128, LSE strides 2 H and 1, the second part offset by
 * 128 H and H) and merges them with mla_lse_merge (B = T_q, S = 2, D = 128).
 * Preconditions (unchecked): cu arrays as stated. */
int mla_prefill_attention(const uint16_t* q, int64_t q_stride_t, int64_t q_stride_h,
                          const uint16_t* k, int64_t k_stride_t, int64_t k_stride_h,
                          const uint16_t* v, int64_t v_stride_t, int64_t v_stride_h,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int N,
                          int max_seqlen_q, int max_seqlen_k, int64_t T_q, int64_t T_k, int H,
                          int causal, float softmax_scale, unsigned qdq_flags,
                          float g_q, float g_k, float g_v, float g_p,
                          void* workspace, size_t workspace_bytes,
                          float* out, int64_t out_stride_t, int64_t out_stride_h,
                          float* lse, int64_t lse_stride_t, int64_t lse_stride_h, void* stream);

/* Gather cached context from the paged NVFP4 latent cache into bf16 rows.
 * [MO-MLA], commit 2 (cached-context prefill chunks gather from the quantized
 * paged cache); [B12X], walkthrough (records found through the block table,
 * the per-layer outer scale restored on read).
 *
 * Output rows [cu_ctx[n], cu_ctx[n+1]) are positions ctx_start[n] + 0, 1, ...
 * of sequence n (ctx_start NULL: from 0), position j being record
 * page_table[n][j / page_size] * page_size + j % page_size.  Latent element:
 * fp32(outer_scale * (s * v)) rounded to bf16 (nearest even), s * v being the
 * exact e4m3-scale times e2m1 value; RoPE: the stored bf16 value, or the
 * e4m3 value (exact in bf16).  A position past the page table or on a page
 * id outside [0, num_pages) gives a zero row.
 *
 *  cache        uint8 [num_pages * page_size, record_bytes] (432 or 368)
 *  page_table   int32 [N, max_pages_per_seq]
 *  cu_ctx       int32 [N + 1], non-decreasing from 0 to T_ctx; N <= 65535
 *  ctx_start    int32 [N] or NULL
 *  max_ctx_len  >= every cu_ctx[n+1] - cu_ctx[n]
 *  kv_c_out     bf16 [T_ctx, 512], row stride (multiple of 8, 16-byte aligned)
 *  k_pe_out     bf16 [T_ctx, 64], row stride (multiple of 8, 16-byte aligned) */
int mla_nvfp4_cache_gather(const uint8_t* cache, int64_t num_pages, int record_bytes, int page_size,
                           const int32_t* page_table, int max_pages_per_seq,
                           const int32_t* cu_ctx, const int32_t* ctx_start, int N, int max_ctx_len,
                           int64_t T_ctx, float outer_scale,
                           uint16_t* kv_c_out, int64_t kv_c_row_stride,
                           uint16_t* k_pe_out, int64_t k_pe_row_stride, void* stream);

/* NVFP4 quantization of fp32 rows with swizzled scales: the stand-alone
 * quantization pass that [FUSED-OUT] (PR description) folds into the prefill
 * epilogue, exposed so the epilogue's arithmetic and layout can be checked
 * bit for bit.  Same per-block rule as the prefill output with multiplier
 * global_scale.
 *
 *  x               fp32 [M, K] dense, K a multiple of 16, 1..65536
 *  codes           uint8 [M, K/2]
 *  scales_swizzled uint8, mla_nvfp4_swizzled_scale_bytes(M, K/16) bytes;
 *                  padding rows and columns are written as zero */
int mla_nvfp4_quantize_rows(const float* x, int64_t M, int K, float global_scale,
                            uint8_t* codes, uint8_t* scales_swizzled, void* stream);

/* Roofline re-measurement helpers (not part of the attention path): an MFMA
 * micro-benchmark and two stream kernels, so that the vendor peaks the
 * roofline fractions are quoted against can be checked on the part.  The
 * caller times the launches (HIP events on `stream`) and derives the rates.
 *
 * mla_roofline_mfma: `blocks` workgroups of 4 wavefronts, each running
 * `iters` iterations of 8 independent fp16 products with operands in
 * registers: shape 0 = v_mfma_f32_16x16x32_f16 (16,384 flops each), shape 1 =
 * v_mfma_f32_32x32x16_f16 (32,768 flops each).  One float per lane is
 * written to `sink` (float [blocks * 256]) so that nothing is removed.
 *
 * mla_roofline_copy: a plain copy of `bytes` (a multiple of 16, 16-byte
 * aligned buffers, not overlapping) from src to dst, 16 bytes per lane.
 *
 * mla_roofline_read: reads `bytes` (a multiple of 16) of src (16-byte
 * aligned) and adds the wrapping 32-bit sum of its little-endian 32-bit words
 * to *sum (device uint32, 4-byte aligned; the caller zeroes it).  bytes == 0
 * launches nothing.
 *
 * All three return MLA_ERR_INVALID_ARGUMENT for arguments outside these
 * ranges, before any launch. */
int mla_roofline_mfma(int shape, int blocks, int iters, float* sink, void* stream);
int mla_roofline_copy(const void* src, void* dst, int64_t bytes, void* stream);
int mla_roofline_read(const void* src, int64_t bytes, uint32_t* sum, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_NVFP4_H */
