// C ABI of libmla_nvfp4.so: argument validation, device check, launches.
// The declarations, with the passages of the pages each call follows, are in
// include/mla_nvfp4.h.  Validation order: pure host checks of the arguments,
// then the no-op cases, then the device check, then the launches.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/mla_nvfp4.h"
#include "launch.hpp"
#include "roofline.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return MLA_OK;
}

bool finite_pos(float x) { return std::isfinite(x) && x > 0.0f; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// A dispatch counts the work-items of each grid dimension in 32 bits, so a
// launch dimension of 256-lane workgroups holds fewer than 2^24 of them.
// Requests whose launches would need more are refused; the caller splits
// them.
constexpr int64_t kMaxBlocks256 = (int64_t(1) << 24) - 1;
int64_t cdiv(int64_t a, int64_t b) { return a / b + (a % b != 0); }   // a >= 0, b > 0
bool blocks_fit(int64_t blocks) { return blocks >= 0 && blocks <= kMaxBlocks256; }
int too_large(const char* what) {
    return fail(MLA_ERR_UNSUPPORTED, "%s: one launch would exceed 2^32 work-items in a grid dimension; split the call",
                what);
}

// Per-device cache of "is gfx950": 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    int state = (dev >= 0 && dev < kMaxDevices) ? g_arch_ok[dev].load(std::memory_order_relaxed) : 0;
    if (state == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail(MLA_ERR_HIP, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
        state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        if (dev >= 0 && dev < kMaxDevices) g_arch_ok[dev].store(state, std::memory_order_relaxed);
        if (state == 2)
            return fail(MLA_ERR_UNSUPPORTED_DEVICE, "device %d is %s; this library is built for gfx950",
                        dev, prop.gcnArchName);
    }
    if (state == 2) return fail(MLA_ERR_UNSUPPORTED_DEVICE, "device %d is not gfx950", dev);
    return MLA_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

int check_record(int record_bytes) {
    if (record_bytes != MLA_RECORD_BYTES_BF16_ROPE && record_bytes != MLA_RECORD_BYTES_FP8_ROPE)
        return fail(MLA_ERR_RECORD_BYTES, "record_bytes=%d is neither the bf16-RoPE width (432) nor the e4m3-RoPE width (368)",
                    record_bytes);
    return MLA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t decode_ws_out_bytes(int B, int H, int S) {
    return align256((size_t)B * S * H * MLA_D_LATENT * sizeof(float));
}

// Common validation of dense and sparse decode arguments.
int check_decode(const uint16_t* q_nope, const uint16_t* q_rope, int64_t q_stride_b, int64_t q_stride_h,
                 const uint8_t* cache, int64_t num_pages, int record_bytes, int page_size,
                 const int32_t* page_table, int max_pages_per_seq, const int32_t* seq_lens, int B, int H,
                 float outer_scale, float softmax_scale, int max_splits, void* workspace,
                 size_t workspace_bytes, float* out, float* lse, bool raw_ok = false) {
    int rc = (raw_ok && record_bytes == MLA_RAW_RECORD_BYTES) ? MLA_OK : check_record(record_bytes);
    if (rc) return rc;
    if (B < 0 || B > 65535 || H < 1 || H > 4096)
        return fail(MLA_ERR_INVALID_ARGUMENT, "need 0 <= B <= 65535 and 1 <= H <= 4096 (B=%d H=%d)", B, H);
    if (page_size < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "page_size must be >= 1 (got %d)", page_size);
    if (max_pages_per_seq < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "max_pages_per_seq must be >= 1");
    if ((int64_t)max_pages_per_seq * page_size > INT32_MAX)
        return fail(MLA_ERR_INVALID_ARGUMENT, "max_pages_per_seq * page_size exceeds int32");
    if (num_pages < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "num_pages must be >= 1");
    if (max_splits < 1 || max_splits > 65535) return fail(MLA_ERR_INVALID_ARGUMENT, "max_splits must be in [1, 65535]");
    if (!std::isfinite(softmax_scale) || softmax_scale < 0.0f)
        return fail(MLA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0");
    if (!finite_pos(outer_scale)) return fail(MLA_ERR_INVALID_ARGUMENT, "outer_scale must be finite and > 0");
    if (B > 0) {
        if (!q_nope || !q_rope || !cache || !page_table || !seq_lens || !out || !lse)
            return fail(MLA_ERR_INVALID_ARGUMENT, "null tensor pointer");
        if (q_stride_b % 8 || q_stride_h % 8 || !aligned(q_nope, 16) || !aligned(q_rope, 16))
            return fail(MLA_ERR_INVALID_ARGUMENT, "q strides must be multiples of 8 elements and q 16-byte aligned");
        if (!aligned(cache, 16) || !aligned(out, 16))
            return fail(MLA_ERR_INVALID_ARGUMENT, "cache and out must be 16-byte aligned");
        if (max_splits > 1) {
            const size_t need = mla_decode_workspace_bytes(B, H, max_splits);
            if (!workspace || workspace_bytes < need)
                return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes needed, %zu given", need,
                            workspace_bytes);
            if (!aligned(workspace, 256)) return fail(MLA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
        }
    }
    return MLA_OK;
}

size_t decode_ws_lse_bytes(int B, int H, int S) { return align256((size_t)B * S * H * sizeof(float)); }
size_t decode_ws_fmt_bytes(int B, int H, int S) { return align256((size_t)B * S * H); }

int run_decode(mla::DecodeArgs& a, void* workspace, hipStream_t stream) {
    if (a.max_splits > 1) {
        char* ws = static_cast<char*>(workspace);
        a.ws_out = reinterpret_cast<float*>(ws);
        a.ws_lse = reinterpret_cast<float*>(ws + decode_ws_out_bytes(a.B, a.H, a.max_splits));
        a.ws_fmt = reinterpret_cast<uint8_t*>(ws + decode_ws_out_bytes(a.B, a.H, a.max_splits) +
                                              decode_ws_lse_bytes(a.B, a.H, a.max_splits));
    } else {
        a.ws_out = nullptr;
        a.ws_lse = nullptr;
        a.ws_fmt = nullptr;
    }
    return hip_status(mla::launch_decode(a, stream), "decode launch");
}

// Scratch memory of mla_decode_nvfp4_noalloc: the decode workspace (split
// partials) for callers that cannot allocate.  Each device holds its own copy
// of this array from the library's load until the process ends; host code
// uses only the per-device address from hipGetSymbolAddress (the array's name
// is a host-side stand-in, not a device address).  Every call on a device
// shares that device's copy.
static __device__ __align__(256) uint8_t scratch[MLA_DECODE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on device d (null until looked up)

// Address of the current device's scratch array, looked up once per device
// with that device current.
int scratch_of_current_device(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERR_UNSUPPORTED_DEVICE, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MLA_OK;
}

int decode_entry(const uint16_t* q_nope, const uint16_t* q_rope, int64_t q_stride_b, int64_t q_stride_h,
                 const uint8_t* cache, int64_t num_pages, int record_bytes, int page_size,
                 const int32_t* page_table, int max_pages_per_seq, const int32_t* seq_lens, int B, int H,
                 float outer_scale, float softmax_scale, int max_splits, void* workspace,
                 size_t workspace_bytes, float* out, float* lse, void* stream) {
    int rc = check_decode(q_nope, q_rope, q_stride_b, q_stride_h, cache, num_pages, record_bytes, page_size,
                          page_table, max_pages_per_seq, seq_lens, B, H, outer_scale, softmax_scale, max_splits,
                          workspace, workspace_bytes, out, lse);
    if (rc) return rc;
    if (B == 0) return ok();
    rc = check_device();
    if (rc) return rc;
    mla::DecodeArgs a{};
    a.q_nope = q_nope;
    a.q_rope = q_rope;
    a.q_stride_b = q_stride_b;
    a.q_stride_h = q_stride_h;
    a.cache = cache;
    a.num_pages = num_pages;
    a.record_bytes = record_bytes;
    a.page_size = page_size;
    a.page_recip = mla::page_recip_of(page_size);
    a.page_table = page_table;
    a.max_pages = max_pages_per_seq;
    a.seq_lens = seq_lens;
    a.indices = nullptr;
    a.topk = 0;
    a.B = B;
    a.H = H;
    a.outer_scale = outer_scale;
    a.softmax_scale = softmax_scale;
    a.max_splits = max_splits;
    a.out = out;
    a.lse = lse;
    return run_decode(a, workspace, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

const char* mla_last_error(void) { return g_last_error.c_str(); }

int mla_nvfp4_record_bytes(int rope_fp8) {
    return rope_fp8 ? MLA_RECORD_BYTES_FP8_ROPE : MLA_RECORD_BYTES_BF16_ROPE;
}

int mla_decode_num_splits(int seq_len, int max_splits) {
    return mla::decode_num_splits(seq_len, max_splits < 1 ? 1 : max_splits);
}

size_t mla_decode_workspace_bytes(int B, int H, int max_splits) {
    if (max_splits <= 1 || B <= 0 || H <= 0) return 0;
    return decode_ws_out_bytes(B, H, max_splits) + decode_ws_lse_bytes(B, H, max_splits) +
           decode_ws_fmt_bytes(B, H, max_splits);
}

int mla_prefill_p_tile(void) { return mla::prefill_p_tile(); }

int mla_raw_cache_write(const uint16_t* kv_c, int64_t kv_c_row_stride, const uint16_t* k_pe, int64_t k_pe_row_stride,
                        const int64_t* slot_mapping, int64_t T, uint8_t* cache, int64_t num_slots, void* stream) {
    if (T < 0 || num_slots < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "T and num_slots must be >= 0");
    if (!blocks_fit(cdiv(T, 4))) return too_large("raw cache write");   // 4 tokens per workgroup
    if (T == 0) return ok();
    if (!kv_c || !k_pe || !slot_mapping || !cache) return fail(MLA_ERR_INVALID_ARGUMENT, "null tensor pointer");
    if (kv_c_row_stride % 8 || k_pe_row_stride % 8 || kv_c_row_stride < MLA_D_LATENT || k_pe_row_stride < MLA_D_ROPE ||
        !aligned(kv_c, 16) || !aligned(k_pe, 16) || !aligned(cache, 16))
        return fail(MLA_ERR_INVALID_ARGUMENT, "kv_c / k_pe rows must be 16-byte aligned with strides >= 512 / 64 "
                    "(multiples of 8), and the cache 16-byte aligned");
    int rc = check_device();
    if (rc) return rc;
    return hip_status(mla::launch_raw_cache_write(kv_c, kv_c_row_stride, k_pe, k_pe_row_stride, slot_mapping, T, cache,
                                                  num_slots, static_cast<hipStream_t>(stream)),
                      "raw cache write launch");
}

int mla_decode_qdq(const uint16_t* q_nope, const uint16_t* q_rope, int64_t q_stride_b, int64_t q_stride_h,
                   const uint8_t* cache, int64_t num_pages, int record_bytes, int page_size,
                   const int32_t* page_table, int max_pages_per_seq, const int32_t* seq_lens, int B, int H,
                   float outer_scale, float softmax_scale, unsigned qdq_flags, float g_q, float g_k, float g_v,
                   float g_p, int max_splits, void* workspace, size_t workspace_bytes, float* out, float* lse,
                   void* stream) {
    int rc = check_decode(q_nope, q_rope, q_stride_b, q_stride_h, cache, num_pages, record_bytes, page_size,
                          page_table, max_pages_per_seq, seq_lens, B, H, outer_scale, softmax_scale, max_splits,
                          workspace, workspace_bytes, out, lse, true);
    if (rc) return rc;
    if (qdq_flags & ~0xFFu) return fail(MLA_ERR_INVALID_ARGUMENT, "unknown qdq_flags bits 0x%x", qdq_flags & ~0xFFu);
    if ((qdq_flags & MLA_QDQ_FP8_MASK) >> 4 & ~qdq_flags & 0xFu)
        return fail(MLA_ERR_INVALID_ARGUMENT, "qdq_flags 0x%x: an FP8 format bit is set for an operand that is not "
                    "quantized", qdq_flags);
    if ((qdq_flags & (MLA_QDQ_K | MLA_QDQ_V)) && record_bytes != MLA_RAW_RECORD_BYTES)
        return fail(MLA_ERR_INVALID_ARGUMENT, "K and V are quantized on read only from raw (%d-byte) records; NVFP4 "
                    "records already hold the quantized latent", MLA_RAW_RECORD_BYTES);
    if (((qdq_flags & MLA_QDQ_Q) && !finite_pos(g_q)) || ((qdq_flags & MLA_QDQ_K) && !finite_pos(g_k)) ||
        ((qdq_flags & MLA_QDQ_V) && !finite_pos(g_v)) || ((qdq_flags & MLA_QDQ_P) && !finite_pos(g_p)))
        return fail(MLA_ERR_INVALID_ARGUMENT, "the scale of every enabled quantizer must be finite and > 0");
    if (((qdq_flags & MLA_QDQ_FP8_Q) && !std::isfinite(1.0f / g_q)) || ((qdq_flags & MLA_QDQ_FP8_K) && !std::isfinite(1.0f / g_k)) ||
        ((qdq_flags & MLA_QDQ_FP8_V) && !std::isfinite(1.0f / g_v)) || ((qdq_flags & MLA_QDQ_FP8_P) && !std::isfinite(1.0f / g_p)))
        return fail(MLA_ERR_INVALID_ARGUMENT, "a per-tensor FP8 multiplier is too small (1/g overflows)");
    if (B == 0) return ok();
    rc = check_device();
    if (rc) return rc;
    mla::DecodeArgs a{};
    a.q_nope = q_nope;
    a.q_rope = q_rope;
    a.q_stride_b = q_stride_b;
    a.q_stride_h = q_stride_h;
    a.cache = cache;
    a.num_pages = num_pages;
    a.record_bytes = record_bytes;
    a.page_size = page_size;
    a.page_recip = mla::page_recip_of(page_size);
    a.page_table = page_table;
    a.max_pages = max_pages_per_seq;
    a.seq_lens = seq_lens;
    a.indices = nullptr;
    a.topk = 0;
    a.B = B;
    a.H = H;
    a.outer_scale = outer_scale;
    a.softmax_scale = softmax_scale;
    a.max_splits = max_splits;
    a.out = out;
    a.lse = lse;
    if (max_splits > 1) {
        char* ws = static_cast<char*>(workspace);
        a.ws_out = reinterpret_cast<float*>(ws);
        a.ws_lse = reinterpret_cast<float*>(ws + decode_ws_out_bytes(B, H, max_splits));
        a.ws_fmt = reinterpret_cast<uint8_t*>(ws + decode_ws_out_bytes(B, H, max_splits) +
                                              decode_ws_lse_bytes(B, H, max_splits));
    }
    return hip_status(mla::launch_decode_qdq(a, qdq_flags, g_q, g_k, g_v, g_p, static_cast<hipStream_t>(stream)),
                      "quantized-operand decode launch");
}

size_t mla_nvfp4_swizzled_scale_bytes(int64_t rows, int64_t scale_cols) {
    if (rows <= 0 || scale_cols <= 0) return 0;
    return (size_t)((rows + 127) / 128 * 128) * (size_t)((scale_cols + 3) / 4 * 4);
}

int mla_nvfp4_cache_write(const uint16_t* kv_c, int64_t kv_c_row_stride, const uint16_t* k_pe,
                          int64_t k_pe_row_stride, const int64_t* slot_mapping, int64_t T, uint8_t* cache,
                          int64_t num_slots, int record_bytes, float outer_scale, void* stream) {
    int rc = check_record(record_bytes);
    if (rc) return rc;
    if (T < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "T must be >= 0");
    if (!finite_pos(outer_scale)) return fail(MLA_ERR_INVALID_ARGUMENT, "outer_scale must be finite and > 0");
    if (num_slots < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "num_slots must be >= 0");
    if (!blocks_fit(cdiv(T, 16))) return too_large("cache write");   // 16 tokens per workgroup
    if (T == 0) return ok();
    if (!kv_c || !k_pe || !slot_mapping || !cache) return fail(MLA_ERR_INVALID_ARGUMENT, "null tensor pointer");
    if (kv_c_row_stride % 8 || !aligned(kv_c, 16) || kv_c_row_stride < MLA_D_LATENT)
        return fail(MLA_ERR_INVALID_ARGUMENT, "kv_c rows must be 16-byte aligned with stride >= 512 (multiple of 8)");
    if (k_pe_row_stride % 2 || !aligned(k_pe, 4) || k_pe_row_stride < MLA_D_ROPE)
        return fail(MLA_ERR_INVALID_ARGUMENT, "k_pe rows must be 4-byte aligned with stride >= 64 (even)");
    if (!aligned(cache, 16)) return fail(MLA_ERR_INVALID_ARGUMENT, "cache must be 16-byte aligned");
    rc = check_device();
    if (rc) return rc;
    return hip_status(mla::launch_cache_write(kv_c, kv_c_row_stride, k_pe, k_pe_row_stride, slot_mapping, T,
                                              cache, num_slots, record_bytes == MLA_RECORD_BYTES_FP8_ROPE,
                                              outer_scale, static_cast<hipStream_t>(stream)),
                      "cache write launch");
}

int mla_decode_nvfp4(const uint16_t* q_nope, const uint16_t* q_rope, int64_t q_stride_b, int64_t q_stride_h,
                     const uint8_t* cache, int64_t num_pages, int record_bytes, int page_size,
                     const int32_t* page_table, int max_pages_per_seq, const int32_t* seq_lens, int B, int H,
                     float outer_scale, float softmax_scale, int max_splits, void* workspace,
                     size_t workspace_bytes, float* out, float* lse, void* stream) {
    return decode_entry(q_nope, q_rope, q_stride_b, q_stride_h, cache, num_pages, record_bytes, page_size,
                        page_table, max_pages_per_seq, seq_lens, B, H, outer_scale, softmax_scale, max_splits,
                        workspace, workspace_bytes, out, lse, stream);
}

int mla_decode_nvfp4_noalloc(const uint16_t* q_nope, const uint16_t* q_rope, int64_t q_stride_b,
                             int64_t q_stride_h, const uint8_t* cache, int64_t num_pages, int record_bytes,
                             int page_size, const int32_t* page_table, int max_pages_per_seq,
                             const int32_t* seq_lens, int B, int H, float outer_scale, float softmax_scale,
                             int max_splits, float* out, float* lse, void* stream) {
    // the size limit first (a pure host check), then the scratch address
    if (B > 0 && H > 0 && max_splits > 1) {
        const size_t need = mla_decode_workspace_bytes(B, H, max_splits);
        if (need > (size_t)MLA_DECODE_NOALLOC_SCRATCH_BYTES)
            return fail(MLA_ERR_WORKSPACE_TOO_SMALL,
                        "B=%d H=%d max_splits=%d need %zu bytes of split scratch; the allocation-free decode "
                        "holds at most %zu (use mla_decode_nvfp4 with a workspace, or fewer splits)",
                        B, H, max_splits, need, (size_t)MLA_DECODE_NOALLOC_SCRATCH_BYTES);
    }
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (B > 0 && max_splits > 1) {
        int rc = check_device();
        if (rc) return rc;
        rc = scratch_of_current_device(&ws);
        if (rc) return rc;
        ws_bytes = MLA_DECODE_NOALLOC_SCRATCH_BYTES;
    }
    return decode_entry(q_nope, q_rope, q_stride_b, q_stride_h, cache, num_pages, record_bytes, page_size,
                        page_table, max_pages_per_seq, seq_lens, B, H, outer_scale, softmax_scale, max_splits,
                        ws, ws_bytes, out, lse, stream);
}

int mla_sparse_decode_nvfp4(const uint16_t* q_nope, const uint16_t* q_rope, int64_t q_stride_b,
                            int64_t q_stride_h, const uint8_t* cache, int64_t num_pages, int record_bytes,
                            int page_size, const int32_t* page_table, int max_pages_per_seq,
                            const int32_t* seq_lens, int B, int H, float outer_scale, float softmax_scale,
                            const int32_t* indices, int topk, int max_splits, void* workspace,
                            size_t workspace_bytes, float* out, float* lse, void* stream) {
    int rc = check_decode(q_nope, q_rope, q_stride_b, q_stride_h, cache, num_pages, record_bytes, page_size,
                          page_table, max_pages_per_seq, seq_lens, B, H, outer_scale, softmax_scale, max_splits,
                          workspace, workspace_bytes, out, lse);
    if (rc) return rc;
    if (topk < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "topk must be >= 1");
    if (B > 0 && !indices) return fail(MLA_ERR_INVALID_ARGUMENT, "null indices");
    if (B == 0) return ok();
    rc = check_device();
    if (rc) return rc;
    mla::DecodeArgs a{};
    a.q_nope = q_nope;
    a.q_rope = q_rope;
    a.q_stride_b = q_stride_b;
    a.q_stride_h = q_stride_h;
    a.cache = cache;
    a.num_pages = num_pages;
    a.record_bytes = record_bytes;
    a.page_size = page_size;
    a.page_recip = mla::page_recip_of(page_size);
    a.page_table = page_table;
    a.max_pages = max_pages_per_seq;
    a.seq_lens = seq_lens;
    a.indices = indices;
    a.topk = topk;
    a.B = B;
    a.H = H;
    a.outer_scale = outer_scale;
    a.softmax_scale = softmax_scale;
    a.max_splits = max_splits;
    a.out = out;
    a.lse = lse;
    return run_decode(a, workspace, static_cast<hipStream_t>(stream));
}

int mla_lse_merge(const float* partial_out, const float* partial_lse, const int32_t* splits_per_seq, int B, int S,
                  int H, int D, float* out, float* lse, void* stream) {
    if (B < 0 || B > 65535 || S < 1 || H < 1 || H > 65536 || D < 4 || D > 4096 || D % 4)
        return fail(MLA_ERR_INVALID_ARGUMENT, "need 0 <= B <= 65535, S >= 1, 1 <= H <= 65536, D in [4, 4096] "
                    "multiple of 4");
    if (B == 0) return ok();
    if (!partial_out || !partial_lse || !out) return fail(MLA_ERR_INVALID_ARGUMENT, "null tensor pointer");
    if (!aligned(partial_out, 16) || !aligned(out, 16))
        return fail(MLA_ERR_INVALID_ARGUMENT, "partial_out and out must be 16-byte aligned");
    int rc = check_device();
    if (rc) return rc;
    mla::MergeArgs m{};
    m.part_out = partial_out;
    m.part_lse = partial_lse;
    m.splits_per_seq = splits_per_seq;
    m.B = B;
    m.S = S;
    m.H = H;
    m.D = D;
    m.out = out;
    m.lse = lse;
    return hip_status(mla::launch_lse_merge(m, static_cast<hipStream_t>(stream)), "merge launch");
}

size_t mla_prefill_workspace_bytes(int64_t T, int H, unsigned qdq_flags) {
    if (T <= 0 || H <= 0) return 0;
    return mla::prefill_workspace_bytes(T, H, qdq_flags);
}

namespace {

// Checks shared by the prefill entry points: flag bits, scales.
int check_prefill_flags(unsigned flags, float softmax_scale, float g_q, float g_k, float g_v, float g_p) {
    const unsigned known = 0xFu | MLA_QDQ_FP8_MASK | MLA_PREFILL_SPARSE_2_4;
    if (flags & ~known) return fail(MLA_ERR_INVALID_ARGUMENT, "unknown qdq_flags bits 0x%x", flags & ~known);
    if ((flags & MLA_QDQ_FP8_MASK) >> 4 & ~flags & 0xFu)
        return fail(MLA_ERR_INVALID_ARGUMENT, "qdq_flags 0x%x: an FP8 format bit is set for an operand that is not "
                    "quantized", flags);
    if (!std::isfinite(softmax_scale) || softmax_scale < 0.0f)
        return fail(MLA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0");
    if (((flags & MLA_QDQ_Q) && !finite_pos(g_q)) || ((flags & MLA_QDQ_K) && !finite_pos(g_k)) ||
        ((flags & MLA_QDQ_V) && !finite_pos(g_v)) || ((flags & MLA_QDQ_P) && !finite_pos(g_p)))
        return fail(MLA_ERR_INVALID_ARGUMENT, "the scale of every enabled quantizer must be finite and > 0");
    // a per-tensor FP8 multiplier must keep 1/g finite in fp32
    if (((flags & MLA_QDQ_FP8_Q) && !std::isfinite(1.0f / g_q)) || ((flags & MLA_QDQ_FP8_K) && !std::isfinite(1.0f / g_k)) ||
        ((flags & MLA_QDQ_FP8_V) && !std::isfinite(1.0f / g_v)) || ((flags & MLA_QDQ_FP8_P) && !std::isfinite(1.0f / g_p)))
        return fail(MLA_ERR_INVALID_ARGUMENT, "a per-tensor FP8 multiplier is too small (1/g overflows)");
    return MLA_OK;
}

}  // namespace

int mla_prefill_nvfp4_out(const uint16_t* q, int64_t q_stride_t, int64_t q_stride_h, const uint16_t* k,
                          int64_t k_stride_t, int64_t k_stride_h, const uint16_t* v, int64_t v_stride_t,
                          int64_t v_stride_h, const int32_t* cu_seqlens, int N, int max_seqlen, int64_t T, int H,
                          float softmax_scale, unsigned qdq_flags, float g_q, float g_k, float g_v, float g_p,
                          float out_global_scale, void* workspace, size_t workspace_bytes, uint8_t* out_fp4,
                          uint8_t* out_scales, float* lse, void* stream) {
    if (N < 0 || N > 65535 || T < 0 || H < 1 || H > 1024 || max_seqlen < 0)
        return fail(MLA_ERR_INVALID_ARGUMENT, "need 0 <= N <= 65535, T >= 0, 1 <= H <= 1024, max_seqlen >= 0");
    int rc0 = check_prefill_flags(qdq_flags, softmax_scale, g_q, g_k, g_v, g_p);
    if (rc0) return rc0;
    if (!finite_pos(out_global_scale)) return fail(MLA_ERR_INVALID_ARGUMENT, "out_global_scale must be finite and > 0");
    if (T > INT32_MAX) return fail(MLA_ERR_INVALID_ARGUMENT, "T must fit in int32");
    // the K / V pre-passes: 12 and 16 work-items per (row, head), and 16 rows
    // of a sequence per workgroup column of V's block quantization
    if (!blocks_fit(cdiv(T * H, 16)) || !blocks_fit(cdiv(max_seqlen, 16))) return too_large("prefill");
    if (T == 0 || N == 0) return ok();
    if (!q || !k || !v || !cu_seqlens || !out_fp4 || !out_scales)
        return fail(MLA_ERR_INVALID_ARGUMENT, "null tensor pointer");
    if (q_stride_t % 8 || q_stride_h % 8 || k_stride_t % 8 || k_stride_h % 8 || v_stride_t % 8 || v_stride_h % 8 ||
        !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
        return fail(MLA_ERR_INVALID_ARGUMENT, "q/k/v strides must be multiples of 8 elements and 16-byte aligned");
    const size_t need = mla_prefill_workspace_bytes(T, H, qdq_flags);
    if (need && (!workspace || workspace_bytes < need))
        return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    if (need && !aligned(workspace, 256)) return fail(MLA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    int rc = check_device();
    if (rc) return rc;
    mla::PrefillArgs a{};
    a.q = q; a.q_st = q_stride_t; a.q_sh = q_stride_h;
    a.k = k; a.k_st = k_stride_t; a.k_sh = k_stride_h;
    a.v = v; a.v_st = v_stride_t; a.v_sh = v_stride_h;
    a.cu_seqlens = cu_seqlens;
    a.cu_k = nullptr;
    a.N = N;
    a.max_seqlen = max_seqlen;
    a.max_seqlen_k = max_seqlen;
    a.T = T;
    a.T_k = T;
    a.H = H;
    a.causal = 1;
    a.softmax_scale = softmax_scale;
    a.flags = qdq_flags;
    a.g_q = g_q; a.g_k = g_k; a.g_v = g_v; a.g_p = g_p; a.g_out = out_global_scale;
    a.workspace = workspace;
    a.out_fp4 = out_fp4;
    a.out_scales = out_scales;
    a.out_f32 = nullptr;
    a.lse = lse;
    a.lse_st = H;
    a.lse_sh = 1;
    hipError_t e = mla::launch_prefill(a, static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) return fail(MLA_ERR_UNSUPPORTED, "prefill kernel not available");
    return hip_status(e, "prefill launch");
}

int mla_prefill_attention(const uint16_t* q, int64_t q_stride_t, int64_t q_stride_h, const uint16_t* k,
                          int64_t k_stride_t, int64_t k_stride_h, const uint16_t* v, int64_t v_stride_t,
                          int64_t v_stride_h, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int N,
                          int max_seqlen_q, int max_seqlen_k, int64_t T_q, int64_t T_k, int H, int causal,
                          float softmax_scale, unsigned qdq_flags, float g_q, float g_k, float g_v, float g_p,
                          void* workspace, size_t workspace_bytes, float* out, int64_t out_stride_t,
                          int64_t out_stride_h, float* lse, int64_t lse_stride_t, int64_t lse_stride_h,
                          void* stream) {
    if (N < 0 || N > 65535 || T_q < 0 || H < 1 || H > 1024 || max_seqlen_q < 0)
        return fail(MLA_ERR_INVALID_ARGUMENT, "need 0 <= N <= 65535, T_q >= 0, 1 <= H <= 1024, max_seqlen_q >= 0");
    if (!causal && (T_k < 0 || max_seqlen_k < 0))
        return fail(MLA_ERR_INVALID_ARGUMENT, "need T_k >= 0 and max_seqlen_k >= 0");
    int rc = check_prefill_flags(qdq_flags, softmax_scale, g_q, g_k, g_v, g_p);
    if (rc) return rc;
    const int64_t Tk = causal ? T_q : T_k;
    if (T_q > INT32_MAX || Tk > INT32_MAX) return fail(MLA_ERR_INVALID_ARGUMENT, "T_q and T_k must fit in int32");
    if (!blocks_fit(cdiv(Tk * H, 16)) || !blocks_fit(cdiv(causal ? max_seqlen_q : max_seqlen_k, 16)))
        return too_large("prefill attention");   // the K / V pre-passes over the keys
    if (T_q == 0 || N == 0) return ok();
    if (!q || !cu_seqlens_q || !out || (!causal && !cu_seqlens_k) || (Tk > 0 && (!k || !v)))
        return fail(MLA_ERR_INVALID_ARGUMENT, "null tensor pointer");
    if (q_stride_t % 8 || q_stride_h % 8 || k_stride_t % 8 || k_stride_h % 8 || v_stride_t % 8 || v_stride_h % 8 ||
        !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
        return fail(MLA_ERR_INVALID_ARGUMENT, "q/k/v strides must be multiples of 8 elements and 16-byte aligned");
    if (out_stride_t % 4 || out_stride_h % 4 || !aligned(out, 16))
        return fail(MLA_ERR_INVALID_ARGUMENT, "out strides must be multiples of 4 elements and out 16-byte aligned");
    const size_t need = mla_prefill_workspace_bytes(Tk, H, qdq_flags);
    if (need && (!workspace || workspace_bytes < need))
        return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    if (need && !aligned(workspace, 256)) return fail(MLA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    rc = check_device();
    if (rc) return rc;
    mla::PrefillArgs a{};
    a.q = q; a.q_st = q_stride_t; a.q_sh = q_stride_h;
    a.k = k; a.k_st = k_stride_t; a.k_sh = k_stride_h;
    a.v = v; a.v_st = v_stride_t; a.v_sh = v_stride_h;
    a.cu_seqlens = cu_seqlens_q;
    a.cu_k = causal ? nullptr : cu_seqlens_k;
    a.N = N;
    a.max_seqlen = max_seqlen_q;
    a.max_seqlen_k = causal ? max_seqlen_q : max_seqlen_k;
    a.T = T_q;
    a.T_k = Tk;
    a.H = H;
    a.causal = causal ? 1 : 0;
    a.softmax_scale = softmax_scale;
    a.flags = qdq_flags;
    a.g_q = g_q; a.g_k = g_k; a.g_v = g_v; a.g_p = g_p; a.g_out = 1.0f;
    a.workspace = workspace;
    a.out_fp4 = nullptr;
    a.out_scales = nullptr;
    a.out_f32 = out;
    a.o_st = out_stride_t;
    a.o_sh = out_stride_h;
    a.lse = lse;
    a.lse_st = lse_stride_t;
    a.lse_sh = lse_stride_h;
    return hip_status(mla::launch_prefill(a, static_cast<hipStream_t>(stream)), "prefill attention launch");
}

int mla_nvfp4_cache_gather(const uint8_t* cache, int64_t num_pages, int record_bytes, int page_size,
                           const int32_t* page_table, int max_pages_per_seq, const int32_t* cu_ctx,
                           const int32_t* ctx_start, int N, int max_ctx_len, int64_t T_ctx, float outer_scale,
                           uint16_t* kv_c_out, int64_t kv_c_row_stride, uint16_t* k_pe_out,
                           int64_t k_pe_row_stride, void* stream) {
    int rc = check_record(record_bytes);
    if (rc) return rc;
    if (N < 0 || N > 65535 || T_ctx < 0 || max_ctx_len < 0 || page_size < 1 || max_pages_per_seq < 1 || num_pages < 1)
        return fail(MLA_ERR_INVALID_ARGUMENT, "need 0 <= N <= 65535, T_ctx, max_ctx_len >= 0 and page_size, "
                    "max_pages_per_seq, num_pages >= 1");
    if (!blocks_fit(cdiv(max_ctx_len, 4))) return too_large("cache gather");
    if ((int64_t)max_pages_per_seq * page_size > INT32_MAX)
        return fail(MLA_ERR_INVALID_ARGUMENT, "max_pages_per_seq * page_size exceeds int32");
    if (!finite_pos(outer_scale)) return fail(MLA_ERR_INVALID_ARGUMENT, "outer_scale must be finite and > 0");
    if (N == 0 || T_ctx == 0 || max_ctx_len == 0) return ok();
    if (!cache || !page_table || !cu_ctx || !kv_c_out || !k_pe_out)
        return fail(MLA_ERR_INVALID_ARGUMENT, "null tensor pointer");
    if (kv_c_row_stride % 8 || k_pe_row_stride % 8 || kv_c_row_stride < MLA_D_LATENT || k_pe_row_stride < MLA_D_ROPE ||
        !aligned(kv_c_out, 16) || !aligned(k_pe_out, 16) || !aligned(cache, 16))
        return fail(MLA_ERR_INVALID_ARGUMENT, "output rows must be 16-byte aligned with strides >= 512 / 64 "
                    "(multiples of 8), and the cache 16-byte aligned");
    rc = check_device();
    if (rc) return rc;
    return hip_status(mla::launch_cache_gather(cache, num_pages, record_bytes == MLA_RECORD_BYTES_FP8_ROPE, page_size,
                                               mla::page_recip_of(page_size), page_table, max_pages_per_seq, cu_ctx,
                                               ctx_start, N, max_ctx_len, outer_scale, kv_c_out, kv_c_row_stride,
                                               k_pe_out, k_pe_row_stride, static_cast<hipStream_t>(stream)),
                      "cache gather launch");
}

int mla_nvfp4_quantize_rows(const float* x, int64_t M, int K, float global_scale, uint8_t* codes,
                            uint8_t* scales_swizzled, void* stream) {
    if (M < 0 || K < 16 || K > 65536 || K % 16)
        return fail(MLA_ERR_INVALID_ARGUMENT, "need M >= 0 and K in [16, 65536], a multiple of 16");
    if (!finite_pos(global_scale)) return fail(MLA_ERR_INVALID_ARGUMENT, "global_scale must be finite and > 0");
    {   // one work-item per (row, padded block column), rows padded to 128
        const int64_t cpad = ((K / 16) + 3) & ~3;
        if (M > kMaxBlocks256 * 256 || !blocks_fit(cdiv(cdiv(M, 128) * 128 * cpad, 256))) return too_large("quantize_rows");
    }
    if (M == 0) return ok();
    if (!x || !codes || !scales_swizzled) return fail(MLA_ERR_INVALID_ARGUMENT, "null tensor pointer");
    if (!aligned(x, 16) || !aligned(codes, 8)) return fail(MLA_ERR_INVALID_ARGUMENT, "x must be 16-byte and codes 8-byte aligned");
    int rc = check_device();
    if (rc) return rc;
    return hip_status(mla::launch_quantize_rows(x, M, K, global_scale, codes, scales_swizzled,
                                                static_cast<hipStream_t>(stream)),
                      "quantize_rows launch");
}

int mla_roofline_mfma(int shape, int blocks, int iters, float* sink, void* stream) {
    if (shape != 0 && shape != 1) return fail(MLA_ERR_INVALID_ARGUMENT, "shape must be 0 (16x16x32) or 1 (32x32x16)");
    if (blocks < 1 || blocks > 65536 || iters < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "need 1 <= blocks <= 65536, iters >= 0");
    if (!sink) return fail(MLA_ERR_INVALID_ARGUMENT, "null sink");
    int rc = check_device();
    if (rc) return rc;
    return hip_status(mla::launch_mfma_rate(shape, blocks, iters, sink, static_cast<hipStream_t>(stream)), "mfma rate launch");
}

int mla_roofline_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (bytes < 0 || bytes % 16) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes must be a non-negative multiple of 16");
    if (bytes == 0) return ok();
    if (!src || !dst) return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
    if (!aligned(src, 16) || !aligned(dst, 16)) return fail(MLA_ERR_INVALID_ARGUMENT, "src and dst must be 16-byte aligned");
    int rc = check_device();
    if (rc) return rc;
    return hip_status(mla::launch_stream_copy(src, dst, bytes, static_cast<hipStream_t>(stream)), "stream copy launch");
}

int mla_roofline_read(const void* src, int64_t bytes, uint32_t* sum, void* stream) {
    if (bytes < 0 || bytes % 16) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes must be a non-negative multiple of 16");
    if (!sum) return fail(MLA_ERR_INVALID_ARGUMENT, "null sum");
    if (bytes == 0) return ok();
    if (!src) return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
    if (!aligned(src, 16) || !aligned(sum, 4)) return fail(MLA_ERR_INVALID_ARGUMENT, "src must be 16-byte and sum 4-byte aligned");
    int rc = check_device();
    if (rc) return rc;
    return hip_status(mla::launch_stream_read(src, bytes, sum, static_cast<hipStream_t>(stream)), "stream read launch");
}

}  // extern "C"
