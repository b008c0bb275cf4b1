// Varlen MLA prefill attention with NVFP4 or FP8 fake quantization of
// Q/K/P/V, optional 2:4 score sparsity, and the output written directly as
// NVFP4 or as fp32 rows with their LSE (gfx950).
//
// [MO-MLA], commit 1 and PR body: varlen prefill with asymmetric head dims
// (qk 192, v 128); each matmul operand quantized once along its own
// contraction axis, in 1x16 NVFP4 blocks or per-tensor FP8 (Q, K along the
// head dim, V along tokens, P along keys after the softmax row sum; the
// denominator stays unquantized); token-exact N:M score sparsity on the
// new-token attention; natural-log LSE, with which chunks of cached context
// merge.  [FUSED-OUT], PR description: the output is written as packed e2m1
// codes plus e4m3 block scales in the 128x4-swizzled layout with an fp32
// global scale, replacing a separate quantization pass (a path for batches
// without cached context).
//
// Attention is causal (queries and keys are the same rows of a sequence) or
// over a sequence's cached context (every query row sees every key row).
//
// Kernels:
//   qk_qdq_kernel   K, one thread per 16-element block along d: the exact
//                   bf16 value s*v (NVFP4) or e4m3 value (FP8) of every
//                   element (the tensor-wide multiplier g is applied later,
//                   in fp32).  Q takes the same steps inside attn_kernel, on
//                   the rows it loads (each Q row is read by one workgroup);
//   v_qdq_kernel    V (NVFP4), one thread per (16-token block of a sequence,
//                   head, 8 dims): blocks start at the sequence start, the
//                   last one may be short;
//   v_fp8_kernel    V (FP8), 8 elements per thread;
//   attn_kernel     one workgroup per (256 query rows, head, sequence):
//                   8 wavefronts x 32 rows.  Keys are visited in tiles of 64
//                   from key 0 (the P-quantization schedule), K/V tiles
//                   staged in registers one tile ahead and stored token-major
//                   in LDS; S^T = K Q^T on v_mfma_f32_32x32x16_bf16; running
//                   max refreshed per tile; P quantized in 16-key blocks
//                   against it (exact in fp16); O^T = V^T P^T with V^T read
//                   by ds_read_b64_tr_b16 (with P and V quantized, the
//                   wavefronts 4-7 run the PV products of a tile one
//                   iteration late, next to the softmax of wavefronts 0-3 on
//                   the same SIMDs; V tiles are triple-buffered for that);
//                   epilogue: O = acc * g_p g_v / l, NVFP4 codes and
//                   swizzled scales (or fp32 rows), LSE = m + ln l;
//   pad_scales_kernel  zero scale bytes of the padding rows of the last
//                   128-row scale tile.
#include "device_common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int kDqk = 192;
constexpr int kDv = 128;
constexpr int kBN = 64;                 // key tile (the P-quantization schedule)
constexpr int kWaves = 8;
constexpr int kRowsPerWave = 32;
constexpr int kBM = kWaves * kRowsPerWave;  // 256 query rows per workgroup
// LDS row pitches (bf16 elements), chosen so the operand reads hit distinct
// banks: K fragments are 16-byte reads of 32 rows per half-wavefront (pitch
// 100 dwords, 4 x odd); V^T fragments are 8-byte transposing reads of 8 rows
// x 16 dwords per wavefront (pitch 80 dwords, 16 x odd).
constexpr int kPitchK = 200;
constexpr int kPitchV = 160;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- Q, K --

// Per-tensor FP8 quantize-dequantize of 8 bf16 values (packed in w4) with
// inv_g = fp32(1/g): code = e4m3(fp32(x * inv_g)) (RNE, satfinite, sign
// kept), returned as the exact bf16 values of the codes (g not applied).
__device__ __forceinline__ u32x4 fp8_qdq8_bf16(u32x4 w4, float inv_g) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t c2 = e4m3_encode2_hw(bf16_lo(w4[i]) * inv_g, bf16_hi(w4[i]) * inv_g);
        const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(c2, false);
        o[i] = pack_bf16_exact(d[0], d[1]);
    }
    return o;
}

template <bool kFp8>
__global__ __launch_bounds__(256) void qk_qdq_kernel(const uint16_t* __restrict__ x, int64_t st, int64_t sh,
                                                     int64_t T, int H, float g, float inv_g,
                                                     uint16_t* __restrict__ out) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // block of 16 along d
    const int64_t nblk = T * H * (kDqk / 16);
    if (idx >= nblk) return;
    const int blk = (int)(idx % (kDqk / 16));
    const int64_t th = idx / (kDqk / 16);
    const int h = (int)(th % H);
    const int64_t t = th / H;
    const u32x4* src = reinterpret_cast<const u32x4*>(x + t * st + (int64_t)h * sh + 16 * blk);
    const u32x4 w0 = src[0], w1 = src[1];
    if constexpr (kFp8) {
        u32x4* dst = reinterpret_cast<u32x4*>(out + (t * H + h) * kDqk + 16 * blk);
        dst[0] = fp8_qdq8_bf16(w0, inv_g);
        dst[1] = fp8_qdq8_bf16(w1, inv_g);
        return;
    }
    float v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_lo(w0[i]);
        v[2 * i + 1] = bf16_hi(w0[i]);
        v[8 + 2 * i] = bf16_lo(w1[i]);
        v[8 + 2 * i + 1] = bf16_hi(w1[i]);
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, __builtin_fabsf(v[i]));
    const Nvfp4Scale sc = nvfp4_block_scale(a, g);
    const float sv = e4m3_decode(sc.code);
    u32x4 o0, o1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // quantize-dequantize: codes by the FP4 conversion, values back exactly
        const f32x2 d0 = e2m1_pair<0>(e2m1_pack2<0>(0u, v[2 * i] * sc.inv, v[2 * i + 1] * sc.inv));
        const f32x2 d1 = e2m1_pair<0>(e2m1_pack2<0>(0u, v[8 + 2 * i] * sc.inv, v[8 + 2 * i + 1] * sc.inv));
        o0[i] = pack_bf16_exact(d0[0] * sv, d0[1] * sv);
        o1[i] = pack_bf16_exact(d1[0] * sv, d1[1] * sv);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(out + (t * H + h) * kDqk + 16 * blk);
    dst[0] = o0;
    dst[1] = o1;
}

// ------------------------------------------------------------------- V --

// grid (ceil(max_seqlen/16), N, ceil(H*128/8/256)); thread = (head, 8 dims):
// 16 tokens x 8 dims in 16-byte loads and stores, eight blocks per thread.
// kF16Out: the exact values s*v are written as fp16 (they fit: at most 6
// significant bits, magnitudes in [2^-10, 2688]) for the fp16 PV products,
// otherwise as bf16.
template <bool kF16Out>
__global__ __launch_bounds__(256) void v_qdq_kernel(const uint16_t* __restrict__ v, int64_t st, int64_t sh,
                                                    const int32_t* __restrict__ cu, int H, float g,
                                                    uint16_t* __restrict__ out) {
    const int n = blockIdx.y;
    const int a = cu[n], e = cu[n + 1];
    const int t0 = a + 16 * blockIdx.x;
    if (t0 >= e) return;
    const int hd8 = blockIdx.z * 256 + threadIdx.x;
    if (hd8 >= H * (kDv / 8)) return;
    const int h = hd8 / (kDv / 8), d0 = 8 * (hd8 % (kDv / 8));
    const int cnt = min(16, e - t0);
    u32x4 raw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int ti = t0 + min(i, cnt - 1);   // (rows past the sequence end are not used)
        raw[i] = *reinterpret_cast<const u32x4*>(v + (int64_t)ti * st + (int64_t)h * sh + d0);
    }
    // x[i][j]: token t0 + i, dim d0 + j (tokens past the end are 0)
    auto x_of = [&](int i, int j) -> float {
        const uint32_t w = raw[i][j >> 1];
        return i < cnt ? ((j & 1) ? bf16_hi(w) : bf16_lo(w)) : 0.0f;
    };
    uint32_t res[16][4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, __builtin_fabsf(x_of(i, j)));
        const Nvfp4Scale sc = nvfp4_block_scale(amax, g);
        const float sv = e4m3_decode(sc.code);
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            const f32x2 dq = e2m1_pair<0>(e2m1_pack2<0>(0u, x_of(i, j) * sc.inv, x_of(i + 1, j) * sc.inv));
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const float q = dq[k] * sv;
                const uint32_t bits = kF16Out ? (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)q) : (f2u(q) >> 16);
                uint32_t& word = res[i + k][j >> 1];
                word = (j & 1) ? ((word & 0xffffu) | (bits << 16)) : bits;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (i < cnt)
            *reinterpret_cast<u32x4*>(out + ((int64_t)(t0 + i) * H + h) * kDv + d0) =
                u32x4{res[i][0], res[i][1], res[i][2], res[i][3]};
    }
}

// V as per-tensor FP8: rows [T, H, 128], 8 elements per thread; the exact
// e4m3 values are written as fp16 (kF16Out) or bf16.
template <bool kF16Out>
__global__ __launch_bounds__(256) void v_fp8_kernel(const uint16_t* __restrict__ v, int64_t st, int64_t sh,
                                                    int64_t T, int H, float inv_g, uint16_t* __restrict__ out) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;   // (token, head, 8 dims)
    if (idx >= T * H * (kDv / 8)) return;
    const int d0 = 8 * (int)(idx % (kDv / 8));
    const int64_t th = idx / (kDv / 8);
    const int h = (int)(th % H);
    const int64_t t = th / H;
    const u32x4 w4 = *reinterpret_cast<const u32x4*>(v + t * st + (int64_t)h * sh + d0);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t c2 = e4m3_encode2_hw(bf16_lo(w4[i]) * inv_g, bf16_hi(w4[i]) * inv_g);
        const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(c2, false);
        if constexpr (kF16Out) {
            const f16x2v hv = {(_Float16)d[0], (_Float16)d[1]};
            o[i] = __builtin_bit_cast(uint32_t, hv);
        } else {
            o[i] = pack_bf16_exact(d[0], d[1]);
        }
    }
    *reinterpret_cast<u32x4*>(out + (t * H + h) * kDv + d0) = o;
}

// ----------------------------------------------------------- attention --

struct AttnParams {
    const uint16_t* q; int64_t q_st, q_sh;   // raw Q
    int q_qdq;                // Q quantize-dequantized on load (multiplier q_g)
    int q_fp8;                // ... as per-tensor FP8 (q_inv = fp32(1/q_g)) instead of NVFP4
    float q_g, q_inv;
    const uint16_t* k; int64_t k_st, k_sh;
    const uint16_t* v; int64_t v_st, v_sh;
    const int32_t* cu;        // query rows of sequence n: [cu[n], cu[n+1])
    const int32_t* ck;        // key rows of sequence n (context attention): [ck[n], ck[n+1])
    int causal;               // keys are the query rows, row i sees keys j <= i
    int H;
    float score_scale_log2;   // softmax_scale * g_q' * g_k' * log2(e)
    float rank_mul;           // 2:4 ranking factor: 1, or 0 when softmax_scale is 0 (every score ties)
    double out_scale;         // g_p' * g_v' (exact in fp64)
    float g_p;                // P multiplier (P quantized only)
    float u_p;                // fp32(6 g_p)
    float inv_u_p;            // fp32(1 / u_p)
    float inv_g_p;            // fp32(1 / g_p) (P as FP8)
    float g_out;              // output global scale
    int64_t T;
    uint8_t* out_fp4;         // NVFP4 output (null: fp32 rows to out_f32)
    uint8_t* out_scales;
    float* out_f32;           // fp32 output rows: element (t, h, d) at t*o_st + h*o_sh + d
    int64_t o_st, o_sh;
    float* lse;               // (t, h) at t*lse_st + h*lse_sh
    int64_t lse_st, lse_sh;
};

struct AttnSmem {
    uint16_t kt[2][kBN * kPitchK];  // 2 x 25600 B
    uint16_t vt[3][kBN * kPitchV];  // 3 x 20480 B
    float pinv[256];                // P block scale code -> fp32(1 / fp32(e4m3(code) g_p)), 0 for d = 0
};

// The P block scale's quotient t = fp32(a / u) is taken as one multiply by
// fp32(1/u), redone as the exact division where scale_quotient_near_tie says
// the code could differ (as nvfp4_block_scale_fast, which the row quantizer
// uses; its tests sweep the e4m3 ties with u not a power of two).

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// D = A (32x16) * B (16x32) + C, fp32 accumulate.  Lane l supplies row
// l % 32 of A and column l % 32 of B with k-slots 8(l/32) .. +7; it receives
// D[8(v/4) + 4(l/32) + v%4][l % 32] in element v.
__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_f16(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

template <bool V>
struct BoolTag {
    static constexpr bool value = V;
};

// Layout of a wavefront's work on one 64-key tile (32 query rows): lane l
// owns query row l % 32 (g2 = l / 32 picks half of the keys).  K and V tile
// rows are stored permuted: within each 32-key half, LDS row 8a + 4g + b
// holds key 16g + 4a + b (tile_row below).  Score tile mt2 = S^T for the
// rows 32 mt2 .. +31; its element v is row 32 mt2 + 8(v/4) + 4 g2 + v%4,
// which holds key 32 mt2 + 16 g2 + v.  So a lane's 16 elements of tile mt2
// are one whole 16-key P block (keys 32 mt2 + 16 g2 .. +15, block 2 mt2 + g2)
// in order, and elements 8h .. 8h+7 of tile mt2 are also the k-slots of
// k-step 2 mt2 + h of the B operand of O^T = V^T P^T (slot j <-> row
// 32 mt2 + 16h + 8(j/4) + 4 g2 + j%4; the V^T operand reads the same rows).
//
// kPMode: 0 P unquantized, 1 NVFP4 blocks along keys, 2 per-tensor FP8.
// kF16: P and V are both quantized, so P^ (s*v or an e4m3 value) and V^ are
// exact in fp16 and the PV products run in fp16, P^ coming straight from the
// FP4 or FP8 conversion; otherwise they run in bf16 (quantized P exact,
// unquantized P split into three bf16 parts).
//
// 2:4 sparsity (kSparse): in a score tile, a lane's elements 4c .. 4c+3
// are 4 consecutive keys starting at a multiple of 4, so each group's choice
// is made within one lane, on the raw fp32 accumulators (the scale factors
// are common to the row and positive; softmax_scale = 0 makes every score
// tie).
template <int kPMode, bool kF16, bool kSparse>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_kernel(AttnParams p) {
    constexpr bool kQuantP = kPMode != 0;
    __shared__ AttnSmem sm;
    if (kPMode == 1 && threadIdx.x < 256) {
        const float d = e4m3_decode(threadIdx.x) * p.g_p;
        sm.pinv[threadIdx.x] = (d == 0.0f) ? 0.0f : 1.0f / d;
    }
    // XCD-aware placement (as for decode): all query tiles of one (sequence,
    // head) run on one XCD when 8 divides the number of (sequence, head)
    // pairs, so that they stream the same K/V tiles through one L2
    int qx, u;
    decode_work_item((int)gridDim.x, (int)(gridDim.y * gridDim.z), qx, u);
    const int h = u % (int)gridDim.y, n = u / (int)gridDim.y;
    const int a = p.cu[n], e = p.cu[n + 1];
    const int L = e - a;                                  // query rows
    const int ka = p.causal ? a : p.ck[n];                // first key row
    const int Lk = p.causal ? L : p.ck[n + 1] - ka;       // key rows
    const int nqt = (L + kBM - 1) / kBM;
    const int qt = nqt - 1 - qx;   // (causal) longest, latest tiles first
    if (qt < 0) return;
    const int r0 = qt * kBM;                     // local row of the tile
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, g2 = lane >> 5;
    const int wr0 = r0 + kRowsPerWave * w;       // first local row of this wavefront
    const bool wave_rows = wr0 < L;
    const int row = wr0 + l32;                   // this lane's query row
    const int lim = p.causal ? row : Lk - 1;     // last key this row sees

    // Q row (B operand of S^T = K Q^T): k-step kk covers dims 16kk + 8 g2 .. +7
    bf16x8 qf[12];
    {
        const int rr = min(row, L - 1);
        const uint16_t* src = p.q + (int64_t)(a + rr) * p.q_st + (int64_t)h * p.q_sh + 8 * g2;
#pragma unroll
        for (int kk = 0; kk < 12; ++kk) qf[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(src + 16 * kk));
    }
    // Q quantize-dequantize, the same steps as qk_qdq_kernel: block kk of
    // the row is this lane's 8 values and those of lane ^ 32
    if (p.q_qdq && p.q_fp8) {
#pragma unroll
        for (int kk = 0; kk < 12; ++kk) qf[kk] = as_bf16x8(fp8_qdq8_bf16(__builtin_bit_cast(u32x4, qf[kk]), p.q_inv));
    } else if (p.q_qdq) {
#pragma unroll
        for (int kk = 0; kk < 12; ++kk) {
            const u32x4 w4 = __builtin_bit_cast(u32x4, qf[kk]);
            float v[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = bf16_lo(w4[i]);
                v[2 * i + 1] = bf16_hi(w4[i]);
            }
            float am = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) am = fmaxf(am, __builtin_fabsf(v[i]));
            am = xor32_max(am);
            const Nvfp4Scale sc = nvfp4_block_scale(am, p.q_g);
            const float scv = e4m3_decode(sc.code);
            u32x4 o4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x2 d = e2m1_pair<0>(e2m1_pack2<0>(0u, v[2 * i] * sc.inv, v[2 * i + 1] * sc.inv));
                o4[i] = pack_bf16_exact(d[0] * scv, d[1] * scv);
            }
            qf[kk] = as_bf16x8(o4);
        }
    }

    // last key tile this workgroup needs; (causal) a wavefront needs tiles up
    // to its last row
    const int rows_end = min(r0 + kBM, L);
    const int nkt = p.causal ? (rows_end + kBN - 1) / kBN : (Lk + kBN - 1) / kBN;
    const int wave_last_row = min(wr0 + kRowsPerWave, L) - 1;

    // K/V tile staging: K 64 rows x 24 chunks (3 per thread), V 64 x 16 (2
    // per thread).  Each thread's chunk pointers are formed once, at its row
    // of tile 0; a whole tile adds a uniform stride, and the last, partial
    // tile clamps rows to key Lk - 1.
    u32x4 sk[3], sv[2];
    const uint16_t* kp[3];
    const uint16_t* vp[2];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int c = tid + 512 * i;
        kp[i] = p.k + (int64_t)(ka + c / 24) * p.k_st + (int64_t)h * p.k_sh + 8 * (c % 24);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + 512 * i;
        vp[i] = p.v + (int64_t)(ka + (c >> 4)) * p.v_st + (int64_t)h * p.v_sh + 8 * (c & 15);
    }
    auto load_tile = [&](int kt) {
        if (kt * kBN + kBN <= Lk) {
            const int64_t ko = (int64_t)(kt * kBN) * p.k_st, vo = (int64_t)(kt * kBN) * p.v_st;
#pragma unroll
            for (int i = 0; i < 3; ++i) sk[i] = *reinterpret_cast<const u32x4*>(kp[i] + ko);
#pragma unroll
            for (int i = 0; i < 2; ++i) sv[i] = *reinterpret_cast<const u32x4*>(vp[i] + vo);
        } else {
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                const int r = (tid + 512 * i) / 24;
                const int j = min(kt * kBN + r, Lk - 1);
                sk[i] = *reinterpret_cast<const u32x4*>(kp[i] + (int64_t)(j - r) * p.k_st);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = (tid + 512 * i) >> 4;
                const int j = min(kt * kBN + r, Lk - 1);
                sv[i] = *reinterpret_cast<const u32x4*>(vp[i] + (int64_t)(j - r) * p.v_st);
            }
        }
    };
    // LDS row of tile key k: within its 32-key half, key 16g + 4a + b goes
    // to row 8a + 4g + b (the layout described above the kernel)
    // (each thread's store offsets are the same for every tile)
    auto tile_row = [](int k) { return (k & 32) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3); };
    int kso[3], vso[2];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int c = tid + 512 * i;
        kso[i] = tile_row(c / 24) * kPitchK + 8 * (c % 24);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + 512 * i;
        vso[i] = tile_row(c >> 4) * kPitchV + 8 * (c & 15);
    }
    auto store_tile = [&](int buf, int vbuf) {
#pragma unroll
        for (int i = 0; i < 3; ++i) *reinterpret_cast<u32x4*>(&sm.kt[buf][kso[i]]) = sk[i];
#pragma unroll
        for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4*>(&sm.vt[vbuf][vso[i]]) = sv[i];
    };

    f32x16 o[4];   // O^T: element v of o[dt] is dim 32dt + 8(v/4) + 4 g2 + v%4 of this row
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.0f;
    const float c_log2 = p.score_scale_log2;

    // P of the current tile, quantized (fp16 B operand of the PV products);
    // wavefronts 4-7 keep it for one iteration when the PV is deferred
    f16x8 hold[4];
    // O^T += V^T P^T.  A fragment (dim tile dt, k-step kb) of the V tile at
    // vb: lane l gets dim 32dt + l%32 and rows 16kb + 4 g2 + 0..3 (slots
    // 0..3) and 16kb + 8 + 4 g2 + 0..3 (slots 4..7) by two transposing reads;
    // in each 16-lane group lane s addresses row k0 + s/4 and dims c0 +
    // 4(s%4) .. +3, and receives the 4 rows of dim c0 + s.
    const int s16 = lane & 15;
    const int vlane = (4 * g2 + (s16 >> 2)) * kPitchV + 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
    auto vfrag = [&](const uint16_t* vb, int kb, int dt) {
        const uint16_t* a0 = vb + vlane + 16 * kb * kPitchV + 32 * dt;
        const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)(const_cast<uint16_t*>(a0)));
        const s16x4 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)(const_cast<uint16_t*>(a0 + 8 * kPitchV)));
        const u32x2 y1 = __builtin_bit_cast(u32x2, x1), y2 = __builtin_bit_cast(u32x2, x2);
        return u32x4{y1[0], y1[1], y2[0], y2[1]};
    };
    // the quantized-P products (fp16); the fragments of k-step kb + 1 are
    // read during k-step kb's products
    auto pv_f16 = [&](const uint16_t* vb, const f16x8 (&pp)[4]) {
        u32x4 vf[2][4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) vf[0][dt] = vfrag(vb, 0, dt);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if (kb + 1 < 4) {
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) vf[(kb + 1) & 1][dt] = vfrag(vb, kb + 1, dt);
            }
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) o[dt] = mfma32_f16(__builtin_bit_cast(f16x8, vf[kb & 1][dt]), pp[kb], o[dt]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto compute = [&](int kt, int buf, int vbuf, auto mask_tag, bool defer) {
        constexpr bool kMask = decltype(mask_tag)::value;
        const uint16_t* kb = sm.kt[buf];
        const uint16_t* vb = sm.vt[vbuf];
        // ---- S^T for keys 32 mt2 .. +31
        f32x16 s[2] = {f32x16{}, f32x16{}};
        auto kfrag = [&](int kk, int mt2) {
            return *reinterpret_cast<const u32x4*>(&kb[(32 * mt2 + l32) * kPitchK + 16 * kk + 8 * g2]);
        };
        // fragments one k-step ahead of their MFMAs
        u32x4 af[2][2];
        af[0][0] = kfrag(0, 0);
        af[0][1] = kfrag(0, 1);
#pragma unroll
        for (int kk = 0; kk < 12; ++kk) {
            if (kk + 1 < 12) {
                af[(kk + 1) & 1][0] = kfrag(kk + 1, 0);
                af[(kk + 1) & 1][1] = kfrag(kk + 1, 1);
            }
#pragma unroll
            for (int mt2 = 0; mt2 < 2; ++mt2) s[mt2] = mfma32_bf16(as_bf16x8(af[kk & 1][mt2]), qf[kk], s[mt2]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- softmax: z in log2 units; the running max refreshed per tile
        // (a tile without masked keys: the max is taken on the raw scores,
        // since fp32(c x) is monotone in x for c >= 0, and each exponent is
        // one fused c * s - m)
        float mx = -INFINITY;
        // element v of score tile mt2 is key 32 mt2 + 16 g2 + v of the tile
        // (the permuted rows above); with 2:4 sparsity, of each group
        // of 4 keys (elements 4c .. 4c+3) the two outranked by two others are
        // dropped: key i beats key j > i when x_i >= x_j (equal scores rank
        // by index), one comparison per pair
        auto two_of = [](bool x, bool y, bool z) { return (x && y) || (z && (x || y)); };
        auto drop_2_4 = [&](float x0, float x1, float x2, float x3, bool (&d)[4]) {
            const bool b01 = x0 >= x1, b02 = x0 >= x2, b03 = x0 >= x3;
            const bool b12 = x1 >= x2, b13 = x1 >= x3, b23 = x2 >= x3;
            d[0] = two_of(!b01, !b02, !b03);
            d[1] = two_of(b01, !b12, !b13);
            d[2] = two_of(b02, b12, !b23);
            d[3] = two_of(b03, b13, b23);
        };
        if constexpr (kMask) {
            // keys past this row's last key are masked; the 2:4 ranking sees
            // them as -inf and ranks the raw scores (times rank_mul: 0 when
            // softmax_scale is 0, which makes every seen score tie)
            const int rel = lim - (kt * kBN + 16 * g2);  // last key offset this lane's row sees
#pragma unroll
            for (int mt2 = 0; mt2 < 2; ++mt2)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    bool seen[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) seen[i] = 32 * mt2 + 4 * c + i <= rel;
                    if constexpr (kSparse) {
                        float x[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) x[i] = seen[i] ? p.rank_mul * s[mt2][4 * c + i] : -INFINITY;
                        bool d[4];
                        drop_2_4(x[0], x[1], x[2], x[3], d);
#pragma unroll
                        for (int i = 0; i < 4; ++i) seen[i] = seen[i] && !d[i];
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float z = seen[i] ? c_log2 * s[mt2][4 * c + i] : -INFINITY;
                        s[mt2][4 * c + i] = z;
                        mx = fmaxf(mx, z);
                    }
                }
        } else {
            // (with 2:4 sparsity the tile is ranked on the raw scores: the
            // caller sends tiles here only when softmax_scale > 0)
            if constexpr (kSparse) {
#pragma unroll
                for (int mt2 = 0; mt2 < 2; ++mt2)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        bool d[4];
                        drop_2_4(s[mt2][4 * c], s[mt2][4 * c + 1], s[mt2][4 * c + 2], s[mt2][4 * c + 3], d);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (d[i]) s[mt2][4 * c + i] = -INFINITY;
                    }
            }
#pragma unroll
            for (int mt2 = 0; mt2 < 2; ++mt2)
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[mt2][v]);
        }
        mx = xor32_max(mx);
        if constexpr (!kMask) mx = c_log2 * mx;
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        float psum = 0.0f;
#pragma unroll
        for (int mt2 = 0; mt2 < 2; ++mt2)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                if constexpr (kMask) s[mt2][v] = __builtin_amdgcn_exp2f(s[mt2][v] - m_use);
                else s[mt2][v] = __builtin_amdgcn_exp2f(__builtin_fmaf(c_log2, s[mt2][v], -m_use));
                psum += s[mt2][v];
            }
        psum = xor32_sum(psum);
        l_run = alpha * l_run + psum;   // unquantized denominator
        m_run = m_new;
        // (multiplying by 1 changes nothing: skipped when no row moved)
        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
        }
        // ---- P operands per 16-key block kb
        bf16x8 ph[4], pm[4], pl[4];
        if constexpr (kPMode == 2) {
            // per-tensor FP8: code = e4m3(fp32(p * fp32(1/g_p))) (p >= 0),
            // its exact value in the fp16 or bf16 operand
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const f32x16& t = s[kb >> 1];
                const int o8 = 8 * (kb & 1);
                float d[8];
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    const uint32_t c2 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                        fminf(t[o8 + i] * p.inv_g_p, 448.0f), fminf(t[o8 + i + 1] * p.inv_g_p, 448.0f), 0, false);
                    const f32x2 dv = __builtin_amdgcn_cvt_pk_f32_fp8(c2, false);
                    d[i] = dv[0];
                    d[i + 1] = dv[1];
                }
                if constexpr (kF16) {
                    hold[kb] = f16x8{(_Float16)d[0], (_Float16)d[1], (_Float16)d[2], (_Float16)d[3],
                                     (_Float16)d[4], (_Float16)d[5], (_Float16)d[6], (_Float16)d[7]};
                } else {
                    ph[kb] = as_bf16x8(u32x4{pack_bf16_exact(d[0], d[1]), pack_bf16_exact(d[2], d[3]),
                                             pack_bf16_exact(d[4], d[5]), pack_bf16_exact(d[6], d[7])});
                }
            }
        } else if constexpr (kQuantP) {
            // this lane's two P blocks (elements 0..15 of s[mt2], block
            // 2 mt2 + g2): maxima and scales side by side (the rare exact
            // divisions in one uniform branch)
            float am[2], tq[2];
            bool nr[2];
            bool any_near = false;
#pragma unroll
            for (int mt2 = 0; mt2 < 2; ++mt2) {
                const f32x16& t = s[mt2];
                float m8[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int o8 = 8 * hh;
                    m8[hh] = fmaxf(fmaxf(fmaxf(t[o8], t[o8 + 1]), fmaxf(t[o8 + 2], t[o8 + 3])),
                                   fmaxf(fmaxf(t[o8 + 4], t[o8 + 5]), fmaxf(t[o8 + 6], t[o8 + 7])));
                }
                am[mt2] = fmaxf(m8[0], m8[1]);
                tq[mt2] = am[mt2] * p.inv_u_p;
                nr[mt2] = scale_quotient_near_tie(tq[mt2]);
                any_near |= nr[mt2];
            }
            if (__any(any_near)) {
#pragma unroll
                for (int mt2 = 0; mt2 < 2; ++mt2) tq[mt2] = nr[mt2] ? am[mt2] / p.u_p : tq[mt2];
            }
            // the two blocks' e4m3 codes by one hardware conversion (tq >= 0;
            // see e4m3_encode_nonneg)
            const uint32_t codes2 =
                (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(tq[0], 448.0f), fminf(tq[1], 448.0f), 0, false);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                // k-step kb: elements 8(kb%2) .. +7 of s[kb/2], block kb/2's scale
                const f32x16& t = s[kb >> 1];
                const int o8 = 8 * (kb & 1);
                const uint32_t code = (codes2 >> (8 * (kb >> 1))) & 0xffu;
                const float inv = sm.pinv[code];
                const float sval = e4m3_decode(code);
                uint32_t c8 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, t[o8] * inv, t[o8 + 1] * inv, 1.0f, 0);
                c8 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c8, t[o8 + 2] * inv, t[o8 + 3] * inv, 1.0f, 1);
                c8 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c8, t[o8 + 4] * inv, t[o8 + 5] * inv, 1.0f, 2);
                c8 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c8, t[o8 + 6] * inv, t[o8 + 7] * inv, 1.0f, 3);
                if constexpr (kF16) {
                    const _Float16 sh = (_Float16)sval;
                    const f16x2 ss = {sh, sh};
                    const f16x2 d0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c8, 1.0f, 0) * ss;
                    const f16x2 d1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c8, 1.0f, 1) * ss;
                    const f16x2 d2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c8, 1.0f, 2) * ss;
                    const f16x2 d3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c8, 1.0f, 3) * ss;
                    hold[kb] = f16x8{d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
                } else {
                    const f32x2 d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c8, 1.0f, 0);
                    const f32x2 d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c8, 1.0f, 1);
                    const f32x2 d2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c8, 1.0f, 2);
                    const f32x2 d3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c8, 1.0f, 3);
                    ph[kb] = as_bf16x8(u32x4{pack_bf16_exact(d0[0] * sval, d0[1] * sval),
                                             pack_bf16_exact(d1[0] * sval, d1[1] * sval),
                                             pack_bf16_exact(d2[0] * sval, d2[1] * sval),
                                             pack_bf16_exact(d3[0] * sval, d3[1] * sval)});
                }
            }
        } else {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                // three bf16 parts (|p - hi - mid - lo| <= 2^-24 |p|)
                const f32x16& t = s[kb >> 1];
                const int o8 = 8 * (kb & 1);
                u32x4 hv, mv, lv;
#pragma unroll
                for (int pr = 0; pr < 4; ++pr) {
                    const float x0 = t[o8 + 2 * pr], x1 = t[o8 + 2 * pr + 1];
                    const uint32_t h1 = pack_bf16_rne(x0, x1);
                    const float e0 = x0 - bf16_lo(h1), e1 = x1 - bf16_hi(h1);
                    const uint32_t m1 = pack_bf16_rne(e0, e1);
                    hv[pr] = h1;
                    mv[pr] = m1;
                    lv[pr] = pack_bf16_rne(e0 - bf16_lo(m1), e1 - bf16_hi(m1));
                }
                ph[kb] = as_bf16x8(hv);
                pm[kb] = as_bf16x8(mv);
                pl[kb] = as_bf16x8(lv);
            }
        }
        if constexpr (kQuantP && kF16) {
            if (!defer) pv_f16(vb, hold);
            return;
        }
        // ---- O^T += V^T P^T in bf16 (P unquantized as three parts, or V
        // unquantized); the fragments of k-step kb + 1 are read during k-step
        // kb's products
        u32x4 vf[2][4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) vf[0][dt] = vfrag(vb, 0, dt);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if (kb + 1 < 4) {
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) vf[(kb + 1) & 1][dt] = vfrag(vb, kb + 1, dt);
            }
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const u32x4 va = vf[kb & 1][dt];
                if constexpr (kF16) {
                    o[dt] = mfma32_f16(__builtin_bit_cast(f16x8, va), hold[kb], o[dt]);
                } else {
                    o[dt] = mfma32_bf16(as_bf16x8(va), ph[kb], o[dt]);
                    if constexpr (!kQuantP) {
                        o[dt] = mfma32_bf16(as_bf16x8(va), pm[kb], o[dt]);
                        o[dt] = mfma32_bf16(as_bf16x8(va), pl[kb], o[dt]);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (nkt > 0) {
        load_tile(0);
        store_tile(0, 0);
    }
    if (nkt > 1) load_tile(1);
    __syncthreads();
    // With P and V quantized, wavefronts 4-7 (which share SIMDs with 0-3)
    // run the PV products of tile kt at the start of iteration kt+1, so that
    // they overlap the softmax of wavefronts 0-3 instead of their products.
    // O sees the same operations in the same order.  Tile kt's K sits in
    // K buffer kt % 2 and its V in V buffer kt % 3, so the V of a deferred
    // tile stays resident for one more iteration.
    const bool defer = (kQuantP && kF16) && w >= 4;
    int held = -1;   // V buffer of the tile whose PV is deferred
    int vbuf = 0;    // V buffer of tile kt
    for (int kt = 0; kt < nkt; ++kt) {
        // (opaque to the compiler, so that it keeps one set of V addresses)
        const int vnext = __builtin_amdgcn_readfirstlane(vbuf == 2 ? 0 : vbuf + 1);
        if constexpr (kQuantP && kF16) {
            if (held >= 0) {
                pv_f16(sm.vt[held], hold);
                held = -1;
            }
        }
        // (causal) a wavefront skips tiles that start after its last row;
        // tiles whose keys all lie within every row's reach need no mask
        // (unless the 2:4 choice masks keys)
        if (wave_rows && (!p.causal || kt * kBN <= wave_last_row)) {
            const bool full = p.causal ? kt * kBN + kBN - 1 <= wr0 : kt * kBN + kBN <= Lk;
            if (full && (!kSparse || p.rank_mul != 0.0f)) compute(kt, kt & 1, vbuf, BoolTag<false>{}, defer);
            else compute(kt, kt & 1, vbuf, BoolTag<true>{}, defer);
            if constexpr (kQuantP && kF16) {
                if (defer) held = vbuf;
            }
        }
        if (kt + 1 < nkt) store_tile((kt + 1) & 1, vnext);   // staged during compute(kt)
        if (kt + 2 < nkt) load_tile(kt + 2);          // lands during compute(kt+1)
        lds_barrier();
        vbuf = vnext;
    }
    if constexpr (kQuantP && kF16) {
        if (held >= 0) pv_f16(sm.vt[held], hold);
    }

    if (!wave_rows) return;
    // ---- epilogue: O = acc * g_p g_v / l in fp64, rounded once to fp32 (when
    // the accumulation is exact, as for a row that sees one key, NVFP4
    // rounding ties then break as in an exact evaluation); output block b
    // (dims 16b .. +15) is elements 8(b%2) .. +7 of o[b/2] in lanes l and
    // l ^ 32: dims 16b + 4 g2 + 0..3 and 16b + 8 + 4 g2 + 0..3.
    const bool ok = row < L;
    const double inv_l = l_run > 0.0f ? p.out_scale / (double)l_run : 0.0;
    const int64_t t = a + row;
    const float lse_v = l_run > 0.0f ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : -INFINITY;
    if (!p.out_fp4) {
        // fp32 rows: block b's elements 0..3 are dims 16b + 4 g2 + 0..3, 4..7
        // are dims 16b + 8 + 4 g2 + 0..3 (a row without keys is 0, lse -inf)
        if (!ok) return;
        float* dst = p.out_f32 + t * p.o_st + (int64_t)h * p.o_sh + 4 * g2;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const f32x16& ob = o[b >> 1];
            const int o8 = 8 * (b & 1);
            f32x4 lo, hi;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lo[i] = (float)((double)ob[o8 + i] * inv_l);
                hi[i] = (float)((double)ob[o8 + 4 + i] * inv_l);
            }
            *reinterpret_cast<f32x4*>(dst + 16 * b) = lo;
            *reinterpret_cast<f32x4*>(dst + 16 * b + 8) = hi;
        }
        if (g2 == 0 && p.lse) p.lse[t * p.lse_st + (int64_t)h * p.lse_sh] = lse_v;
        return;
    }
    uint8_t* codes_row = p.out_fp4 + (t * p.H + h) * (kDv / 2);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        float x[8];
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i] = (float)((double)o[b >> 1][8 * (b & 1) + i] * inv_l);
            am = fmaxf(am, __builtin_fabsf(x[i]));
        }
        am = xor32_max(am);
        const Nvfp4Scale sc = nvfp4_block_scale(am, p.g_out);
        // codes of dims 16b + 4 g2 + 0..3 (bytes 2 g2, 2 g2 + 1) and
        // 16b + 8 + 4 g2 + 0..3 (bytes 4 + 2 g2, 5 + 2 g2)
        const uint32_t c8 = e2m1_encode8(x, sc.inv);
        const uint32_t c01 = c8 & 0xffffu, c23 = c8 >> 16;
        if (ok) {
            *reinterpret_cast<uint16_t*>(codes_row + 8 * b + 2 * g2) = (uint16_t)c01;
            *reinterpret_cast<uint16_t*>(codes_row + 8 * b + 4 + 2 * g2) = (uint16_t)c23;
            if (g2 == 0) {
                const int64_t cpad = (int64_t)p.H * 8;
                p.out_scales[swizzled_scale_offset(t, (int64_t)h * 8 + b, cpad)] = (uint8_t)sc.code;
            }
        }
    }
    if (ok && g2 == 0 && p.lse) p.lse[t * p.lse_st + (int64_t)h * p.lse_sh] = lse_v;
}

// Zero the scale bytes of rows T .. ceil(T/128)*128 - 1 (all columns).
__global__ __launch_bounds__(256) void pad_scales_kernel(uint8_t* scales, int64_t T, int64_t cpad) {
    const int64_t tpad = (T + 127) / 128 * 128;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n = (tpad - T) * cpad;
    if (idx >= n) return;
    const int64_t m = T + idx / cpad, c = idx % cpad;
    scales[swizzled_scale_offset(m, c, cpad)] = 0;
}

template <int kPMode, bool kF16>
void launch_attn(bool sparse, dim3 grid, dim3 block, hipStream_t stream, const AttnParams& p) {
    if (sparse) hipLaunchKernelGGL((attn_kernel<kPMode, kF16, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((attn_kernel<kPMode, kF16, false>), grid, block, 0, stream, p);
}

}  // namespace

int prefill_p_tile() { return kBN; }

size_t prefill_workspace_bytes(int64_t T, int H, unsigned flags) {
    size_t b = 0;
    const size_t rows = (size_t)T * H;
    if (flags & 2u) b += rows * kDqk * 2;
    if (flags & 8u) b += rows * kDv * 2;
    return b;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    const int H = a.H;
    const int64_t T = a.T;
    const bool causal = a.causal != 0;
    const int64_t Tk = causal ? T : a.T_k;
    const int32_t* cuk = causal ? a.cu_seqlens : a.cu_k;
    const int max_k = causal ? a.max_seqlen : a.max_seqlen_k;
    const unsigned f = a.flags;
    const bool qP = f & 4u, qV = f & 8u;
    uint16_t* ws = static_cast<uint16_t*>(a.workspace);
    AttnParams p{};
    p.q = a.q; p.q_st = a.q_st; p.q_sh = a.q_sh;
    p.k = a.k; p.k_st = a.k_st; p.k_sh = a.k_sh;
    p.v = a.v; p.v_st = a.v_st; p.v_sh = a.v_sh;
    float gq = 1.0f, gk = 1.0f, gv = 1.0f, gp = 1.0f;
    if (f & 1u) {   // (in attn_kernel)
        p.q_qdq = 1;
        p.q_fp8 = (f & 16u) ? 1 : 0;
        p.q_g = a.g_q;
        p.q_inv = 1.0f / a.g_q;
        gq = a.g_q;
    }
    if ((f & 2u) && Tk > 0) {
        const int64_t nqk_blocks = Tk * H * (kDqk / 16);
        const dim3 grid((unsigned)((nqk_blocks + 255) / 256));
        if (f & 32u)
            hipLaunchKernelGGL(qk_qdq_kernel<true>, grid, dim3(256), 0, stream, a.k, a.k_st, a.k_sh, Tk, H, a.g_k,
                               1.0f / a.g_k, ws);
        else
            hipLaunchKernelGGL(qk_qdq_kernel<false>, grid, dim3(256), 0, stream, a.k, a.k_st, a.k_sh, Tk, H, a.g_k,
                               1.0f / a.g_k, ws);
        p.k = ws; p.k_st = (int64_t)H * kDqk; p.k_sh = kDqk;
        ws += (size_t)Tk * H * kDqk;
    }
    if (f & 2u) gk = a.g_k;
    if (qV && Tk > 0) {
        if (f & 128u) {
            const int64_t n8 = Tk * H * (kDv / 8);
            const dim3 grid((unsigned)((n8 + 255) / 256));
            if (qP)
                hipLaunchKernelGGL(v_fp8_kernel<true>, grid, dim3(256), 0, stream, a.v, a.v_st, a.v_sh, Tk, H,
                                   1.0f / a.g_v, ws);
            else
                hipLaunchKernelGGL(v_fp8_kernel<false>, grid, dim3(256), 0, stream, a.v, a.v_st, a.v_sh, Tk, H,
                                   1.0f / a.g_v, ws);
        } else {
            const dim3 grid((unsigned)((max_k + 15) / 16), (unsigned)a.N, (unsigned)((H * (kDv / 8) + 255) / 256));
            if (qP)
                hipLaunchKernelGGL(v_qdq_kernel<true>, grid, dim3(256), 0, stream, a.v, a.v_st, a.v_sh, cuk, H,
                                   a.g_v, ws);
            else
                hipLaunchKernelGGL(v_qdq_kernel<false>, grid, dim3(256), 0, stream, a.v, a.v_st, a.v_sh, cuk, H,
                                   a.g_v, ws);
        }
        p.v = ws; p.v_st = (int64_t)H * kDv; p.v_sh = kDv;
        ws += (size_t)Tk * H * kDv;
    }
    if (qV) gv = a.g_v;
    if (qP) gp = a.g_p;
    p.cu = a.cu_seqlens;
    p.ck = cuk;
    p.causal = causal ? 1 : 0;
    p.H = H;
    p.score_scale_log2 = a.softmax_scale * gq * gk * kLog2e;
    p.rank_mul = a.softmax_scale > 0.0f ? 1.0f : 0.0f;
    p.out_scale = (double)gp * (double)gv;
    p.g_p = a.g_p;
    p.u_p = 6.0f * a.g_p;
    p.inv_u_p = 1.0f / p.u_p;
    p.inv_g_p = 1.0f / a.g_p;
    p.g_out = a.g_out;
    p.T = T;
    p.out_fp4 = a.out_fp4;
    p.out_scales = a.out_scales;
    p.out_f32 = a.out_f32;
    p.o_st = a.o_st;
    p.o_sh = a.o_sh;
    p.lse = a.lse;
    p.lse_st = a.lse_st;
    p.lse_sh = a.lse_sh;
    if (a.max_seqlen > 0) {
        const dim3 grid((unsigned)((a.max_seqlen + kBM - 1) / kBM), (unsigned)H, (unsigned)a.N);
        const dim3 block(kWaves * 64);
        const bool fp8p = f & 64u;
        const bool sp = f & 256u;
        if (qP && qV) {
            if (fp8p) launch_attn<2, true>(sp, grid, block, stream, p);
            else launch_attn<1, true>(sp, grid, block, stream, p);
        } else if (qP) {
            if (fp8p) launch_attn<2, false>(sp, grid, block, stream, p);
            else launch_attn<1, false>(sp, grid, block, stream, p);
        } else {
            launch_attn<0, false>(sp, grid, block, stream, p);
        }
    }
    if (a.out_fp4) {
        const int64_t cpad = (int64_t)H * 8;
        const int64_t npad = ((T + 127) / 128 * 128 - T) * cpad;
        if (npad > 0)
            hipLaunchKernelGGL(pad_scales_kernel, dim3((unsigned)((npad + 255) / 256)), dim3(256), 0, stream,
                               a.out_scales, T, cpad);
    }
    return hipGetLastError();
}

}  // namespace mla
