// Paged absorbed split-K MLA decode with quantized attention operands
// (gfx950): P quantized in the loop, Q quantized by the caller in an fp32
// carrier, and a raw bf16 latent cache whose K and V are quantized on read.
//
// [MO-MLA], PR body and commit 4: every attention matmul operand is
// fake-quantized once along its own contraction axis; the decode quantizes
// P after the softmax row sum (the denominator unquantized) and takes the
// caller's Q in an FP32 carrier; with a raw latent cache it quantizes K along
// the feature axis and V along the token axis, independently, V in blocks of
// 16 at absolute token positions.  NVFP4 (1x16 blocks, e4m3 scale) or
// per-tensor FP8 per operand, as in the prefill.  [B12X], walkthrough: the
// NVFP4 records are dequantized on read with the per-layer outer scale.
//
// Work item: workgroup (split s, sequence b, group of 128 heads) of 8
// wavefronts (two per SIMD), each owning 16 heads, so that a tile is staged
// once for all 128 heads.  The split's tokens are walked in tiles of 32;
// every wavefront sees all of them in order, so each holds one running max,
// refreshed per tile, against which P is quantized.  Per tile:
//   offsets   threads 0..31 walk the page table two tiles ahead (three
//             offset slots in LDS);
//   staging   the workgroup dequantizes (NVFP4 records: s*v, exact in fp16)
//             or quantizes (raw records: K in 16-feature blocks, V in
//             16-token blocks per dim, from the bf16 values) the tile into a
//             K tile (576 columns; RoPE columns bf16) and a V tile (512
//             columns) in LDS; a raw tile's K words are loaded during the
//             previous tile's softmax and PV products;
//   compute   (wavefronts that own heads) S^T = K Q^T on
//             v_mfma_f32_16x16x32 (Q's first kQLdsLatent latent k-steps and
//             its RoPE k-steps in LDS, the others in registers; latent
//             k-steps fp16, or bf16 for raw unquantized K; RoPE k-steps
//             bf16), fragments one k-step ahead of their products, latent
//             and RoPE partial scores scaled separately; online softmax in
//             base 2;
//             P quantized per 16-key block (NVFP4) or per element (FP8),
//             exact in the fp16 / bf16 B operand, or unquantized as fp16
//             hi + lo (bf16 V: three bf16 parts); O^T = V^T P^T with V^T
//             read by ds_read_b64_tr_b16.
// Epilogue: out = vmul * O / l (vmul: the V and P multipliers), lse = m +
// ln l, to the output (one split) or to the workspace as fp32 partials, which
// split_merge_kernel merges.
#include "device_common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int kTile = 32;
constexpr int kPitch = kQK + 16;   // elements per tile row (592: 1184 B, conflict-free fragment reads)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeadsPerGroup = 16 * kWaves;
// Q k-steps kept in LDS (B-operand layout, 16 B per lane): the first
// kQLdsLatent latent k-steps and the two RoPE k-steps; the others stay in
// registers.
constexpr int kQLdsLatent = 8;
constexpr int kQLds = kQLdsLatent + 2;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

struct QdqSmem {
    uint16_t kt[kTile * kPitch];   // K tile: latent (fp16 or bf16) then RoPE (bf16)
    uint16_t vt[kTile * kPitch];   // V tile: latent (fp16 or bf16)
    u32x4 qs[kWaves][kQLds][64];   // each wavefront's LDS-held Q B-operand fragments (slot, lane)
    int64_t offs[3][kTile];        // record byte offsets of tiles t .. t+2 (masked tokens: 0)
    uint32_t valid[3];             // bit i: token i of the tile is unmasked
};

__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    const f16x2 h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// Packed operand values (fp16 pairs when kF16, bf16 pairs otherwise) of 8
// floats that the target type holds exactly.
template <bool kF16>
__device__ __forceinline__ u32x4 pack8_exact(const float* x) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = kF16 ? pack_f16(x[2 * i], x[2 * i + 1]) : pack_bf16_exact(x[2 * i], x[2 * i + 1]);
    return r;
}

// Quantize-dequantize of 16 values along their block: NVFP4 (multiplier g,
// u = fp32(6 g) and inv_u = fp32(1/u) given; the exact values s*v are
// returned, g not applied) or per-tensor FP8 (inv_g = fp32(1/g); the exact
// e4m3 values are returned).
__device__ __forceinline__ void qdq16(float* x, bool fp8, float g, float inv_g, float u, float inv_u) {
    if (fp8) {
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(e4m3_encode2_hw(x[i] * inv_g, x[i + 1] * inv_g), false);
            x[i] = d[0];
            x[i + 1] = d[1];
        }
        return;
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, __builtin_fabsf(x[i]));
    const Nvfp4Scale sc = nvfp4_block_scale_fast(a, g, u, inv_u);
    const float sv = e4m3_decode(sc.code);
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
        const f32x2 d = e2m1_pair<0>(e2m1_pack2<0>(0u, x[i] * sc.inv, x[i + 1] * sc.inv));
        x[i] = d[0] * sv;
        x[i + 1] = d[1] * sv;
    }
}

struct QdqParams {
    DecodeArgs d;
    unsigned flags;           // 1 Q, 2 K, 4 P, 8 V; 16/32/64/128 FP8 formats
    float g_q, g_k, g_v, g_p;
    // Per-call constants formed on the host in IEEE fp32 (the same values the
    // device would compute), so that they stay in scalar registers rather
    // than a vector register per lane: 1/g_k, 1/g_v, 1/g_p, the units 6 g of
    // K's, V's and P's block scales and their reciprocals, the RoPE score
    // multiplier and the output multiplier.
    float inv_g_k, inv_g_v, inv_g_p, u_k, inv_u_k, u_v, inv_u_v, u_p, inv_u_p, sc_rope, v_mul;
};

// kCache: 0 NVFP4 records with bf16 RoPE, 1 NVFP4 with e4m3 RoPE, 2 raw bf16
// records (1152 B).  kKF16 / kVF16: the latent K / V tile holds fp16 (exact
// s*v or e4m3 values) rather than bf16 (raw values).
template <int kCache, bool kKF16, bool kVF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_qdq_kernel(QdqParams pp) {
    constexpr bool kRaw = kCache == 2;
    constexpr int kRec = kCache == 0 ? 432 : (kCache == 1 ? 368 : 1152);
    const DecodeArgs& p = pp.d;
    __shared__ QdqSmem sm;

    // Placement: workgroups are dispatched round-robin over the 8 XCDs in
    // linear-id order.  When 8 divides B, sequence b runs on XCD b % 8 and the
    // head groups of one (sequence, split) are consecutive there, so that
    // they run together and all but the first read the records from that
    // XCD's L2 (a bijection onto splits x sequences x head groups).
    int s, b, hg;
    {
        const int G = (int)gridDim.z, S = p.max_splits;
        const int L = (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
        if ((p.B & 7) == 0) {
            const int k = L >> 3;
            hg = k % G;
            s = (k / G) % S;
            b = (L & 7) + 8 * (k / (G * S));
        } else {
            hg = L % G;
            s = (L / G) % S;
            b = L / (G * S);
        }
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int gq = lane >> 4, c16 = lane & 15;
    const int hq = hg * kHeadsPerGroup + 16 * w + c16;
    const bool hok = hq < p.H;
    const bool wave_active = hg * kHeadsPerGroup + 16 * w < p.H;   // (wavefront-uniform)

    int L = p.seq_lens[b];
    const int Lmax = p.max_pages * p.page_size;
    L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
    const int ns = decode_num_splits(L, p.max_splits);
    if (s >= ns) return;
    const int ct = decode_chunk_tiles(L, p.max_splits);   // in 64-token tiles
    const int i0 = 64 * ct * s;
    const int i1 = min(L, i0 + 64 * ct);
    const int ntiles = (i1 - i0 + kTile - 1) / kTile;

    const bool qQ = pp.flags & 1u, qK = pp.flags & 2u, qP = pp.flags & 4u, qV = pp.flags & 8u;
    const bool fQ = pp.flags & 16u, fK = pp.flags & 32u, fP = pp.flags & 64u, fV = pp.flags & 128u;

    // ---- Q (B operand): lane holds head c16, dims 32kk + 8gq .. +7 (kk 16,
    // 17: RoPE).  Quantized: NVFP4 blocks of 16 features (block 2kk + gq/2
    // spans lanes gq and gq ^ 1) or per-tensor FP8, the exact values kept.
    // Raw with fp16 K: scaled by 2^(14 - E) per head (exact).
    // (k-steps kQLdsLatent..15 in registers qf, the others in LDS sm.qs)
    float q_mul_lat = 1.0f;
    u32x4 qf[16 - kQLdsLatent];
    {
        const int64_t qoff = (int64_t)b * p.q_stride_b + (int64_t)(hok ? hq : 0) * p.q_stride_h + 8 * gq;
        const u32x4 zero = {0u, 0u, 0u, 0u};
        float x[18][8];
#pragma unroll
        for (int kk = 0; kk < 18; ++kk) {
            const u32x4 r = hok ? *reinterpret_cast<const u32x4*>((kk < 16 ? p.q_nope + 32 * kk : p.q_rope + 32 * (kk - 16)) + qoff)
                                : zero;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[kk][2 * j] = bf16_lo(r[j]);
                x[kk][2 * j + 1] = bf16_hi(r[j]);
            }
        }
        if (qQ) {
            const float inv_g = 1.0f / pp.g_q;
#pragma unroll
            for (int kk = 0; kk < 18; ++kk) {
                if (fQ) {
#pragma unroll
                    for (int i = 0; i < 8; i += 2) {
                        const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(
                            e4m3_encode2_hw(x[kk][i] * inv_g, x[kk][i + 1] * inv_g), false);
                        x[kk][i] = d[0];
                        x[kk][i + 1] = d[1];
                    }
                } else {
                    float a = 0.0f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) a = fmaxf(a, __builtin_fabsf(x[kk][i]));
                    a = xor16_max(a);
                    const Nvfp4Scale sc = nvfp4_block_scale(a, pp.g_q);
                    const float sv = e4m3_decode(sc.code);
#pragma unroll
                    for (int i = 0; i < 8; i += 2) {
                        const f32x2 d = e2m1_pair<0>(e2m1_pack2<0>(0u, x[kk][i] * sc.inv, x[kk][i + 1] * sc.inv));
                        x[kk][i] = d[0] * sv;
                        x[kk][i + 1] = d[1] * sv;
                    }
                }
            }
            q_mul_lat = pp.g_q;
        } else if (kKF16) {
            float amax = 0.0f;
#pragma unroll
            for (int kk = 0; kk < 16; ++kk)
#pragma unroll
                for (int i = 0; i < 8; ++i) amax = fmaxf(amax, __builtin_fabsf(x[kk][i]));
            amax = xor32_max(xor16_max(amax));
            int E = amax > 0.0f ? (int)((f2u(amax) >> 23) & 0xffu) - 127 : 0;
            E = E < -100 ? -100 : E;
            q_mul_lat = __builtin_ldexpf(1.0f, E - 14);
#pragma unroll
            for (int kk = 0; kk < 16; ++kk)
#pragma unroll
                for (int i = 0; i < 8; ++i) x[kk][i] = __builtin_ldexpf(x[kk][i], 14 - E);
        }
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            if (kk < kQLdsLatent) sm.qs[w][kk][lane] = pack8_exact<kKF16>(x[kk]);
            else qf[kk - kQLdsLatent] = pack8_exact<kKF16>(x[kk]);
        }
#pragma unroll
        for (int kk = 16; kk < 18; ++kk) sm.qs[w][kQLdsLatent + kk - 16][lane] = pack8_exact<false>(x[kk]);
    }
    // multipliers of the stored operands: NVFP4 latent * outer; raw K or V
    // quantized * g_k, g_v; P quantized * g_p
    const float k_mul_lat = kRaw ? (qK ? pp.g_k : 1.0f) : p.outer_scale;
    const float sc_lat = p.softmax_scale * kLog2e * q_mul_lat * k_mul_lat;
    const float sc_rope = pp.sc_rope, v_mul = pp.v_mul;
    const float u_p = pp.u_p, inv_u_p = pp.inv_u_p, inv_g_p = pp.inv_g_p;
    const float inv_gk = pp.inv_g_k, inv_gv = pp.inv_g_v;

    f32x4 o[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    const uint8_t* __restrict__ cache = p.cache;
    // Page walk of tile t into offset slot t % 3 by threads 0..31, two tiles
    // ahead: the page-table entry of tile t + 2 is requested at the start of
    // tile t and its offsets stored at the end, so that the load overlaps the
    // tile's work; a raw cache's K words of tile t + 1 are loaded after tile
    // t's score products and land during its softmax and PV (registers kw).
    constexpr int kKBlk = kTile * 36, kKIt = (kKBlk + kThreads - 1) / kThreads;   // K: 32 tokens x 36 blocks of 16 features
    u32x4 kw[kKIt][2];
    auto load_k_raw = [&](const int64_t* offs) {
        // (indices clamped, so every address is a record of the tile;
        // wavefronts with no block at step j load nothing)
        const int t0 = 64 * w + lane_now();
#pragma unroll
        for (int j = 0; j < kKIt; ++j) {
            if (kThreads * j + 64 * w >= kKBlk) break;
            const int i = min(t0 + kThreads * j, kKBlk - 1);
            const u32x4* src = reinterpret_cast<const u32x4*>(cache + offs[i / 36] + 32 * (i % 36));
            kw[j][0] = src[0];
            kw[j][1] = src[1];
        }
    };
    int pg_next = -1;
    auto walk_request = [&](int t) {
        const int pos = i0 + kTile * t + tid;
        int pi, rem;
        page_divmod(min(pos, max(i1 - 1, 0)), p.page_size, p.page_recip, pi, rem);
        pg_next = p.page_table[(int64_t)b * p.max_pages + pi];
    };
    auto walk_store = [&](int t) {
        const int pos = i0 + kTile * t + tid;
        int64_t off = -1;
        if (t < ntiles && pos < i1 && pg_next >= 0 && pg_next < p.num_pages) {
            int pi, rem;
            page_divmod(pos, p.page_size, p.page_recip, pi, rem);
            off = ((int64_t)pg_next * p.page_size + rem) * kRec;
        }
        const uint64_t vm = __ballot(off >= 0);
        sm.offs[t % 3][tid] = off < 0 ? 0 : off;
        if (tid == 0) sm.valid[t % 3] = (uint32_t)vm;
    };
    if (tid < kTile && ntiles > 0) {
        walk_request(0);
        walk_store(0);
        walk_request(1);
        walk_store(1);
    }
    __syncthreads();
    if constexpr (kRaw) {
        if (ntiles > 0) load_k_raw(sm.offs[0]);
    }
    for (int t = 0; t < ntiles; ++t) {
        if (tid < kTile) walk_request(t + 2);
        const int64_t* offs = sm.offs[t % 3];
        // (one word for the workgroup: read into a scalar register; the
        // masks below shift it per tile rather than testing loop-invariant
        // bit masks, which would each hold a register across the loop)
        const uint32_t vmask = __builtin_amdgcn_readfirstlane(sm.valid[t % 3]);
        // ---- staging
        if constexpr (!kRaw) {
            // 32 tokens x 64 chunks of 8 latent elements: code word + block scale
#pragma unroll
            for (int k = 0; k < 2048 / kThreads; ++k) {
                const int tok = w + (kThreads / 64) * k, ch = lane;   // chunk tid + kThreads k
                const uint8_t* rp = cache + offs[tok];
                const uint32_t cw = *reinterpret_cast<const uint32_t*>(rp + 4 * ch);
                const float scf = ((vmask >> tok) & 1u) ? e4m3_decode(rp[256 + (ch >> 1)]) : 0.0f;
                const _Float16 sh = (_Float16)scf;
                const f16x2 ss = {sh, sh};
                const f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0) * ss;
                const f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1) * ss;
                const f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2) * ss;
                const f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3) * ss;
                const u32x4 wv = {__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
                                  __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3)};
                *reinterpret_cast<u32x4*>(&sm.kt[tok * kPitch + 8 * ch]) = wv;
                *reinterpret_cast<u32x4*>(&sm.vt[tok * kPitch + 8 * ch]) = wv;
            }
            if (tid < 256) {   // RoPE: 32 tokens x 8 units of 8 values
                const int tok = tid >> 3, un = tid & 7;
                const uint8_t* rp = cache + offs[tok];
                u32x4 wv;
                if (kCache == 1) {
                    const u32x2 r2 = *reinterpret_cast<const u32x2*>(rp + 288 + 8 * un);
                    const u32x2 y0 = e4m3x4_to_bf16(r2[0]), y1 = e4m3x4_to_bf16(r2[1]);
                    wv = u32x4{y0[0], y0[1], y1[0], y1[1]};
                } else {
                    wv = *reinterpret_cast<const u32x4*>(rp + 288 + 16 * un);
                }
                const u32x4 zero = {0u, 0u, 0u, 0u};
                *reinterpret_cast<u32x4*>(&sm.kt[tok * kPitch + kLatent + 8 * un]) = ((vmask >> tok) & 1u) ? wv : zero;
            }
        } else {
            // K: 32 tokens x 36 blocks of 16 features (32 latent, 4 RoPE),
            // loaded during the previous tile.  The latent words also go to
            // the V tile as they are (masked tokens 0); a quantized V is then
            // formed there in place: 2 blocks of 16 tokens (absolute
            // positions base, base + 16) x 256 pairs of dims.
            const int half = __builtin_amdgcn_readfirstlane(tid >> 8), d0 = 2 * (tid & 255);
            const int t0 = 64 * w + lane_now();
#pragma unroll
            for (int j = 0; j < kKIt; ++j) {
                const int i = t0 + kThreads * j;
                if (i >= kKBlk) break;
                const int tok = i / 36, blk = i % 36;
                const bool ok = (vmask >> tok) & 1u;
                const u32x4 w0 = kw[j][0], w1 = kw[j][1];
                if (blk < 32) {
                    const u32x4 zero = {0u, 0u, 0u, 0u};
                    u32x4* vdst = reinterpret_cast<u32x4*>(&sm.vt[tok * kPitch + 16 * blk]);
                    vdst[0] = ok ? w0 : zero;
                    vdst[1] = ok ? w1 : zero;
                }
                float x[16];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    x[2 * jj] = ok ? bf16_lo(w0[jj]) : 0.0f;
                    x[2 * jj + 1] = ok ? bf16_hi(w0[jj]) : 0.0f;
                    x[8 + 2 * jj] = ok ? bf16_lo(w1[jj]) : 0.0f;
                    x[8 + 2 * jj + 1] = ok ? bf16_hi(w1[jj]) : 0.0f;
                }
                if (qK) qdq16(x, fK, pp.g_k, inv_gk, pp.u_k, pp.inv_u_k);
                u32x4 a, c;
                if (blk < 32 && kKF16) {
                    a = pack8_exact<true>(x);
                    c = pack8_exact<true>(x + 8);
                } else {
                    a = pack8_exact<false>(x);
                    c = pack8_exact<false>(x + 8);
                }
                u32x4* dst = reinterpret_cast<u32x4*>(&sm.kt[tok * kPitch + 16 * blk]);
                dst[0] = a;
                dst[1] = c;
            }
            // V quantized: per dim the block's amax (NVFP4) or each element
            // (FP8); unquantized, the tile already holds the operand
            if (qV) {
                __syncthreads();   // the V tile's raw words are all written
                float x[2][16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const uint32_t r = *reinterpret_cast<const uint32_t*>(&sm.vt[(16 * half + i) * kPitch + d0]);
                    x[0][i] = bf16_lo(r);
                    x[1][i] = bf16_hi(r);
                }
#pragma unroll
                for (int d = 0; d < 2; ++d) qdq16(x[d], fV, pp.g_v, inv_gv, pp.u_v, pp.inv_u_v);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int tok = 16 * half + i;
                    *reinterpret_cast<uint32_t*>(&sm.vt[tok * kPitch + d0]) =
                        kVF16 ? pack_f16(x[0][i], x[1][i]) : pack_bf16_exact(x[0][i], x[1][i]);
                }
            }
        }
        __syncthreads();

        // (wavefronts past the last head only stage and prefetch)
        // ---- S^T = K Q^T: rows 16tt + c16 (tokens), latent and RoPE apart
        f32x4 sl[2], sr[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            sl[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            sr[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (wave_active) {
            // fragments (and LDS-held Q) one k-step ahead of their MFMAs
            auto q_lds = [](int kk) { return kk < kQLdsLatent || kk >= 16; };
            auto q_slot = [](int kk) { return kk < 16 ? kk : kQLdsLatent + kk - 16; };
            auto kt_frag = [&](int kk, int tt) {
                return *reinterpret_cast<const u32x4*>(&sm.kt[(16 * tt + c16) * kPitch + 32 * kk + 8 * gq]);
            };
            u32x4 f0[2], f1[2], qb[2];
            f0[0] = kt_frag(0, 0);
            f1[0] = kt_frag(0, 1);
            qb[0] = sm.qs[w][q_slot(0)][lane];
#pragma unroll
            for (int kk = 0; kk < 18; ++kk) {
                if (kk + 1 < 18) {
                    f0[(kk + 1) & 1] = kt_frag(kk + 1, 0);
                    f1[(kk + 1) & 1] = kt_frag(kk + 1, 1);
                    if (q_lds(kk + 1)) qb[(kk + 1) & 1] = sm.qs[w][q_slot(kk + 1)][lane];
                }
                const u32x4 qv = q_lds(kk) ? qb[kk & 1] : qf[kk - kQLdsLatent];
                const u32x4 a0 = f0[kk & 1], a1 = f1[kk & 1];
                if (kk >= 16) {
                    sr[0] = mfma16x16x32(as_bf16x8(a0), as_bf16x8(qv), sr[0]);
                    sr[1] = mfma16x16x32(as_bf16x8(a1), as_bf16x8(qv), sr[1]);
                } else if (kKF16) {
                    sl[0] = mfma_f16(__builtin_bit_cast(f16x8, a0), __builtin_bit_cast(f16x8, qv), sl[0]);
                    sl[1] = mfma_f16(__builtin_bit_cast(f16x8, a1), __builtin_bit_cast(f16x8, qv), sl[1]);
                } else {
                    sl[0] = mfma16x16x32(as_bf16x8(a0), as_bf16x8(qv), sl[0]);
                    sl[1] = mfma16x16x32(as_bf16x8(a1), as_bf16x8(qv), sl[1]);
                }
                if (kk + 1 < 18) {   // the next k-step's reads ahead of this step's products
                    if (q_lds(kk + 1)) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
                    else __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (kRaw) {   // the next tile's K words land during this tile's softmax and PV
            if (t + 1 < ntiles) load_k_raw(sm.offs[(t + 1) % 3]);
        }
        if (wave_active) {
            // ---- softmax (log2 units): token 16tt + 4gq + i of head c16
            float z[2][4];
            float mx = -INFINITY;
            const uint32_t vq = vmask >> ((lane_now() >> 2) & 12);   // bits from token 4 gq
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    z[tt][i] = ((vq >> (16 * tt + i)) & 1u) ? sc_lat * sl[tt][i] + sc_rope * sr[tt][i] : -INFINITY;
                    mx = fmaxf(mx, z[tt][i]);
                }
            mx = xor32_max(xor16_max(mx));
            const float m_new = fmaxf(m_run, mx);
            const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
            const float m_use = m_new == -INFINITY ? 0.0f : m_new;
            float pv[2][4];
            float psum = 0.0f;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pv[tt][i] = __builtin_amdgcn_exp2f(z[tt][i] - m_use);   // masked: 0
                    psum += pv[tt][i];
                }
            psum = xor32_sum(xor16_sum(psum));
            l_run = alpha * l_run + psum;   // unquantized denominator
            m_run = m_new;
            if (__any(alpha != 1.0f)) {
#pragma unroll
                for (int c = 0; c < 32; ++c) o[c] *= alpha;
            }
            // ---- P (B operand; k-slot j < 4: token 4gq + j, j >= 4: token
            // 16 + 4gq + j - 4).  P block tt (16 keys) of head c16: this lane's 4
            // values and those of lanes c16 + 16g'.
            float ph[2][4], pm[2][4], plo[2][4];
            int sweeps = 1;
            if (qP) {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    if (fP) {
#pragma unroll
                        for (int i = 0; i < 4; i += 2) {
                            const uint32_t c2 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                                fminf(pv[tt][i] * inv_g_p, 448.0f), fminf(pv[tt][i + 1] * inv_g_p, 448.0f), 0, false);
                            const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(c2, false);
                            ph[tt][i] = d[0];
                            ph[tt][i + 1] = d[1];
                        }
                    } else {
                        float a = fmaxf(fmaxf(pv[tt][0], pv[tt][1]), fmaxf(pv[tt][2], pv[tt][3]));
                        a = xor32_max(xor16_max(a));
                        float tq = a * inv_u_p;
                        if (scale_quotient_near_tie(tq)) tq = a / u_p;
                        const uint32_t code = e4m3_encode_nonneg(tq);
                        const float sv = e4m3_decode(code);
                        const float dd = sv * pp.g_p;
                        const float inv = dd == 0.0f ? 0.0f : 1.0f / dd;
#pragma unroll
                        for (int i = 0; i < 4; i += 2) {
                            const f32x2 d = e2m1_pair<0>(e2m1_pack2<0>(0u, pv[tt][i] * inv, pv[tt][i + 1] * inv));
                            ph[tt][i] = d[0] * sv;
                            ph[tt][i + 1] = d[1] * sv;
                        }
                    }
                }
            } else {
                // unquantized: fp16 hi + lo (fp16 V), or three bf16 parts (bf16 V)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float x = pv[tt][i];
                        if (kVF16) {
                            ph[tt][i] = (float)(_Float16)x;
                            pm[tt][i] = (float)(_Float16)(x - ph[tt][i]);
                        } else {
                            ph[tt][i] = bf16_lo(pack_bf16_rne(x, 0.0f));
                            const float r = x - ph[tt][i];
                            pm[tt][i] = bf16_lo(pack_bf16_rne(r, 0.0f));
                            plo[tt][i] = bf16_lo(pack_bf16_rne(r - pm[tt][i], 0.0f));
                        }
                    }
                sweeps = kVF16 ? 2 : 3;
            }
            // ---- O^T += V^T P^T: V^T fragment of column tile c by transposing
            // reads (tokens 4gq + s/4 and 16 + 4gq + s/4 in each 16-lane group)
            const uint16_t* vb1 = sm.vt + (4 * gq + (c16 >> 2)) * kPitch + 4 * (c16 & 3);
            const uint16_t* vb2 = sm.vt + (16 + 4 * gq + (c16 >> 2)) * kPitch + 4 * (c16 & 3);
            auto vt_frag = [&](int c) {
                const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)(const_cast<uint16_t*>(vb1 + 16 * c)));
                const s16x4 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)(const_cast<uint16_t*>(vb2 + 16 * c)));
                const u32x2 y1 = __builtin_bit_cast(u32x2, x1), y2 = __builtin_bit_cast(u32x2, x2);
                return u32x4{y1[0], y1[1], y2[0], y2[1]};
            };
            for (int sw = 0; sw < sweeps; ++sw) {
                float pp8[8];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) pp8[4 * tt + i] = sw == 0 ? ph[tt][i] : (sw == 1 ? pm[tt][i] : plo[tt][i]);
                const u32x4 bp = kVF16 ? u32x4{pack_f16(pp8[0], pp8[1]), pack_f16(pp8[2], pp8[3]),
                                               pack_f16(pp8[4], pp8[5]), pack_f16(pp8[6], pp8[7])}
                                       : pack8_exact<false>(pp8);
                // two column tiles per step, fragments one step ahead of their products
                u32x4 va = vt_frag(0), vb = vt_frag(1);
#pragma unroll
                for (int c = 0; c < 32; c += 2) {
                    u32x4 na = va, nb = vb;
                    if (c + 2 < 32) {
                        na = vt_frag(c + 2);
                        nb = vt_frag(c + 3);
                    }
                    if (kVF16) {
                        o[c] = mfma_f16(__builtin_bit_cast(f16x8, va), __builtin_bit_cast(f16x8, bp), o[c]);
                        o[c + 1] = mfma_f16(__builtin_bit_cast(f16x8, vb), __builtin_bit_cast(f16x8, bp), o[c + 1]);
                    } else {
                        o[c] = mfma16x16x32(as_bf16x8(va), as_bf16x8(bp), o[c]);
                        o[c + 1] = mfma16x16x32(as_bf16x8(vb), as_bf16x8(bp), o[c + 1]);
                    }
                    if (c + 2 < 32) {
                        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    va = na;
                    vb = nb;
                }
            }
        }
        if (tid < kTile) walk_store(t + 2);
        __syncthreads();   // the tiles are restaged next iteration
    }

    // ---- epilogue
    const bool any = l_run > 0.0f;
    const float so = any ? v_mul / l_run : 0.0f;
    const float lse_v = any ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : -INFINITY;
    if (!hok) return;
    float* dst;
    if (ns == 1) {
        dst = p.out + ((int64_t)b * p.H + hq) * kLatent;
        if (gq == 0) p.lse[(int64_t)b * p.H + hq] = lse_v;
    } else {
        const int64_t row = ((int64_t)b * p.max_splits + s) * p.H + hq;
        dst = p.ws_out + row * kLatent;
        if (gq == 0) {
            p.ws_lse[row] = lse_v;
            p.ws_fmt[row] = 0;   // fp32 partial
        }
    }
#pragma unroll
    for (int c = 0; c < 32; ++c) *reinterpret_cast<f32x4*>(dst + 16 * c + 4 * gq) = o[c] * so;
}

template <int kCache, bool kKF16, bool kVF16>
hipError_t launch_qdq_t(const QdqParams& pp, hipStream_t stream) {
    const dim3 grid((unsigned)pp.d.max_splits, (unsigned)pp.d.B, (unsigned)((pp.d.H + kHeadsPerGroup - 1) / kHeadsPerGroup));
    hipLaunchKernelGGL((decode_qdq_kernel<kCache, kKF16, kVF16>), grid, dim3(kWaves * 64), 0, stream, pp);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_qdq(const DecodeArgs& a, unsigned flags, float g_q, float g_k, float g_v, float g_p,
                             hipStream_t stream) {
    // NVFP4 records, more than 16 heads, P quantized: the 128-head decode
    // kernel with P (and Q) quantization (same schedule: each wavefront walks
    // its split's 32-token tiles in order with one running max)
    if (a.record_bytes != 1152 && a.H > 16 && (flags & 4u)) {
        DecodeArgs b = a;
        b.qdq_flags = flags;
        b.g_q = g_q;
        b.g_p = g_p;
        return launch_decode_pq(b, stream);
    }
    QdqParams pp{a, flags, g_q, g_k, g_v, g_p};
    {
        // (the kernel's multipliers: scores ((scale log2 e) q_mul) k_mul with
        // q_mul = g_q when Q is quantized, k_mul = g_k for a quantized raw K;
        // output V multiplier times g_p when P is quantized)
        const bool raw = a.record_bytes == 1152;
        const float q_mul_rope = (flags & 1u) ? g_q : 1.0f;
        const float k_mul_rope = (raw && (flags & 2u)) ? g_k : 1.0f;
        pp.inv_g_k = 1.0f / g_k;
        pp.inv_g_v = 1.0f / g_v;
        pp.inv_g_p = 1.0f / g_p;
        pp.u_k = 6.0f * g_k;
        pp.inv_u_k = 1.0f / pp.u_k;
        pp.u_v = 6.0f * g_v;
        pp.inv_u_v = 1.0f / pp.u_v;
        pp.u_p = 6.0f * g_p;
        pp.inv_u_p = 1.0f / pp.u_p;
        pp.sc_rope = a.softmax_scale * kLog2e * q_mul_rope * k_mul_rope;
        pp.v_mul = (raw ? ((flags & 8u) ? g_v : 1.0f) : a.outer_scale) * ((flags & 4u) ? g_p : 1.0f);
    }
    hipError_t e;
    if (a.record_bytes == 1152) {
        const bool kf = flags & 2u, vf = flags & 8u;
        if (kf && vf) e = launch_qdq_t<2, true, true>(pp, stream);
        else if (kf) e = launch_qdq_t<2, true, false>(pp, stream);
        else if (vf) e = launch_qdq_t<2, false, true>(pp, stream);
        else e = launch_qdq_t<2, false, false>(pp, stream);
    } else if (a.record_bytes == 368) {
        e = launch_qdq_t<1, true, true>(pp, stream);
    } else {
        e = launch_qdq_t<0, true, true>(pp, stream);
    }
    if (e != hipSuccess || a.max_splits <= 1) return e;
    return launch_split_merge(a, stream);
}

}  // namespace mla
