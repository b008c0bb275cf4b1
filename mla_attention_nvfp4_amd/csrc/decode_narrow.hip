// Paged absorbed split-K MLA decode over the NVFP4 latent cache for narrow
// head groups (H <= 16), where the path is bound by HBM: every wavefront
// streams its own tokens, with no workgroup barrier in the token loop.
//
// [MO-MLA], commit 1: split-K absorbed MQA decode over the paged latent with
// grouped query heads and a natural-log LSE for merging; commit 3: V is the
// stored latent itself.  [B12X], walkthrough and sequence diagram: the
// decode kernel stages NVFP4 data, dequantizes it and accumulates, restoring
// the per-layer outer scale on read; review 2: Q is not quantized.
//
// Work item: workgroup (split s, sequence b) of 4 wavefronts; wavefront w
// takes the split's 32-token tiles w, w+4, ... (two 16-token halves whose
// chains interleave).  Per tile, software-pipelined: page-table walk two
// tiles ahead, record loads one tile ahead into registers, then
//   S^T = K Q^T (per half: 16 tokens x 16 heads).  Lane l covers token l%16 of each half and the
//     latent dims 128(l/16) .. +127 (k-step kk: dims 128(l/16) + 8kk .. +7;
//     the k-slot order is a permutation shared by both operands), so each
//     lane dequantizes the 64 code bytes and 8 scales of its own token
//     straight into the MFMA operand: e2m1 x e4m3 is exact in fp16 (at most
//     6 significant bits, magnitudes in [2^-10, 2688]), by the gfx950 FP4
//     conversion and one packed fp16 multiply per two elements.  Q's latent
//     part is held in fp16 after an exact per-head power-of-two scaling
//     (bf16 has 8 significant bits); the RoPE k-steps stay in bf16, since
//     arbitrary bf16 RoPE values need not fit fp16's range.
//   online softmax in base 2 with lazy rescaling; P as fp16 hi + lo
//     (|p - hi - lo| <= 2^-22 |p|);
//   O^T = V^T P^T with v_mfma_f32_16x16x32_f16 (k = the tile's 32 tokens):
//     the dequantized latent goes to this wavefront's own LDS tile
//     (token-major) and V^T is read back by ds_read_b64_tr_b16.
// The four wavefronts then merge their (O, m, l) in LDS; single-split
// sequences are written out, split ones go to the workspace for
// split_merge_kernel.
#include "device_common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kNW = 4;            // wavefronts per workgroup
constexpr int kNT = 32;           // tokens per wavefront tile (two 16-token halves)
constexpr int kVP = 528;          // fp16 per V tile row (1056 B: conflict-free writes and transposed reads)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;
// PV precision: P enters V^T P^T rounded to fp16 (relative error <= 2^-11,
// so the output moves by at most 2^-11 max|V|); a tile whose dequantized
// latent may exceed kSinglePBound in magnitude (outer x 6 x block scale)
// adds a second sweep with the residual p - fp16(p).
constexpr float kSinglePBound = 8.0f;

struct NarrowSmem {
    _Float16 vt[kNW][kNT * kVP];  // 4 x 33,792 B; reused for the output merge
    float m[kNW][16], l[kNW][16];
    uint32_t wide[kNW];           // wavefront w saw a tile above the single-pass bound
};

__device__ __forceinline__ f32x4 mfma_k32_f16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// D = A (16x16) * B (16x16) + C; lane l supplies row / column l % 16 with
// k-slots 4*(l/16) .. +3 and receives D[4*(l/16) + i][l % 16].


// The record bytes one lane needs for its token: 64 code bytes, 8 scale
// bytes, and its RoPE share (32 B bf16 or 16 B e4m3).
struct Staged {
    u32x4 c[4];
    u32x2 sc;
    u32x4 r[2];
};

template <bool kRopeFp8, bool kSparse>
__global__ __launch_bounds__(kNW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_narrow_kernel(DecodeArgs p) {
    constexpr int kRec = kRopeFp8 ? 368 : 432;
    __shared__ NarrowSmem sm;

    int s, b;
    decode_work_item(p.max_splits, p.B, s, b);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c16 = lane & 15, gq = lane >> 4;

    // The sequence length and Q are requested together (the length first,
    // so that it can be waited for alone); the page-table entries of the
    // first tiles are requested before Q is processed.
    const bool hok = c16 < p.H;
    int L = p.seq_lens[b];
    u32x4 qraw[16], qrraw[2];
    {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const uint16_t* qn = p.q_nope + (int64_t)b * p.q_stride_b + (int64_t)(hok ? c16 : 0) * p.q_stride_h + 128 * gq;
        const uint16_t* qp = p.q_rope + (int64_t)b * p.q_stride_b + (int64_t)(hok ? c16 : 0) * p.q_stride_h + 16 * gq;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) qraw[kk] = hok ? *reinterpret_cast<const u32x4*>(qn + 8 * kk) : zero;
#pragma unroll
        for (int kr = 0; kr < 2; ++kr) qrraw[kr] = hok ? *reinterpret_cast<const u32x4*>(qp + 8 * kr) : zero;
    }
    const int Lmax = p.max_pages * p.page_size;
    L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
    const int n_items = kSparse ? p.topk : L;
    const int ns = decode_num_splits(n_items, p.max_splits);
    if (s >= ns) return;
    const int ct = decode_chunk_tiles(n_items, p.max_splits);   // in 64-item units
    const int i0 = 64 * ct * s;
    const int i1 = min(n_items, i0 + 64 * ct);
    const int ntiles = (i1 - i0 + kNT - 1) / kNT;
    const int nmine = ntiles > w ? (ntiles - w + kNW - 1) / kNW : 0;   // tiles w, w+4, ...

    // ---- Q.  Latent (B operand of the fp16 k-steps): lane holds head c16,
    // dims 128gq + 8kk .. +7 for kk = 0..15, scaled by 2^(14 - E) where 2^E
    // <= max |q_nope| of the head < 2^(E+1) (exact; the largest value lands
    // in [2^14, 2^15)).  RoPE (bf16 k-steps kr = 0, 1): dims 16gq + 8kr .. +7.
    f16x8 qf[16];
    bf16x8 qr[2];
    float q_unscale;   // 2^(E - 14)
    auto setup_q = [&]() {
        float amax = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                amax = fmaxf(amax, fmaxf(__builtin_fabsf(bf16_lo(qraw[kk][j])), __builtin_fabsf(bf16_hi(qraw[kk][j]))));
        amax = xor32_max(xor16_max(amax));
        int E = amax > 0.0f ? (int)((f2u(amax) >> 23) & 0xffu) - 127 : 0;
        E = E < -100 ? -100 : E;
        const int sh = 14 - E;
        q_unscale = __builtin_ldexpf(1.0f, E - 14);
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            f16x8 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[2 * j] = (_Float16)__builtin_ldexpf(bf16_lo(qraw[kk][j]), sh);
                v[2 * j + 1] = (_Float16)__builtin_ldexpf(bf16_hi(qraw[kk][j]), sh);
            }
            qf[kk] = v;
        }
#pragma unroll
        for (int kr = 0; kr < 2; ++kr) qr[kr] = as_bf16x8(qrraw[kr]);
    };

    const uint8_t* __restrict__ cache = p.cache;
    const float outer = p.outer_scale;
    const float sc_rope = p.softmax_scale * kLog2e;
    float sc_lat = 0.0f;   // set with Q
    const float wide_scale = kSinglePBound / (6.0f * outer);   // block scales above this need the residual sweep

    // ---- token addressing: tile j of this wavefront covers items
    // i0 + kNT*(w + kNW*j) .. +31; lane l handles item + 16 h2 + c16 of half h2.
    auto item_of = [&](int j, int h2) { return i0 + kNT * (w + kNW * j) + 16 * h2 + c16; };
    // The raw entry (the item itself, or the top-k index, loaded from a
    // clamped address) is taken one iteration before it is validated, so
    // that the index load is not waited for right after it is issued.
    auto raw_of = [&](int j, int h2) -> int {
        const int ic = min(item_of(j, h2), max(n_items - 1, 0));
        return kSparse ? p.indices[(int64_t)b * p.topk + ic] : ic;
    };
    auto position_from = [&](int j, int h2, int raw) -> int {
        const int item = item_of(j, h2);
        return (j < nmine && item < i1 && raw >= 0 && raw < L) ? raw : -1;
    };
    auto position_of = [&](int j, int h2) -> int { return position_from(j, h2, raw_of(j, h2)); };
    auto page_of = [&](int pos) -> int {
        int pi, rem;
        page_divmod(pos < 0 ? 0 : pos, p.page_size, p.page_recip, pi, rem);
        return p.page_table[(int64_t)b * p.max_pages + pi];
    };
    auto page_rem = [&](int pos) -> int {
        int q, r;
        page_divmod(pos < 0 ? 0 : pos, p.page_size, p.page_recip, q, r);
        return r;
    };
    auto offset_of = [&](int pos, int pg) -> int64_t {
        return (pos >= 0 && pg >= 0 && pg < p.num_pages)
                   ? ((int64_t)pg * p.page_size + page_rem(pos)) * kRec : int64_t(-1);
    };
    // masked tokens load record 0 (always present) and are zeroed at dequant
    auto load = [&](Staged& st, int64_t off) {
        const uint8_t* rp = cache + (off < 0 ? 0 : off);
#pragma unroll
        for (int k = 0; k < 4; ++k) st.c[k] = *reinterpret_cast<const u32x4*>(rp + 64 * gq + 16 * k);
        st.sc = *reinterpret_cast<const u32x2*>(rp + 256 + 8 * gq);
        if (kRopeFp8) {
            st.r[0] = *reinterpret_cast<const u32x4*>(rp + 288 + 16 * gq);
            st.r[1] = st.r[0];
        } else {
            st.r[0] = *reinterpret_cast<const u32x4*>(rp + 288 + 32 * gq);
            st.r[1] = *reinterpret_cast<const u32x4*>(rp + 288 + 32 * gq + 16);
        }
    };

    f32x4 o[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;
    bool wide_seen = false;   // some tile of this wavefront exceeded the single-pass bound
    _Float16* vt = sm.vt[w];

    // one tile: halves h2 = 0, 1 (tokens 16 h2 .. +15 of the tile)
    auto compute = [&](const Staged (&st)[2], const int64_t (&off)[2]) {
        const bool valid0 = off[0] >= 0, valid1 = off[1] >= 0;
        // validity of tokens 0..31 (lane c16 of group 0 holds token 16 h2 + c16)
        const uint32_t vm = ((uint32_t)__ballot(valid0 && gq == 0) & 0xffffu) |
                            (((uint32_t)__ballot(valid1 && gq == 0) & 0xffffu) << 16);
        // ---- S^T of each half: RoPE k-steps (bf16), then the latent ones
        // (fp16), the two halves' chains interleaved
        f32x4 s_r[2], s_l[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            s_r[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
            s_l[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kr = 0; kr < 2; ++kr) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                u32x4 a;
                if (kRopeFp8) {
                    const uint32_t x0 = st[h2].r[0][2 * kr], x1 = st[h2].r[0][2 * kr + 1];
                    const u32x2 y0 = e4m3x4_to_bf16(x0), y1 = e4m3x4_to_bf16(x1);
                    a = u32x4{y0[0], y0[1], y1[0], y1[1]};
                } else {
                    a = st[h2].r[kr];
                }
                const u32x4 zero = {0u, 0u, 0u, 0u};
                s_r[h2] = mfma16x16x32(as_bf16x8((h2 ? valid1 : valid0) ? a : zero), qr[kr], s_r[h2]);
            }
        }
        // the lane's 8 block scales per half (e4m3 -> fp32 by the hardware
        // FP8 conversion, exact); a masked token gets scale 0, hence zero K, V
        f32x2 sf[2][4];
        bool big = false;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const bool v = h2 ? valid1 : valid0;
            const uint32_t sw0 = v ? st[h2].sc[0] : 0u, sw1 = v ? st[h2].sc[1] : 0u;
            sf[h2][0] = __builtin_amdgcn_cvt_pk_f32_fp8(sw0, false);
            sf[h2][1] = __builtin_amdgcn_cvt_pk_f32_fp8(sw0, true);
            sf[h2][2] = __builtin_amdgcn_cvt_pk_f32_fp8(sw1, false);
            sf[h2][3] = __builtin_amdgcn_cvt_pk_f32_fp8(sw1, true);
#pragma unroll
            for (int k = 0; k < 4; ++k) big = big || fmaxf(sf[h2][k][0], sf[h2][k][1]) > wide_scale;
        }
        const bool residual = __any(big);   // uniform: the wavefront's tile needs the second sweep
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const uint32_t cw = st[h2].c[kk >> 2][kk & 3];
                const _Float16 sv = (_Float16)sf[h2][kk >> 2][(kk >> 1) & 1];
                const f16x2 ss = {sv, sv};
                const f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0) * ss;
                const f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1) * ss;
                const f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2) * ss;
                const f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3) * ss;
                const f16x8 a = {v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
                s_l[h2] = mfma_k32_f16(a, qf[kk], s_l[h2]);
                // 16-byte chunk j of a tile row is stored at j ^ ((j >> 4) & 1):
                // the 64 lanes of one store then cover every bank once
                *reinterpret_cast<f16x8*>(&vt[(16 * h2 + c16) * kVP + 128 * gq + 8 * (kk ^ (gq & 1))]) = a;
            }
        }
        // ---- online softmax: z[h2][i] is token 16 h2 + 4gq + i of head c16
        float z[2][4];
        float mx = -INFINITY;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                z[h2][i] = ((vm >> (16 * h2 + 4 * gq + i)) & 1u) ? sc_lat * s_l[h2][i] + sc_rope * s_r[h2][i]
                                                                 : -INFINITY;
                mx = fmaxf(mx, z[h2][i]);
            }
        mx = xor32_max(xor16_max(mx));
        const bool move = mx > m_run + kRescaleSlack;
        const float m_new = move ? mx : m_run;
        const bool live = m_new != -INFINITY;
        const float alpha = (move && m_run != -INFINITY) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        float psum = 0.0f;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                z[h2][i] = live ? __builtin_amdgcn_exp2f(z[h2][i] - m_new) : 0.0f;
                psum += z[h2][i];
            }
        psum = xor32_sum(xor16_sum(psum));
        l_run = alpha * l_run + psum;
        m_run = m_new;
        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int c = 0; c < 32; ++c) o[c] *= alpha;
        }
        // P as fp16 hi (+ lo = the residual); B operand of O^T = V^T P^T (k =
        // 32 tokens): slot j < 4 is token 4gq + j, slot j >= 4 is token
        // 16 + 4gq + j - 4
        f16x8 ph, pl;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ph[4 * h2 + i] = (_Float16)z[h2][i];
                pl[4 * h2 + i] = (_Float16)(z[h2][i] - (float)ph[4 * h2 + i]);
            }
        // ---- O^T = V^T P^T on v_mfma_f32_16x16x32_f16: A fragment of dim
        // tile c by two transposing reads (tokens 4gq .. +3 and 16 + 4gq ..
        // +3); in each 16-lane group lane s addresses token row k0 + s/4 and
        // dims 16c + 4(s%4) .. +3, and receives the 4 tokens of dim 16c + s.
        // (chunk 2c + (s%4)/2 sits at 2c + ((s%4)/2 ^ 1) in dim tiles c with bit 3 set)
        const _Float16* vb0 = vt + (4 * gq + (c16 >> 2)) * kVP + 4 * (c16 & 3);
        const _Float16* vb1 = vt + (4 * gq + (c16 >> 2)) * kVP + 8 * (((c16 & 3) >> 1) ^ 1) + 4 * (c16 & 1);
        auto vfrag = [&](int c) {
            const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(
                const_cast<__attribute__((address_space(3))) _Float16*>(
                    (__attribute__((address_space(3))) const _Float16*)(((c >> 3) & 1 ? vb1 : vb0) + 16 * c))));
            const s16x4 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(
                const_cast<__attribute__((address_space(3))) _Float16*>(
                    (__attribute__((address_space(3))) const _Float16*)(((c >> 3) & 1 ? vb1 : vb0) + 16 * kVP + 16 * c))));
            const f16x4 y1 = __builtin_bit_cast(f16x4, x1), y2 = __builtin_bit_cast(f16x4, x2);
            return f16x8{y1[0], y1[1], y1[2], y1[3], y2[0], y2[1], y2[2], y2[3]};
        };
        // fragments in groups of 8 dim tiles, the next group read during
        // this group's products
        auto pv_sweep = [&](const f16x8& pp) {
            f16x8 vf[2][8];
#pragma unroll
            for (int c = 0; c < 8; ++c) vf[0][c] = vfrag(c);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (g + 1 < 4) {
#pragma unroll
                    for (int c = 0; c < 8; ++c) vf[(g + 1) & 1][c] = vfrag(8 * (g + 1) + c);
                }
#pragma unroll
                for (int c = 0; c < 8; ++c) o[8 * g + c] = mfma_k32_f16(vf[g & 1][c], pp, o[8 * g + c]);
            }
        };
        pv_sweep(ph);
        if (residual) pv_sweep(pl);
        wide_seen = wide_seen || residual;
    };

    // ---- token loop: records of tile j+1 in flight, page-table entries of
    // tile j+2 loading, indices of tile j+3 loading (sparse)
    if (nmine > 0) {
        Staged cur[2], nxt[2];
        int64_t offA[2], offB[2];
        int posC[2], rawD[2];
        int p0[2], p1[2], g0[2], g1[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            p0[h2] = position_of(0, h2);
            p1[h2] = position_of(1, h2);
            g0[h2] = page_of(p0[h2]);
            g1[h2] = page_of(p1[h2]);
        }
        setup_q();
        sc_lat = sc_rope * outer * q_unscale;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            offA[h2] = offset_of(p0[h2], g0[h2]);
            offB[h2] = offset_of(p1[h2], g1[h2]);
            posC[h2] = position_of(2, h2);
            rawD[h2] = raw_of(3, h2);
        }
        load(cur[0], offA[0]);
        load(cur[1], offA[1]);
        for (int j = 0; j < nmine; ++j) {
            int pgC[2], posD[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                pgC[h2] = page_of(posC[h2]);              // tile j+2, used at the end
                posD[h2] = position_from(j + 3, h2, rawD[h2]);
                rawD[h2] = raw_of(j + 4, h2);             // tile j+4 (sparse: index load)
            }
            load(nxt[0], offB[0]);                        // tile j+1 (masked reloads past the end)
            load(nxt[1], offB[1]);
            compute(cur, offA);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                cur[h2] = nxt[h2];
                offA[h2] = offB[h2];
                offB[h2] = offset_of(posC[h2], pgC[h2]);
                posC[h2] = posD[h2];
            }
        }
    }

    // ---- merge the four wavefronts: weights 2^(m_w - M) per head
    if (gq == 0) {
        sm.m[w][c16] = m_run;
        sm.l[w][c16] = l_run;
    }
    if (lane == 0) sm.wide[w] = wide_seen ? 1u : 0u;
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kNW; ++v) M = fmaxf(M, sm.m[v][c16]);
    float ltot = 0.0f, aw = 0.0f;
#pragma unroll
    for (int v = 0; v < kNW; ++v) {
        const float mv = sm.m[v][c16];
        const float a = (mv == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mv - M);
        ltot += a * sm.l[v][c16];
        if (v == w) aw = a;
    }
#pragma unroll
    for (int c = 0; c < 32; ++c) o[c] *= aw;
    // sum of the four O's through LDS: each wavefront stores its weighted O
    // over its own V tile (f32x4 per (dim tile, lane)); then wavefront w
    // sums dim tiles 8w .. 8w+7 of all four, as (O0 + O2) + (O1 + O3), and
    // writes them
    {
        f32x4* mine = reinterpret_cast<f32x4*>(&sm.vt[w][0]);
#pragma unroll
        for (int c = 0; c < 32; ++c) mine[c * 64 + lane] = o[c];
    }
    __syncthreads();
    f32x4 r[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int c = 8 * w + k;
        const f32x4 v0 = reinterpret_cast<const f32x4*>(&sm.vt[0][0])[c * 64 + lane];
        const f32x4 v1 = reinterpret_cast<const f32x4*>(&sm.vt[1][0])[c * 64 + lane];
        const f32x4 v2 = reinterpret_cast<const f32x4*>(&sm.vt[2][0])[c * 64 + lane];
        const f32x4 v3 = reinterpret_cast<const f32x4*>(&sm.vt[3][0])[c * 64 + lane];
        r[k] = (v0 + v2) + (v1 + v3);
    }

    const bool any = ltot > 0.0f;
    const float so = any ? outer / ltot : 0.0f;
    const float lse_v = any ? (M + __builtin_amdgcn_logf(ltot)) * kLn2 : -INFINITY;
    if (!hok) return;
    // element i of r[k]: dim 16(8w + k) + 4gq + i of head c16
    float* dst;
    if (ns == 1) {
        dst = p.out + ((int64_t)b * p.H + c16) * kLatent;
        if (w == 0 && gq == 0) p.lse[(int64_t)b * p.H + c16] = lse_v;
    } else {
        // split partial: fp16 in the first half of its row when no tile of
        // the split exceeded the latent bound (|partial| <= 8, absolute
        // rounding <= 2^-8), fp32 otherwise
        const int64_t row = ((int64_t)b * p.max_splits + s) * p.H + c16;
        const bool wide = (sm.wide[0] | sm.wide[1] | sm.wide[2] | sm.wide[3]) != 0u;
        dst = p.ws_out + row * kLatent;
        if (w == 0 && gq == 0) {
            p.ws_lse[row] = lse_v;
            p.ws_fmt[row] = wide ? 0 : 1;
        }
        if (!wide) {
            _Float16* dh = reinterpret_cast<_Float16*>(dst);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const f32x4 v = r[k] * so;
                *reinterpret_cast<f16x4*>(dh + 16 * (8 * w + k) + 4 * gq) =
                    f16x4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
            }
            return;
        }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) *reinterpret_cast<f32x4*>(dst + 16 * (8 * w + k) + 4 * gq) = r[k] * so;
}

template <bool kRopeFp8, bool kSparse>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((decode_narrow_kernel<kRopeFp8, kSparse>), dim3((unsigned)a.max_splits, (unsigned)a.B),
                       dim3(kNW * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_narrow(const DecodeArgs& a, hipStream_t stream) {
    const bool fp8 = a.record_bytes == 368;
    if (a.indices) return fp8 ? launch_t<true, true>(a, stream) : launch_t<false, true>(a, stream);
    return fp8 ? launch_t<true, false>(a, stream) : launch_t<false, false>(a, stream);
}

}  // namespace mla
