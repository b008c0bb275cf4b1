// Paged absorbed split-K MLA decode over the NVFP4 latent cache (gfx950),
// dense and top-k sparse from one template, plus the LSE merge kernel.
//
// [MO-MLA], commit 1: split-K absorbed MQA decode over the paged latent with
// grouped query heads and a natural-log LSE for merging; commit 3: V is the
// stored latent itself.  [B12X], walkthrough and sequence diagram: the
// decode kernel stages NVFP4 data, dequantizes it and accumulates, restoring
// the per-layer outer scale on read; review 2: Q is staged as bf16 with no
// Q quantization.
//
// Work item: workgroup (split s, sequence b, head group hg) of NW (= 8)
// wavefronts, each owning 16 query heads.  The split's tokens are walked in
// tiles of 32, software-pipelined:
//   offsets   record byte offsets (page-table walk) of tile t+3 into a ring
//             of 4 LDS slots (the position / index load one iteration
//             earlier than the page-table load, so no load is waited for
//             right after it is issued);
//   staging   each wavefront loads its own 32/NW records of tile t+2 into
//             registers (coalesced runs per record; no cross-wave traffic);
//   dequant   each wavefront dequantizes its own records of tile t+1 into
//             the free token-major tile: latent as fp16 (e2m1 code x e4m3
//             scale is exact in fp16; the outer scale is not folded), RoPE
//             as bf16 in columns 512..575;
//   compute   tile t: S^T = K Q^T on v_mfma_f32_16x16x32 (A = tile rows,
//             B = the wavefront's Q; latent k-steps in fp16 with Q scaled
//             by a power of two per head, then the accumulator scaled by
//             outer * 2^(E-14), then the RoPE k-steps in bf16); online
//             softmax in base 2 with lazy rescaling; P rounded to fp16 (B
//             operand) for O^T = V^T P^T, whose A operand is read from the
//             same token-major tile with the transposing LDS load
//             ds_read_b64_tr_b16 (V is the latent); a tile whose latent may
//             exceed the single-pass bound adds a sweep with the residual
//             p - fp16(p).
// The epilogue writes out = outer * O / l and lse = m + ln l (natural log)
// to the output when the sequence has one split; otherwise it writes the
// partial to the workspace, and split_merge_kernel (launched after the
// decode kernel) merges each sequence's partials in split order.
#include "device_common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int kTile = 32;            // tokens per tile
constexpr int kKsPitch = kQK + 16;   // bf16 elements per tile row (592: 1184 B, conflict-free)
constexpr int kRing = 4;             // offset ring slots
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;
// PV precision.  P enters V^T P^T rounded to fp16 (relative error <= 2^-11),
// so the output moves by at most 2^-11 max|V| from that rounding; a tile
// whose dequantized latent may exceed kSinglePBound in magnitude (outer x 6 x
// block scale) adds a second product with the residual p - fp16(p), which
// makes P exact to about 2^-22 relative.  With the bound at 8 the single-pass
// error stays below 4e-3 absolute.
constexpr float kSinglePBound = 8.0f;

template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x32_f16, same lane layout as the bf16 form
__device__ __forceinline__ f32x4 mfma_k32_f16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Q k-steps kept in LDS (B-operand layout, 16 B per lane) instead of
// registers: the RoPE part and the first kQLdsLatent latent k-steps.
constexpr int kQLdsLatent = 6;
constexpr int kQLds = kQLdsLatent + 2;

template <int NW>
struct DecodeSmem {
    uint16_t ks[2][kTile * kKsPitch];     // 2 x 37888 B
    u32x4 qs[NW][kQLds][64];              // NW x 8 KB
    int64_t offs[kRing][kTile];           // record byte offset (masked tokens: 0, see valid)
    uint32_t valid[kRing];                // bit i: token i of the tile is unmasked
    alignas(16) uint32_t wide[kRing][NW];  // wavefront w's records of the tile exceed the single-pass bound
};




// kPQ: 0 plain decode; 1 P quantized as NVFP4 (16-key blocks), 2 as
// per-tensor FP8 (the quantized-operand decode on NVFP4 records: the running
// max is then exact, refreshed per tile, and P is quantized against it; the
// quantized values are exact in the fp16 B operand, so one PV sweep).  Q may
// be quantized at set-up (p.qdq_flags bit 1), its exact values kept.
template <int NW, bool kRopeFp8, bool kSparse, int kPQ>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void decode_kernel(DecodeArgs p) {
    constexpr int kRec = kRopeFp8 ? 368 : 432;
    constexpr int kRpw = kTile / NW;                         // records per wavefront
    static_assert(NW == 8, "the per-tile flags are read as two 4-word vectors");
    __shared__ DecodeSmem<NW> sm;

    int s, u;
    decode_work_item(p.max_splits, p.B * (int)gridDim.z, s, u);
    const int b = u % p.B, hg = u / p.B;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // (wavefront-uniform)
    const int gq = lane >> 4, c16 = lane & 15;

    const int h_base = hg * (16 * NW) + 16 * w;
    const bool wave_active = h_base < p.H;
    const int hq = h_base + c16;

    // The sequence length and this wavefront's Q rows are requested
    // together (the length first, so that it can be waited for alone); the
    // page-table entries of the first tiles are requested before Q is
    // processed.
    int L = p.seq_lens[b];
    const bool qok = hq < p.H;
    const int64_t qoff = (int64_t)b * p.q_stride_b + (int64_t)(qok ? hq : 0) * p.q_stride_h + 8 * gq;
    u32x4 qraw[16], qrope[2];
    {
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) qraw[kk] = qok ? *reinterpret_cast<const u32x4*>(p.q_nope + qoff + 32 * kk) : zero;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) qrope[kk] = qok ? *reinterpret_cast<const u32x4*>(p.q_rope + qoff + 32 * kk) : zero;
    }
    const int Lmax = p.max_pages * p.page_size;
    L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
    const int n_items = kSparse ? p.topk : L;
    const int ns = decode_num_splits(n_items, p.max_splits);
    if (s >= ns) return;
    const int ct = decode_chunk_tiles(n_items, p.max_splits);  // in 64-token tiles
    const int T0 = 2 * s * ct;
    const int T1 = min((n_items + kTile - 1) / kTile, T0 + 2 * ct);

    // Q as the B operand of S^T = K Q^T: k-step kk covers d = 32kk..32kk+31
    // (kk 16, 17: RoPE).  Latent k-steps are fp16, scaled by 2^(14 - E)
    // where 2^E <= max |q_nope| of the head < 2^(E+1) (bf16 -> fp16 exact
    // down to 2^-24 of the head's largest value); RoPE k-steps stay bf16.
    // Latent k-steps kQLdsLatent..15 stay in registers (qf[kk -
    // kQLdsLatent]); the others go to this wavefront's LDS slots (slot kk
    // for kk < kQLdsLatent, kQLdsLatent + kk - 16 for RoPE).
    f16x8 qf[16 - kQLdsLatent];
    float q_unscale;   // 2^(E - 14)
    float q_mul = 1.0f;   // Q quantized: its tensor-wide multiplier (applied to the whole score)
    auto setup_q_quantized = [&]() {
        // blocks of 16 features: block 2kk + gq/2 of k-step kk is this lane's 8
        // values and those of lane ^ 16; the exact values s*v (or e4m3 values)
        // are kept, fp16 for the latent (no scaling needed), bf16 for RoPE
        const bool fp8 = p.qdq_flags & 16u;
        const float inv_g = 1.0f / p.g_q;
        auto qdq8 = [&](u32x4 r, float* x) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[2 * j] = bf16_lo(r[j]);
                x[2 * j + 1] = bf16_hi(r[j]);
            }
            if (fp8) {
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(e4m3_encode2_hw(x[i] * inv_g, x[i + 1] * inv_g), false);
                    x[i] = d[0];
                    x[i + 1] = d[1];
                }
            } else {
                float a = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) a = fmaxf(a, __builtin_fabsf(x[i]));
                a = xor16_max(a);
                const Nvfp4Scale sc = nvfp4_block_scale(a, p.g_q);
                const float sv = e4m3_decode(sc.code);
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    const f32x2 d = e2m1_pair<0>(e2m1_pack2<0>(0u, x[i] * sc.inv, x[i + 1] * sc.inv));
                    x[i] = d[0] * sv;
                    x[i + 1] = d[1] * sv;
                }
            }
        };
        q_unscale = 1.0f;
        q_mul = p.g_q;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float x[8];
            qdq8(qraw[kk], x);
            f16x8 v;
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = (_Float16)x[i];
            if (kk < kQLdsLatent) sm.qs[w][kk][lane] = __builtin_bit_cast(u32x4, v);
            else qf[kk - kQLdsLatent] = v;
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            float x[8];
            qdq8(qrope[kk], x);
            sm.qs[w][kQLdsLatent + kk][lane] =
                u32x4{pack_bf16_exact(x[0], x[1]), pack_bf16_exact(x[2], x[3]), pack_bf16_exact(x[4], x[5]),
                      pack_bf16_exact(x[6], x[7])};
        }
    };
    auto setup_q = [&]() {
        if (kPQ != 0 && (p.qdq_flags & 1u)) {
            setup_q_quantized();
            return;
        }
        float amax = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                amax = fmaxf(amax, fmaxf(__builtin_fabsf(bf16_lo(qraw[kk][j])), __builtin_fabsf(bf16_hi(qraw[kk][j]))));
        amax = xor32_max(xor16_max(amax));   // over the head's four lanes c16 + 16gq
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
            if (kk < kQLdsLatent) sm.qs[w][kk][lane] = __builtin_bit_cast(u32x4, v);
            else qf[kk - kQLdsLatent] = v;
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) sm.qs[w][kQLdsLatent + kk][lane] = qrope[kk];
    };

    const uint8_t* __restrict__ cache = p.cache;
    const float outer = p.outer_scale;
    // P quantized: u = fp32(6 g_p), 1/u, 1/g_p
    const float p_u = 6.0f * p.g_p, p_inv_u = kPQ != 0 ? 1.0f / p_u : 0.0f, p_inv_g = kPQ != 0 ? 1.0f / p.g_p : 0.0f;
    float lat_scale = 0.0f;                               // latent partial sum -> outer * q.k (set with Q)
    float score_scale = p.softmax_scale * kLog2e;         // log2 units (times Q's multiplier, set with Q)
    const float wide_scale = kSinglePBound / (6.0f * outer);   // block scales above this need the residual pass

    // ---- offsets.  Loads are issued by every lane of wavefront 0 from
    // clamped (always valid) addresses and masked afterwards, so the
    // control flow stays uniform and the compiler's load counters exact.
    // The raw entry (the item itself, or the top-k index, loaded from a
    // clamped address) is taken one iteration before it is validated, so
    // that the index load is not waited for right after it is issued.
    auto raw_of = [&](int t) -> int {
        const int item = t * kTile + (lane & (kTile - 1));
        const int ic = min(item, max(n_items - 1, 0));
        return kSparse ? p.indices[(int64_t)b * p.topk + ic] : ic;
    };
    auto position_from = [&](int t, int raw) -> int {
        const int item = t * kTile + (lane & (kTile - 1));
        return (t < T1 && item < n_items && raw >= 0 && raw < L) ? raw : -1;   // (tiles past the split: masked)
    };
    auto position_of = [&](int t) -> int { return position_from(t, raw_of(t)); };
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
    auto store_offs = [&](int slot, int64_t off) {
        const uint64_t vm = __ballot(lane < kTile && off >= 0);
        if (lane < kTile) sm.offs[slot][lane] = off < 0 ? 0 : off;   // masked: record 0, zeroed later
        if (lane == 0) sm.valid[slot] = (uint32_t)vm;
    };

    // ---- staging: this wavefront's records kRpw*w .. +kRpw-1 of a tile in
    // registers.  Lane l holds code word l (elements 8l..8l+7) and the
    // matching scale byte of each record, plus one 16-byte RoPE unit
    // (record l/8, unit l%8); every load is a contiguous run per record.
    // Masked tokens load record 0 (always present) and are zeroed.
    uint32_t rc[kRpw], rs[kRpw];
    u32x4 rr;
    // (the loaded words are used as they are; masking happens in dequant,
    // one iteration later, so that no load is waited for here)
    auto load_raw = [&](int slot) {
#pragma unroll
        for (int r = 0; r < kRpw; ++r) {
            const uint8_t* rp = cache + sm.offs[slot][kRpw * w + r];
            rc[r] = *reinterpret_cast<const uint32_t*>(rp + 4 * lane);
            rs[r] = rp[256 + (lane >> 1)];
        }
        const int r = (lane >> 3) % kRpw, u = lane & 7;
        const uint8_t* rp = cache + sm.offs[slot][kRpw * w + r];
        if (kRopeFp8) {
            const u32x2 v2 = *reinterpret_cast<const u32x2*>(rp + 288 + 8 * u);
            rr = u32x4{v2[0], v2[1], 0u, 0u};
        } else {
            rr = *reinterpret_cast<const u32x4*>(rp + 288 + 16 * u);
        }
    };

    // ---- dequant of the staged records into tile rows kRpw*w + r:
    // lane = 16-byte column chunk (8 latent elements)
    auto dequant = [&](int kbuf, int slot) {
        uint16_t* ks = sm.ks[kbuf];
        const uint32_t vmask = __builtin_amdgcn_readfirstlane(sm.valid[slot]);   // (one word)
        bool big = false;
#pragma unroll
        for (int r = 0; r < kRpw; ++r) {
            const int tok = kRpw * w + r;
            const bool valid = (vmask >> tok) & 1u;
            // masked: scale 0 (the code word of record 0 is finite)
            const float scf = e4m3_hw<0>(valid ? rs[r] : 0u);
            big = big || scf > wide_scale;
            const _Float16 sc = (_Float16)scf;
            const f16x2 ss = {sc, sc};
            const uint32_t c = rc[r];
            const f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 0) * ss;
            const f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 1) * ss;
            const f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 2) * ss;
            const f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 3) * ss;
            const f16x8 wv = {v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
            *reinterpret_cast<f16x8*>(&ks[tok * kKsPitch + 8 * lane]) = wv;
        }
        const bool wbig = __any(big);
        if (lane == 0) sm.wide[slot][w] = wbig ? 1u : 0u;
        // RoPE: kRpw tokens x 8 units of 8 elements
        if (lane < 8 * kRpw) {
            const int tok = kRpw * w + (lane >> 3), u = lane & 7;
            const bool valid = (vmask >> tok) & 1u;
            u32x4 wv;
            if (kRopeFp8) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const u32x2 y = e4m3x4_to_bf16(rr[j]);
                    wv[2 * j] = y[0];
                    wv[2 * j + 1] = y[1];
                }
            } else {
                wv = rr;
            }
            const u32x4 zero = {0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(&ks[tok * kKsPitch + kLatent + 8 * u]) = valid ? wv : zero;
        }
    };

    f32x4 o[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;
    bool wide_seen = false;   // some tile of this split exceeded the single-pass bound

    auto compute = [&](int kbuf, int slot) {
        const uint16_t* ks = sm.ks[kbuf];
        // S^T accumulators, one per 16-token half of the tile (consecutive
        // MFMAs alternate between them): the latent k-steps (fp16) go first,
        // the accumulators are then multiplied by outer * 2^(E - 14), and
        // the RoPE k-steps (bf16) follow.
        f32x4 sa[2];
        sa[0] = sa[1] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto ks_frag = [&](int kk, int tt) {
            return *reinterpret_cast<const u32x4*>(&ks[(16 * tt + c16) * kKsPitch + 32 * kk + 8 * gq]);
        };
        auto q_lds = [](int kk) { return kk < kQLdsLatent || kk >= 16; };
        auto q_slot = [](int kk) { return kk < kQLdsLatent ? kk : kQLdsLatent + kk - 16; };
        // fragments (and LDS-held Q) one k-step ahead of their MFMAs
        u32x4 f0[2], f1[2], qb[2];
        f0[0] = ks_frag(0, 0);
        f1[0] = ks_frag(0, 1);
        qb[0] = sm.qs[w][q_slot(0)][lane];
#pragma unroll
        for (int kk = 0; kk < 18; ++kk) {
            if (kk + 1 < 18) {
                f0[(kk + 1) & 1] = ks_frag(kk + 1, 0);
                f1[(kk + 1) & 1] = ks_frag(kk + 1, 1);
                if (q_lds(kk + 1)) qb[(kk + 1) & 1] = sm.qs[w][q_slot(kk + 1)][lane];
            }
            if (kk < 16) {
                const f16x8 qv = q_lds(kk) ? __builtin_bit_cast(f16x8, qb[kk & 1]) : qf[kk - kQLdsLatent];
                sa[0] = mfma_k32_f16(__builtin_bit_cast(f16x8, f0[kk & 1]), qv, sa[0]);
                sa[1] = mfma_k32_f16(__builtin_bit_cast(f16x8, f1[kk & 1]), qv, sa[1]);
            } else {
                if (kk == 16) {
                    sa[0] *= lat_scale;
                    sa[1] *= lat_scale;
                }
                const bf16x8 qv = as_bf16x8(qb[kk & 1]);
                sa[0] = mfma16x16x32(as_bf16x8(f0[kk & 1]), qv, sa[0]);
                sa[1] = mfma16x16x32(as_bf16x8(f1[kk & 1]), qv, sa[1]);
            }
            // the next k-step's LDS reads are issued ahead of this step's
            // two products
            if (kk + 1 < 18) {
                if (q_lds(kk + 1)) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
                else __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // scores (log2 units) of tokens 16tt + 4gq + i for head c16
        float z[2][4];
        float mx = -INFINITY;
        const uint32_t vmask = __builtin_amdgcn_readfirstlane(sm.valid[slot]);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) z[tt][i] = score_scale * sa[tt][i];
        if (vmask != 0xffffffffu) {   // (uniform) a tile with masked tokens
            const uint32_t vq = vmask >> ((lane_now() >> 2) & 12);   // bits from token 4 gq
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!((vq >> (16 * tt + i)) & 1u)) z[tt][i] = -INFINITY;
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, z[tt][i]);
        mx = xor32_max(xor16_max(mx));
        // Lazy rescaling: the reference max moves only when a score exceeds
        // it by more than kRescaleSlack (log2 units), so p <= 2^8 and O is
        // rescaled rarely.  Same softmax; only the rounding differs.  With P
        // quantized the max is exact (P is quantized against it).
        const bool move = kPQ != 0 ? mx > m_run : mx > m_run + kRescaleSlack;
        const float m_new = move ? mx : m_run;
        const bool live = m_new != -INFINITY;
        const float alpha = (move && m_run != -INFINITY) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        float pv[2][4];
        float psum = 0.0f;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pv[tt][i] = live ? __builtin_amdgcn_exp2f(z[tt][i] - m_new) : 0.0f;
                psum += pv[tt][i];
            }
        psum = xor32_sum(xor16_sum(psum));
        l_run = alpha * l_run + psum;
        m_run = m_new;
        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int c = 0; c < 32; ++c) o[c] *= alpha;
        }
        // P as fp16 (B operand): k-slot j < 4 is token 4gq + j, j >= 4 is
        // token 16 + 4gq + j - 4 (the same slots as the V^T fragment below);
        // the residual p - fp16(p) is formed only for a tile that needs it.
        f16x8 ph;
        if constexpr (kPQ == 0) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) ph[4 * tt + i] = (_Float16)pv[tt][i];
        } else {
            // P block tt (16 keys) of head c16: this lane's 4 values and those
            // of lanes c16 + 16g'; the quantized values are exact in fp16
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                if constexpr (kPQ == 2) {
#pragma unroll
                    for (int i = 0; i < 4; i += 2) {
                        const uint32_t c2 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                            fminf(pv[tt][i] * p_inv_g, 448.0f), fminf(pv[tt][i + 1] * p_inv_g, 448.0f), 0, false);
                        const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(c2, false);
                        ph[4 * tt + i] = (_Float16)d[0];
                        ph[4 * tt + i + 1] = (_Float16)d[1];
                    }
                } else {
                    float a = fmaxf(fmaxf(pv[tt][0], pv[tt][1]), fmaxf(pv[tt][2], pv[tt][3]));
                    a = xor32_max(xor16_max(a));
                    float tq = a * p_inv_u;
                    const bool near = scale_quotient_near_tie(tq);
                    if (__any(near)) {   // (the exact division only when a lane needs it)
                        __asm__ volatile("");
                        const float q = a / p_u;
                        tq = near ? q : tq;
                    }
                    const uint32_t code = e4m3_encode_nonneg(tq);
                    const float sv = e4m3_decode(code);
                    const float dd = sv * p.g_p;
                    const float inv = dd == 0.0f ? 0.0f : 1.0f / dd;
#pragma unroll
                    for (int i = 0; i < 4; i += 2) {
                        const f32x2 d = e2m1_pair<0>(e2m1_pack2<0>(0u, pv[tt][i] * inv, pv[tt][i + 1] * inv));
                        ph[4 * tt + i] = (_Float16)(d[0] * sv);
                        ph[4 * tt + i + 1] = (_Float16)(d[1] * sv);
                    }
                }
            }
        }
        // V^T fragment of column tile c by transposing reads: within each
        // 16-lane group, lane s addresses token 4gq + s/4 (+16 for the
        // second half) and columns 16c + 4(s%4) .. +3; lane i receives the 4
        // tokens of column 16c + i.
        const lds_s16x4* vb1 = reinterpret_cast<const lds_s16x4*>(
            (__attribute__((address_space(3))) const uint16_t*)(ks + (4 * gq + (c16 >> 2)) * kKsPitch + 4 * (c16 & 3)));
        const lds_s16x4* vb2 = reinterpret_cast<const lds_s16x4*>(
            (__attribute__((address_space(3))) const uint16_t*)(ks + (16 + 4 * gq + (c16 >> 2)) * kKsPitch + 4 * (c16 & 3)));
        auto vt_frag = [&](int c) {
            const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_s16x4*>(vb1 + 4 * c));
            const s16x4 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_s16x4*>(vb2 + 4 * c));
            const u32x2 y1 = __builtin_bit_cast(u32x2, x1), y2 = __builtin_bit_cast(u32x2, x2);
            return __builtin_bit_cast(f16x8, u32x4{y1[0], y1[1], y2[0], y2[1]});
        };
        // two column tiles per step, fragments one step ahead of their
        // products; the residual pass (rare) is a second sweep
        auto pv_sweep = [&](const f16x8& pp) {
            f16x8 va = vt_frag(0), vb = vt_frag(1);
#pragma unroll
            for (int c = 0; c < 32; c += 2) {
                f16x8 na = va, nb = vb;
                if (c + 2 < 32) {
                    na = vt_frag(c + 2);
                    nb = vt_frag(c + 3);
                }
                o[c] = mfma_k32_f16(va, pp, o[c]);
                o[c + 1] = mfma_k32_f16(vb, pp, o[c + 1]);
                if (c + 2 < 32) {   // the next fragments' reads ahead of these products
                    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                va = na;
                vb = nb;
            }
        };
        pv_sweep(ph);
        const u32x4 wa = *reinterpret_cast<const u32x4*>(&sm.wide[slot][0]);
        const u32x4 wb = *reinterpret_cast<const u32x4*>(&sm.wide[slot][4]);
        const u32x4 wo = wa | wb;
        // (the flags are the same in every lane: a uniform branch)
        const bool wide = __builtin_amdgcn_readfirstlane(wo[0] | wo[1] | wo[2] | wo[3]) != 0u;
        wide_seen = wide_seen || wide;
        if (kPQ == 0 && wide) {
            f16x8 pl;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) pl[4 * tt + i] = (_Float16)(pv[tt][i] - (float)ph[4 * tt + i]);
            pv_sweep(pl);
        }
    };

    if (T0 < T1) {
        {
            // page-table entries of tiles T0..T0+2 requested by every
            // wavefront (uniform control flow), Q processed meanwhile
            int pos0[3], pg0[3];
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                pos0[k] = position_of(T0 + k);
                pg0[k] = page_of(pos0[k]);
            }
            setup_q();
            lat_scale = outer * q_unscale;
            score_scale *= q_mul;
            if (w == 0) {
#pragma unroll
                for (int k = 0; k < 3; ++k) store_offs(k, offset_of(pos0[k], pg0[k]));
            }
        }
        __syncthreads();
        load_raw(0);
        dequant(0, 0);
        int raw_next = raw_of(T0 + 3);   // (before the records, as in the loop)
        load_raw(1);
        __syncthreads();
        for (int t = T0; t < T1; ++t) {
            const int i = t - T0;
            // tile t+3 in two stages: its page-table entry is requested now
            // and its offsets stored at the end.  Every wavefront issues the
            // same loads every iteration (tiles past the split are masked and
            // read record 0), so the compiler's load counters stay exact and
            // the wait for the page-table entry does not also wait for the
            // records of tile t+2; wavefront 0 stores.
            const int pos_cur = position_from(t + 3, raw_next);
            const int pg_cur = page_of(pos_cur);
            raw_next = raw_of(t + 4);
            // Dequant first, so that the records of tile t+2 are issued at
            // the start of the iteration and have the whole compute phase of
            // tile t (and the barrier) to land.  (Running the two halves of
            // the workgroup in opposite phase order measured slower: the
            // late-issued loads of one half then held the barrier.)
            dequant((i + 1) & 1, (i + 1) & 3);
            load_raw((i + 2) & 3);   // lands during tile t
            if (wave_active) compute(i & 1, i & 3);
            if (w == 0) store_offs((i + 3) & 3, offset_of(pos_cur, pg_cur));
            lds_barrier();
        }
    }

    const bool any = l_run > 0.0f;
    const float so = any ? (kPQ != 0 ? outer * p.g_p : outer) / l_run : 0.0f;
    const float lse_v = any ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : -INFINITY;
    const bool has_head = wave_active && hq < p.H;
    if (ns == 1) {
        if (!has_head) return;
        float* dst = p.out + ((int64_t)b * p.H + hq) * kLatent;
        if (gq == 0) p.lse[(int64_t)b * p.H + hq] = lse_v;
#pragma unroll
        for (int c = 0; c < 32; ++c) *reinterpret_cast<f32x4*>(dst + 16 * c + 4 * gq) = o[c] * so;
        return;
    }

    // Split: write the partial; split_merge_kernel combines them.  When no
    // tile of the split exceeded the latent bound (|V| <= 8), the partial
    // (a convex combination of V rows) is within 8 in magnitude and is
    // stored as fp16 (absolute rounding <= 2^-8) in the first half of its row.
    if (!has_head) return;
    const int64_t row = ((int64_t)b * p.max_splits + s) * p.H + hq;
    float* dst = p.ws_out + row * kLatent;
    if (gq == 0) {
        p.ws_lse[row] = lse_v;
        p.ws_fmt[row] = wide_seen ? 0 : 1;
    }
    if (!wide_seen) {
        _Float16* dh = reinterpret_cast<_Float16*>(dst);
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            const f32x4 v = o[c] * so;
            *reinterpret_cast<f16x4*>(dh + 16 * c + 4 * gq) =
                f16x4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
        }
    } else {
#pragma unroll
        for (int c = 0; c < 32; ++c) *reinterpret_cast<f32x4*>(dst + 16 * c + 4 * gq) = o[c] * so;
    }
}

// Merge of the split partials of a decode launch, one wavefront per (b, h)
// (same rule as lse_merge_kernel, splits in order); sequences with a single
// split were written directly by the decode kernel.  Up to 64 splits, lane s
// fetches split s's LSE and format byte together with the sequence length,
// and the fp16 partial rows of the first four splits are loaded in the same
// round (every row exists, and fp16 is the usual format); rows past the
// sequence's split count hold stale values and are masked once the count is
// known.  A split stored as fp32 is re-read, and further splits are read
// four at a time.
__device__ __forceinline__ float wave_max64(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v = wave_xor_max(v, m);
    return v;
}
__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v = wave_xor_sum(v, m);
    return v;
}

template <bool kSparse>
__global__ __launch_bounds__(256) void split_merge_kernel(DecodeArgs p) {
    // Workgroup: sequence b, heads 4hq..4hq+3, on a (HQ, B) grid dispatched
    // in linear order.  When B is a multiple of 8, sequence b's workgroups
    // are placed on XCD b % 8, where the decode kernels ran all of its
    // splits, so the partials are read from the L2 they were written to (a
    // bijection; otherwise the identity).
    const int HQ = (p.H + 3) / 4, wg = (int)(blockIdx.x + gridDim.x * blockIdx.y);
    int b, hq;
    if ((p.B & 7) == 0) {
        const int k = wg >> 3;
        b = (wg & 7) + 8 * (k / HQ);
        hq = k % HQ;
    } else {
        b = wg / HQ;
        hq = wg % HQ;
    }
    const int h = 4 * hq + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (h >= p.H) return;
    const int64_t row0 = (int64_t)b * p.max_splits * p.H + h;   // split s at row0 + s*H
    float* dst = p.out + ((int64_t)b * p.H + h) * kLatent + 8 * lane;
    const int64_t rl = row0 + (int64_t)(lane < p.max_splits ? lane : 0) * p.H;
    const float lv = p.ws_lse[rl];
    const uint32_t fv = p.ws_fmt[rl];
    f16x8 spec[4];   // fp16 rows of splits 0..3, loaded before the split count is known
#pragma unroll
    for (int j = 0; j < 4; ++j)
        spec[j] = *reinterpret_cast<const f16x8*>(
            reinterpret_cast<const _Float16*>(p.ws_out + (row0 + (int64_t)(j < p.max_splits ? j : 0) * p.H) * kLatent) + 8 * lane);
    int L = p.seq_lens[b];
    const int Lmax = p.max_pages * p.page_size;
    L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
    const int ns = decode_num_splits(kSparse ? p.topk : L, p.max_splits);
    if (ns <= 1) return;
    auto load_row = [&](int64_t row, bool f16, f32x4& x0, f32x4& x1) {
        if (f16) {   // fp16 partial in the row's first half
            const f16x8 v = *reinterpret_cast<const f16x8*>(reinterpret_cast<const _Float16*>(p.ws_out + row * kLatent) + 8 * lane);
            x0 = f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
            x1 = f32x4{(float)v[4], (float)v[5], (float)v[6], (float)v[7]};
        } else {
            const float* src = p.ws_out + row * kLatent + 8 * lane;
            x0 = *reinterpret_cast<const f32x4*>(src);
            x1 = *reinterpret_cast<const f32x4*>(src + 4);
        }
    };
    float M, wsum;
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    if (ns <= 64) {
        const float l = lane < ns ? lv : -INFINITY;
        M = wave_max64(l);
        const float wl = (l == -INFINITY || M == -INFINITY) ? 0.0f : expf(l - M);
        wsum = wave_sum64(wl);
        for (int s0 = 0; s0 < ns; s0 += 4) {
            f32x4 x0[4], x1[4];
            float wg[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool in = s0 + j < ns;
                const int sj = in ? s0 + j : s0;   // (uniform)
                wg[j] = __int_as_float(in ? __builtin_amdgcn_readlane(__float_as_int(wl), sj) : 0);
                const bool f16 = __builtin_amdgcn_readlane(fv, sj) != 0u;
                if (s0 == 0 && f16 && in) {
                    const f16x8 v = spec[j];
                    x0[j] = f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
                    x1[j] = f32x4{(float)v[4], (float)v[5], (float)v[6], (float)v[7]};
                } else {
                    load_row(row0 + (int64_t)sj * p.H, f16, x0[j], x1[j]);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (wg[j] != 0.0f) {   // (uniform) splits past the count and those without tokens add nothing
                    a0 += wg[j] * x0[j];
                    a1 += wg[j] * x1[j];
                }
            }
        }
    } else {
        M = -INFINITY;
        for (int s = 0; s < ns; ++s) M = fmaxf(M, p.ws_lse[row0 + (int64_t)s * p.H]);
        wsum = 0.0f;
        for (int s = 0; s < ns; ++s) {
            const int64_t row = row0 + (int64_t)s * p.H;
            const float l = p.ws_lse[row];
            if (l == -INFINITY) continue;
            f32x4 x0, x1;
            load_row(row, p.ws_fmt[row] != 0, x0, x1);
            const float wgt = expf(l - M);
            wsum += wgt;
            a0 += wgt * x0;
            a1 += wgt * x1;
        }
    }
    if (M == -INFINITY) {
        *reinterpret_cast<f32x4*>(dst) = f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
        if (lane == 0) p.lse[(int64_t)b * p.H + h] = -INFINITY;
        return;
    }
    const float inv = 1.0f / wsum;
    *reinterpret_cast<f32x4*>(dst) = a0 * inv;
    *reinterpret_cast<f32x4*>(dst + 4) = a1 * inv;
    if (lane == 0) p.lse[(int64_t)b * p.H + h] = M + logf(wsum);
}

// One wavefront merges one (b, h).  Up to 64 splits, lane s reads split
// s's LSE once and the weights come from wavefront reductions; the partial
// rows are then read four splits at a time, added in split order.  More
// splits take a plain loop over the splits.
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeArgs a) {
    // grid (heads / 4, B): wavefront w of workgroup (x, b) merges head 4x + w
    const int b = blockIdx.y, h = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (h >= a.H) return;
    int n = a.splits_per_seq ? a.splits_per_seq[b] : a.S;
    n = n < 0 ? 0 : (n > a.S ? a.S : n);
    const int64_t base = (int64_t)b * a.S * a.H + h;  // row of split s: base + s*H
    float* out = a.out + ((int64_t)b * a.H + h) * a.D;
    float M, wsum;
    if (n <= 64) {
        const float l = lane < n ? a.part_lse[base + (int64_t)lane * a.H] : -INFINITY;
        M = wave_max64(l);
        const float wl = (l == -INFINITY || M == -INFINITY) ? 0.0f : expf(l - M);
        wsum = wave_sum64(wl);
        if (M != -INFINITY) {
            const float inv = 1.0f / wsum;
            for (int c = 4 * lane; c < a.D; c += 256) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int s0 = 0; s0 < n; s0 += 4) {
                    f32x4 x[4];
                    float wg[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bool in = s0 + j < n;
                        const int sj = in ? s0 + j : s0;   // (uniform)
                        wg[j] = __int_as_float(in ? __builtin_amdgcn_readlane(__float_as_int(wl), sj) : 0);
                        x[j] = *reinterpret_cast<const f32x4*>(a.part_out + (base + (int64_t)sj * a.H) * a.D + c);
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (wg[j] != 0.0f) acc += wg[j] * x[j];   // (uniform) splits without tokens add nothing
                }
                *reinterpret_cast<f32x4*>(out + c) = acc * inv;
            }
        }
    } else {
        M = -INFINITY;
        for (int s = 0; s < n; ++s) M = fmaxf(M, a.part_lse[base + (int64_t)s * a.H]);
        wsum = 0.0f;
        for (int s = 0; s < n; ++s) {
            const float l = a.part_lse[base + (int64_t)s * a.H];
            wsum += (l == -INFINITY || M == -INFINITY) ? 0.0f : expf(l - M);
        }
        if (M != -INFINITY) {
            const float inv = 1.0f / wsum;
            for (int c = 4 * lane; c < a.D; c += 256) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int s = 0; s < n; ++s) {
                    const float l = a.part_lse[base + (int64_t)s * a.H];
                    if (l == -INFINITY) continue;
                    const float wgt = expf(l - M);
                    acc += wgt * *reinterpret_cast<const f32x4*>(a.part_out + (base + (int64_t)s * a.H) * a.D + c);
                }
                *reinterpret_cast<f32x4*>(out + c) = acc * inv;
            }
        }
    }
    if (M == -INFINITY) {
        for (int c = 4 * lane; c < a.D; c += 256) *reinterpret_cast<f32x4*>(out + c) = f32x4{0.f, 0.f, 0.f, 0.f};
        if (a.lse && lane == 0) a.lse[(int64_t)b * a.H + h] = -INFINITY;
        return;
    }
    if (a.lse && lane == 0) a.lse[(int64_t)b * a.H + h] = M + logf(wsum);
}

template <int NW, bool kRopeFp8, bool kSparse, int kPQ = 0>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    const int hg = 16 * NW;
    const dim3 grid((unsigned)a.max_splits, (unsigned)a.B, (unsigned)((a.H + hg - 1) / hg));
    hipLaunchKernelGGL((decode_kernel<NW, kRopeFp8, kSparse, kPQ>), grid, dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

template <int NW>
hipError_t launch_decode_w(const DecodeArgs& a, hipStream_t stream) {
    const bool fp8 = a.record_bytes == 368;
    if (a.indices)
        return fp8 ? launch_decode_t<NW, true, true>(a, stream) : launch_decode_t<NW, false, true>(a, stream);
    return fp8 ? launch_decode_t<NW, true, false>(a, stream) : launch_decode_t<NW, false, false>(a, stream);
}

}  // namespace

// Up to 16 heads: the narrow kernel (each wavefront its own tokens); more:
// 128 heads per workgroup.  Split sequences are then merged by
// split_merge_kernel.
// Dense decode on NVFP4 records with P quantized (and Q, by p.qdq_flags), for
// more than 16 heads; the split merge follows.
hipError_t launch_decode_pq(const DecodeArgs& a, hipStream_t stream) {
    const bool fp8r = a.record_bytes == 368, fp8p = a.qdq_flags & 64u;
    hipError_t e;
    if (fp8p) e = fp8r ? launch_decode_t<8, true, false, 2>(a, stream) : launch_decode_t<8, false, false, 2>(a, stream);
    else e = fp8r ? launch_decode_t<8, true, false, 1>(a, stream) : launch_decode_t<8, false, false, 1>(a, stream);
    if (e != hipSuccess || a.max_splits <= 1) return e;
    return launch_split_merge(a, stream);
}

hipError_t launch_split_merge(const DecodeArgs& a, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    const dim3 grid((unsigned)((a.H + 3) / 4), (unsigned)a.B);   // (4 heads, sequence)
    if (a.indices)
        hipLaunchKernelGGL((split_merge_kernel<true>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((split_merge_kernel<false>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    const hipError_t e = a.H <= 16 ? launch_decode_narrow(a, stream) : launch_decode_w<8>(a, stream);
    if (e != hipSuccess || a.max_splits <= 1) return e;
    return launch_split_merge(a, stream);
}

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream) {
    if (a.B == 0 || a.H == 0) return hipSuccess;
    hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)((a.H + 3) / 4), (unsigned)a.B), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mla
