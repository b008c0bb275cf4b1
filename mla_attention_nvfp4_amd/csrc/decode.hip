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
// Work item: workgroup (split s, sequence b, head group hg) with NW
// wavefronts, wavefront w owning 16 query heads.  The token range of the
// split is walked in tiles of 64 tokens:
//   phase A  every thread dequantizes an 8-token x 8-element block of the
//            latent (e2m1 code x e4m3 scale, exact in bf16; the outer scale
//            is NOT folded in) and writes it twice to LDS: token-major (Ks,
//            the QK^T operand) and element-major (Vt, the PV operand); the
//            RoPE part goes to Ks columns 512..575.  The global loads of the
//            next tile are issued before the MMA phase of this one.
//   phase B  each wavefront: S^T = K Q^T with v_mfma_f32_16x16x32_bf16
//            (A = Ks rows from LDS, B = the wave's 16 Q rows held in VGPRs),
//            two accumulators (latent and RoPE) so that
//            z = scale * (outer * s_nope + s_rope) in fp32; online softmax
//            in base 2; P, split into bf16 hi + lo parts, stays in
//            registers as the B operand of O^T = V^T P^T (A = Vt rows from
//            LDS, each fragment used by two MFMAs).
// The epilogue writes out = outer * O / l and lse = m + ln l (natural log)
// to the output when the sequence has one split; otherwise it writes the
// partial to the workspace and the last workgroup of the sequence and head
// group to finish merges the partials (same rule as lse_merge_kernel).
#include "device_common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int kTile = 64;            // tokens per tile
constexpr int kKsPitch = kQK + 8;    // bf16 elements per Ks row (584)
constexpr int kVtPitch = kTile + 8;  // bf16 elements per Vt row (72)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;

struct DecodeSmem {
    uint16_t ks[kTile * kKsPitch];        // [token][576 (+8)]  74752 B
    uint16_t vt[kLatent * kVtPitch];      // [element][64 (+8)] 73728 B
    int64_t offs[2][kTile];               // record byte offset, -1 = masked
    int last;                             // this workgroup merges the splits
};

template <int NW, bool kRopeFp8, bool kSparse>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_kernel(DecodeArgs p) {
    constexpr int kRec = kRopeFp8 ? 368 : 432;
    constexpr int kG = 8 / NW;            // 8-token groups per thread
    constexpr int kR = 512 / (64 * NW);   // RoPE 16-byte units per thread
    __shared__ DecodeSmem sm;

    const int s = blockIdx.x, b = blockIdx.y, hg = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int gq = lane >> 4, c16 = lane & 15;

    int L = p.seq_lens[b];
    const int Lmax = p.max_pages * p.page_size;
    L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
    const int n_items = kSparse ? p.topk : L;
    const int ns = decode_num_splits(n_items, p.max_splits);
    if (s >= ns) return;
    const int ct = decode_chunk_tiles(n_items, p.max_splits);
    const int nt = (n_items + kTile - 1) / kTile;
    const int t_begin = s * ct;
    const int t_end = min(nt, t_begin + ct);

    const int h_base = hg * 16 * NW + 16 * w;
    const bool wave_active = h_base < p.H;
    const int hq = h_base + c16;

    // Q as the B operand of S^T = K Q^T: k-step kk covers d = 32kk..32kk+31.
    bf16x8 qf[18];
    {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const bool ok = hq < p.H;
        const int64_t qoff = (int64_t)b * p.q_stride_b + (int64_t)hq * p.q_stride_h + 8 * gq;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk)
            qf[kk] = as_bf16x8(ok ? *reinterpret_cast<const u32x4*>(p.q_nope + qoff + 32 * kk) : zero);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            qf[16 + kk] = as_bf16x8(ok ? *reinterpret_cast<const u32x4*>(p.q_rope + qoff + 32 * kk) : zero);
    }

    const uint8_t* __restrict__ cache = p.cache;
    const float scale_log2 = p.softmax_scale * kLog2e;
    const float outer = p.outer_scale;

    auto compute_offs = [&](int t, int buf) {
        // threads 0..63: record offset of the tile's tokens
        const int item = t * kTile + tid;
        int64_t off = -1;
        if (item < n_items) {
            const int pos = kSparse ? p.indices[(int64_t)b * p.topk + item] : item;
            if (pos >= 0 && pos < L) {
                const int pg = p.page_table[(int64_t)b * p.max_pages + pos / p.page_size];
                if (pg >= 0 && pg < p.num_pages)
                    off = ((int64_t)pg * p.page_size + pos % p.page_size) * kRec;
            }
        }
        sm.offs[buf][tid] = off;
    };

    // per-thread staging registers for one tile
    uint32_t codes[kG][8], scl[kG][8];
    u32x4 rope[kR];

    // Masked tokens load record 0 (always present) and are zeroed, so the
    // loads need no branches.
    auto load_tile = [&](int buf) {
#pragma unroll
        for (int g = 0; g < kG; ++g) {
            const int chunk = 8 * (w * kG + g) + (lane & 7);
            const int tg = lane >> 3;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int64_t off = sm.offs[buf][tg * 8 + r];
                const uint8_t* rp = cache + (off < 0 ? 0 : off);
                const uint32_t cw = *reinterpret_cast<const uint32_t*>(rp + 4 * chunk);
                const uint32_t sw = rp[256 + (chunk >> 1)];
                codes[g][r] = off < 0 ? 0u : cw;
                scl[g][r] = off < 0 ? 0u : sw;
            }
        }
#pragma unroll
        for (int i = 0; i < kR; ++i) {
            const int item = tid + i * NW * 64;
            const int64_t off = sm.offs[buf][item >> 3];
            const uint8_t* rp = cache + (off < 0 ? 0 : off);
            const int u = item & 7;
            u32x4 v;
            if (kRopeFp8) {
                const u32x2 v2 = *reinterpret_cast<const u32x2*>(rp + 288 + 8 * u);
                v = u32x4{v2[0], v2[1], 0u, 0u};
            } else {
                v = *reinterpret_cast<const u32x4*>(rp + 288 + 16 * u);
            }
            const u32x4 zero = {0u, 0u, 0u, 0u};
            rope[i] = off < 0 ? zero : v;
        }
    };

    auto dequant_tile = [&]() {
#pragma unroll
        for (int g = 0; g < kG; ++g) {
            const int chunk = 8 * (w * kG + g) + (lane & 7);
            const int tg = lane >> 3;
            // kw[r][j]: bf16 pair (elements 2j, 2j+1) of token row r
            uint32_t kw[8][4];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float sc = e4m3_decode(scl[g][r]);
                const uint32_t c = codes[g][r];
                {
                    const f32x2 v0 = e2m1_pair<0>(c), v1 = e2m1_pair<1>(c);
                    const f32x2 v2 = e2m1_pair<2>(c), v3 = e2m1_pair<3>(c);
                    kw[r][0] = pack_bf16_exact(v0[0] * sc, v0[1] * sc);
                    kw[r][1] = pack_bf16_exact(v1[0] * sc, v1[1] * sc);
                    kw[r][2] = pack_bf16_exact(v2[0] * sc, v2[1] * sc);
                    kw[r][3] = pack_bf16_exact(v3[0] * sc, v3[1] * sc);
                }
                const u32x4 wv = {kw[r][0], kw[r][1], kw[r][2], kw[r][3]};
                *reinterpret_cast<u32x4*>(&sm.ks[(tg * 8 + r) * kKsPitch + 8 * chunk]) = wv;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // element e of rows (2i, 2i+1): low or high halves of kw[.][e/2]
                const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                u32x4 wv;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    wv[i] = __builtin_amdgcn_perm(kw[2 * i + 1][e >> 1], kw[2 * i][e >> 1], sel);
                *reinterpret_cast<u32x4*>(&sm.vt[(8 * chunk + e) * kVtPitch + 8 * tg]) = wv;
            }
        }
#pragma unroll
        for (int i = 0; i < kR; ++i) {
            const int item = tid + i * NW * 64;
            const int tok = item >> 3, u = item & 7;
            u32x4 wv;
            if (kRopeFp8) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const uint32_t x = rope[i][j];
                    wv[2 * j] = pack_bf16_exact(e4m3_decode(x & 0xffu), e4m3_decode((x >> 8) & 0xffu));
                    wv[2 * j + 1] = pack_bf16_exact(e4m3_decode((x >> 16) & 0xffu), e4m3_decode(x >> 24));
                }
            } else {
                wv = rope[i];
            }
            *reinterpret_cast<u32x4*>(&sm.ks[tok * kKsPitch + kLatent + 8 * u]) = wv;
        }
    };

    f32x4 o[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    auto mma_tile = [&](int buf) {
        f32x4 sn[4], sr[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            sn[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            sr[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // A fragments double-buffered one k-step ahead; the scheduling
        // barrier keeps the compiler from hoisting every LDS read at once.
        auto ks_frag = [&](int kk, int tt) {
            return *reinterpret_cast<const u32x4*>(&sm.ks[(16 * tt + c16) * kKsPitch + 32 * kk + 8 * gq]);
        };
        u32x4 acur[4], anxt[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acur[tt] = ks_frag(0, tt);
#pragma unroll
        for (int kk = 0; kk < 18; ++kk) {
            if (kk + 1 < 18) {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) anxt[tt] = ks_frag(kk + 1, tt);
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                if (kk < 16) sn[tt] = mfma16x16x32(as_bf16x8(acur[tt]), qf[kk], sn[tt]);
                else sr[tt] = mfma16x16x32(as_bf16x8(acur[tt]), qf[kk], sr[tt]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) acur[tt] = anxt[tt];
        }
        // scores (log2 units) of tokens 16tt + 4gq + i for head c16
        float z[4][4];
        float mx = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool valid = sm.offs[buf][16 * tt + 4 * gq + i] >= 0;
                const float v = scale_log2 * (outer * sn[tt][i] + sr[tt][i]);
                z[tt][i] = valid ? v : -INFINITY;
                mx = fmaxf(mx, z[tt][i]);
            }
        }
        mx = wave_xor_max(mx, 16);
        mx = wave_xor_max(mx, 32);
        // Lazy rescaling: the reference max m_run moves only when a score
        // exceeds it by more than kRescaleSlack (log2 units), so p <= 2^8 and
        // O is rescaled rarely (a rescale costs AGPR round trips).  The result
        // is the same softmax; only rounding differs.
        const bool move = mx > m_run + kRescaleSlack;
        const float m_new = move ? mx : m_run;
        const bool live = m_new != -INFINITY;
        const float alpha = (move && m_run != -INFINITY) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        float psum = 0.0f;
        float pv[4][4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pv[tt][i] = live ? __builtin_amdgcn_exp2f(z[tt][i] - m_new) : 0.0f;
                psum += pv[tt][i];
            }
        }
        psum = wave_xor_sum(psum, 16);
        psum = wave_xor_sum(psum, 32);
        l_run = alpha * l_run + psum;
        m_run = m_new;
        // any lane of the wave moving its max triggers the (rare) rescale
        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int c = 0; c < 32; ++c) o[c] *= alpha;
        }
        // P as hi + lo bf16 parts (|p - hi - lo| <= 2^-16 |p|): one bf16
        // rounding of P alone can exceed the output tolerance when V has
        // large outliers, so PV runs twice per V fragment.
        bf16x8 ph[2], pl[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            u32x4 h, lo;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float* src = pv[2 * k2 + j];
                h[2 * j] = pack_bf16_rne(src[0], src[1]);
                h[2 * j + 1] = pack_bf16_rne(src[2], src[3]);
                lo[2 * j] = pack_bf16_rne(src[0] - bf16_lo(h[2 * j]), src[1] - bf16_hi(h[2 * j]));
                lo[2 * j + 1] = pack_bf16_rne(src[2] - bf16_lo(h[2 * j + 1]), src[3] - bf16_hi(h[2 * j + 1]));
            }
            ph[k2] = as_bf16x8(h);
            pl[k2] = as_bf16x8(lo);
        }
        auto vt_frag = [&](int c, int k2) {
            // tokens 32k2 + 4gq .. +3 and 32k2 + 16 + 4gq .. +3 of element row 16c + c16
            const uint16_t* rp = &sm.vt[(16 * c + c16) * kVtPitch + 32 * k2 + 4 * gq];
            const u32x2 lo = *reinterpret_cast<const u32x2*>(rp);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(rp + 16);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
        u32x4 vcur[2], vnxt[2];
        vcur[0] = vt_frag(0, 0);
        vcur[1] = vt_frag(0, 1);
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            if (c + 1 < 32) {
                vnxt[0] = vt_frag(c + 1, 0);
                vnxt[1] = vt_frag(c + 1, 1);
            }
            o[c] = mfma16x16x32(as_bf16x8(vcur[0]), ph[0], o[c]);
            o[c] = mfma16x16x32(as_bf16x8(vcur[1]), ph[1], o[c]);
            o[c] = mfma16x16x32(as_bf16x8(vcur[0]), pl[0], o[c]);
            o[c] = mfma16x16x32(as_bf16x8(vcur[1]), pl[1], o[c]);
            __builtin_amdgcn_sched_barrier(0);
            vcur[0] = vnxt[0];
            vcur[1] = vnxt[1];
        }
    };

    if (t_begin < t_end) {
        if (tid < kTile) compute_offs(t_begin, 0);
        __syncthreads();
        for (int t = t_begin; t < t_end; ++t) {
            const int buf = (t - t_begin) & 1;
            load_tile(buf);
            dequant_tile();
            if (t + 1 < t_end && tid < kTile) compute_offs(t + 1, buf ^ 1);
            __syncthreads();
            if (wave_active) mma_tile(buf);
            __syncthreads();
        }
    }

    const bool has_head = wave_active && hq < p.H;
    const bool any = l_run > 0.0f;
    const float so = any ? outer / l_run : 0.0f;
    const float lse_v = any ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : -INFINITY;
    if (ns == 1) {
        if (!has_head) return;
        float* dst = p.out + ((int64_t)b * p.H + hq) * kLatent;
        if (gq == 0) p.lse[(int64_t)b * p.H + hq] = lse_v;
#pragma unroll
        for (int c = 0; c < 32; ++c) *reinterpret_cast<f32x4*>(dst + 16 * c + 4 * gq) = o[c] * so;
        return;
    }

    // Split: write the partial, then the last workgroup of (b, hg) to arrive
    // merges all ns partials in split order (so the result does not depend
    // on arrival order) and resets the arrival counter for the next call.
    if (has_head) {
        const int64_t row = ((int64_t)b * p.max_splits + s) * p.H + hq;
        float* dst = p.ws_out + row * kLatent;
        if (gq == 0) p.ws_lse[row] = lse_v;
#pragma unroll
        for (int c = 0; c < 32; ++c) *reinterpret_cast<f32x4*>(dst + 16 * c + 4 * gq) = o[c] * so;
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        int* cnt = p.ws_count + (int64_t)b * p.count_stride + hg;
        const int old = atomicAdd(cnt, 1);
        sm.last = (old == ns - 1);
        if (old == ns - 1) atomicExch(cnt, 0);
    }
    __syncthreads();
    if (!sm.last || !wave_active) return;
    __threadfence();
    for (int j = 0; j < 16; ++j) {
        const int h = h_base + j;
        if (h >= p.H) break;
        const int64_t row0 = (int64_t)b * p.max_splits * p.H + h;   // split s2 at row0 + s2*H
        float M = -INFINITY;
        for (int s2 = 0; s2 < ns; ++s2) M = fmaxf(M, p.ws_lse[row0 + (int64_t)s2 * p.H]);
        float* dst = p.out + ((int64_t)b * p.H + h) * kLatent + 8 * lane;
        if (M == -INFINITY) {
            *reinterpret_cast<f32x4*>(dst) = f32x4{0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<f32x4*>(dst + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
            if (lane == 0) p.lse[(int64_t)b * p.H + h] = -INFINITY;
            continue;
        }
        float wsum = 0.0f;
        f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
        for (int s2 = 0; s2 < ns; ++s2) {
            const int64_t row = row0 + (int64_t)s2 * p.H;
            const float l = p.ws_lse[row];
            if (l == -INFINITY) continue;
            const float wgt = expf(l - M);
            wsum += wgt;
            const float* src = p.ws_out + row * kLatent + 8 * lane;
            a0 += wgt * *reinterpret_cast<const f32x4*>(src);
            a1 += wgt * *reinterpret_cast<const f32x4*>(src + 4);
        }
        const float inv = 1.0f / wsum;
        *reinterpret_cast<f32x4*>(dst) = a0 * inv;
        *reinterpret_cast<f32x4*>(dst + 4) = a1 * inv;
        if (lane == 0) p.lse[(int64_t)b * p.H + h] = M + logf(wsum);
    }
}

// One wavefront merges one (b, h).
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeArgs a) {
    const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (wid >= a.B * a.H) return;
    const int b = wid / a.H, h = wid % a.H;
    int n = a.splits_per_seq ? a.splits_per_seq[b] : a.S;
    n = n < 0 ? 0 : (n > a.S ? a.S : n);
    const int64_t base = (int64_t)b * a.S * a.H + h;  // row of split s: base + s*H
    float M = -INFINITY;
    for (int s = 0; s < n; ++s) M = fmaxf(M, a.part_lse[base + (int64_t)s * a.H]);
    float* out = a.out + ((int64_t)b * a.H + h) * a.D;
    if (M == -INFINITY) {
        for (int c = 4 * lane; c < a.D; c += 256) *reinterpret_cast<f32x4*>(out + c) = f32x4{0.f, 0.f, 0.f, 0.f};
        if (a.lse && lane == 0) a.lse[(int64_t)b * a.H + h] = -INFINITY;
        return;
    }
    float wsum = 0.0f;
    for (int s = 0; s < n; ++s) {
        const float l = a.part_lse[base + (int64_t)s * a.H];
        wsum += (l == -INFINITY) ? 0.0f : expf(l - M);
    }
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
    if (a.lse && lane == 0) a.lse[(int64_t)b * a.H + h] = M + logf(wsum);
}

template <int NW, bool kRopeFp8, bool kSparse>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)a.max_splits, (unsigned)a.B, (unsigned)((a.H + 16 * NW - 1) / (16 * NW)));
    hipLaunchKernelGGL((decode_kernel<NW, kRopeFp8, kSparse>), grid, dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    const bool fp8 = a.record_bytes == 368;
    const bool sparse = a.indices != nullptr;
    if (sparse) return fp8 ? launch_decode_t<4, true, true>(a, stream) : launch_decode_t<4, false, true>(a, stream);
    return fp8 ? launch_decode_t<4, true, false>(a, stream) : launch_decode_t<4, false, false>(a, stream);
}

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream) {
    const int waves = a.B * a.H;
    if (waves == 0) return hipSuccess;
    hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mla
