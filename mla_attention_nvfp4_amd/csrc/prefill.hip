// Varlen causal MLA prefill with NVFP4 fake quantization of Q/K/P/V and the
// output written directly as NVFP4 (gfx950).
//
// [MO-MLA], commit 1 and PR body: varlen prefill with asymmetric head dims
// (qk 192, v 128); each matmul operand quantized once along its own
// contraction axis in 1x16 NVFP4 blocks (Q, K along the head dim, V along
// tokens, P along keys after the softmax row sum; the denominator stays
// unquantized); natural-log LSE.  [FUSED-OUT], PR description: the output is
// written as packed e2m1 codes plus e4m3 block scales in the 128x4-swizzled
// layout with an fp32 global scale, replacing a separate quantization pass.
//
// Kernels:
//   qk_qdq_kernel   Q and K, one thread per 16-element block along d: the
//                   exact bf16 value s*v of every element (the tensor-wide
//                   multiplier g is applied later, in fp32);
//   v_qdq_kernel    V, one thread per (16-token block of a sequence, head,
//                   dim): blocks start at the sequence start, the last one
//                   may be short;
//   attn_kernel     one workgroup per (256 query rows, head, sequence):
//                   8 wavefronts x 32 rows.  Keys are visited in tiles of 64
//                   from key 0 (the P-quantization schedule), K/V tiles
//                   staged in registers one tile ahead and stored token-major
//                   in LDS; S^T = K Q^T on v_mfma_f32_16x16x32_bf16; running
//                   max refreshed per tile; P quantized in 16-key blocks
//                   against it (exact in bf16); O^T = V^T P^T with V^T read
//                   by ds_read_b64_tr_b16; epilogue: O = acc * g_p g_v / l,
//                   NVFP4 codes and swizzled scales, LSE = m + ln l;
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
constexpr int kPitch = 208;             // bf16 elements per LDS row (416 B): conflict-free
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ---------------------------------------------------------------- Q, K --

__global__ __launch_bounds__(256) void qk_qdq_kernel(const uint16_t* __restrict__ x, int64_t st, int64_t sh,
                                                     int64_t T, int H, float g, uint16_t* __restrict__ out) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // block of 16 along d
    const int64_t nblk = T * H * (kDqk / 16);
    if (idx >= nblk) return;
    const int blk = (int)(idx % (kDqk / 16));
    const int64_t th = idx / (kDqk / 16);
    const int h = (int)(th % H);
    const int64_t t = th / H;
    const u32x4* src = reinterpret_cast<const u32x4*>(x + t * st + (int64_t)h * sh + 16 * blk);
    const u32x4 w0 = src[0], w1 = src[1];
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
        o0[i] = pack_bf16_exact(e2m1_decode(e2m1_encode(v[2 * i] * sc.inv)) * sv,
                                e2m1_decode(e2m1_encode(v[2 * i + 1] * sc.inv)) * sv);
        o1[i] = pack_bf16_exact(e2m1_decode(e2m1_encode(v[8 + 2 * i] * sc.inv)) * sv,
                                e2m1_decode(e2m1_encode(v[8 + 2 * i + 1] * sc.inv)) * sv);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(out + (t * H + h) * kDqk + 16 * blk);
    dst[0] = o0;
    dst[1] = o1;
}

// ------------------------------------------------------------------- V --

// grid (ceil(max_seqlen/16), N, ceil(H*128/256)); thread = (head, dim)
__global__ __launch_bounds__(256) void v_qdq_kernel(const uint16_t* __restrict__ v, int64_t st, int64_t sh,
                                                    const int32_t* __restrict__ cu, int H, float g,
                                                    uint16_t* __restrict__ out) {
    const int n = blockIdx.y;
    const int a = cu[n], e = cu[n + 1];
    const int t0 = a + 16 * blockIdx.x;
    if (t0 >= e) return;
    const int hd = blockIdx.z * 256 + threadIdx.x;
    if (hd >= H * kDv) return;
    const int h = hd / kDv, d = hd % kDv;
    const int cnt = min(16, e - t0);
    float x[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        x[i] = 0.0f;
        if (i < cnt) {
            const uint16_t bits = v[(int64_t)(t0 + i) * st + (int64_t)h * sh + d];
            x[i] = u2f((uint32_t)bits << 16);
            amax = fmaxf(amax, __builtin_fabsf(x[i]));
        }
    }
    const Nvfp4Scale sc = nvfp4_block_scale(amax, g);
    const float sv = e4m3_decode(sc.code);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (i < cnt) {
            const float q = e2m1_decode(e2m1_encode(x[i] * sc.inv)) * sv;
            out[((int64_t)(t0 + i) * H + h) * kDv + d] = (uint16_t)(f2u(q) >> 16);
        }
    }
}

// ----------------------------------------------------------- attention --

struct AttnParams {
    const uint16_t* q; int64_t q_st, q_sh;   // Q operand (exact bf16 s*v, or raw)
    const uint16_t* k; int64_t k_st, k_sh;
    const uint16_t* v; int64_t v_st, v_sh;
    const int32_t* cu;
    int H;
    float score_scale_log2;   // softmax_scale * g_q' * g_k' * log2(e)
    double out_scale;         // g_p' * g_v' (exact in fp64)
    float g_p;                // P multiplier (P quantized only)
    float u_p;                // fp32(6 g_p)
    float inv_u_p;            // fp32(1 / u_p)
    float g_out;              // output global scale
    int64_t T;
    uint8_t* out_fp4;
    uint8_t* out_scales;
    float* lse;
};

struct AttnSmem {
    uint16_t kt[2][kBN * kPitch];   // 2 x 26624 B
    uint16_t vt[2][kBN * kPitch];   // 2 x 26624 B
    float pinv[256];                // P block scale code -> fp32(1 / fp32(e4m3(code) g_p)), 0 for d = 0
};

// e4m3 code of a P block with amax a >= 0: the quantizer's t = fp32(a / u)
// by one multiply with fp32(1/u); the product lies within two ulps of the
// quotient, so the code can differ only when it is within a few ulps of an
// e4m3 rounding tie (or in the subnormal range, where the rounding is done
// on t * 512): those lanes redo the exact division.
__device__ __forceinline__ uint32_t p_scale_code(float a, float u, float inv_u) {
    const float tq = a * inv_u;
    const uint32_t rem = f2u(tq) & 0xfffffu;
    const bool near = tq < 0.015625f || (rem > 0x80000u - 8u && rem < 0x80000u + 8u);
    return e4m3_encode(near ? a / u : tq);
}

// Values of the two e2m1 codes in byte kSel of w, unit scale.
template <int kSel>
__device__ __forceinline__ f32x2 fp4_pair(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, kSel);
}

template <bool kQuantP>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_kernel(AttnParams p) {
    __shared__ AttnSmem sm;
    if (kQuantP && threadIdx.x < 256) {
        const float d = e4m3_decode(threadIdx.x) * p.g_p;
        sm.pinv[threadIdx.x] = (d == 0.0f) ? 0.0f : 1.0f / d;
    }
    const int n = blockIdx.z, h = blockIdx.y;
    const int a = p.cu[n], e = p.cu[n + 1];
    const int L = e - a;
    const int nqt = (L + kBM - 1) / kBM;
    const int qt = nqt - 1 - (int)blockIdx.x;   // longest (latest) tiles first
    if (qt < 0) return;
    const int r0 = qt * kBM;                     // local row of the tile
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int gq = lane >> 4, c16 = lane & 15;
    const int wr0 = r0 + kRowsPerWave * w;       // first local row of this wavefront
    const bool wave_rows = wr0 < L;

    // Q rows of the wavefront: B operand of S^T = K Q^T (2 row groups of 16)
    bf16x8 qf[2][6];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
        const int row = min(wr0 + 16 * rg + c16, L - 1);
        const uint16_t* src = p.q + (int64_t)(a + row) * p.q_st + (int64_t)h * p.q_sh + 8 * gq;
#pragma unroll
        for (int kk = 0; kk < 6; ++kk) qf[rg][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(src + 32 * kk));
    }

    // last key tile this workgroup needs; a wavefront needs tiles up to its last row
    const int rows_end = min(r0 + kBM, L);
    const int nkt = (rows_end + kBN - 1) / kBN;
    const int wave_last_row = min(wr0 + kRowsPerWave, L) - 1;

    // K/V tile staging: K 64 rows x 24 chunks (3 per thread), V 64 x 16 (2 per thread)
    u32x4 sk[3], sv[2];
    auto load_tile = [&](int kt) {
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int c = tid + 512 * i;
            const int row = c / 24, col = c % 24;
            const int j = min(kt * kBN + row, L - 1);
            sk[i] = *reinterpret_cast<const u32x4*>(p.k + (int64_t)(a + j) * p.k_st + (int64_t)h * p.k_sh + 8 * col);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + 512 * i;
            const int row = c >> 4, col = c & 15;
            const int j = min(kt * kBN + row, L - 1);
            sv[i] = *reinterpret_cast<const u32x4*>(p.v + (int64_t)(a + j) * p.v_st + (int64_t)h * p.v_sh + 8 * col);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int c = tid + 512 * i;
            *reinterpret_cast<u32x4*>(&sm.kt[buf][(c / 24) * kPitch + 8 * (c % 24)]) = sk[i];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + 512 * i;
            *reinterpret_cast<u32x4*>(&sm.vt[buf][(c >> 4) * kPitch + 8 * (c & 15)]) = sv[i];
        }
    };

    f32x4 o[2][8];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[rg][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.0f, 0.0f};

    auto compute = [&](int kt, int buf) {
        const uint16_t* kb = sm.kt[buf];
        const uint16_t* vb = sm.vt[buf];
        // S^T [64 keys x 32 rows]: 4 key m-tiles x 2 row groups
        f32x4 s[2][4];
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) s[rg][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 6; ++kk) {
            u32x4 af[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                af[mt] = *reinterpret_cast<const u32x4*>(&kb[(16 * mt + c16) * kPitch + 32 * kk + 8 * gq]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int rg = 0; rg < 2; ++rg) s[rg][mt] = mfma16x16x32(as_bf16x8(af[mt]), qf[rg][kk], s[rg][mt]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // softmax + P quantization per row group; lane holds keys
        // 16mt + 4gq + i (local in the tile) of row wr0 + 16rg + c16
        bf16x8 ph[2][2], pm[2][2], pl[2][2];
        float alpha[2];
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) {
            const int row = wr0 + 16 * rg + c16;
            float z[4][4];
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = kt * kBN + 16 * mt + 4 * gq + i;
                    z[mt][i] = (key <= row) ? p.score_scale_log2 * s[rg][mt][i] : -INFINITY;
                    mx = fmaxf(mx, z[mt][i]);
                }
            mx = xor32_max(xor16_max(mx));
            const float m_new = fmaxf(m_run[rg], mx);
            const bool live = m_new != -INFINITY;
            alpha[rg] = (m_run[rg] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run[rg] - m_new);
            float pv[4][4];
            float psum = 0.0f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pv[mt][i] = live ? __builtin_amdgcn_exp2f(z[mt][i] - m_new) : 0.0f;
                    psum += pv[mt][i];
                }
            psum = xor32_sum(xor16_sum(psum));
            l_run[rg] = alpha[rg] * l_run[rg] + psum;   // unquantized denominator
            m_run[rg] = m_new;
            if constexpr (kQuantP) {
                // 16-key block = key m-tile mt: amax over its 4 lane groups
                float am[4];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    am[mt] = xor32_max(xor16_max(fmaxf(fmaxf(pv[mt][0], pv[mt][1]), fmaxf(pv[mt][2], pv[mt][3]))));
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const uint32_t code = p_scale_code(am[mt], p.u_p, p.inv_u_p);
                    const float inv = sm.pinv[code];
                    const float sval = e4m3_decode(code);
                    uint32_t codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, pv[mt][0] * inv,
                                                                             pv[mt][1] * inv, 1.0f, 0);
                    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, pv[mt][2] * inv,
                                                                    pv[mt][3] * inv, 1.0f, 1);
                    const f32x2 d0 = fp4_pair<0>(codes), d1 = fp4_pair<1>(codes);
                    pv[mt][0] = d0[0] * sval;
                    pv[mt][1] = d0[1] * sval;
                    pv[mt][2] = d1[0] * sval;
                    pv[mt][3] = d1[1] * sval;
                }
            }
            // B operand of O^T = V^T P^T, k-step k2 (keys 32k2 .. +31): slot
            // j < 4 is key 32k2 + 4gq + j (m-tile 2k2), j >= 4 is key
            // 32k2 + 16 + 4gq + j - 4 (m-tile 2k2 + 1).  Quantized P is
            // exact in bf16; unquantized P is split into three bf16 parts
            // (|p - hi - mid - lo| <= 2^-24 |p|).
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                u32x4 hv, mv, lv;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const float* src = pv[2 * k2 + hh];
#pragma unroll
                    for (int pr = 0; pr < 2; ++pr) {
                        const float x0 = src[2 * pr], x1 = src[2 * pr + 1];
                        if constexpr (kQuantP) {
                            hv[2 * hh + pr] = pack_bf16_exact(x0, x1);
                            mv[2 * hh + pr] = 0u;
                            lv[2 * hh + pr] = 0u;
                        } else {
                            const uint32_t h1 = pack_bf16_rne(x0, x1);
                            const float r0 = x0 - bf16_lo(h1), r1 = x1 - bf16_hi(h1);
                            const uint32_t m1 = pack_bf16_rne(r0, r1);
                            hv[2 * hh + pr] = h1;
                            mv[2 * hh + pr] = m1;
                            lv[2 * hh + pr] = pack_bf16_rne(r0 - bf16_lo(m1), r1 - bf16_hi(m1));
                        }
                    }
                }
                ph[rg][k2] = as_bf16x8(hv);
                pm[rg][k2] = as_bf16x8(mv);
                pl[rg][k2] = as_bf16x8(lv);
            }
        }
        // (multiplying by 1 changes nothing: skipped when no row moved)
        if (__any(alpha[0] != 1.0f || alpha[1] != 1.0f)) {
#pragma unroll
            for (int rg = 0; rg < 2; ++rg)
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) o[rg][dt] *= alpha[rg];
        }
        // V^T fragments by transposing reads: within each 16-lane group,
        // lane s addresses key 32k2 + 4gq + s/4 (+16 for the second half)
        // and dims 16dt + 4(s%4) .. +3
        const uint16_t* vbase = vb + (4 * gq + (c16 >> 2)) * kPitch + 4 * (c16 & 3);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const uint16_t* p1 = vbase + 32 * k2 * kPitch + 16 * dt;
                const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)(const_cast<uint16_t*>(p1)));
                const s16x4 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(__attribute__((address_space(3))) uint16_t*)(const_cast<uint16_t*>(p1 + 16 * kPitch)));
                const u32x2 y1 = __builtin_bit_cast(u32x2, x1), y2 = __builtin_bit_cast(u32x2, x2);
                const bf16x8 va = as_bf16x8(u32x4{y1[0], y1[1], y2[0], y2[1]});
#pragma unroll
                for (int rg = 0; rg < 2; ++rg) {
                    o[rg][dt] = mfma16x16x32(va, ph[rg][k2], o[rg][dt]);
                    if constexpr (!kQuantP) {
                        o[rg][dt] = mfma16x16x32(va, pm[rg][k2], o[rg][dt]);
                        o[rg][dt] = mfma16x16x32(va, pl[rg][k2], o[rg][dt]);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    load_tile(0);
    store_tile(0);
    if (nkt > 1) load_tile(1);
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
        // a wavefront skips tiles that start after its last row
        if (wave_rows && kt * kBN <= wave_last_row) compute(kt, kt & 1);
        if (kt + 1 < nkt) store_tile((kt + 1) & 1);   // staged during compute(kt)
        if (kt + 2 < nkt) load_tile(kt + 2);          // lands during compute(kt+1)
        lds_barrier();
    }

    if (!wave_rows) return;
    // epilogue: lane holds O^T[dim 16dt + 4gq + i][row c16] of row group rg
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
        const int row = wr0 + 16 * rg + c16;
        const bool ok = row < L;
        // O = acc * g_p g_v / l in fp64, rounded once to fp32: when the
        // accumulation is exact (a row that sees one key) this is the
        // correctly rounded value, so NVFP4 rounding ties break as in an
        // exact evaluation.
        const double inv_l = l_run[rg] > 0.0f ? p.out_scale / (double)l_run[rg] : 0.0;
        const int64_t t = a + row;
        uint8_t* codes_row = p.out_fp4 + (t * p.H + h) * (kDv / 2);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            float x[4];
            float am = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = (float)((double)o[rg][dt][i] * inv_l);
                am = fmaxf(am, __builtin_fabsf(x[i]));
            }
            am = xor32_max(xor16_max(am));
            const Nvfp4Scale sc = nvfp4_block_scale(am, p.g_out);
            const uint32_t c2 = e2m1_encode(x[0] * sc.inv) | (e2m1_encode(x[1] * sc.inv) << 4) |
                                (e2m1_encode(x[2] * sc.inv) << 8) | (e2m1_encode(x[3] * sc.inv) << 12);
            if (ok) {
                *reinterpret_cast<uint16_t*>(codes_row + 8 * dt + 2 * gq) = (uint16_t)c2;
                if (gq == 0) {
                    const int64_t cpad = (int64_t)p.H * 8;
                    p.out_scales[swizzled_scale_offset(t, (int64_t)h * 8 + dt, cpad)] = (uint8_t)sc.code;
                }
            }
        }
        if (ok && gq == 0 && p.lse)
            p.lse[t * p.H + h] = l_run[rg] > 0.0f ? (m_run[rg] + __builtin_amdgcn_logf(l_run[rg])) * kLn2 : -INFINITY;
    }
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

}  // namespace

size_t prefill_workspace_bytes(int64_t T, int H, unsigned flags) {
    size_t b = 0;
    const size_t rows = (size_t)T * H;
    if (flags & 1u) b += rows * kDqk * 2;
    if (flags & 2u) b += rows * kDqk * 2;
    if (flags & 8u) b += rows * kDv * 2;
    return b;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    const int H = a.H;
    const int64_t T = a.T;
    uint16_t* ws = static_cast<uint16_t*>(a.workspace);
    AttnParams p{};
    p.q = a.q; p.q_st = a.q_st; p.q_sh = a.q_sh;
    p.k = a.k; p.k_st = a.k_st; p.k_sh = a.k_sh;
    p.v = a.v; p.v_st = a.v_st; p.v_sh = a.v_sh;
    float gq = 1.0f, gk = 1.0f, gv = 1.0f, gp = 1.0f;
    const int64_t nqk_blocks = T * H * (kDqk / 16);
    if (a.flags & 1u) {
        hipLaunchKernelGGL(qk_qdq_kernel, dim3((unsigned)((nqk_blocks + 255) / 256)), dim3(256), 0, stream, a.q,
                           a.q_st, a.q_sh, T, H, a.g_q, ws);
        p.q = ws; p.q_st = (int64_t)H * kDqk; p.q_sh = kDqk;
        gq = a.g_q;
        ws += (size_t)T * H * kDqk;
    }
    if (a.flags & 2u) {
        hipLaunchKernelGGL(qk_qdq_kernel, dim3((unsigned)((nqk_blocks + 255) / 256)), dim3(256), 0, stream, a.k,
                           a.k_st, a.k_sh, T, H, a.g_k, ws);
        p.k = ws; p.k_st = (int64_t)H * kDqk; p.k_sh = kDqk;
        gk = a.g_k;
        ws += (size_t)T * H * kDqk;
    }
    if (a.flags & 8u) {
        const dim3 grid((unsigned)((a.max_seqlen + 15) / 16), (unsigned)a.N, (unsigned)((H * kDv + 255) / 256));
        hipLaunchKernelGGL(v_qdq_kernel, grid, dim3(256), 0, stream, a.v, a.v_st, a.v_sh, a.cu_seqlens, H, a.g_v, ws);
        p.v = ws; p.v_st = (int64_t)H * kDv; p.v_sh = kDv;
        gv = a.g_v;
        ws += (size_t)T * H * kDv;
    }
    if (a.flags & 4u) gp = a.g_p;
    p.cu = a.cu_seqlens;
    p.H = H;
    p.score_scale_log2 = a.softmax_scale * gq * gk * kLog2e;
    p.out_scale = (double)gp * (double)gv;
    p.g_p = a.g_p;
    p.u_p = 6.0f * a.g_p;
    p.inv_u_p = 1.0f / p.u_p;
    p.g_out = a.g_out;
    p.T = T;
    p.out_fp4 = a.out_fp4;
    p.out_scales = a.out_scales;
    p.lse = a.lse;
    if (a.max_seqlen > 0) {
        const dim3 grid((unsigned)((a.max_seqlen + kBM - 1) / kBM), (unsigned)H, (unsigned)a.N);
        if (a.flags & 4u)
            hipLaunchKernelGGL(attn_kernel<true>, grid, dim3(kWaves * 64), 0, stream, p);
        else
            hipLaunchKernelGGL(attn_kernel<false>, grid, dim3(kWaves * 64), 0, stream, p);
    }
    const int64_t cpad = (int64_t)H * 8;
    const int64_t npad = ((T + 127) / 128 * 128 - T) * cpad;
    if (npad > 0)
        hipLaunchKernelGGL(pad_scales_kernel, dim3((unsigned)((npad + 255) / 256)), dim3(256), 0, stream,
                           a.out_scales, T, cpad);
    return hipGetLastError();
}

}  // namespace mla
