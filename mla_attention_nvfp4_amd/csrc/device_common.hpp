// Device helpers shared by the gfx950 kernels: NVFP4 element/scale codecs,
// bf16 packing, MFMA operand types and wavefront reductions.
//
// Formats (public definitions; the pages only name them): e2m1 is the OCP MX
// FP4 element (sign, 2-bit exponent with bias 1, 1-bit mantissa; magnitudes
// 0, 0.5, 1, 1.5, 2, 3, 4, 6) and e4m3 the OCP FP8 E4M3FN scale (bias 7,
// max 448, no infinities).  Encoders round to nearest, ties to even, and
// saturate to the largest finite magnitude.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kQK = kLatent + kRope;  // 576

__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }

// ---------------------------------------------------------------- e4m3 --

// e4m3 code of an fp32 value: RNE, satfinite (|t| >= 448 -> 0x7E), sign kept.
// Branch-free: the three cases are computed and selected.
__device__ __forceinline__ uint32_t e4m3_encode(float t) {
    const uint32_t bits = f2u(t);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const uint32_t a = bits & 0x7fffffffu;
    // below 2^-6: multiples of 2^-9 (exact scaling, RNE)
    const uint32_t sub = (uint32_t)__builtin_rintf(u2f(a) * 512.0f);
    // normal: round the mantissa to 3 bits, rebias
    const uint32_t nrm = ((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
    const uint32_t code = a >= 0x43e00000u ? 0x7eu : (a < 0x3c800000u ? sub : nrm);   // >= 448 (and inf)
    return sign | code;
}

// e4m3 code of t >= 0 by the gfx950 FP8 conversion (round to nearest even):
// the same code as e4m3_encode for every fp32 value in [0, 448] (checked on
// the device over all of them).  Larger values, +inf and NaN are clamped to
// 448 first, whose code (0x7E) is the one e4m3_encode gives them.
__device__ __forceinline__ uint32_t e4m3_encode_nonneg(float t) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(t, 448.0f), 0.0f, 0, false) & 0xffu;
}

// e4m3 codes of two signed values by one FP8 conversion, in bytes 0 and 1:
// the sign bit over the code of min(|t|, 448) (as e4m3_encode_nonneg), which
// is e4m3_encode's code for every fp32 input, +-inf and NaN included (they
// saturate to 0x7E).
__device__ __forceinline__ uint32_t e4m3_encode2_hw(float t0, float t1) {
    const uint32_t mag = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(__builtin_fabsf(t0), 448.0f),
                                                                   fminf(__builtin_fabsf(t1), 448.0f), 0, false) & 0xffffu;
    return mag | ((f2u(t0) >> 24) & 0x80u) | ((f2u(t1) >> 16) & 0x8000u);
}

// fp32 value of an e4m3 code by the gfx950 FP8 conversion (OCP E4M3FN,
// exact; codes 0x7F/0xFF are NaN and never produced by the encoders here).
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
    return __builtin_amdgcn_cvt_f32_fp8(b & 0xffu, 0);
}

// fp32 value of e4m3 byte `sel` of x (as e4m3_decode), and four such bytes
// as two packed bf16 pairs (exact: e4m3 fits bf16).
template <int kSel>
__device__ __forceinline__ float e4m3_hw(uint32_t x) {
    return __builtin_amdgcn_cvt_f32_fp8(x, kSel);
}
__device__ __forceinline__ u32x2 e4m3x4_to_bf16(uint32_t x) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(x, false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(x, true);
    return u32x2{__builtin_amdgcn_perm(f2u(lo[1]), f2u(lo[0]), 0x07060302u),
                 __builtin_amdgcn_perm(f2u(hi[1]), f2u(hi[0]), 0x07060302u)};
}

// ---------------------------------------------------------------- e2m1 --

// e2m1 codes of a and b written as byte kSel of w (a in the low nibble) by
// the gfx950 FP4 conversion with a unit scale: round to nearest, ties to
// even (tied values go to the even code: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1,
// 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4), saturating at 6, sign bit kept also
// when the result is 0.  Checked on the device against a comparison-based
// encoder of that rule over all bf16 bit patterns, infinities included,
// times a set of scale factors: no difference (NaN inputs are unspecified).
template <int kSel>
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t w, float a, float b) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, kSel);
}

// e2m1 codes of x[0..7] * s (each product one fp32 rounding), low nibble first.
__device__ __forceinline__ uint32_t e2m1_encode8(const float* x, float s) {
    uint32_t w = e2m1_pack2<0>(0u, x[0] * s, x[1] * s);
    w = e2m1_pack2<1>(w, x[2] * s, x[3] * s);
    w = e2m1_pack2<2>(w, x[4] * s, x[5] * s);
    return e2m1_pack2<3>(w, x[6] * s, x[7] * s);
}

// Values of the two e2m1 codes in byte `sel` (0..3) of `w` (low nibble
// first), by the gfx950 FP4 conversion with a unit scale (exact: checked
// against the e2m1 value table for all 256 bytes).
template <int kSel>
__device__ __forceinline__ f32x2 e2m1_pair(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, kSel);
}

// The lane's index within its wavefront, read afresh (v_mbcnt) where it is
// used: the volatile statement is not moved out of a loop, so values
// derived from the lane (masks, addresses) are formed in the loop body
// instead of each holding a register, or a spill slot, across the loop.
__device__ __forceinline__ int lane_now() {
    int l;
    __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// ------------------------------------------------------- NVFP4 blocks --

// Two-level NVFP4 block scale for a block with amax `a` and dequant
// multiplier g: t = a / (6 g), s = e4m3(t), d = s * g, inv = 1/d (0 when
// d == 0); each step one IEEE fp32 operation (this file is compiled with
// contraction off and correctly rounded division).
struct Nvfp4Scale {
    uint32_t code;
    float inv;
};

__device__ __forceinline__ Nvfp4Scale nvfp4_block_scale(float a, float g) {
    const float u = 6.0f * g;
    const float t = a / u;
    const uint32_t s = e4m3_encode_nonneg(t);   // t >= 0 (or NaN)
    const float d = e4m3_decode(s) * g;
    return Nvfp4Scale{s, (d == 0.0f) ? 0.0f : 1.0f / d};
}

// The scale quotient t = fp32(a / u) taken as one multiply by
// inv_u = fp32(1 / u): the product lies within two ulps of the correctly
// rounded quotient, so its e4m3 code can differ only where it is within a few
// ulps of an e4m3 rounding tie (the 20 mantissa bits below the kept 3 near
// one half) or in the subnormal range (below 2^-6, where the rounding is done
// on t * 512).  Such values must redo the exact division.
__device__ __forceinline__ bool scale_quotient_near_tie(float tq) {
    const uint32_t rem = f2u(tq) & 0xfffffu;
    return tq < 0.015625f || (rem > 0x80000u - 8u && rem < 0x80000u + 8u);
}

// nvfp4_block_scale with the quotient by multiplication: u = fp32(6 g) and
// inv_u = fp32(1 / u) are given; the exact division is redone only where
// scale_quotient_near_tie says the code could differ, so the scale code and
// inv are those of nvfp4_block_scale.
__device__ __forceinline__ Nvfp4Scale nvfp4_block_scale_fast(float a, float g, float u, float inv_u) {
    float t = a * inv_u;
    const bool near = scale_quotient_near_tie(t);
    if (__any(near)) {
        // (a wavefront divides only when one of its lanes needs it; the empty
        // statement keeps the compiler from computing the quotient in every
        // lane and selecting it)
        __asm__ volatile("");
        const float q = a / u;
        t = near ? q : t;
    }
    const uint32_t s = e4m3_encode_nonneg(t);
    const float d = e4m3_decode(s) * g;
    return Nvfp4Scale{s, (d == 0.0f) ? 0.0f : 1.0f / d};
}

// Byte offset of scale (m, c) in the 128x4-swizzled layout with cpad
// (a multiple of 4) scale columns: tiles of 128 rows x 4 columns (512 B),
// row-tile major; inside a tile (m % 32) * 16 + ((m % 128) / 32) * 4 + c % 4.
__device__ __forceinline__ int64_t swizzled_scale_offset(int64_t m, int64_t c, int64_t cpad) {
    return ((m >> 7) * (cpad >> 2) + (c >> 2)) * 512 + (m & 31) * 16 + ((m & 127) >> 5) * 4 + (c & 3);
}

// ------------------------------------------------------------ bf16 pack --

// Pack the bf16 numbers held exactly by two fp32 values (low half = a).
__device__ __forceinline__ uint32_t pack_bf16_exact(float a, float b) {
    return __builtin_amdgcn_perm(f2u(b), f2u(a), 0x07060302u);
}

// Round two fp32 values to bf16 (nearest even) and pack them (low half = a).
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
    uint32_t ua = f2u(a), ub = f2u(b);
    ua = (ua + 0x7fffu + ((ua >> 16) & 1u)) >> 16;
    ub = (ub + 0x7fffu + ((ub >> 16) & 1u)) & 0xffff0000u;
    return ua | ub;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return u2f(w & 0xffff0000u); }

// ----------------------------------------------------------------- MFMA --

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D = A (16x32) * B (32x16) + C, fp32 accumulate.  Lane l supplies row
// l % 16 of A and column l % 16 of B, each with 8 consecutive k-slots
// 8*(l/16) .. 8*(l/16)+7 (the same slots in A and B); it receives
// D[4*(l/16) + i][l % 16] in element i.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------ wavefront --

__device__ __forceinline__ float wave_xor_max(float v, int mask) {
    return fmaxf(v, __shfl_xor(v, mask, 64));
}
__device__ __forceinline__ float wave_xor_sum(float v, int mask) {
    return v + __shfl_xor(v, mask, 64);
}

// op(x[l], x[l ^ 16]) and op(x[l], x[l ^ 32]) by the gfx950 row-swap
// permutes (VALU; each returns {x[l], x[l ^ 16 or 32]} in some order).
__device__ __forceinline__ float xor16_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
    return fmaxf(u2f(r[0]), u2f(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
    return fmaxf(u2f(r[0]), u2f(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
    return u2f(r[0]) + u2f(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
    return u2f(r[0]) + u2f(r[1]);
}

// LDS-only workgroup barrier: this wavefront's LDS operations are complete
// before it arrives; outstanding global loads stay in flight.  (The asm's
// memory clobber keeps the compiler from moving memory accesses across.)
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace mla
