"""e2m1 and e4m3 codecs and the NVFP4 two-level block quantizer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The element format (e2m1, "FP4") and the scale format (e4m3, "FP8 E4M3FN") are
taken from their public definitions (OCP Microscaling spec for E2M1, OCP 8-bit
floating point spec for E4M3), not from the pages: the pages only name them.
Encoding is "nearest representable value, ties to the value whose last mantissa
bit is 0", with saturation to the largest finite magnitude.

The block quantizer follows [MO-MLA], PR body, contract notes: NVFP4 is a 1x16
block along the contraction axis with an e4m3 block scale, the scale being the
block amax over (6 * 448) times a tensor-wide factor; and [B12X], PR description:
the latent carries a per-layer fp32 outer scale restored on read.  Both readings
are one rule with a dequant multiplier ``g`` (finite, > 0):

    a    = max |x| over the block                      (fp32)
    u    = fp32(6 * g)
    t    = fp32(a / u)
    s    = e4m3(t)                                      (scale code)
    d    = fp32(value(s) * g)
    inv  = 0 if d == 0 else fp32(1 / d)
    code = e2m1(fp32(x * inv))

and dequantization is x_hat = g * (value(s) * value(code)), where
value(s) * value(code) is exact (at most 6 significant bits).  The exact binary32
operation order is this project's convention: the pages give the formula, not
the rounding sequence.
"""

from __future__ import annotations

import numpy as np

F32 = np.float32

#: magnitude of an e2m1 code's low three bits (sign is bit 3)
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
E4M3_MAX = 448.0
BLOCK = 16


def _e4m3_table() -> np.ndarray:
    """Values of the 127 non-negative finite e4m3 codes 0x00..0x7E, by code.

    Exponent field E (4 bits, bias 7), mantissa M (3 bits): E == 0 is
    subnormal M * 2**-9, otherwise (1 + M/8) * 2**(E-7).  Code 0x7F is NaN;
    E4M3FN has no infinities.
    """
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        e, m = code >> 3, code & 7
        vals[code] = m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()  # ascending in code


def _nearest_ties_even(a: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the entry of ascending ``table`` nearest to each a >= 0.

    Equal distances go to the even index (the representable value whose last
    mantissa bit is zero: in both formats the code's low bit is the mantissa's
    low bit).  Values above the last entry map to the last entry (saturation).
    """
    a = np.asarray(a, dtype=np.float64)
    hi = np.searchsorted(table, a, side="left")          # table[hi-1] < a <= table[hi]
    hi = np.minimum(hi, len(table) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = np.abs(a - table[lo])
    d_hi = np.abs(table[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    # above the largest entry the distances to the last two entries can round
    # to the same float64 (huge a): saturation decides, not the distance
    return np.where(a > table[-1], len(table) - 1, np.where(pick_hi, hi, lo))


def e2m1_value(code) -> np.ndarray:
    """Value of e2m1 codes (bit 3 sign, bits 2..0 magnitude index)."""
    code = np.asarray(code, dtype=np.int64)
    mag = E2M1_MAGNITUDES[code & 7]
    return np.where((code >> 3) & 1, -mag, mag)


def e2m1_encode(q) -> np.ndarray:
    """e2m1 code of each fp32 value: round to nearest, ties to even, saturate.

    The sign bit is the input's sign bit, so -0.0 and negative values that
    round to zero give code 0x8.  Inputs must not be NaN.
    """
    q = np.asarray(q, dtype=F32)
    mag = _nearest_ties_even(np.abs(q).astype(np.float64), E2M1_MAGNITUDES)
    return (mag | (np.signbit(q).astype(np.int64) << 3)).astype(np.uint8)


def e4m3_value(code) -> np.ndarray:
    """Value of e4m3 (FN) codes; 0x7F and 0xFF are NaN."""
    code = np.asarray(code, dtype=np.int64)
    mag_code = code & 0x7F
    mag = np.where(mag_code == 0x7F, np.nan, E4M3_VALUES[np.minimum(mag_code, 126)])
    return np.where((code >> 7) & 1, -mag, mag)


def e4m3_encode(t) -> np.ndarray:
    """e4m3 (FN) code of each fp32 value: RNE with satfinite.

    |t| >= 448 gives the largest finite code 0x7E (0xFE if negative); the sign
    bit is kept, so -0.0 gives 0x80.  Inputs must not be NaN.
    """
    t = np.asarray(t, dtype=F32)
    mag = _nearest_ties_even(np.abs(t).astype(np.float64), E4M3_VALUES)
    return (mag | (np.signbit(t).astype(np.int64) << 7)).astype(np.uint8)


def nvfp4_quantize(x, g, axis: int = -1):
    """NVFP4 block quantization of fp32 ``x`` in blocks of 16 along ``axis``.

    ``axis`` length must be a multiple of 16.  Returns ``(codes, scales)``:
    ``codes`` uint8 e2m1 codes with the shape of ``x``; ``scales`` uint8 e4m3
    codes with ``axis`` divided by 16.  ``g`` is the dequant multiplier
    (finite, > 0): the outer scale for the latent cache, the tensor-wide scale
    for prefill operands and output.
    """
    x = np.moveaxis(np.asarray(x, dtype=F32), axis, -1)
    n = x.shape[-1]
    if n % BLOCK:
        raise ValueError(f"length {n} along the block axis is not a multiple of {BLOCK}")
    xb = x.reshape(x.shape[:-1] + (n // BLOCK, BLOCK))
    codes, scales = _quantize_blocks(xb, g)
    codes = np.moveaxis(codes.reshape(x.shape), -1, axis)
    scales = np.moveaxis(scales, -1, axis)
    return codes, scales


def _quantize_blocks(xb: np.ndarray, g):
    """The quantizer on an array whose last axis is one block (any length >= 1)."""
    g = F32(g)
    a = np.max(np.abs(xb), axis=-1)                      # fp32, exact
    u = F32(F32(6.0) * g)
    t = (a / u).astype(F32)                              # IEEE fp32 division
    s = e4m3_encode(t)
    d = (e4m3_value(s).astype(F32) * g).astype(F32)
    with np.errstate(divide="ignore"):
        inv = np.where(d == 0, F32(0.0), (F32(1.0) / d)).astype(F32)
    q = (xb * inv[..., None]).astype(F32)
    return e2m1_encode(q), s


def nvfp4_quantize_ragged(x, g, axis: int = -1):
    """Blocks of 16 along ``axis`` where the last block may be shorter.

    Used for prefill V, whose blocks run along tokens from the start of each
    sequence ([MO-MLA], PR body: V is quantized along the token axis in blocks
    of 16); a sequence whose length is not a multiple of 16 ends in a short
    block whose amax is taken over the elements it has.  Returns per-element
    codes and a per-element copy of the block's scale code.
    """
    x = np.moveaxis(np.asarray(x, dtype=F32), axis, -1)
    n = x.shape[-1]
    codes = np.empty(x.shape, dtype=np.uint8)
    scl = np.empty(x.shape, dtype=np.uint8)
    for b0 in range(0, n, BLOCK):
        b1 = min(n, b0 + BLOCK)
        c, s = _quantize_blocks(x[..., b0:b1], g)
        codes[..., b0:b1] = c
        scl[..., b0:b1] = s[..., None]
    return np.moveaxis(codes, -1, axis), np.moveaxis(scl, -1, axis)


def nvfp4_dequantize(codes, scales, g, axis: int = -1) -> np.ndarray:
    """float64 x_hat = g * (scale * element) with one scale per 16 along axis."""
    codes = np.moveaxis(np.asarray(codes), axis, -1)
    scales = np.moveaxis(np.asarray(scales), axis, -1)
    s = np.repeat(e4m3_value(scales), BLOCK, axis=-1)
    return np.moveaxis(float(F32(g)) * (s * e2m1_value(codes)), -1, axis)


def nvfp4_qdq(x, g, axis: int = -1) -> np.ndarray:
    """Quantize then dequantize (fake quantization), float64 result."""
    c, s = nvfp4_quantize(x, g, axis)
    return nvfp4_dequantize(c, s, g, axis)


def nvfp4_qdq_ragged(x, g, axis: int = -1) -> np.ndarray:
    """Fake quantization with a possibly short last block (see above)."""
    c, s = nvfp4_quantize_ragged(x, g, axis)
    return float(F32(g)) * (e4m3_value(s) * e2m1_value(c))


def fp8_quantize(x, g):
    """Per-tensor FP8 quantization: one multiplier ``g`` (finite, > 0) for the
    whole tensor ([MO-MLA], commit 1: the prefill operands may be NVFP4 in
    1x16 blocks or per-tensor FP8).  The rule mirrors the NVFP4 element step:
    inv = fp32(1 / g), code = e4m3(fp32(x * inv)) (RNE, satfinite, sign kept).
    Returns the e4m3 codes."""
    g = F32(g)
    inv = (F32(1.0) / g).astype(F32)
    return e4m3_encode((np.asarray(x, dtype=F32) * inv).astype(F32))


def fp8_qdq(x, g) -> np.ndarray:
    """Per-tensor FP8 fake quantization: float64 x_hat = g * value(code)."""
    return float(F32(g)) * e4m3_value(fp8_quantize(x, g))


def f32_to_bf16_bits(x) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of fp32 values, round to nearest even
    (finite inputs)."""
    u = np.asarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to fp32."""
    bits = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (bits << 16).view(F32)

