"""NVFP4 latent cache record: pack, unpack, cache write.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[B12X], review 1 (the api.py record guard) fixes the record sizes: an NVFP4
latent record is 432 bytes with a bf16 RoPE part and 368 bytes with an fp8 RoPE
part, and any other width is an error.  [B12X], PR description: the 512-d
latent ``kv_c`` is stored as NVFP4 with a per-layer fp32 outer scale restored in
the kernel on read, and the RoPE part may be stored as fp8.  [FUSED-OUT], review
of the output view: packed e2m1 is two codes per byte.

The byte layout inside the record is this project's reading (the pages give
only the totals):

    [0, 256)     512 e2m1 codes; element 2i in the low nibble of byte i,
                 element 2i+1 in the high nibble
    [256, 288)   32 e4m3 block scales; scale j covers elements 16j..16j+15
    [288, 416)   64 bf16 RoPE values, little-endian      (432-byte record)
    [288, 352)   64 e4m3 RoPE values (RNE, satfinite, no scaling) (368-byte)
    last 16 B    reserved, written as zero

256 + 32 + 128 + 16 = 432 and 256 + 32 + 64 + 16 = 368.  The outer scale
multiplies the 512-d latent only; the RoPE part is stored unscaled.
"""

from __future__ import annotations

import numpy as np

from .formats import (F32, bf16_to_f32, e2m1_value, e4m3_encode, e4m3_value,
                      f32_to_bf16_bits, nvfp4_quantize)

D_LATENT = 512
D_ROPE = 64
CODE_BYTES = D_LATENT // 2         # 256
SCALE_BYTES = D_LATENT // 16       # 32
RESERVED_BYTES = 16
RECORD_BYTES_BF16_ROPE = CODE_BYTES + SCALE_BYTES + 2 * D_ROPE + RESERVED_BYTES  # 432
RECORD_BYTES_FP8_ROPE = CODE_BYTES + SCALE_BYTES + D_ROPE + RESERVED_BYTES       # 368


def record_bytes(rope_fp8: bool) -> int:
    return RECORD_BYTES_FP8_ROPE if rope_fp8 else RECORD_BYTES_BF16_ROPE


def rope_is_fp8(rec_bytes: int) -> bool:
    """The record width decides the RoPE storage type; other widths are errors."""
    if rec_bytes == RECORD_BYTES_FP8_ROPE:
        return True
    if rec_bytes == RECORD_BYTES_BF16_ROPE:
        return False
    raise ValueError(f"record width {rec_bytes} is neither 432 (bf16 RoPE) nor 368 (e4m3 RoPE)")


def pack_records(kv_c_bits, k_pe_bits, outer_scale, rec_bytes: int) -> np.ndarray:
    """Records for T tokens.

    ``kv_c_bits`` uint16 [T, 512] and ``k_pe_bits`` uint16 [T, 64] are bf16 bit
    patterns; ``outer_scale`` is the fp32 per-layer scale (the dequant
    multiplier of the latent).  Returns uint8 [T, rec_bytes].
    """
    fp8 = rope_is_fp8(rec_bytes)
    kv = bf16_to_f32(kv_c_bits)
    pe_bits = np.asarray(k_pe_bits, dtype=np.uint16)
    T = kv.shape[0]
    codes, scales = nvfp4_quantize(kv, outer_scale, axis=-1)     # [T,512], [T,32]
    out = np.zeros((T, rec_bytes), dtype=np.uint8)
    out[:, :CODE_BYTES] = (codes[:, 0::2] & 0xF) | ((codes[:, 1::2] & 0xF) << 4)
    out[:, CODE_BYTES:CODE_BYTES + SCALE_BYTES] = scales
    r0 = CODE_BYTES + SCALE_BYTES
    if fp8:
        out[:, r0:r0 + D_ROPE] = e4m3_encode(bf16_to_f32(pe_bits))
    else:
        out[:, r0:r0 + 2 * D_ROPE] = pe_bits.astype("<u2").view(np.uint8).reshape(T, 2 * D_ROPE)
    return out


def unpack_records(rec, outer_scale):
    """Dequantized (latent [T,512] float64 including the outer scale,
    rope [T,64] float64) from uint8 records [T, rec_bytes]."""
    rec = np.asarray(rec, dtype=np.uint8)
    fp8 = rope_is_fp8(rec.shape[-1])
    packed = rec[..., :CODE_BYTES].astype(np.int64)
    codes = np.empty(rec.shape[:-1] + (D_LATENT,), dtype=np.int64)
    codes[..., 0::2] = packed & 0xF
    codes[..., 1::2] = packed >> 4
    scales = rec[..., CODE_BYTES:CODE_BYTES + SCALE_BYTES]
    s = np.repeat(e4m3_value(scales), 16, axis=-1)
    latent = float(F32(outer_scale)) * (s * e2m1_value(codes))
    r0 = CODE_BYTES + SCALE_BYTES
    if fp8:
        rope = e4m3_value(rec[..., r0:r0 + D_ROPE]).astype(np.float64)
    else:
        bits = rec[..., r0:r0 + 2 * D_ROPE].copy().view("<u2")
        rope = bf16_to_f32(bits).astype(np.float64)
    return latent, rope


def gather_bf16(rec, outer_scale):
    """Cached-context gather: records back to the bf16 tensors a prefill over
    the cached prefix consumes ([MO-MLA], commit 2: cached-context prefill
    chunks are gathered from the quantized paged cache).  Latent element i:
    one fp32 multiply of the outer scale by the exact value s * v, then
    rounded to bf16 (nearest even).  RoPE: the stored bf16 value, or the e4m3
    value (exact in bf16).  Returns uint16 bit patterns (kv_c [T,512],
    k_pe [T,64])."""
    rec = np.asarray(rec, dtype=np.uint8)
    fp8 = rope_is_fp8(rec.shape[-1])
    packed = rec[..., :CODE_BYTES].astype(np.int64)
    codes = np.empty(rec.shape[:-1] + (D_LATENT,), dtype=np.int64)
    codes[..., 0::2] = packed & 0xF
    codes[..., 1::2] = packed >> 4
    scales = rec[..., CODE_BYTES:CODE_BYTES + SCALE_BYTES]
    sv = (np.repeat(e4m3_value(scales), 16, axis=-1) * e2m1_value(codes)).astype(F32)   # exact
    kv = f32_to_bf16_bits((F32(outer_scale) * sv).astype(F32))
    r0 = CODE_BYTES + SCALE_BYTES
    if fp8:
        pe = f32_to_bf16_bits(e4m3_value(rec[..., r0:r0 + D_ROPE]).astype(F32))
    else:
        pe = rec[..., r0:r0 + 2 * D_ROPE].copy().view("<u2").astype(np.uint16)
    return kv, pe


def cache_write(cache, kv_c_bits, k_pe_bits, slot_mapping, outer_scale) -> None:
    """In place: cache.reshape(-1, rec)[slot] = record(token) for each token
    whose slot is >= 0; every other byte of ``cache`` is left as it was.

    [MO-MLA], commits 1-2: the latent is quantized once, before the cache
    write, and decode consumes that stored representation as is.
    """
    flat = cache.reshape(-1, cache.shape[-1])
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    if not np.any(keep):
        return
    recs = pack_records(np.asarray(kv_c_bits)[keep], np.asarray(k_pe_bits)[keep],
                        outer_scale, cache.shape[-1])
    flat[slots[keep]] = recs
