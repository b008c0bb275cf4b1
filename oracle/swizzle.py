"""NVFP4 output quantization and the 128x4-swizzled block-scale layout.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[FUSED-OUT], PR description: the prefill writes its output as packed e2m1 codes,
an fp32 global scale, and e4m3 block scales laid out in the 128x4-swizzled
layout that the NVFP4 GEMMs consume; the buffer's 128-row tiles belong to one
producer.  The page names the layout only; its index formula below is the
public block-scale layout of those GEMM libraries, restated:

A logical scale matrix SF[M, C] (row m = output row, column c = block of 16
along the row) is stored in tiles of 128 rows x 4 columns, 512 bytes each,
tiles ordered row-tile major.  Inside a tile, entry (m, c) sits at
(m % 32) * 16 + ((m % 128) // 32) * 4 + (c % 4).  So

    offset(m, c) = ((m // 128) * (C' // 4) + c // 4) * 512
                   + (m % 32) * 16 + ((m % 128) // 32) * 4 + c % 4

with C' = C rounded up to a multiple of 4.  The buffer has ceil(M/128)*128*C'
bytes; entries of padding rows and columns are zero.
"""

from __future__ import annotations

import numpy as np

from .formats import F32, nvfp4_quantize


def padded_cols(C: int) -> int:
    return (C + 3) // 4 * 4


def buffer_bytes(M: int, C: int) -> int:
    return (M + 127) // 128 * 128 * padded_cols(C)


def swizzled_offset(m, c, C: int):
    m = np.asarray(m, dtype=np.int64)
    c = np.asarray(c, dtype=np.int64)
    return ((m // 128) * (padded_cols(C) // 4) + c // 4) * 512 \
        + (m % 32) * 16 + ((m % 128) // 32) * 4 + c % 4


def swizzle(sf) -> np.ndarray:
    """Byte buffer holding SF[M, C] (uint8) in the swizzled layout."""
    sf = np.asarray(sf, dtype=np.uint8)
    M, C = sf.shape
    buf = np.zeros(buffer_bytes(M, C), dtype=np.uint8)
    mm, cc = np.meshgrid(np.arange(M), np.arange(C), indexing="ij")
    buf[swizzled_offset(mm, cc, C)] = sf
    return buf


def unswizzle(buf, M: int, C: int) -> np.ndarray:
    mm, cc = np.meshgrid(np.arange(M), np.arange(C), indexing="ij")
    return np.asarray(buf, dtype=np.uint8)[swizzled_offset(mm, cc, C)]


def pack_codes(codes) -> np.ndarray:
    """Two e2m1 codes per byte along the last axis, element 2i in the low
    nibble ([FUSED-OUT], review of the output view: packed e2m1, two per byte)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return ((codes[..., 0::2] & 0xF) | ((codes[..., 1::2] & 0xF) << 4)).astype(np.uint8)


def unpack_codes(packed) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def quantize_rows(x, global_scale):
    """NVFP4 quantization of fp32 rows x [M, K] (K a multiple of 16) with the
    fp32 global scale as dequant multiplier: returns (packed codes [M, K/2],
    swizzled scale buffer)."""
    x = np.asarray(x, dtype=F32)
    codes, sf = nvfp4_quantize(x, global_scale, axis=-1)
    return pack_codes(codes), swizzle(sf)
