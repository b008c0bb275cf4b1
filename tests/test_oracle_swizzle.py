"""Pins of the oracle's 128x4 block-scale swizzle and row quantizer."""
import numpy as np

from conftest import golden_rows
from oracle import formats as F
from oracle import swizzle as S


def test_swizzle_golden_offsets():
    for row in golden_rows("swizzle.txt"):
        m, c, C, off = (int(t) for t in row.split()[:4])
        assert int(S.swizzled_offset(m, c, C)) == off, row


def test_swizzle_is_a_bijection_onto_tiles():
    for M, C in ((1, 4), (128, 8), (200, 1024), (257, 6), (129, 3)):
        mm, cc = np.meshgrid(np.arange(M), np.arange(C), indexing="ij")
        off = S.swizzled_offset(mm, cc, C).ravel()
        assert len(np.unique(off)) == M * C
        assert off.min() >= 0 and off.max() < S.buffer_bytes(M, C)
        # each 512-byte tile holds 128 rows x 4 columns of one row tile
        tile = off // 512
        assert np.array_equal(tile, ((mm // 128) * (S.padded_cols(C) // 4) + cc // 4).ravel())


def test_swizzle_round_trip_and_zero_padding():
    rng = np.random.default_rng(20)
    sf = rng.integers(1, 256, (150, 10), dtype=np.uint8)
    buf = S.swizzle(sf)
    assert buf.size == 256 * 12
    assert np.array_equal(S.unswizzle(buf, 150, 10), sf)
    used = np.zeros(buf.size, bool)
    mm, cc = np.meshgrid(np.arange(150), np.arange(10), indexing="ij")
    used[S.swizzled_offset(mm, cc, 10)] = True
    assert not buf[~used].any() and used.sum() == 1500


def test_quantize_rows_is_blockwise_nvfp4():
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((130, 64)) * 3).astype(np.float32)
    packed, buf = S.quantize_rows(x, 0.01)
    codes = S.unpack_codes(packed)
    sf = S.unswizzle(buf, 130, 4)
    for i in range(130):
        c, s = F.nvfp4_quantize(x[i], 0.01)
        assert np.array_equal(codes[i], c) and np.array_equal(sf[i], s)
    # hand example: first block of row 0 as in the golden block table
    y = np.zeros((1, 32), np.float32)
    y[0, :4] = [6, 3, -1.5, 0.2]
    packed, buf = S.quantize_rows(y, 1.0)
    assert list(packed[0, :2]) == [0x57, 0x0B]
    assert buf[0] == 0x38 and buf.size == 128 * 4
