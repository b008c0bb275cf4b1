"""Pins of the oracle's number formats and NVFP4 block quantizer.

Each check ties the oracle to something other than itself: hand-derived tables
(tests/golden), exhaustive round trips of every code, brute-force nearest-value
search, PyTorch's own float8_e4m3fn conversion, and closed-form properties.
"""
import math

import numpy as np
import pytest
import torch

from conftest import golden_rows
from oracle import formats as F


def test_e2m1_golden_table():
    for row in golden_rows("e2m1_encode.txt"):
        val, code = row.split()[:2]
        got = int(F.e2m1_encode(np.float32(float(val))))
        assert got == int(code, 16), (val, hex(got), code)


def test_e2m1_all_codes_round_trip():
    codes = np.arange(16)
    vals = F.e2m1_value(codes)
    # -0.0 must keep its sign bit so that code 0x8 survives the round trip
    vals = np.where(codes == 8, -0.0, vals).astype(np.float32)
    assert np.array_equal(F.e2m1_encode(vals), codes.astype(np.uint8))


def test_e2m1_matches_brute_force():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-8, 8, 20000), rng.uniform(-1, 1, 20000),
                        np.arange(-7, 7.01, 0.125)]).astype(np.float32)
    mags = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    for v in x:
        a = abs(float(v))
        dist = [abs(a - m) for m in mags]
        best = min(dist)
        cands = [i for i, dd in enumerate(dist) if dd == best]
        mag = [c for c in cands if c % 2 == 0][0] if len(cands) > 1 else cands[0]
        want = mag | (8 if math.copysign(1.0, float(v)) < 0 else 0)
        assert int(F.e2m1_encode(v)) == want, v


def test_e4m3_golden_table():
    for row in golden_rows("e4m3_encode.txt"):
        val, code = row.split()[:2]
        got = int(F.e4m3_encode(np.float32(float(val))))
        assert got == int(code, 16), (val, hex(got), code)


def test_e4m3_all_finite_codes_round_trip():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert codes.size == 254
    vals = F.e4m3_value(codes).astype(np.float32)
    vals = np.where(codes == 0x80, np.float32(-0.0), vals)
    assert np.array_equal(F.e4m3_encode(vals), codes.astype(np.uint8))
    assert np.isnan(F.e4m3_value(0x7F)) and np.isnan(F.e4m3_value(0xFF))


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = F.e4m3_value(np.arange(256))
    both_nan = np.isnan(ref) & np.isnan(mine)
    assert np.array_equal(np.where(both_nan, 0, ref), np.where(both_nan, 0, mine))


def test_e4m3_encode_matches_torch_in_range():
    """PyTorch rounds to nearest even inside the finite range; beyond it the
    two conventions differ (torch gives NaN, the quantizer saturates)."""
    rng = np.random.default_rng(1)
    vals = F.E4M3_VALUES
    mids = (vals[1:] + vals[:-1]) / 2
    x = np.concatenate([rng.uniform(0, 448, 50000), np.exp(rng.uniform(-12, 6, 50000)),
                        mids, vals, -vals]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_encode(x), ref)


def _block_rows():
    for row in golden_rows("nvfp4_blocks.txt"):
        g, xs, sc, packed, deq = [c.strip() for c in row.split("|")]
        x = np.zeros(16, np.float32)
        xv = [float(t) for t in xs.split()]
        x[: len(xv)] = xv
        yield (float(g), x, int(sc, 16), [int(b, 16) for b in packed.split()],
               [float(t) for t in deq.split()])


def test_nvfp4_golden_blocks():
    n = 0
    for g, x, sc, packed, deq in _block_rows():
        codes, scales = F.nvfp4_quantize(x, g)
        assert int(scales[0]) == sc, (x, hex(int(scales[0])))
        got = [int(codes[0] | (codes[1] << 4)), int(codes[2] | (codes[3] << 4))]
        assert got == packed, (x, [hex(b) for b in got])
        xh = F.nvfp4_dequantize(codes, scales, g)
        assert np.array_equal(xh[: len(deq)], np.array(deq)), (x, xh[: len(deq)])
        n += 1
    assert n == 8


def test_scale_times_element_exact_in_bf16():
    """Every e4m3 scale times every e2m1 value is a bf16 number, so a kernel
    can dequantize to bf16 MFMA operands without rounding."""
    s = F.E4M3_VALUES[1:]
    prod = (s[:, None] * F.E2M1_MAGNITUDES[None, :]).ravel()
    as_bf16 = torch.from_numpy(prod).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(as_bf16, prod)


def test_quantizer_error_bound_and_range():
    """Closed-form properties of the rule: when the scale does not saturate,
    each element is within one unit of d = g*value(s) (the widest gap between
    adjacent e2m1 magnitudes, 4 to 6, is 2) and the block amax lands on 4 or 6."""
    rng = np.random.default_rng(2)
    for g in (1.0, 0.7, 1.9, 1 / 2688):
        x = (rng.standard_normal((4000, 16)) * rng.uniform(0.01, 50, (4000, 1)) * g).astype(np.float32)
        codes, s = F.nvfp4_quantize(x, g)
        s = s[:, 0]
        d = F.e4m3_value(s) * np.float32(g)
        xh = F.nvfp4_dequantize(codes, s[:, None], g)
        ok = (F.e4m3_value(s) < 448) & (F.e4m3_value(s) > 2 ** -6)
        err = np.abs(xh - x) / d[:, None]
        assert np.all(err[ok] <= 1.0 + 1e-6)
        amax_code = np.take_along_axis(codes & 7, np.argmax(np.abs(x), axis=1)[:, None], 1)[:, 0]
        assert np.all(np.isin(amax_code[ok], [6, 7]))


def test_quantizer_block_independence_and_axis():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 64)).astype(np.float32)
    c_all, s_all = F.nvfp4_quantize(x, 1.0)
    for j in range(4):
        c, s = F.nvfp4_quantize(x[:, 16 * j:16 * j + 16], 1.0)
        assert np.array_equal(c, c_all[:, 16 * j:16 * j + 16]) and np.array_equal(s[:, 0], s_all[:, j])
    c_t, s_t = F.nvfp4_quantize(x.T.copy(), 1.0, axis=0)
    assert np.array_equal(c_t.T, c_all) and np.array_equal(s_t.T, s_all)


def test_ragged_blocks_equal_zero_padded():
    """A short last block quantizes like a block padded with zeros."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((21, 5)).astype(np.float32)
    got = F.nvfp4_qdq_ragged(x, 0.5, axis=0)
    pad = np.zeros((32, 5), np.float32)
    pad[:21] = x
    want = F.nvfp4_qdq(pad, 0.5, axis=0)[:21]
    assert np.array_equal(got, want)


def test_encoders_saturate_far_above_range():
    """Satfinite far above the largest magnitude (the quantizer reaches such
    element values when a block's scale saturates at 448): e2m1 gives +-6
    (codes 7 and 15), e4m3 gives +-448 (0x7E and 0xFE), for every float32
    exponent above the range, up to the largest finite float32."""
    big = np.float32(2.0) ** np.arange(3, 128, dtype=np.float32)
    big = np.concatenate([big, [np.finfo(np.float32).max, np.float32(4.5535715e36)]]).astype(np.float32)
    assert np.all(F.e2m1_encode(big) == 7)
    assert np.all(F.e2m1_encode(-big) == 15)
    big4 = big[big > 448]
    assert np.all(F.e4m3_encode(big4) == 0x7E)
    assert np.all(F.e4m3_encode(-big4) == 0xFE)
