"""GPU parity: NVFP4 row quantization with swizzled scales, bit for bit."""
import numpy as np
import pytest
import torch

from mla_attention_nvfp4_amd import ops
from oracle import swizzle as S

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,g", [(1, 16, 1.0), (130, 64, 0.01), (257, 2048, 1 / 2688), (128, 16384, 0.003)])
def test_quantize_rows_bit_exact(M, K, g):
    rng = np.random.default_rng(M + K)
    x = (rng.standard_normal((M, K)) * rng.uniform(0.01, 30, (M, 1))).astype(np.float32)
    x[0, :16] = 0.0                      # an all-zero block
    if K >= 32:
        x[0, 16:32] = [6, 3, -1.5, 0.2] + [0] * 12
    codes, scales = ops.quantize_rows(torch.from_numpy(x).cuda(), g)
    torch.cuda.synchronize()
    want_codes, want_scales = S.quantize_rows(x, g)
    assert np.array_equal(codes.cpu().numpy(), want_codes)
    assert np.array_equal(scales.cpu().numpy(), want_scales)


def _scale_sweep_amax(n_blocks: int, seed: int) -> np.ndarray:
    """Block maxima that probe the e4m3 rounding of the block scale: every
    positive e4m3 value and every midpoint between neighbours (the ties),
    each with its fp32 neighbours two ulps either side, values above the
    e4m3 maximum 448, and random values over [0, 500] and [2^-12, 500]."""
    from oracle import formats as F
    vals = np.sort(np.unique(F.e4m3_value(np.arange(0, 0x7F)).astype(np.float64)))
    mids = (vals[:-1] + vals[1:]) / 2
    base = np.concatenate([vals, mids, [448.0, 449.0, 464.0, 480.0, 1e4, 3.4e38]]).astype(np.float32)
    pts = [base]
    for d in (1, 2):
        up, dn = base.copy(), base.copy()
        for _ in range(d):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(0))
        pts += [up, dn]
    rng = np.random.default_rng(seed)
    fixed = np.concatenate(pts)
    rest = n_blocks - fixed.size
    rand = np.concatenate([rng.uniform(0, 500, rest // 2),
                           np.exp2(rng.uniform(-12, np.log2(500), rest - rest // 2))]).astype(np.float32)
    amax = np.concatenate([fixed, rand])[:n_blocks]
    assert amax.size == n_blocks and np.all(amax >= 0)
    return amax


def test_quantize_rows_scale_rounding_sweep():
    """With g = fp32(1/6), 6g rounds to 1 in fp32, so a block's scale code is
    the e4m3 rounding of its maximum itself: a dense sweep of maxima (ties
    and their neighbours included) checks the block-scale encoding bit for
    bit, codes and swizzled scales, against the oracle."""
    M, K = 256, 2048
    amax = _scale_sweep_amax(M * K // 16, 7)
    rng = np.random.default_rng(8)
    frac = rng.uniform(-1, 1, (amax.size, 16)).astype(np.float32)
    frac[:, 0] = 1.0
    blocks = (frac * amax[:, None]).astype(np.float32)
    blocks[:, 0] = amax                      # the exact maximum
    x = blocks.reshape(M, K)
    g = float(np.float32(1 / 6))
    assert np.float32(6) * np.float32(g) == np.float32(1.0)
    codes, scales = ops.quantize_rows(torch.from_numpy(x).cuda(), g)
    torch.cuda.synchronize()
    want_codes, want_scales = S.quantize_rows(x, g)
    assert np.array_equal(scales.cpu().numpy(), want_scales)
    assert np.array_equal(codes.cpu().numpy(), want_codes)


def test_quantize_rows_scale_quotient_sweep():
    """The scale quotient t = a / (6 g) is formed as a * fp32(1 / (6 g)) with
    the division redone near e4m3 rounding ties (the P blocks of the prefill
    form it the same way).  With g = fp32(1/2688), the P multiplier, 6g is not
    a power of two and the product can differ from the quotient in its last
    bits.  The block maxima here put the quotient on every e4m3 value and
    every midpoint between neighbours, and up to 6 fp32 ulps of the maximum
    either side, plus the subnormal range and saturation: codes and swizzled
    scales must equal the oracle's (true division) bit for bit."""
    from oracle import formats as F
    g32 = np.float32(1 / 2688)
    u = np.float32(np.float32(6) * g32)
    vals = np.sort(np.unique(F.e4m3_value(np.arange(0, 0x7F)).astype(np.float64)))
    ties = np.concatenate([vals, (vals[:-1] + vals[1:]) / 2, [448.0, 464.0, 2.0 ** -10, 3 * 2.0 ** -11]])
    a0 = (ties * np.float64(u)).astype(np.float32)
    pts = [a0]
    up, dn = a0.copy(), a0.copy()
    for _ in range(6):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(0))
        pts += [up.copy(), dn.copy()]
    amax = np.concatenate(pts)
    M, K = 64, (amax.size + 63) // 64 * 16
    rng = np.random.default_rng(9)
    amax = np.concatenate([amax, rng.uniform(0, 1.2, M * K // 16 - amax.size).astype(np.float32)])
    frac = rng.uniform(-1, 1, (amax.size, 16)).astype(np.float32)
    blocks = (frac * amax[:, None]).astype(np.float32)
    blocks[:, 0] = amax
    x = blocks.reshape(M, K)
    # the fixture holds blocks where the plain product a * fp32(1/u) would
    # take another scale code than the quotient: those the redo must fix
    inv_u = np.float32(np.float32(1) / u)
    differs = F.e4m3_encode((amax * inv_u).astype(np.float32)) != F.e4m3_encode((amax / u).astype(np.float32))
    assert int(differs.sum()) >= 20
    codes, scales = ops.quantize_rows(torch.from_numpy(x).cuda(), float(g32))
    torch.cuda.synchronize()
    want_codes, want_scales = S.quantize_rows(x, float(g32))
    assert np.array_equal(scales.cpu().numpy(), want_scales)
    assert np.array_equal(codes.cpu().numpy(), want_codes)
