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
