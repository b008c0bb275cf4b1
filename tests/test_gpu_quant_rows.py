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
