"""Pins of the oracle's prefill: textbook attention, schedule-free operand
quantization, hand-worked P quantization under the tile schedule, output."""
import math

import numpy as np
import torch

from oracle import formats as F
from oracle import prefill as P
from oracle import swizzle as S


def _bf16_f32(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def _inputs(rng, lens, H):
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q = _bf16_f32(rng.standard_normal((T, H, 192)))
    k = _bf16_f32(rng.standard_normal((T, H, 192)))
    v = _bf16_f32(rng.standard_normal((T, H, 128)))
    return q, k, v, cu


def _sdpa_causal(q, k, v, scale):
    # one sequence, [L, H, d] float64 -> [L, H, dv]
    qq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    kk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    vv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True, scale=scale)
    return o[0].numpy().transpose(1, 0, 2)


def _lse_causal(q, k, scale):
    z = scale * np.einsum("ihd,jhd->hij", q, k)
    L = z.shape[1]
    z = np.where(np.tril(np.ones((L, L), bool))[None], z, -np.inf)
    m = z.max(-1, keepdims=True)
    return (m + np.log(np.exp(z - m).sum(-1, keepdims=True)))[..., 0].T


def test_no_quantization_is_textbook_causal_attention():
    rng = np.random.default_rng(30)
    q, k, v, cu = _inputs(rng, [1, 70, 130, 0, 17], 2)
    O, lse = P.prefill(q, k, v, cu, 0.09, 0, 1, 1, 1, 1)
    for a, b in zip(cu[:-1], cu[1:]):
        if b == a:
            continue
        ref = _sdpa_causal(q[a:b].astype(np.float64), k[a:b].astype(np.float64),
                           v[a:b].astype(np.float64), 0.09)
        assert np.allclose(O[a:b], ref, rtol=1e-11, atol=1e-12)
        assert np.allclose(lse[a:b], _lse_causal(q[a:b].astype(np.float64), k[a:b].astype(np.float64), 0.09),
                           rtol=0, atol=1e-11)


def test_operand_quantization_is_schedule_free():
    """Q/K/V flags only: textbook attention on the fake-quantized operands,
    whatever the tile schedule."""
    rng = np.random.default_rng(31)
    q, k, v, cu = _inputs(rng, [150, 33], 2)
    gq, gk, gv = (float(np.float32(np.abs(t).max() / 2688)) for t in (q, k, v))
    O, lse = P.prefill(q, k, v, cu, 0.07, P.FLAG_Q | P.FLAG_K | P.FLAG_V, gq, gk, gv, 1)
    for a, b in zip(cu[:-1], cu[1:]):
        qh = F.nvfp4_qdq(q[a:b], gq)
        kh = F.nvfp4_qdq(k[a:b], gk)
        vh = F.nvfp4_qdq_ragged(v[a:b], gv, axis=0)
        ref = _sdpa_causal(qh, kh, vh, 0.07)
        assert np.allclose(O[a:b], ref, rtol=1e-11, atol=1e-12)
        assert np.allclose(lse[a:b], _lse_causal(qh, kh, 0.07), rtol=0, atol=1e-11)


def _p_case(L, kz, vsel):
    q = np.zeros((L, 1, 192), np.float32)
    q[:, 0, 0] = 1
    k = np.zeros((L, 1, 192), np.float32)
    k[:, 0, 0] = kz
    v = np.zeros((L, 1, 128), np.float32)
    for j, c in vsel.items():
        v[j, 0, c] = 1
    return q, k, v


def test_p_quantization_hand_worked_single_tile():
    """tests/golden/prefill_p_schedule.txt, case A."""
    g = float(np.float32(1 / 2688))
    q, k, v = _p_case(2, [0, -1], {0: 0, 1: 1})
    O, lse = P.prefill(q, k, v, [0, 2], 1.0, P.FLAG_P, 1, 1, 1, g)
    l = 1 + math.exp(-1)
    assert np.allclose(O[1, 0, :3], [2688 * g / l, 896 * g / l, 0], rtol=1e-14, atol=0)
    assert abs(lse[1, 0] - math.log(l)) < 1e-14
    assert np.allclose(O[0, 0, :2], [2688 * g, 0], rtol=1e-14) and lse[0, 0] == 0


def test_p_quantization_hand_worked_running_max():
    """tests/golden/prefill_p_schedule.txt, case B: the running max changes
    at the second 64-key tile."""
    g = float(np.float32(1 / 2688))
    kz = np.full(65, -1024.0)
    kz[0], kz[1], kz[64] = 0, -1, 1
    q, k, v = _p_case(65, kz, {0: 0, 1: 1, 64: 2})
    O, lse = P.prefill(q, k, v, [0, 65], 1.0, P.FLAG_P, 1, 1, 1, g, rows_of=lambda n, L: [64])
    e1, e2 = math.exp(-1), math.exp(-2)
    l = 1 + e1 + e2
    assert np.allclose(O[64, 0, :3], [2688 * g * e1 / l, 896 * g * e1 / l, 2688 * g / l], rtol=1e-13, atol=0)
    assert abs(lse[64, 0] - (1 + math.log(l))) < 1e-13


def test_row_subsets_and_head_subsets_agree_with_full():
    rng = np.random.default_rng(32)
    q, k, v, cu = _inputs(rng, [140, 70], 3)
    args = (cu, 0.08, 15, 0.002, 0.002, 0.002, 1 / 2688)
    O, lse = P.prefill(q, k, v, *args)
    O2, lse2 = P.prefill(q, k, v, *args, heads=[2, 0], rows_of=lambda n, L: [0, L - 1, 64, 65])
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        for r in (0, b - a - 1, 64, 65):
            for h in (0, 2):
                assert np.allclose(O[a + r, h], O2[a + r, h], rtol=1e-12, atol=1e-13)
                assert abs(lse[a + r, h] - lse2[a + r, h]) < 1e-12
    assert np.all(np.isnan(O2[:, 1]))


def test_output_quantization_layout():
    rng = np.random.default_rng(33)
    O = rng.standard_normal((131, 2, 128))
    packed, buf = P.output_nvfp4_swizzled(O, 0.003)
    assert packed.shape == (131, 2, 64) and buf.size == 256 * 16
    sf = S.unswizzle(buf, 131, 16)
    for t in (0, 77, 130):
        for h in (0, 1):
            c, s = F.nvfp4_quantize(O[t, h].astype(np.float32), 0.003)
            assert np.array_equal(S.unpack_codes(packed[t, h]), c)
            assert np.array_equal(sf[t, 8 * h:8 * h + 8], s)
