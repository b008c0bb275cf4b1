"""Pins of the oracle's per-tensor FP8 operands, 2:4 score sparsity, context
attention over a cached prefix, the chunked-prefill merge and the cached-context
gather: hand-worked values, brute force, textbook attention and invariants."""
import itertools
import math

import numpy as np
import torch

from conftest import golden_rows
from oracle import formats as F
from oracle import prefill as P
from oracle import record as R


def _bf16_f32(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def _sdpa(q, k, v, scale, mask=None):
    """q [Lq,H,d], k [Lk,H,d], v [Lk,H,dv] float64; mask [Lq,Lk] bool or None."""
    qq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    kk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    vv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=m, scale=scale)
    return o[0].numpy().transpose(1, 0, 2)


def _lse(q, k, scale, mask=None):
    z = scale * np.einsum("ihd,jhd->hij", q, k)
    if mask is not None:
        z = np.where(mask[None], z, -np.inf)
    m = z.max(-1, keepdims=True)
    return (m + np.log(np.exp(z - m).sum(-1, keepdims=True)))[..., 0].T


# ------------------------------------------------------------------ FP8 --

def test_fp8_qdq_golden():
    for row in golden_rows("fp8_qdq.txt"):
        g, x, code, want = (f.strip() for f in row.split("|"))
        c = F.fp8_quantize(np.float32(float(x)), float(g))
        assert int(c) == int(code, 16), row
        xh = F.fp8_qdq(np.float32(float(x)), float(g))
        assert xh == float(want) and np.signbit(xh) == np.signbit(float(want)), row


def test_fp8_qdq_round_trips_representable_values_and_bounds_error():
    g = np.float32(0.75)
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    vals = (F.e4m3_value(codes) * np.float64(g)).astype(np.float32)
    # x = g * value is representable: with inv = fp32(1/g) the product may be
    # off by an ulp, but never by half an e4m3 step
    assert np.array_equal(F.fp8_qdq(vals, g), float(g) * F.e4m3_value(codes))
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(10000) * 50).astype(np.float32)
    err = np.abs(F.fp8_qdq(x, g) - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, float(g) * 2.0 ** -10) * 1.0001)


def test_fp8_operands_are_schedule_free_textbook_attention():
    """Q, K, V per-tensor FP8 only: textbook causal attention on the fake-
    quantized operands."""
    rng = np.random.default_rng(2)
    lens = [70, 130]
    T = sum(lens)
    cu = [0, 70, 200]
    q = _bf16_f32(rng.standard_normal((T, 2, 192)))
    k = _bf16_f32(rng.standard_normal((T, 2, 192)))
    v = _bf16_f32(rng.standard_normal((T, 2, 128)))
    g = [float(np.float32(np.abs(t).max() / 448)) for t in (q, k, v)]
    flags = P.FLAG_Q | P.FLAG_K | P.FLAG_V | P.FP8_Q | P.FP8_K | P.FP8_V
    O, lse = P.prefill(q, k, v, cu, 0.07, flags, *g, 1.0)
    qh, kh, vh = (F.fp8_qdq(t, gg) for t, gg in zip((q, k, v), g))
    for a, b in zip(cu[:-1], cu[1:]):
        L = b - a
        mask = np.tril(np.ones((L, L), bool))
        assert np.allclose(O[a:b], _sdpa(qh[a:b], kh[a:b], vh[a:b], 0.07, mask), rtol=1e-11, atol=1e-12)
        assert np.allclose(lse[a:b], _lse(qh[a:b], kh[a:b], 0.07, mask), rtol=0, atol=1e-11)


def test_fp8_p_hand_worked_case_c():
    """tests/golden/prefill_p_schedule.txt, case C (P as per-tensor FP8)."""
    g = float(np.float32(1 / 448))
    q = np.zeros((2, 1, 192), np.float32)
    q[:, 0, 0] = 1
    k = np.zeros((2, 1, 192), np.float32)
    k[:, 0, 0] = [0, -1]
    v = np.zeros((2, 1, 128), np.float32)
    v[0, 0, 0] = v[1, 0, 1] = 1
    O, lse = P.prefill(q, k, v, [0, 2], 1.0, P.FLAG_P | P.FP8_P, 1, 1, 1, g)
    l = 1 + math.exp(-1)
    assert np.allclose(O[1, 0, :3], [448 * g / l, 160 * g / l, 0], rtol=1e-14, atol=0)
    assert abs(lse[1, 0] - math.log(l)) < 1e-14
    assert np.allclose(O[0, 0, :2], [448 * g, 0], rtol=1e-14) and lse[0, 0] == 0


# ------------------------------------------------------------------ 2:4 --

def test_keep_2_4_golden():
    for row in golden_rows("sparse_2_4.txt"):
        sc, va, kept = (f.split() for f in row.split("|"))
        got = P.keep_2_4(np.array([[float(x) for x in sc]]), np.array([[x == "1" for x in va]]))
        assert sorted(np.nonzero(got[0])[0].tolist()) == [int(x) for x in kept], row


def _brute_keep(z, valid):
    keep = np.zeros(z.shape, bool)
    for r in range(z.shape[0]):
        for g0 in range(0, z.shape[1], 4):
            cand = [j for j in range(g0, g0 + 4) if valid[r, j]]
            # sort by (score descending, index ascending); the first two valid keys
            cand.sort(key=lambda j: (-z[r, j], j))
            for j in cand[:2]:
                keep[r, j] = True
    return keep


def test_keep_2_4_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(50):
        z = rng.integers(-3, 4, (5, 16)).astype(np.float64)       # many ties
        valid = rng.uniform(size=(5, 16)) < 0.8
        assert np.array_equal(P.keep_2_4(z, valid), _brute_keep(z, valid))


def test_sparse_2_4_no_quantization_is_masked_textbook_attention():
    """Flags 2:4 only: causal attention with the 2:4 mask chosen by brute force
    on the exact scores (fp64 SDPA with that mask)."""
    rng = np.random.default_rng(4)
    lens = [1, 3, 70, 133]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    # a coarse grid keeps every score exact and produces ties
    q = (rng.integers(-2, 3, (T, 2, 192)) / 4.0).astype(np.float32)
    k = (rng.integers(-2, 3, (T, 2, 192)) / 4.0).astype(np.float32)
    v = _bf16_f32(rng.standard_normal((T, 2, 128)))
    O, lse = P.prefill(q, k, v, cu, 0.05, P.SPARSE_2_4, 1, 1, 1, 1)
    for a, b in zip(cu[:-1], cu[1:]):
        L = int(b - a)
        n4 = (L + 3) // 4 * 4
        for h in range(2):
            z = np.zeros((L, n4))
            z[:, :L] = q[a:b, h].astype(np.float64) @ k[a:b, h].astype(np.float64).T
            causal = np.arange(n4)[None, :] <= np.arange(L)[:, None]
            mask = _brute_keep(z, causal)[:, :L]
            qh, kh, vh = (t[a:b, h:h + 1].astype(np.float64) for t in (q, k, v))
            assert np.allclose(O[a:b, h:h + 1], _sdpa(qh, kh, vh, 0.05, mask), rtol=1e-11, atol=1e-12)
            assert np.allclose(lse[a:b, h:h + 1], _lse(qh, kh, 0.05, mask), rtol=0, atol=1e-11)
            # two keys per full group, and the diagonal group keeps min(2, unmasked)
            kept = mask.sum(1)
            full = np.arange(L) // 4 * 2 + np.minimum(np.arange(L) % 4 + 1, 2)
            assert np.array_equal(kept, full)


def test_sparse_2_4_with_zero_softmax_scale_keeps_the_first_two_of_each_group():
    rng = np.random.default_rng(5)
    q = _bf16_f32(rng.standard_normal((9, 1, 192)))
    k = _bf16_f32(rng.standard_normal((9, 1, 192)))
    v = _bf16_f32(rng.standard_normal((9, 1, 128)))
    O, lse = P.prefill(q, k, v, [0, 9], 0.0, P.SPARSE_2_4, 1, 1, 1, 1)
    # row 8 keeps keys 0, 1, 4, 5, 8: the mean of those V rows
    assert np.allclose(O[8, 0], v[[0, 1, 4, 5, 8], 0].astype(np.float64).mean(0), rtol=1e-13, atol=1e-14)
    assert abs(lse[8, 0] - math.log(5)) < 1e-14


def test_sparse_2_4_decision_ignores_tensor_multipliers():
    """With Q and K quantized, the decision is the one on the unscaled
    operand values: scaling both global multipliers by powers of two (which
    scales every quantized value exactly) changes nothing but the scores."""
    rng = np.random.default_rng(6)
    q = _bf16_f32(rng.standard_normal((40, 1, 192)))
    k = _bf16_f32(rng.standard_normal((40, 1, 192)))
    v = _bf16_f32(rng.standard_normal((40, 1, 128)))
    fl = P.FLAG_Q | P.FLAG_K | P.SPARSE_2_4
    gq, gk = float(np.float32(np.abs(q).max() / 2688)), float(np.float32(np.abs(k).max() / 2688))
    O1, l1 = P.prefill(q, k, v, [0, 40], 0.1, fl, gq, gk, 1, 1)
    O2, l2 = P.prefill(q * 4, k * 8, v, [0, 40], 0.1 / 32, fl, gq * 4, gk * 8, 1, 1)
    assert np.allclose(O1, O2, rtol=1e-12, atol=1e-13) and np.allclose(l1, l2, rtol=0, atol=1e-12)


# ----------------------------------------------------- context attention --

def _ctx_inputs(rng, new_lens, ctx_lens, H=2):
    cu_q = np.concatenate([[0], np.cumsum(new_lens)]).astype(np.int64)
    cu_c = np.concatenate([[0], np.cumsum(ctx_lens)]).astype(np.int64)
    Tq, Tc = int(cu_q[-1]), int(cu_c[-1])
    q = _bf16_f32(rng.standard_normal((Tq, H, 192)))
    k = _bf16_f32(rng.standard_normal((Tq, H, 192)))
    v = _bf16_f32(rng.standard_normal((Tq, H, 128)))
    ck = _bf16_f32(rng.standard_normal((Tc, H, 192)))
    cv = _bf16_f32(rng.standard_normal((Tc, H, 128)))
    return q, k, v, cu_q, ck, cv, cu_c


def test_context_attention_is_textbook_unmasked_attention():
    rng = np.random.default_rng(7)
    q, _, _, cu_q, ck, cv, cu_c = _ctx_inputs(rng, [5, 40, 3], [100, 1, 0])
    O, lse = P.attention(q, ck, cv, cu_q, cu_c, 0.08, 0, 1, 1, 1, 1, False)
    for n in range(3):
        a, b, ca, cb = cu_q[n], cu_q[n + 1], cu_c[n], cu_c[n + 1]
        if cb == ca:       # no context: zero output, lse -inf
            assert np.all(O[a:b] == 0) and np.all(np.isneginf(lse[a:b]))
            continue
        qh, kh, vh = (t.astype(np.float64) for t in (q[a:b], ck[ca:cb], cv[ca:cb]))
        assert np.allclose(O[a:b], _sdpa(qh, kh, vh, 0.08), rtol=1e-11, atol=1e-12)
        assert np.allclose(lse[a:b], _lse(qh, kh, 0.08), rtol=0, atol=1e-11)


def test_chunked_prefill_merge_equals_attention_over_the_whole_sequence():
    """Without quantization, the LSE merge of the context part and the causal
    new-token part is causal attention over context followed by the new tokens
    (new token i sees the whole context and new tokens 0..i)."""
    rng = np.random.default_rng(8)
    q, k, v, cu_q, ck, cv, cu_c = _ctx_inputs(rng, [30, 7, 12], [50, 130, 0])
    O, lse = P.chunked_prefill(q, k, v, cu_q, ck, cv, cu_c, 0.06, 0, 1, 1, 1, 1)
    for n in range(3):
        a, b, ca, cb = cu_q[n], cu_q[n + 1], cu_c[n], cu_c[n + 1]
        C, L = int(cb - ca), int(b - a)
        kk = np.concatenate([ck[ca:cb], k[a:b]]).astype(np.float64)
        vv = np.concatenate([cv[ca:cb], v[a:b]]).astype(np.float64)
        mask = np.arange(C + L)[None, :] <= (C + np.arange(L))[:, None]
        qh = q[a:b].astype(np.float64)
        assert np.allclose(O[a:b], _sdpa(qh, kk, vv, 0.06, mask), rtol=1e-11, atol=1e-12)
        assert np.allclose(lse[a:b], _lse(qh, kk, 0.06, mask), rtol=0, atol=1e-11)


def test_chunked_prefill_with_operand_quantization_equals_one_pass():
    """Q/K/V quantized (schedule-free) and a context of whole 16-token blocks:
    V's token blocks then fall the same in the context, the new tokens and
    their concatenation, so the chunked result is the single causal prefill
    over the concatenated sequence, restricted to the new rows."""
    rng = np.random.default_rng(9)
    q, k, v, cu_q, ck, cv, cu_c = _ctx_inputs(rng, [20, 33], [64, 112])
    fl = P.FLAG_Q | P.FLAG_K | P.FLAG_V
    g = (0.002, 0.003, 0.0021)
    O, lse = P.chunked_prefill(q, k, v, cu_q, ck, cv, cu_c, 0.07, fl, *g, 1.0)
    for n in range(2):
        a, b, ca, cb = cu_q[n], cu_q[n + 1], cu_c[n], cu_c[n + 1]
        C, L = int(cb - ca), int(b - a)
        qq = np.concatenate([np.zeros((C, 2, 192), np.float32), q[a:b]])
        kk = np.concatenate([ck[ca:cb], k[a:b]])
        vv = np.concatenate([cv[ca:cb], v[a:b]])
        Of, lf = P.prefill(qq, kk, vv, [0, C + L], 0.07, fl, *g, 1.0, rows_of=lambda n_, L_: np.arange(C, C + L))
        assert np.allclose(O[a:b], Of[C:], rtol=1e-11, atol=1e-12)
        assert np.allclose(lse[a:b], lf[C:], rtol=0, atol=1e-11)


# ------------------------------------------------------------ gather --

def test_gather_golden():
    for row in golden_rows("gather_bf16.txt"):
        f = [x.strip() for x in row.split("|")]
        if f[0] == "ROPE":
            rec = np.zeros((1, 368), np.uint8)
            rec[0, 288] = int(f[1], 16)
            _, pe = R.gather_bf16(rec, 1.0)
            assert int(pe[0, 0]) == int(f[2], 16), row
            continue
        rec = np.zeros((1, 432), np.uint8)
        rec[0, 256] = int(f[1], 16)
        rec[0, 0] = int(f[2], 16)
        kv, _ = R.gather_bf16(rec, float(f[0]))
        want = [int(x, 16) for x in f[3].split()]
        assert [int(kv[0, 0]), int(kv[0, 1])] == want, row


def test_gather_rounds_the_dequantized_latent_once():
    """With a power-of-two outer scale the gather is exact (the dequantized
    latent itself); otherwise within half a bf16 ulp of the fp32 product; the
    bf16 RoPE part is copied bit for bit."""
    rng = np.random.default_rng(10)
    kv = torch.from_numpy(rng.standard_normal((20, 512)).astype(np.float32)).to(torch.bfloat16)
    pe = torch.from_numpy(rng.standard_normal((20, 64)).astype(np.float32)).to(torch.bfloat16)
    kvb = kv.view(torch.int16).numpy().view(np.uint16)
    peb = pe.view(torch.int16).numpy().view(np.uint16)
    for g in (0.5, 2.0, 0.7, 1.37):
        rec = R.pack_records(kvb, peb, g, 432)
        lat, _ = R.unpack_records(rec, g)
        gk, gp = R.gather_bf16(rec, g)
        got = F.bf16_to_f32(gk).astype(np.float64)
        if g in (0.5, 2.0):
            assert np.array_equal(got, lat)
        else:
            assert np.all(np.abs(got - lat) <= np.abs(lat) * 2.0 ** -8 + 1e-30)
        assert np.array_equal(gp, peb)
