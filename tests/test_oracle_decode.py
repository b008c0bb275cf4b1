"""Pins of the oracle's decode: library attention, closed forms, invariants."""
import math

import numpy as np
import scipy.special
import torch

from conftest import golden_rows
from oracle import decode as D
from oracle import record as R


def _bf16(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16)


def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def _setup(rng, B, H, L_max, page_size, rec_bytes, s_l, n_pages_extra=3, shuffle=True):
    pages_per_seq = (L_max + page_size - 1) // page_size
    n_pages = B * pages_per_seq + n_pages_extra
    perm = rng.permutation(n_pages) if shuffle else np.arange(n_pages)
    page_table = perm[: B * pages_per_seq].reshape(B, pages_per_seq).astype(np.int32)
    cache = np.zeros((n_pages, page_size, rec_bytes), np.uint8)
    kv = _bf16(rng.standard_normal((B, pages_per_seq * page_size, 512)))
    pe = _bf16(rng.standard_normal((B, pages_per_seq * page_size, 64)))
    for b in range(B):
        slots = D.slots_of(page_table[b], page_size, np.arange(pages_per_seq * page_size))
        R.cache_write(cache, _bits(kv[b]), _bits(pe[b]), slots, s_l)
    q = _bf16(rng.standard_normal((B, H, 576))).to(torch.float32).numpy()
    return cache, page_table, q


def test_dense_matches_torch_sdpa_on_decoded_tokens():
    rng = np.random.default_rng(10)
    for rec in (432, 368):
        cache, pt, q = _setup(rng, 2, 3, 5, 2, rec, 0.75)
        seq = np.array([5, 3])
        out, lse = D.dense_decode(q[..., :512], q[..., 512:], cache, pt, seq, 2, 0.75, 0.11)
        for b in range(2):
            lat, rope = D.tokens_of(cache, pt[b], 2, np.arange(seq[b]), 0.75)
            k = torch.from_numpy(np.concatenate([lat, rope], 1))[None, None]
            v = torch.from_numpy(lat)[None, None]
            qq = torch.from_numpy(q[b].astype(np.float64))[None, :, None, :]
            ref = torch.nn.functional.scaled_dot_product_attention(
                qq, k.expand(1, 3, -1, -1), v.expand(1, 3, -1, -1), scale=0.11)[0, :, 0]
            assert np.allclose(out[b], ref.numpy(), rtol=1e-12, atol=1e-12)
            z = 0.11 * (q[b].astype(np.float64) @ np.concatenate([lat, rope], 1).T)
            assert np.allclose(lse[b], scipy.special.logsumexp(z, axis=1), rtol=0, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(11)
    cache, pt, q = _setup(rng, 1, 4, 64, 64, 432, 1.5)
    # L = 1: out is the single latent, lse its score
    out, lse = D.dense_decode(q[..., :512], q[..., 512:], cache, pt, [1], 64, 1.5, 0.3)
    lat, rope = D.tokens_of(cache, pt[0], 64, [0], 1.5)
    assert np.allclose(out[0], np.broadcast_to(lat[0], (4, 512)), rtol=0, atol=0)
    z0 = 0.3 * (q[0, :, :512].astype(np.float64) @ lat[0] + q[0, :, 512:].astype(np.float64) @ rope[0])
    assert np.allclose(lse[0], z0, rtol=1e-14, atol=1e-14)
    # softmax_scale = 0: uniform average and lse = ln L
    out, lse = D.dense_decode(q[..., :512], q[..., 512:], cache, pt, [40], 64, 1.5, 0.0)
    lat, _ = D.tokens_of(cache, pt[0], 64, np.arange(40), 1.5)
    assert np.allclose(out[0], lat.mean(0), rtol=1e-12, atol=1e-14)
    assert np.allclose(lse[0], math.log(40), rtol=0, atol=1e-14)
    # q = 0 gives equal scores too
    z = np.zeros_like(q)
    out, lse = D.dense_decode(z[..., :512], z[..., 512:], cache, pt, [7], 64, 1.5, 1.0)
    lat, _ = D.tokens_of(cache, pt[0], 64, np.arange(7), 1.5)
    assert np.allclose(out[0], lat.mean(0), rtol=1e-12, atol=1e-14)
    # L = 0: zero output, lse = -inf
    out, lse = D.dense_decode(q[..., :512], q[..., 512:], cache, pt, [0], 64, 1.5, 1.0)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))


def test_outer_scale_enters_latent_only():
    """The outer scale multiplies the stored latent on read ([B12X], PR
    description: restored in-kernel on read) and not the RoPE part: reading
    the same records with twice the outer scale and half the softmax scale,
    with q_rope = 0, repeats the weights and doubles out; with q_nope = 0 the
    scores ignore the outer scale."""
    rng = np.random.default_rng(12)
    kv = _bf16(rng.standard_normal((64, 512)))
    pe = _bf16(rng.standard_normal((64, 64)))
    c = np.zeros((1, 64, 432), np.uint8)
    R.cache_write(c, _bits(kv), _bits(pe), np.arange(64), 0.5)
    q = _bf16(rng.standard_normal((1, 2, 576))).to(torch.float32).numpy()
    pt = np.zeros((1, 1), np.int32)
    qn = q.copy()
    qn[..., 512:] = 0
    o1, l1 = D.dense_decode(qn[..., :512], qn[..., 512:], c, pt, [64], 64, 0.5, 0.2)
    o2, l2 = D.dense_decode(qn[..., :512], qn[..., 512:], c, pt, [64], 64, 1.0, 0.1)
    assert np.allclose(2 * o1, o2, rtol=1e-12, atol=1e-14)
    assert np.allclose(l1, l2, rtol=1e-13, atol=1e-13)
    qr = q.copy()
    qr[..., :512] = 0
    o1, l1 = D.dense_decode(qr[..., :512], qr[..., 512:], c, pt, [64], 64, 0.5, 0.2)
    o2, l2 = D.dense_decode(qr[..., :512], qr[..., 512:], c, pt, [64], 64, 1.0, 0.2)
    assert np.allclose(2 * o1, o2, rtol=1e-12, atol=1e-14)
    assert np.array_equal(l1, l2)


def test_paging_is_transparent():
    rng = np.random.default_rng(13)
    cache, pt, q = _setup(rng, 2, 2, 150, 16, 368, 1.0)
    seq = np.array([150, 77])
    out, lse = D.dense_decode(q[..., :512], q[..., 512:], cache, pt, seq, 16, 1.0, 0.05)
    for b in range(2):
        flat = cache.reshape(-1, 368)
        slots = D.slots_of(pt[b], 16, np.arange(seq[b]))
        linear = np.zeros((1, 160, 368), np.uint8)
        linear[0, : seq[b]] = flat[slots]
        o2, l2 = D.dense_decode(q[b:b + 1, :, :512], q[b:b + 1, :, 512:], linear,
                                np.zeros((1, 1), np.int32), [seq[b]], 160, 1.0, 0.05)
        assert np.array_equal(out[b], o2[0]) and np.array_equal(lse[b], l2[0])


def test_merge_golden():
    for row in golden_rows("merge.txt"):
        parts = [p.split() for p in row.split(";")]
        pairs = [(float(a), float(b)) for a, b in parts[:-2]]
        want_o, want_l = float(parts[-2][0]), float(parts[-1][0])
        po = np.array([[p[1]] for p in pairs])          # [S, 1]
        pl = np.array([p[0] for p in pairs])            # [S]
        o, l = D.lse_merge(po, pl)
        assert abs(o[0] - want_o) < 1e-12, row
        assert (np.isneginf(l) and np.isneginf(want_l)) or abs(l - want_l) < 1e-12, row


def test_split_merge_equals_single_pass():
    rng = np.random.default_rng(14)
    cache, pt, q = _setup(rng, 1, 3, 300, 64, 432, 0.9)
    out, lse = D.dense_decode(q[..., :512], q[..., 512:], cache, pt, [300], 64, 0.9, 0.07)
    for _ in range(5):
        cuts = np.sort(rng.integers(0, 301, rng.integers(1, 6)))
        bounds = [0, *cuts.tolist(), 300]                 # may contain empty chunks
        po, pl = D.split_decode(q[0, :, :512], q[0, :, 512:], cache, pt[0], 64, 0.9, 0.07, bounds)
        o, l = D.lse_merge(po, pl)
        assert np.allclose(o, out[0], rtol=1e-12, atol=1e-14)
        assert np.allclose(l, lse[0], rtol=1e-13, atol=1e-13)


def test_sparse_pins():
    rng = np.random.default_rng(15)
    cache, pt, q = _setup(rng, 2, 2, 200, 64, 432, 1.25)
    seq = np.array([200, 130])
    dense, dl = D.dense_decode(q[..., :512], q[..., 512:], cache, pt, seq, 64, 1.25, 0.04)
    # all positions, in order and permuted, with masked entries mixed in
    idx = np.full((2, 260), -1, np.int64)
    idx[0, :200] = np.arange(200)
    idx[1, :130] = rng.permutation(130)
    idx[1, 130:140] = [130, 131, 199, 500, -7, 10**6, 130, 150, 199, -1]   # all >= L or < 0
    for b in range(2):
        idx[b] = idx[b][rng.permutation(260)]
    out, lse = D.sparse_decode(q[..., :512], q[..., 512:], cache, pt, seq, 64, 1.25, 0.04, idx)
    assert np.allclose(out, dense, rtol=1e-12, atol=1e-14)
    assert np.allclose(lse, dl, rtol=1e-13, atol=1e-13)
    # a subset equals dense decode over exactly those tokens, gathered by hand
    sub = np.array([[5, 77, 3, 190, -1, 64]])
    out, lse = D.sparse_decode(q[:1, :, :512], q[:1, :, 512:], cache, pt[:1], seq[:1], 64, 1.25, 0.04, sub)
    lat, rope = D.tokens_of(cache, pt[0], 64, [5, 77, 3, 190, 64], 1.25)
    o2, l2 = D.attend(q[0, :, :512], q[0, :, 512:], lat, rope, 0.04)
    assert np.allclose(out[0], o2, rtol=1e-13) and np.allclose(lse[0], l2, rtol=1e-13)
    # nothing valid
    out, lse = D.sparse_decode(q[:1, :, :512], q[:1, :, 512:], cache, pt[:1], seq[:1], 64, 1.25, 0.04,
                               np.full((1, 8), -1))
    assert np.all(out == 0) and np.all(np.isneginf(lse))
