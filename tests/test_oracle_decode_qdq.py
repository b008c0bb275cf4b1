"""Pins of the oracle's decode with quantized operands: hand-worked P
schedule and V token blocks, closed forms, and reductions to plain decode."""
import math

import numpy as np
import torch

from conftest import golden_rows
from oracle import decode as D
from oracle import decode_qdq as DQ
from oracle import formats as F
from oracle import record as R


def _bits(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _raw_cache(latent, rope, page_size=64, shuffle_seed=None):
    """Raw records of one sequence in a paged cache (page table in order, or
    shuffled)."""
    L = latent.shape[0]
    n_pages = max(1, (L + page_size - 1) // page_size)
    order = np.arange(n_pages) if shuffle_seed is None else np.random.default_rng(shuffle_seed).permutation(n_pages)
    cache = np.zeros((n_pages, page_size, DQ.RAW_RECORD_BYTES), np.uint8)
    recs = DQ.raw_records(_bits(latent), _bits(rope))
    slots = D.slots_of(order, page_size, np.arange(L))
    cache.reshape(-1, DQ.RAW_RECORD_BYTES)[slots] = recs
    return cache, order[None].astype(np.int32)


def _expr(s):
    return eval(s.replace("^", "**").replace("e**", "math.e**").replace("ln(", "math.log("), {"math": math})


def _case_tokens(case, L):
    lat = np.zeros((L, 512), np.float32)
    if case == "D":
        lat[:, 0] = -1024
        lat[0, 0], lat[1, 0], lat[32, 0] = 0, -1, 1
        marks = {0: 10, 1: 11, 32: 12}
    else:
        lat[:, 0] = -1024
        lat[0, 0], lat[192, 0], lat[193, 0] = 5, 0, -1
        marks = {0: 10, 192: 11, 193: 12}
    for j, d in marks.items():
        lat[j, d] = 1
    return lat, list(marks)


def test_p_schedule_golden():
    g = float(np.float32(1 / 2688))
    for row in golden_rows("decode_qdq.txt"):
        case, ms, coef, den, lse_s = (f.strip() for f in row.split("|"))
        if case == "V":
            continue
        L = 33 if case == "D" else 300
        lat, keys = _case_tokens(case, L)
        cache, pt = _raw_cache(lat, np.zeros((L, 64)), shuffle_seed=1)
        q = np.zeros((1, 1, 576))
        q[0, 0, 0] = 1
        out, lse = DQ.decode_qdq(q[..., :512], q[..., 512:], cache, pt, [L], 64, 1.0, 1.0, DQ.FLAG_P, 1, 1, 1, g,
                                 int(ms))
        c = [_expr(x) for x in coef.split()]
        dn = _expr(den)
        # marker dims 10, 11, 12 carry the weights of the three keys
        assert np.allclose(out[0, 0, 10:13], [x * g / dn for x in c], rtol=1e-13, atol=0), row
        assert abs(lse[0, 0] - _expr(lse_s)) < 1e-12, row


def test_v_token_blocks_golden():
    row = [r for r in golden_rows("decode_qdq.txt") if r.startswith("V")][0]
    want = float(row.split("|")[2])
    lat = np.zeros((20, 512), np.float32)
    lat[:16, 0] = 6
    lat[16:, 0] = [0.1, 0.2, 0.3, 0.4]
    cache, pt = _raw_cache(lat, np.zeros((20, 64)), page_size=16, shuffle_seed=2)
    q = np.zeros((1, 1, 576))
    for ms in (1, 2, 7):
        out, lse = DQ.decode_qdq(q[..., :512], q[..., 512:], cache, pt, [20], 16, 1.0, 0.0, DQ.FLAG_V, 1, 1, 1.0,
                                 1, ms)
        assert out[0, 0, 0] == want and abs(lse[0, 0] - math.log(20)) < 1e-14


def test_split_bounds_follow_the_documented_policy():
    assert DQ.split_bounds(4096, 4) == [0, 1024, 2048, 3072, 4096]
    assert DQ.split_bounds(300, 2) == [0, 192, 300]
    assert DQ.split_bounds(257, 8) == [0, 192, 257]
    assert DQ.split_bounds(100, 8) == [0, 100]
    assert DQ.split_bounds(0, 4) == [0, 0]
    assert DQ.split_bounds(17000, 80) [:3] == [0, 256, 512] and len(DQ.split_bounds(17000, 80)) == 68


def _rand(seed, L, H, rec):
    rng = np.random.default_rng(seed)
    kv = rng.standard_normal((L, 512)).astype(np.float32)
    pe = rng.standard_normal((L, 64)).astype(np.float32)
    q = torch.tensor(rng.standard_normal((1, H, 576)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    if rec == DQ.RAW_RECORD_BYTES:
        cache, pt = _raw_cache(kv, pe, shuffle_seed=seed)
    else:
        n_pages = (L + 63) // 64
        cache = np.zeros((n_pages, 64, rec), np.uint8)
        pt = np.random.default_rng(seed).permutation(n_pages)[None].astype(np.int32)
        R.cache_write(cache, _bits(kv), _bits(pe), D.slots_of(pt[0], 64, np.arange(L)), 0.8)
    return q, cache, pt, kv, pe


def test_no_flags_is_plain_decode():
    for rec in (432, 368):
        q, cache, pt, _, _ = _rand(3, 300, 3, rec)
        a = DQ.decode_qdq(q[..., :512], q[..., 512:], cache, pt, [300], 64, 0.8, 0.05, 0, 1, 1, 1, 1, 2)
        b = D.dense_decode(q[..., :512], q[..., 512:], cache, pt, [300], 64, 0.8, 0.05)
        assert np.allclose(a[0], b[0], rtol=1e-12, atol=1e-14) and np.allclose(a[1], b[1], rtol=0, atol=1e-12)


def test_raw_cache_without_flags_is_textbook_attention():
    q, cache, pt, kv, pe = _rand(4, 150, 2, DQ.RAW_RECORD_BYTES)
    kv64 = F.bf16_to_f32(_bits(kv)).astype(np.float64)
    pe64 = F.bf16_to_f32(_bits(pe)).astype(np.float64)
    k = torch.from_numpy(np.concatenate([kv64, pe64], 1))[None, None].expand(1, 2, -1, -1)
    v = torch.from_numpy(kv64)[None, None].expand(1, 2, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q[0].astype(np.float64))[None, :, None],
                                                           k, v, scale=0.04)[0, :, 0].numpy()
    for ms in (1, 3):
        out, _ = DQ.decode_qdq(q[..., :512], q[..., 512:], cache, pt, [150], 64, 1.0, 0.04, 0, 1, 1, 1, 1, ms)
        assert np.allclose(out[0], ref, rtol=1e-11, atol=1e-13)


def test_k_quantized_on_read_matches_the_nvfp4_record():
    """Raw records with K quantized along features (NVFP4, multiplier g)
    score like NVFP4 records written with outer scale g (RoPE zero, so only
    the latent's 32 blocks are quantized): the LSE is the same."""
    rng = np.random.default_rng(5)
    L, g = 200, 0.6
    kv = rng.standard_normal((L, 512)).astype(np.float32)
    pe = np.zeros((L, 64), np.float32)
    raw, pt = _raw_cache(kv, pe, shuffle_seed=5)
    nv = np.zeros((raw.shape[0], 64, 432), np.uint8)
    R.cache_write(nv, _bits(kv), _bits(pe), D.slots_of(pt[0], 64, np.arange(L)), g)
    q = torch.tensor(rng.standard_normal((1, 2, 576)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    _, l1 = DQ.decode_qdq(q[..., :512], q[..., 512:], raw, pt, [L], 64, 1.0, 0.07, DQ.FLAG_K, 1, g, 1, 1, 1)
    _, l2 = D.dense_decode(q[..., :512], q[..., 512:], nv, pt, [L], 64, g, 0.07)
    assert np.allclose(l1, l2, rtol=0, atol=1e-12)


def test_q_quantization_closed_form():
    """One token: lse = z = softmax_scale * q_hat . k.  The first block of q
    is the hand-derived NVFP4 block [6, 3, -1.5, 0.2] -> [6, 3, -1.5, 0]."""
    lat = np.zeros((1, 512), np.float32)
    lat[0, :4] = [1, 10, 100, 1000]
    cache, pt = _raw_cache(lat, np.zeros((1, 64)))
    q = np.zeros((1, 1, 576))
    q[0, 0, :4] = [6, 3, -1.5, 0.2]
    _, lse = DQ.decode_qdq(q[..., :512], q[..., 512:], cache, pt, [1], 64, 1.0, 0.5, DQ.FLAG_Q, 1.0, 1, 1, 1, 1)
    assert lse[0, 0] == 0.5 * (6 + 30 - 150 + 0)
    _, lse = DQ.decode_qdq(q[..., :512], q[..., 512:], cache, pt, [1], 64, 1.0, 0.5, 0, 1.0, 1, 1, 1, 1)
    assert abs(lse[0, 0] - 0.5 * (6 + 30 - 150 + 1000 * 0.2)) < 1e-12


def test_without_p_the_chunks_do_not_matter():
    q, cache, pt, _, _ = _rand(6, 700, 2, DQ.RAW_RECORD_BYTES)
    fl = DQ.FLAG_Q | DQ.FLAG_K | DQ.FLAG_V | DQ.FP8_K
    ref = DQ.decode_qdq(q[..., :512], q[..., 512:], cache, pt, [700], 64, 1.0, 0.05, fl, 0.003, 0.01, 0.002, 1, 1)
    for ms in (2, 3, 8):
        o, l = DQ.decode_qdq(q[..., :512], q[..., 512:], cache, pt, [700], 64, 1.0, 0.05, fl, 0.003, 0.01, 0.002, 1,
                             ms)
        assert np.allclose(o, ref[0], rtol=1e-11, atol=1e-13) and np.allclose(l, ref[1], rtol=0, atol=1e-12)


def test_empty_sequence():
    q, cache, pt, _, _ = _rand(7, 64, 2, DQ.RAW_RECORD_BYTES)
    o, l = DQ.decode_qdq(q[..., :512], q[..., 512:], cache, pt, [0], 64, 1.0, 0.05, 15, 0.01, 0.01, 0.01,
                         float(np.float32(1 / 2688)), 4)
    assert np.all(o == 0) and np.all(np.isneginf(l))
