"""Pins of the oracle's page walk and of its sparse multiset reading.

The slots come from hand-worked rows (``golden/page_walk.txt``), and the cache
records are built byte by byte here, not through the oracle's packer: slot s
holds a record whose latent block j is 6 when bit j of (s + 1) is set and 0
otherwise (codes 0x77 with scale 0x38 = 1.0, or codes 0x00 with scale 0x00),
with a zero RoPE part.  A decode of one token then returns that token's latent
exactly, which names the slot the oracle read.
"""
import math

import numpy as np

from conftest import golden_rows
from oracle import decode as D
from oracle import record as R

REC = 432


def _walks():
    out = []
    for row in golden_rows("page_walk.txt"):
        ps, pt, pos, slots = (f.split() for f in row.split("|"))
        out.append((int(ps[0]), np.array(pt, np.int32), np.array(pos, np.int64), np.array(slots, np.int64)))
    return out


def _latent_of_slot(s):
    bits = np.array([((s + 1) >> j) & 1 for j in range(32)], np.float64)
    return np.repeat(6.0 * bits, 16)


def _record_of_slot(s):
    rec = np.zeros(REC, np.uint8)
    for j in range(32):
        if ((s + 1) >> j) & 1:
            rec[8 * j:8 * j + 8] = 0x77       # 16 codes of value 6
            rec[256 + j] = 0x38               # e4m3 1.0
    return rec


def _cache(page_size, n_pages):
    cache = np.zeros((n_pages, page_size, REC), np.uint8)
    flat = cache.reshape(-1, REC)
    for s in range(flat.shape[0]):
        flat[s] = _record_of_slot(s)
    return cache


def test_slots_of_golden():
    for ps, pt, pos, slots in _walks():
        assert np.array_equal(D.slots_of(pt, ps, pos), slots), (ps, pt, pos)


def test_hand_built_record_decodes_to_its_pattern():
    lat, rope = R.unpack_records(_record_of_slot(12)[None], 1.0)
    assert np.array_equal(lat[0], _latent_of_slot(12)) and not rope.any()


def test_single_token_reads_the_golden_slot():
    """Sparse decode with one index returns the latent of exactly the slot
    the hand-worked walk names (closed form L = 1: out = v, lse = z)."""
    for ps, pt, pos, slots in _walks():
        cache = _cache(ps, int(pt.max()) + 1)
        q = np.zeros((1, 2, 576))
        q[0, 1, :512] = 1.0
        L = int(pos.max()) + 1
        for j, s in zip(pos, slots):
            out, lse = D.sparse_decode(q[..., :512], q[..., 512:], cache, pt[None], [L], ps, 1.0, 0.5,
                                       np.array([[j]]))
            want = _latent_of_slot(int(s))
            assert np.array_equal(out[0, 0], want) and np.array_equal(out[0, 1], want), (ps, j, s)
            assert lse[0, 0] == 0.0 and lse[0, 1] == 0.5 * want.sum(), (ps, j, s)


def test_dense_walks_every_golden_slot():
    """Dense decode over positions 0..L-1 of a golden row listing all of them,
    with softmax_scale = 0: out is the mean latent of the listed slots and
    lse = ln L."""
    for ps, pt, pos, slots in _walks():
        if not np.array_equal(pos, np.arange(pos.size)):
            continue
        cache = _cache(ps, int(pt.max()) + 1)
        q = np.ones((1, 1, 576))
        out, lse = D.dense_decode(q[..., :512], q[..., 512:], cache, pt[None], [pos.size], ps, 1.0, 0.0)
        want = np.mean([_latent_of_slot(int(s)) for s in slots], axis=0)
        assert np.allclose(out[0, 0], want, rtol=0, atol=1e-13), (ps, pt)
        assert abs(lse[0, 0] - math.log(pos.size)) < 1e-14


def test_sparse_duplicate_index_counts_twice():
    """A valid position listed twice is two members of the attended multiset
    ([B12X] walkthrough: top-k indices select tokens; the reading of a repeat
    is this project's, stated in the oracle).  Indices [a, a, b] weigh token a
    2:1 against token b."""
    ps, pt = 4, np.array([3, 0, 2], np.int32)
    cache = _cache(ps, 4)
    a, b = 5, 9                               # slots 1 and 9 (golden row 1)
    va, vb = _latent_of_slot(1), _latent_of_slot(9)
    q = np.zeros((1, 1, 576))
    # softmax_scale = 0: out = (2 va + vb) / 3, lse = ln 3
    out, lse = D.sparse_decode(q[..., :512], q[..., 512:], cache, pt[None], [12], ps, 1.0, 0.0,
                               np.array([[a, -1, a, b, 40]]))
    assert np.allclose(out[0, 0], (2 * va + vb) / 3, rtol=0, atol=1e-13)
    assert abs(lse[0, 0] - math.log(3)) < 1e-14
    # with scores: q_nope = 1, softmax_scale = 1/96, so z = 6 * 16 * popcount / 96 = popcount(slot + 1)
    q[0, 0, :512] = 1.0
    za, zb = bin(1 + 1).count("1"), bin(9 + 1).count("1")     # 1 and 2
    out, lse = D.sparse_decode(q[..., :512], q[..., 512:], cache, pt[None], [12], ps, 1.0, 1.0 / 96,
                               np.array([[b, a, a]]))
    den = 2 * math.exp(za) + math.exp(zb)
    assert np.allclose(out[0, 0], (2 * math.exp(za) * va + math.exp(zb) * vb) / den, rtol=1e-14, atol=1e-14)
    assert abs(lse[0, 0] - math.log(den)) < 1e-13
