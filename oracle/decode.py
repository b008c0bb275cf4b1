"""Absorbed MLA decode over the paged NVFP4 latent cache: dense, sparse, merge.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed ([MO-MLA], commit 1 and PR body; [B12X], walkthrough and
sequence diagram): one query token per sequence and H query heads share one
latent (absorbed MQA).  For sequence b with L = seq_lens[b] tokens and query
head h, each cached token j < L contributes

    k_j = s_l * dequant(latent part of record j)     (512-d; s_l = outer scale)
    r_j = RoPE part of record j                      (64-d, bf16 or e4m3)
    z_j = softmax_scale * (q_nope . k_j + q_rope . r_j)
    v_j = k_j                                        (V is the latent itself:
                                                      [MO-MLA], commit 3)

    out = sum_j e^(z_j - m) v_j / sum_j e^(z_j - m),  m = max_j z_j
    lse = m + ln sum_j e^(z_j - m)                   (natural log, so that
                                                      chunks merge: [MO-MLA],
                                                      commit 1)

Record j of sequence b sits at slot page_table[b][j // P] * P + j % P of the
cache viewed as [slots, record_bytes].  L = 0 gives out = 0 and lse = -inf.
The query is bf16 and is used unquantized ([B12X], review 2: the NVFP4 path
stages Q as bf16 with no Q quantization).  All arithmetic here is float64.
"""

from __future__ import annotations

import numpy as np

from .record import D_LATENT, unpack_records


def slots_of(page_table_row, page_size: int, positions) -> np.ndarray:
    """Cache slots of logical token positions of one sequence."""
    pos = np.asarray(positions, dtype=np.int64)
    pages = np.asarray(page_table_row, dtype=np.int64)[pos // page_size]
    return pages * page_size + pos % page_size


def attend(q_nope, q_rope, latent, rope, softmax_scale):
    """Softmax attention of H query rows over N tokens (float64).

    q_nope [H,512], q_rope [H,64], latent [N,512] (outer scale included),
    rope [N,64].  Returns out [H,512], lse [H].
    """
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    H = q_nope.shape[0]
    if latent.shape[0] == 0:
        return np.zeros((H, D_LATENT)), np.full(H, -np.inf)
    z = float(softmax_scale) * (q_nope @ latent.T + q_rope @ rope.T)     # [H, N]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e @ latent) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def tokens_of(cache, page_table_row, page_size, positions, outer_scale):
    """Dequantized (latent, rope) of the given logical positions."""
    flat = np.asarray(cache).reshape(-1, cache.shape[-1])
    recs = flat[slots_of(page_table_row, page_size, positions)]
    return unpack_records(recs, outer_scale)


def dense_decode(q_nope, q_rope, cache, page_table, seq_lens, page_size,
                 outer_scale, softmax_scale, batch=None):
    """out [B,H,512], lse [B,H] (float64).  ``batch`` restricts the work to a
    subset of sequences; other rows are NaN."""
    q_nope = np.asarray(q_nope, dtype=np.float64)
    B, H = q_nope.shape[:2]
    out = np.full((B, H, D_LATENT), np.nan)
    lse = np.full((B, H), np.nan)
    for b in (range(B) if batch is None else batch):
        L = int(seq_lens[b])
        lat, rope = tokens_of(cache, page_table[b], page_size, np.arange(L), outer_scale)
        out[b], lse[b] = attend(q_nope[b], q_rope[b], lat, rope, softmax_scale)
    return out, lse


def sparse_decode(q_nope, q_rope, cache, page_table, seq_lens, page_size,
                  outer_scale, softmax_scale, indices, batch=None):
    """Top-k sparse decode ([B12X], walkthrough: sparse MLA decode on the NVFP4
    cache).  indices [B, topk] are logical positions of sequence b, shared by
    all heads; an entry < 0 or >= seq_lens[b] is masked.  The attended set is
    the multiset of valid entries (a duplicate counts twice).  No valid entry
    gives out = 0, lse = -inf."""
    q_nope = np.asarray(q_nope, dtype=np.float64)
    B, H = q_nope.shape[:2]
    out = np.full((B, H, D_LATENT), np.nan)
    lse = np.full((B, H), np.nan)
    for b in (range(B) if batch is None else batch):
        L = int(seq_lens[b])
        idx = np.asarray(indices[b], dtype=np.int64)
        pos = idx[(idx >= 0) & (idx < L)]
        lat, rope = tokens_of(cache, page_table[b], page_size, pos, outer_scale)
        out[b], lse[b] = attend(q_nope[b], q_rope[b], lat, rope, softmax_scale)
    return out, lse


def lse_merge(partial_out, partial_lse):
    """Merge S partial results of disjoint token sets ([MO-MLA], commit 1:
    split-K decode with a natural-log LSE used to merge chunks).

    partial_out [S,...,D], partial_lse [S,...].  With M = max_s lse_s:
    w_s = e^(lse_s - M), out = sum_s w_s out_s / sum_s w_s,
    lse = M + ln sum_s w_s; all lse_s = -inf gives (0, -inf).
    """
    po = np.asarray(partial_out, dtype=np.float64)
    pl = np.asarray(partial_lse, dtype=np.float64)
    M = pl.max(axis=0)
    empty = np.isneginf(M)
    Msafe = np.where(empty, 0.0, M)
    w = np.where(np.isneginf(pl), 0.0, np.exp(pl - Msafe))
    wsum = w.sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = (w[..., None] * np.where(np.isneginf(pl)[..., None], 0.0, po)).sum(axis=0) \
            / wsum[..., None]
        lse = Msafe + np.log(wsum)
    out = np.where(empty[..., None], 0.0, out)
    lse = np.where(empty, -np.inf, lse)
    return out, lse


def split_decode(q_nope, q_rope, cache, page_table_row, page_size, outer_scale,
                 softmax_scale, bounds):
    """Partial results of one sequence over contiguous chunks
    [bounds[s], bounds[s+1]): returns (out [S,H,512], lse [S,H])."""
    outs, lses = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        lat, rope = tokens_of(cache, page_table_row, page_size, np.arange(a, b), outer_scale)
        o, l = attend(q_nope, q_rope, lat, rope, softmax_scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)
