"""Varlen MLA prefill with NVFP4 or FP8 fake quantization, optional 2:4 score
sparsity, chunked-context attention, and NVFP4 output.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[MO-MLA], commit 1 and PR body: varlen prefill with asymmetric head dims
(qk 192 = 128 nope + 64 rope, v 128), each attention matmul operand
fake-quantized once along its own contraction axis, as NVFP4 1x16 blocks or
as per-tensor FP8: Q and K along the head dim, V along tokens, P along keys
after the softmax row-sum, the softmax denominator itself unquantized;
token-exact N:M score sparsity on the new-token attention; natural-log LSE,
which merges a chunk of new tokens with the cached-context chunks.
[FUSED-OUT], PR description: the output is written directly as NVFP4 with a
128x4-swizzled scale buffer and an fp32 global scale (``swizzle.py``); the
fusion is limited to batches without cached context.

The algorithm, per sequence n with query rows r in [cu_q[n], cu_q[n+1])
(local index i) and key rows in [cu_k[n], cu_k[n+1]) (local index j), and
head h:

1. Operand quantization, each switched by a flag bit (Q=1, K=2, P=4, V=8),
   with the format bit (Q=16, K=32, P=64, V=128) choosing per-tensor FP8
   instead of NVFP4:
   Q_hat, K_hat = block QDQ along d with multipliers g_q, g_k;
   V_hat = block QDQ along local key position (blocks [16k, 16k+16), the last
   one possibly short) per head and dim, multiplier g_v.
2. z_ij = softmax_scale * Q_hat_i . K_hat_j.  Causal attention (queries and
   keys are the same rows): keys j <= i.  Context attention (queries are new
   tokens, keys the cached prefix): every key.
   2:4 sparsity (bit 256): in each group of 4 keys starting at a local key
   index divisible by 4, the 2 largest scores of the row are kept and the
   others masked; a masked key counts as -inf, and of equal scores the lower
   key index ranks first.
3. Keys are taken in tiles of BN_P = 64 from j = 0 upward.  Start m = -inf,
   l = 0, acc = 0.  Per tile: m' = max(m, max of the tile's unmasked z);
   alpha = e^(m - m') (0 while m = -inf); p_j = e^(z_ij - m') on unmasked keys,
   0 on masked ones; l <- alpha*l + sum p  (unquantized); p_hat = QDQ of
   fp32(p) with multiplier g_p (NVFP4: blocks along keys aligned to the local
   key index, masked zeros included; FP8: per element); acc <- alpha*acc +
   sum_j p_hat_j V_hat_j; m <- m'.
4. O_i = acc / l,  LSE_i = m + ln l.

Step 3's tile width is a convention of this project: [MO-MLA], commit 1, says
its golden oracles replicate the kernel schedules, and P's quantization depends
on the running maximum the kernel holds when it quantizes, so the schedule is
part of the definition.  The running maximum is refreshed at every 64-key tile
and the accumulator always rescaled.  With the P flag off the schedule drops
out and step 3 is textbook softmax attention.

The 2:4 decision compares exact scores: the dot products are taken on the
operands without their tensor-wide multipliers (values that float64 holds
and sums exactly here), since those multipliers and softmax_scale > 0 are
common to a row; softmax_scale = 0 makes every score equal.
"""

from __future__ import annotations

import numpy as np

from .decode import lse_merge
from .formats import F32, fp8_qdq, nvfp4_qdq, nvfp4_qdq_ragged
from .swizzle import pack_codes, swizzle
from .formats import nvfp4_quantize

BN_P = 64
D_QK = 192
D_V = 128
FLAG_Q, FLAG_K, FLAG_P, FLAG_V = 1, 2, 4, 8
FP8_Q, FP8_K, FP8_P, FP8_V = 16, 32, 64, 128
SPARSE_2_4 = 256


def _qdq(x, flags, on, fp8, g, axis=-1):
    if not flags & on:
        return x.astype(np.float64)
    return fp8_qdq(x, g) if flags & fp8 else nvfp4_qdq(x, g, axis=axis)


def operand_multipliers(flags, g_q, g_k):
    """The tensor-wide multipliers inside Q_hat and K_hat (1 when raw)."""
    return (float(F32(g_q)) if flags & FLAG_Q else 1.0), (float(F32(g_k)) if flags & FLAG_K else 1.0)


def quantize_q(q, flags, g_q, heads=None):
    """Q_hat [T, len(heads), 192] (float64): along d, NVFP4 or FP8."""
    heads = np.arange(q.shape[1]) if heads is None else np.asarray(heads)
    return _qdq(np.asarray(q, dtype=F32)[:, heads], flags, FLAG_Q, FP8_Q, g_q)


def quantize_kv(k, v, cu_k, flags, g_k, g_v, heads=None):
    """(K_hat [T,.,192], V_hat [T,.,128]) float64: K along d; V along the
    local key position of each sequence of ``cu_k`` (NVFP4 blocks of 16 from
    the sequence's first row, the last possibly short) or per-tensor FP8."""
    heads = np.arange(k.shape[1]) if heads is None else np.asarray(heads)
    ks = np.asarray(k, dtype=F32)[:, heads]
    vs = np.asarray(v, dtype=F32)[:, heads]
    kh = _qdq(ks, flags, FLAG_K, FP8_K, g_k)
    if flags & FLAG_V and flags & FP8_V:
        vh = fp8_qdq(vs, g_v)
    elif flags & FLAG_V:
        vh = np.empty(vs.shape, dtype=np.float64)
        for a, b in zip(cu_k[:-1], cu_k[1:]):
            if b > a:
                vh[a:b] = nvfp4_qdq_ragged(vs[a:b], g_v, axis=0)
    else:
        vh = vs.astype(np.float64)
    return kh, vh


def quantize_operands(q, k, v, cu_seqlens, flags, g_q, g_k, g_v, heads=None):
    """Step 1 for the given heads of a causal prefill (queries and keys are
    the same rows): (Q_hat, K_hat, V_hat) as float64 arrays [T, len(heads), d]."""
    kh, vh = quantize_kv(k, v, cu_seqlens, flags, g_k, g_v, heads)
    return quantize_q(q, flags, g_q, heads), kh, vh


def keep_2_4(score, valid):
    """Step 2's 2:4 selection on one tile of rows: ``score`` [R, n] exact
    scores, ``valid`` [R, n] unmasked keys, n a multiple of 4 (groups of 4
    consecutive keys from key 0).  Returns the kept-key mask: in each group
    the two highest-ranked keys, ranking masked keys as -inf and equal
    scores by lower key index."""
    R, n = score.shape
    z = np.where(valid, score, -np.inf).reshape(R, n // 4, 4)
    # rank of key a in its group: keys that beat it (higher, or equal and earlier)
    beats = (z[..., None, :] > z[..., :, None])
    earlier = np.arange(4)[None, :] < np.arange(4)[:, None]          # [a, b]: b < a
    beats |= (z[..., None, :] == z[..., :, None]) & earlier
    rank = beats.sum(axis=-1)
    return (rank < 2).reshape(R, n) & valid


def attend_rows(qh, kh, vh, rows, softmax_scale, quantize_p, g_p, p_quantizer=None, *,
                causal=True, sparse_2_4=False, p_fp8=False, multipliers=(1.0, 1.0), keep_fn=None):
    """Steps 2-4 for one sequence and one head.

    qh [Lq,192], kh [Lk,192], vh [Lk,128] (this sequence, float64); ``rows``
    local query indices.  Causal: key j is seen by row i when j <= i (queries
    and keys are the same rows); otherwise every key is.  Returns
    O [len(rows),128], LSE [len(rows)].

    ``multipliers`` are the tensor-wide factors inside qh and kh (the 2:4
    decision uses qh/g_q . kh/g_k, which recovers the exact operand values).
    ``p_quantizer(p32, t0)``, if given, replaces step 3's P QDQ for the tile
    starting at key t0 (p32: the tile's fp32 probabilities [R, 64]); it lets a
    test examine the alternatives of P rounding decisions that lie on a
    rounding boundary.  ``keep_fn(score, valid)``, likewise, replaces the 2:4
    choice (``keep_2_4``), for the alternatives of near-equal scores.
    """
    rows = np.asarray(rows, dtype=np.int64)
    R = rows.size
    if R == 0:
        return np.zeros((0, D_V)), np.zeros(0)
    nk = int(rows.max()) + 1 if causal else kh.shape[0]
    if nk == 0:
        return np.zeros((R, D_V)), np.full(R, -np.inf)
    z = float(softmax_scale) * (qh[rows] @ kh[:nk].T)                 # [R, nk]
    if sparse_2_4:
        n4 = (nk + 3) // 4 * 4
        exact = np.zeros((R, n4))
        if softmax_scale != 0:
            exact[:, :nk] = (qh[rows] / multipliers[0]) @ (kh[:nk] / multipliers[1]).T
        keys4 = np.arange(n4)
        valid4 = (keys4[None, :] <= rows[:, None]) if causal else np.broadcast_to(keys4 < nk, (R, n4))
        kept = (keep_fn or keep_2_4)(exact, valid4)[:, :nk]
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    acc = np.zeros((R, D_V))
    for t0 in range(0, nk, BN_P):
        t1 = min(nk, t0 + BN_P)
        keys = np.arange(t0, t0 + BN_P)
        if causal:
            valid = keys[None, :] <= rows[:, None]                     # [R, 64]
        else:
            valid = np.broadcast_to(keys[None, :] < nk, (R, BN_P))
        if sparse_2_4:
            kv = np.zeros((R, BN_P), bool)
            kv[:, : t1 - t0] = kept[:, t0:t1]
            valid = valid & kv
        zt = np.full((R, BN_P), -np.inf)
        zt[:, : t1 - t0] = z[:, t0:t1]
        zt = np.where(valid, zt, -np.inf)
        m_new = np.maximum(m, zt.max(axis=1))
        live = ~np.isneginf(m_new)                                     # row has a key so far
        m_safe = np.where(live, m_new, 0.0)
        alpha = np.where(np.isneginf(m), 0.0, np.exp(m - m_safe))
        p = np.where(valid, np.exp(zt - m_safe[:, None]), 0.0)
        l = alpha * l + p.sum(axis=1)
        if quantize_p and p_quantizer is not None:
            p_hat = p_quantizer(p.astype(F32), t0)
        elif quantize_p and p_fp8:
            p_hat = fp8_qdq(p.astype(F32), g_p)
        elif quantize_p:
            p_hat = nvfp4_qdq(p.astype(F32), g_p, axis=-1)
        else:
            p_hat = p
        vt = np.zeros((BN_P, D_V))
        vt[: t1 - t0] = vh[t0:t1]
        acc = alpha[:, None] * acc + p_hat @ vt
        m = np.where(live, m_new, m)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(l[:, None] > 0, acc / np.where(l > 0, l, 1.0)[:, None], 0.0)
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return out, lse


def attention(q, k, v, cu_q, cu_k, softmax_scale, flags, g_q, g_k, g_v, g_p, causal,
              heads=None, rows_of=None):
    """O [Tq,H,128] and LSE [Tq,H] (float64) of the varlen attention of the
    query rows of each sequence over its key rows (causal: the same rows;
    otherwise the key rows are the sequence's cached context).

    q [Tq,H,192], k [Tk,H,192] and v [Tk,H,128] are fp32 arrays holding the
    bf16 inputs.  ``heads`` restricts the computation to a subset of heads;
    ``rows_of(n, L)`` may return the local query rows of sequence n to compute.
    Rows and heads not computed are NaN.  A query row with no key gives O = 0,
    LSE = -inf.
    """
    cq = [int(c) for c in cu_q]
    ck = [int(c) for c in cu_k]
    Tq, H = q.shape[:2]
    heads = np.arange(H) if heads is None else np.asarray(heads)
    qh = quantize_q(q, flags, g_q, heads)
    kh, vh = quantize_kv(k, v, ck, flags, g_k, g_v, heads)
    mult = operand_multipliers(flags, g_q, g_k)
    O = np.full((Tq, H, D_V), np.nan)
    lse = np.full((Tq, H), np.nan)
    for n, (a, b) in enumerate(zip(cq[:-1], cq[1:])):
        Lq = b - a
        if Lq == 0:
            continue
        ka, kb = ck[n], ck[n + 1]
        rows = np.arange(Lq) if rows_of is None else np.asarray(rows_of(n, Lq), dtype=np.int64)
        for hi, h in enumerate(heads):
            o, s = attend_rows(qh[a:b, hi], kh[ka:kb, hi], vh[ka:kb, hi], rows, softmax_scale,
                               bool(flags & FLAG_P), g_p, causal=causal, sparse_2_4=bool(flags & SPARSE_2_4),
                               p_fp8=bool(flags & FP8_P), multipliers=mult)
            O[a + rows, h] = o
            lse[a + rows, h] = s
    return O, lse


def prefill(q, k, v, cu_seqlens, softmax_scale, flags, g_q, g_k, g_v, g_p,
            heads=None, rows_of=None):
    """O [T,H,128] and LSE [T,H] (float64) of the varlen causal prefill
    (queries and keys are the same rows of each sequence)."""
    return attention(q, k, v, cu_seqlens, cu_seqlens, softmax_scale, flags, g_q, g_k, g_v, g_p, True,
                     heads=heads, rows_of=rows_of)


def chunked_prefill(q, k, v, cu_q, ctx_k, ctx_v, cu_ctx, softmax_scale, flags, g_q, g_k, g_v, g_p,
                    ctx_flags=None, heads=None):
    """A chunk of new tokens whose sequences already hold a cached context:
    the causal attention of the new tokens over themselves (with ``flags``,
    2:4 sparsity included) and their context attention over the cached
    prefix (with ``ctx_flags``, default ``flags`` without 2:4: the sparsity is
    for new-token attention), merged by their natural-log LSEs
    ([MO-MLA], commit 1: the prefill's LSE merges chunked context; commit 2:
    cached-context chunks are gathered from the quantized cache and quantized
    again as prefill operands).  ctx_k [Tc,H,192] and ctx_v [Tc,H,128] are
    the context keys and values (the model's projection of the gathered
    latent).  Returns O [T,H,128], LSE [T,H]."""
    ctx_flags = (flags & ~SPARSE_2_4) if ctx_flags is None else ctx_flags
    o_new, l_new = attention(q, k, v, cu_q, cu_q, softmax_scale, flags, g_q, g_k, g_v, g_p, True, heads)
    o_ctx, l_ctx = attention(q, ctx_k, ctx_v, cu_q, cu_ctx, softmax_scale, ctx_flags, g_q, g_k, g_v, g_p,
                             False, heads)
    return lse_merge(np.stack([o_ctx, o_new]), np.stack([l_ctx, l_new]))


def output_nvfp4(O, out_global_scale):
    """The fused NVFP4 output of rows O [T,H,128]: packed codes [T,H,64] and
    the scale matrix SF [T, H*8] (unswizzled; ``swizzle.swizzle`` lays it
    out).  The quantizer input is the fp32 value of O."""
    T, H, D = O.shape
    codes, sf = nvfp4_quantize(np.asarray(O).astype(F32), out_global_scale, axis=-1)
    return pack_codes(codes), sf.reshape(T, H * (D // 16))


def output_nvfp4_swizzled(O, out_global_scale):
    packed, sf = output_nvfp4(O, out_global_scale)
    return packed, swizzle(sf)
