"""Varlen causal MLA prefill with NVFP4 fake quantization and NVFP4 output.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[MO-MLA], commit 1 and PR body: varlen prefill with asymmetric head dims
(qk 192 = 128 nope + 64 rope, v 128), each attention matmul operand
fake-quantized once along its own contraction axis in NVFP4 1x16 blocks:
Q and K along the head dim, V along tokens, P along keys after the softmax
row-sum, the softmax denominator itself unquantized; natural-log LSE.
[FUSED-OUT], PR description: the output is written directly as NVFP4 with a
128x4-swizzled scale buffer and an fp32 global scale (``swizzle.py``).

The algorithm, per sequence n (rows r in [cu[n], cu[n+1]), local index
i = r - cu[n]) and head h:

1. Operand quantization, each switched by a flag bit (Q=1, K=2, P=4, V=8):
   Q_hat, K_hat = block QDQ along d with multipliers g_q, g_k;
   V_hat = block QDQ along local token position (blocks [16k, 16k+16), the
   last one possibly short) per head and dim, multiplier g_v.
2. z_ij = softmax_scale * Q_hat_i . K_hat_j for keys j <= i (causal).
3. Keys are taken in tiles of BN_P = 64 from j = 0 upward.  Start m = -inf,
   l = 0, acc = 0.  Per tile: m' = max(m, max of the tile's unmasked z);
   alpha = e^(m - m') (0 while m = -inf); p_j = e^(z_ij - m') on unmasked keys,
   0 on masked ones; l <- alpha*l + sum p  (unquantized); p_hat = block QDQ of
   fp32(p) along keys with multiplier g_p, blocks aligned to the local key
   index, masked zeros included; acc <- alpha*acc + sum_j p_hat_j V_hat_j;
   m <- m'.
4. O_i = acc / l,  LSE_i = m + ln l.

Step 3's tile width is a convention of this project: [MO-MLA], commit 1, says
its golden oracles replicate the kernel schedules, and P's quantization depends
on the running maximum the kernel holds when it quantizes, so the schedule is
part of the definition.  The running maximum is refreshed at every 64-key tile
and the accumulator always rescaled.  With the P flag off the schedule drops
out and step 3 is textbook causal softmax attention.
"""

from __future__ import annotations

import numpy as np

from .formats import F32, nvfp4_qdq, nvfp4_qdq_ragged
from .swizzle import pack_codes, swizzle
from .formats import nvfp4_quantize

BN_P = 64
D_QK = 192
D_V = 128
FLAG_Q, FLAG_K, FLAG_P, FLAG_V = 1, 2, 4, 8


def quantize_operands(q, k, v, cu_seqlens, flags, g_q, g_k, g_v, heads=None):
    """Step 1 for the given heads: (Q_hat, K_hat, V_hat) as float64 arrays
    [T, len(heads), d]."""
    heads = np.arange(q.shape[1]) if heads is None else np.asarray(heads)
    qs = np.asarray(q, dtype=F32)[:, heads]
    ks = np.asarray(k, dtype=F32)[:, heads]
    vs = np.asarray(v, dtype=F32)[:, heads]
    qh = nvfp4_qdq(qs, g_q, axis=-1) if flags & FLAG_Q else qs.astype(np.float64)
    kh = nvfp4_qdq(ks, g_k, axis=-1) if flags & FLAG_K else ks.astype(np.float64)
    if flags & FLAG_V:
        vh = np.empty(vs.shape, dtype=np.float64)
        for a, b in zip(cu_seqlens[:-1], cu_seqlens[1:]):
            if b > a:
                vh[a:b] = nvfp4_qdq_ragged(vs[a:b], g_v, axis=0)
    else:
        vh = vs.astype(np.float64)
    return qh, kh, vh


def attend_rows(qh, kh, vh, rows, softmax_scale, quantize_p, g_p, p_quantizer=None):
    """Steps 2-4 for one sequence and one head.

    qh [L,192], kh [L,192], vh [L,128] (this sequence, float64); ``rows``
    local query indices.  Returns O [len(rows),128], LSE [len(rows)].

    ``p_quantizer(p32, t0)``, if given, replaces step 3's P block QDQ for the
    tile starting at key t0 (p32: the tile's fp32 probabilities [R, 64]); it
    lets a test examine the alternatives of P rounding decisions that lie on
    a rounding boundary.  The default is the NVFP4 block QDQ.
    """
    rows = np.asarray(rows, dtype=np.int64)
    R = rows.size
    if R == 0:
        return np.zeros((0, D_V)), np.zeros(0)
    nk = int(rows.max()) + 1
    z = float(softmax_scale) * (qh[rows] @ kh[:nk].T)                 # [R, nk]
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    acc = np.zeros((R, D_V))
    for t0 in range(0, nk, BN_P):
        t1 = min(nk, t0 + BN_P)
        keys = np.arange(t0, t0 + BN_P)
        valid = keys[None, :] <= rows[:, None]                         # [R, 64]
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
        elif quantize_p:
            p_hat = nvfp4_qdq(p.astype(F32), g_p, axis=-1)
        else:
            p_hat = p
        vt = np.zeros((BN_P, D_V))
        vt[: t1 - t0] = vh[t0:t1]
        acc = alpha[:, None] * acc + p_hat @ vt
        m = np.where(live, m_new, m)
    out = acc / l[:, None]
    lse = m + np.log(l)
    return out, lse


def prefill(q, k, v, cu_seqlens, softmax_scale, flags, g_q, g_k, g_v, g_p,
            heads=None, rows_of=None):
    """O [T,H,128] and LSE [T,H] (float64) of the varlen causal prefill.

    q, k [T,H,192] and v [T,H,128] are fp32 arrays holding the bf16 inputs.
    ``heads`` restricts the computation to a subset of heads; ``rows_of(n, L)``
    may return the local rows of sequence n to compute.  Rows and heads not
    computed are NaN.
    """
    cu = [int(c) for c in cu_seqlens]
    T, H = q.shape[:2]
    heads = np.arange(H) if heads is None else np.asarray(heads)
    qh, kh, vh = quantize_operands(q, k, v, cu, flags, g_q, g_k, g_v, heads)
    O = np.full((T, H, D_V), np.nan)
    lse = np.full((T, H), np.nan)
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        L = b - a
        if L == 0:
            continue
        rows = np.arange(L) if rows_of is None else np.asarray(rows_of(n, L), dtype=np.int64)
        for hi, h in enumerate(heads):
            o, s = attend_rows(qh[a:b, hi], kh[a:b, hi], vh[a:b, hi], rows,
                               softmax_scale, bool(flags & FLAG_P), g_p)
            O[a + rows, h] = o
            lse[a + rows, h] = s
    return O, lse


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
