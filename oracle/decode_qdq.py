"""Decode with quantized attention operands: P quantized in the decode loop,
Q quantized by the caller in an fp32 carrier, and a raw (bf16) latent cache
whose K and V are quantized on read.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[MO-MLA], PR body and commit 4: every attention matmul operand is
fake-quantized once along its own contraction axis.  The split-K absorbed
decode quantizes P in the kernel (after the softmax row sum, the denominator
unquantized) and takes Q quantized by the caller in an FP32 carrier (the
dequantized values are not rounded back to bf16).  In the raw-cache model the
latent cache stays bf16 and the decode quantizes K along the feature axis and
V along the token axis, independently, V in blocks of 16 at absolute token
positions so that the split boundaries do not move them (the last, open block
holds only the tokens the sequence has).  The formats are those of the
prefill: NVFP4 1x16 blocks or per-tensor FP8, chosen per operand.

Cache records: the NVFP4 latent records (432 / 368 bytes, ``record.py``),
whose K and V are the stored latent (quantizing K or V again on read is not
offered: that would be the double quantization the pages move away from), or
raw records of 1152 bytes: the 512 bf16 latent values then the 64 bf16 RoPE
values, little-endian.

The computation, per sequence b (L tokens) and head h:

1. k_j (576-d) and v_j (512-d): NVFP4 records give k_j = [s_l * dequant(latent),
   rope] and v_j = s_l * dequant(latent).  Raw records give k_j = [latent,
   rope] and v_j = latent, each then quantized when its flag is set: K along
   the 576 features (NVFP4: 36 blocks of 16; or per-tensor FP8) with g_k;
   V along tokens (NVFP4: blocks [16k, 16k+16) of positions < L per dim; or
   per-tensor FP8) with g_v.
2. q (576-d): quantized along its features with g_q when its flag is set.
3. z_j = softmax_scale * q_hat . k_hat_j.
4. The tokens are cut into the decode's split-K chunks (the split policy of
   the library, written out in ``split_bounds``).  In each chunk, keys are
   taken in tiles of 32 from the chunk start, in order, with a running max m
   refreshed per tile: p_j = e^(z_j - m'), l <- alpha l + sum p (unquantized),
   p_hat = QDQ of fp32(p) with g_p (NVFP4: 16-key blocks aligned to the tile,
   keys past L included as zeros; or per-tensor FP8), acc <- alpha acc +
   sum p_hat v_hat.  Each chunk gives (acc / l, m + ln l); the chunks merge by
   their natural-log LSE (``decode.lse_merge``).

With P unquantized, step 4 is plain softmax attention whatever the chunks.
Which running max quantizes P is the kernels' schedule, and the pages say
their oracles replicate the kernel schedules; the 32-key tile and the chunks
are this project's convention.
"""

from __future__ import annotations

import numpy as np

from .decode import lse_merge, slots_of
from .formats import F32, bf16_to_f32, fp8_qdq, nvfp4_qdq, nvfp4_qdq_ragged
from .record import D_LATENT, D_ROPE, unpack_records

RAW_RECORD_BYTES = 2 * (D_LATENT + D_ROPE)     # 1152
TILE = 32
FLAG_Q, FLAG_K, FLAG_P, FLAG_V = 1, 2, 4, 8
FP8_Q, FP8_K, FP8_P, FP8_V = 16, 32, 64, 128


def split_bounds(n: int, max_splits: int):
    """The decode's split-K chunks of n tokens: with tiles of 64, want =
    clamp(ceil(n / 256), 1, max_splits) chunks of ceil(tiles / want) tiles
    each (the last possibly shorter); one chunk when n <= 0."""
    if n <= 0:
        return [0, 0]
    tiles = (n + 63) // 64
    want = min(max(1, (n + 255) // 256), max(1, max_splits))
    chunk = (tiles + want - 1) // want
    bounds = list(range(0, n, 64 * chunk)) + [n]
    return bounds


def raw_records(kv_c_bits, k_pe_bits) -> np.ndarray:
    """Raw cache records of T tokens from bf16 bit patterns: uint8 [T, 1152]."""
    kv = np.asarray(kv_c_bits, dtype=np.uint16)
    pe = np.asarray(k_pe_bits, dtype=np.uint16)
    return np.concatenate([kv, pe], axis=-1).astype("<u2").view(np.uint8)


def unpack_raw(rec):
    """(latent [T,512], rope [T,64]) float64 from raw records."""
    bits = np.asarray(rec, dtype=np.uint8).copy().view("<u2")
    vals = bf16_to_f32(bits).astype(np.float64)
    return vals[..., :D_LATENT], vals[..., D_LATENT:]


def _qdq(x, flags, on, fp8, g, axis=-1):
    if not flags & on:
        return np.asarray(x, dtype=np.float64)
    x32 = np.asarray(x, dtype=F32)
    return fp8_qdq(x32, g) if flags & fp8 else nvfp4_qdq(x32, g, axis=axis)


def operands(cache, page_table_row, page_size, L, outer_scale, flags, g_k, g_v):
    """Step 1 for one sequence: (k_hat [L,576], v_hat [L,512]) float64."""
    flat = np.asarray(cache).reshape(-1, cache.shape[-1])
    recs = flat[slots_of(page_table_row, page_size, np.arange(L))]
    if cache.shape[-1] != RAW_RECORD_BYTES:
        if flags & (FLAG_K | FLAG_V):
            raise ValueError("K and V are quantized on read only for raw records")
        lat, rope = unpack_records(recs, outer_scale)
        return np.concatenate([lat, rope], axis=-1), lat
    lat, rope = unpack_raw(recs)
    k = _qdq(np.concatenate([lat, rope], axis=-1), flags, FLAG_K, FP8_K, g_k)
    if flags & FLAG_V and flags & FP8_V:
        v = fp8_qdq(lat.astype(F32), g_v)
    elif flags & FLAG_V:
        v = nvfp4_qdq_ragged(lat.astype(F32), g_v, axis=0) if L else lat
    else:
        v = lat
    return k, v


def _chunk(k, v, z, a, b, flags, g_p, p_quantizer=None):
    """Step 4 over tokens [a, b) of one head's row: (out, lse).
    ``p_quantizer(p32, t0)``, if given, replaces the P QDQ of the tile at
    token t0 (a test hook for P decisions that lie on a rounding boundary)."""
    m, l = -np.inf, 0.0
    acc = np.zeros(D_LATENT)
    for t0 in range(a, b, TILE):
        t1 = min(b, t0 + TILE)
        zt = np.full(TILE, -np.inf)
        zt[: t1 - t0] = z[t0:t1]
        m_new = max(m, zt.max())
        alpha = 0.0 if m == -np.inf else np.exp(m - m_new)
        p = np.where(np.isneginf(zt), 0.0, np.exp(zt - m_new))
        l = alpha * l + p.sum()
        if flags & FLAG_P and p_quantizer is not None:
            p_hat = p_quantizer(p.astype(F32), t0)
        elif flags & FLAG_P:
            p32 = p.astype(F32)
            p_hat = fp8_qdq(p32, g_p) if flags & FP8_P else nvfp4_qdq(p32, g_p)
        else:
            p_hat = p
        vt = np.zeros((TILE, D_LATENT))
        vt[: t1 - t0] = v[t0:t1]
        acc = alpha * acc + p_hat @ vt
        m = m_new
    if l == 0.0:
        return np.zeros(D_LATENT), -np.inf
    return acc / l, m + np.log(l)


def decode_qdq(q_nope, q_rope, cache, page_table, seq_lens, page_size, outer_scale, softmax_scale,
               flags, g_q, g_k, g_v, g_p, max_splits, batch=None, p_quantizer=None):
    """out [B,H,512], lse [B,H] (float64); ``batch`` restricts the work to a
    subset of sequences (other rows NaN).  ``cache`` is [pages, page_size,
    record] with NVFP4 (432 / 368 B) or raw (1152 B) records.
    ``p_quantizer``: see ``_chunk``."""
    q = np.concatenate([np.asarray(q_nope, np.float64), np.asarray(q_rope, np.float64)], axis=-1)
    B, H = q.shape[:2]
    out = np.full((B, H, D_LATENT), np.nan)
    lse = np.full((B, H), np.nan)
    for b in (range(B) if batch is None else batch):
        L = int(seq_lens[b])
        k, v = operands(cache, page_table[b], page_size, L, outer_scale, flags, g_k, g_v)
        qh = _qdq(q[b], flags, FLAG_Q, FP8_Q, g_q)                     # [H, 576]
        z = float(softmax_scale) * (qh @ k.T)                          # [H, L]
        bounds = split_bounds(L, max_splits)
        for h in range(H):
            parts = [_chunk(k, v, z[h], a, e, flags, g_p, p_quantizer) for a, e in zip(bounds[:-1], bounds[1:])]
            po = np.stack([o for o, _ in parts])
            pl = np.array([s for _, s in parts])
            out[b, h], lse[b, h] = lse_merge(po, pl)
    return out, lse
