"""Seeded synthetic inputs for the NVFP4 MLA workloads.

This module only draws inputs (it holds none of the method's arithmetic) and
serves both the GPU path and the CPU oracle.  Everything is drawn on the CPU
with ``torch.Generator`` seeded ``20260000 + workload number``, so the data do
not depend on the GPU.

Workloads (sizes as stated for each; the pages publish no benchmark suite):

0  tiny decode: B=1, H=16, L=256, pages of 64 in identity order, outer scale
   1.0, bf16 RoPE (432-byte records), softmax_scale = 1/sqrt(576), 1 split.
1  dense decode, DeepSeek-V3 shape: B=64, H=128, L=4096 for every sequence,
   pages of 64 in a shuffled page table, outer scale ~ U[0.5, 2] (one draw),
   432-byte records, 4 splits + merge.
2  ragged decode with fp8 RoPE: B=128, H=128, L ~ U{1024..32768}, pages of
   64 shuffled, e4m3 RoPE (368-byte records), latent N(0,1) with each element
   multiplied by 20 with probability 0.01, outer scale ~ U[0.5, 2], split
   count chosen per sequence (up to 8 splits).
3  sparse top-k decode: B=32, H=128, L=65536 per sequence, pages of 64
   shuffled, 432-byte records, outer scale ~ U[0.5, 2]; indices [32, 2048]
   drawn without replacement from [0, 65536) with 205 entries per row
   (round(0.1 * 2048)) set to -1 at random positions; up to 8 splits.
4  varlen causal prefill: N=8 sequences with L ~ U{2048..8192}, H=128, Q and
   K bf16 N(0,1) [T,128,192], V bf16 N(0,1) [T,128,128]; Q/K/P/V quantized;
   the tensor-wide dequant multipliers are the caller's choice
   g_x = fp32(max|x| / (6 * 448)) per input, g_p = fp32(1 / (6 * 448)), and
   the output global scale g_out = g_v; softmax_scale = 1/sqrt(192).

q, kv_c, k_pe, Q, K, V are N(0,1) rounded to bf16.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

SEED_BASE = 20260000
PAGE = 64
D_LATENT, D_ROPE = 512, 64


def _gen(workload: int) -> torch.Generator:
    return torch.Generator().manual_seed(SEED_BASE + workload)


def _randn_bf16(g: torch.Generator, shape, chunk_rows: int = 1 << 16) -> torch.Tensor:
    """N(0,1) rounded to bf16, drawn in row chunks to bound fp32 temporaries."""
    shape = tuple(shape)
    out = torch.empty(shape, dtype=torch.bfloat16)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = torch.randn((r1 - r0, flat.shape[1]), generator=g).to(torch.bfloat16)
    return out


@dataclasses.dataclass
class DecodeInputs:
    """Decode workload on the CPU.  Token j of sequence b is row
    token_offsets[b] + j of kv_c / k_pe and is written to cache slot
    slot_mapping of that row."""
    name: str
    B: int
    H: int
    page_size: int
    record_bytes: int
    outer_scale: float
    softmax_scale: float
    max_splits: int
    q: torch.Tensor             # bf16 [B, H, 576]
    kv_c: torch.Tensor          # bf16 [T, 512]
    k_pe: torch.Tensor          # bf16 [T, 64]
    seq_lens: torch.Tensor      # int32 [B]
    token_offsets: torch.Tensor  # int64 [B + 1]
    page_table: torch.Tensor    # int32 [B, max_pages] (-1 past the end)
    slot_mapping: torch.Tensor  # int64 [T]
    num_pages: int
    indices: torch.Tensor | None = None   # int32 [B, topk] (sparse)

    @property
    def topk(self) -> int:
        return 0 if self.indices is None else int(self.indices.shape[1])


def _paged(g, lens, page_size, shuffle):
    lens = [int(x) for x in lens]
    pages_per = [(L + page_size - 1) // page_size for L in lens]
    num_pages = max(1, sum(pages_per))
    order = torch.randperm(num_pages, generator=g) if shuffle else torch.arange(num_pages)
    max_pages = max(1, max(pages_per))
    pt = torch.full((len(lens), max_pages), -1, dtype=torch.int32)
    slots = []
    k = 0
    for b, (L, npg) in enumerate(zip(lens, pages_per)):
        pages = order[k:k + npg]
        k += npg
        pt[b, :npg] = pages.to(torch.int32)
        j = torch.arange(L, dtype=torch.int64)
        slots.append(pages.to(torch.int64)[j // page_size] * page_size + j % page_size)
    offs = torch.zeros(len(lens) + 1, dtype=torch.int64)
    offs[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0)
    return pt, torch.cat(slots) if slots else torch.zeros(0, dtype=torch.int64), offs, num_pages


def decode_workload(n: int, H: int | None = None) -> DecodeInputs:
    """Decode workloads 0-3; ``H`` overrides the head count (e.g. 16)."""
    g = _gen(n)
    if n == 0:
        B, Hd, lens, shuffle, rec, outer, splits = 1, 16, [256], False, 432, 1.0, 1
    elif n == 1:
        B, Hd, shuffle, rec, splits = 64, 128, True, 432, 4
        lens = [4096] * B
        outer = float(torch.empty(()).uniform_(0.5, 2.0, generator=g))
    elif n == 2:
        B, Hd, shuffle, rec, splits = 128, 128, True, 368, 8
        lens = torch.randint(1024, 32768 + 1, (B,), generator=g).tolist()
        outer = float(torch.empty(()).uniform_(0.5, 2.0, generator=g))
    elif n == 3:
        B, Hd, shuffle, rec, splits = 32, 128, True, 432, 8
        lens = [65536] * B
        outer = float(torch.empty(()).uniform_(0.5, 2.0, generator=g))
    else:
        raise ValueError(f"no decode workload {n}")
    H = Hd if H is None else H
    q = _randn_bf16(g, (B, H, D_LATENT + D_ROPE), chunk_rows=B)
    pt, slots, offs, num_pages = _paged(g, lens, PAGE, shuffle)
    T = int(offs[-1])
    kv_c = _randn_bf16(g, (T, D_LATENT))
    if n == 2:
        for r0 in range(0, T, 1 << 16):
            r1 = min(T, r0 + (1 << 16))
            hit = torch.rand((r1 - r0, D_LATENT), generator=g) < 0.01
            blk = kv_c[r0:r1]
            blk[hit] = (blk[hit].to(torch.float32) * 20).to(torch.bfloat16)
    k_pe = _randn_bf16(g, (T, D_ROPE))
    indices = None
    if n == 3:
        topk, n_bad = 2048, round(0.1 * 2048)
        indices = torch.empty((B, topk), dtype=torch.int32)
        for b in range(B):
            row = torch.randperm(lens[b], generator=g)[:topk].to(torch.int32)
            bad = torch.randperm(topk, generator=g)[:n_bad]
            row[bad] = -1
            indices[b] = row
    return DecodeInputs(
        name=f"decode{n}", B=B, H=H, page_size=PAGE, record_bytes=rec, outer_scale=outer,
        softmax_scale=1.0 / math.sqrt(D_LATENT + D_ROPE), max_splits=splits, q=q, kv_c=kv_c,
        k_pe=k_pe, seq_lens=torch.tensor(lens, dtype=torch.int32), token_offsets=offs,
        page_table=pt, slot_mapping=slots, num_pages=num_pages, indices=indices)


def small_decode(seed: int, B: int, H: int, lens, page_size: int = 64, rec: int = 432,
                 outer: float = 1.0, softmax_scale: float | None = None, max_splits: int = 1,
                 shuffle: bool = True, outliers: bool = False, topk: int = 0,
                 invalid_frac: float = 0.0, kv_gain: float = 1.0) -> DecodeInputs:
    """A small decode case for parity tests (same recipe as the workloads;
    kv_gain multiplies the latent before it is rounded to bf16)."""
    g = torch.Generator().manual_seed(seed)
    q = _randn_bf16(g, (B, H, D_LATENT + D_ROPE), chunk_rows=max(1, B))
    pt, slots, offs, num_pages = _paged(g, lens, page_size, shuffle)
    T = int(offs[-1])
    kv_c = _randn_bf16(g, (max(T, 0), D_LATENT))
    if kv_gain != 1.0:
        kv_c = (kv_c.to(torch.float32) * kv_gain).to(torch.bfloat16)
    if outliers and T:
        hit = torch.rand((T, D_LATENT), generator=g) < 0.01
        kv_c[hit] = (kv_c[hit].to(torch.float32) * 20).to(torch.bfloat16)
    k_pe = _randn_bf16(g, (max(T, 0), D_ROPE))
    indices = None
    if topk:
        indices = torch.empty((B, topk), dtype=torch.int32)
        for b in range(B):
            L = int(lens[b])
            # positions drawn with replacement over a range a bit beyond L,
            # so that out-of-range entries appear too
            row = torch.randint(-1, max(L + 8, 1), (topk,), generator=g).to(torch.int32)
            if invalid_frac:
                bad = torch.rand(topk, generator=g) < invalid_frac
                row[bad] = -1
            indices[b] = row
    return DecodeInputs(
        name=f"small{seed}", B=B, H=H, page_size=page_size, record_bytes=rec, outer_scale=outer,
        softmax_scale=(1.0 / math.sqrt(D_LATENT + D_ROPE)) if softmax_scale is None else softmax_scale,
        max_splits=max_splits, q=q, kv_c=kv_c, k_pe=k_pe,
        seq_lens=torch.tensor(list(lens), dtype=torch.int32), token_offsets=offs, page_table=pt,
        slot_mapping=slots, num_pages=num_pages, indices=indices)


@dataclasses.dataclass
class PrefillInputs:
    name: str
    H: int
    q: torch.Tensor            # bf16 [T, H, 192]
    k: torch.Tensor            # bf16 [T, H, 192]
    v: torch.Tensor            # bf16 [T, H, 128]
    cu_seqlens: torch.Tensor   # int32 [N + 1]
    max_seqlen: int
    softmax_scale: float
    flags: int
    g_q: float
    g_k: float
    g_v: float
    g_p: float
    g_out: float

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])


FP8_BIT = {"q": 16, "k": 32, "p": 64, "v": 128}


def _amax_scale(x: torch.Tensor, fp8: bool = False) -> float:
    # the caller's tensor-wide multiplier: fp32(max|x| / (6 * 448)) for NVFP4
    # (block scales up to 448 times elements up to 6), fp32(max|x| / 448) for
    # per-tensor FP8
    return float(np.float32(float(x.abs().max().float()) / (448.0 if fp8 else 2688.0)))


def _p_scale(flags: int) -> float:
    # probabilities are at most 1: fp32(1 / 448) for FP8, fp32(1 / (6 * 448)) for NVFP4
    return float(np.float32(1.0 / (448.0 if flags & FP8_BIT["p"] else 2688.0)))


def _cu(lens) -> torch.Tensor:
    cu = torch.zeros(len(lens) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int32), 0)
    return cu


def prefill_inputs(seed: int, lens, H: int, flags: int = 15, name: str | None = None) -> PrefillInputs:
    g = torch.Generator().manual_seed(seed)
    lens = [int(x) for x in lens]
    T = sum(lens)
    q = _randn_bf16(g, (T, H, 192), chunk_rows=4096)
    k = _randn_bf16(g, (T, H, 192), chunk_rows=4096)
    v = _randn_bf16(g, (T, H, 128), chunk_rows=4096)
    gq, gk, gv = (_amax_scale(t, bool(flags & FP8_BIT[n])) if T else 1.0 for t, n in ((q, "q"), (k, "k"), (v, "v")))
    return PrefillInputs(name=name or f"prefill{seed}", H=H, q=q, k=k, v=v, cu_seqlens=_cu(lens),
                         max_seqlen=max(lens) if lens else 0, softmax_scale=1.0 / math.sqrt(192),
                         flags=flags, g_q=gq, g_k=gk, g_v=gv, g_p=_p_scale(flags), g_out=gv)


def grid_prefill_inputs(seed: int, lens, H: int, flags: int, name: str | None = None) -> PrefillInputs:
    """As prefill_inputs, but Q and K drawn from the grid {-1, -0.75, ..., 1}:
    every score is then a multiple of 1/16 below 192 in magnitude (exact in
    fp32 whatever the summation order), and equal scores are common."""
    inp = prefill_inputs(seed, lens, H, flags, name)
    g = torch.Generator().manual_seed(seed + 7919)
    T = inp.T
    inp.q = (torch.randint(-4, 5, (T, H, 192), generator=g).float() / 4).to(torch.bfloat16)
    inp.k = (torch.randint(-4, 5, (T, H, 192), generator=g).float() / 4).to(torch.bfloat16)
    if T:
        inp.g_q = _amax_scale(inp.q, bool(flags & FP8_BIT["q"]))
        inp.g_k = _amax_scale(inp.k, bool(flags & FP8_BIT["k"]))
    return inp


@dataclasses.dataclass
class ContextInputs:
    """A chunk of new tokens per sequence plus that sequence's cached context
    as prefill operands (the model's projection of the gathered latent):
    q, k, v new-token rows [T, H, 192/192/128] with cu_q; ctx_k, ctx_v
    context rows [Tc, H, 192/128] with cu_ctx."""
    new: PrefillInputs
    ctx_k: torch.Tensor
    ctx_v: torch.Tensor
    cu_ctx: torch.Tensor

    @property
    def max_ctx(self) -> int:
        c = self.cu_ctx.tolist()
        return max([b - a for a, b in zip(c[:-1], c[1:])] + [0])


def context_inputs(seed: int, new_lens, ctx_lens, H: int, flags: int) -> ContextInputs:
    """Seeded new-token and context operands, N(0,1) rounded to bf16; K and V
    multipliers cover both (their amax over new and context rows)."""
    new = prefill_inputs(seed, new_lens, H, flags)
    g = torch.Generator().manual_seed(seed + 104729)
    Tc = sum(int(x) for x in ctx_lens)
    ck = _randn_bf16(g, (Tc, H, 192), chunk_rows=4096)
    cv = _randn_bf16(g, (Tc, H, 128), chunk_rows=4096)
    if Tc and new.T:
        new.g_k = _amax_scale(torch.cat([new.k.reshape(-1), ck.reshape(-1)]), bool(flags & FP8_BIT["k"]))
        new.g_v = _amax_scale(torch.cat([new.v.reshape(-1), cv.reshape(-1)]), bool(flags & FP8_BIT["v"]))
        new.g_out = new.g_v
    return ContextInputs(new=new, ctx_k=ck, ctx_v=cv, cu_ctx=_cu(ctx_lens))


def prefill_workload(n: int = 4) -> PrefillInputs:
    if n != 4:
        raise ValueError(f"no prefill workload {n}")
    g = _gen(4)
    lens = torch.randint(2048, 8192 + 1, (8,), generator=g).tolist()
    return prefill_inputs(SEED_BASE + 4, lens, 128, 15, name="prefill4")
