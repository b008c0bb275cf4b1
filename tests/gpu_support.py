"""Helpers shared by the GPU parity tests: run a workload through the HIP
library and through the CPU oracle, and compare to the stated tolerances.

Tolerances (decode and merge outputs): relative L2 error <= 2e-3 and max
absolute error <= 1e-2 on out; absolute error <= 1e-3 on the natural-log LSE.
Integer and byte outputs (cache records, codes, swizzled scales) are compared
bit for bit.
"""
import numpy as np
import torch

from mla_attention_nvfp4_amd import ops
from oracle import decode as OD
from oracle import record as OR

REL_L2 = 2e-3
MAX_ABS = 1e-2
LSE_ABS = 1e-3


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def gpu_cache(inp, fill: int = 0) -> torch.Tensor:
    cache = torch.full((inp.num_pages, inp.page_size, inp.record_bytes), fill, dtype=torch.uint8,
                       device="cuda")
    if inp.kv_c.shape[0]:
        ops.cache_write(inp.kv_c.cuda(), inp.k_pe.cuda(), inp.slot_mapping.cuda(), cache, inp.outer_scale)
    return cache


def oracle_positions(inp, b: int) -> np.ndarray:
    """Logical positions of sequence b whose records the oracle needs."""
    L = int(inp.seq_lens[b])
    if inp.indices is None:
        return np.arange(L)
    idx = inp.indices[b].numpy().astype(np.int64)
    return np.unique(idx[(idx >= 0) & (idx < L)])


def oracle_cache(inp, batch) -> np.ndarray:
    cache = np.zeros((inp.num_pages, inp.page_size, inp.record_bytes), np.uint8)
    offs = inp.token_offsets.numpy()
    for b in batch:
        pos = oracle_positions(inp, b)
        rows = offs[b] + pos
        OR.cache_write(cache, bits(inp.kv_c[rows]), bits(inp.k_pe[rows]),
                       inp.slot_mapping.numpy()[rows], inp.outer_scale)
    return cache


def oracle_decode(inp, batch):
    cache = oracle_cache(inp, batch)
    q = inp.q.float().numpy()
    args = (q[..., :512], q[..., 512:], cache, inp.page_table.numpy(), inp.seq_lens.numpy(), inp.page_size,
            inp.outer_scale, inp.softmax_scale)
    if inp.indices is None:
        return OD.dense_decode(*args, batch=batch)
    return OD.sparse_decode(*args, inp.indices.numpy(), batch=batch)


def gpu_decode(inp, cache, max_splits=None):
    q = inp.q.cuda()
    splits = inp.max_splits if max_splits is None else max_splits
    args = (q[..., :512], q[..., 512:], cache, inp.page_table.cuda(), inp.seq_lens.cuda())
    if inp.indices is None:
        out, lse = ops.decode(*args, inp.outer_scale, inp.softmax_scale, splits)
    else:
        out, lse = ops.sparse_decode(*args, inp.indices.cuda(), inp.outer_scale, inp.softmax_scale, splits)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), lse.cpu().double().numpy()


def compare(out, lse, ref_out, ref_lse, batch, what=""):
    """Assert the stated tolerances on the rows in ``batch``; returns the
    measured (rel_l2, max_abs, lse_abs)."""
    o, r = out[batch], ref_out[batch]
    lo, lr = lse[batch], ref_lse[batch]
    empty = np.isneginf(lr)
    assert np.array_equal(np.isneginf(lo), empty), f"{what}: -inf LSE pattern differs"
    assert np.all(o[empty] == 0), f"{what}: rows without tokens must be zero"
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    num = np.linalg.norm(o - r)
    den = np.linalg.norm(r)
    rel = num / den if den > 0 else num
    mab = float(np.max(np.abs(o - r))) if o.size else 0.0
    lab = float(np.max(np.abs(lo[~empty] - lr[~empty]))) if (~empty).any() else 0.0
    print(f"  {what}: rel_l2={rel:.3e} max_abs={mab:.3e} lse_abs={lab:.3e}", flush=True)
    assert rel <= REL_L2, f"{what}: rel L2 {rel:.3e}"
    assert mab <= MAX_ABS, f"{what}: max abs {mab:.3e}"
    assert lab <= LSE_ABS, f"{what}: lse abs {lab:.3e}"
    return rel, mab, lab
