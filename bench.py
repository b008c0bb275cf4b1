#!/usr/bin/env python3
"""Benchmark of the NVFP4 MLA decode step on one MI355X.

Step (timed unit): one decode serving step of the dense workload B=64
sequences x 128 heads x 4096 cached tokens (pages of 64, 432-byte records,
4 splits + merge): the NVFP4 cache write of the batch's 64 new tokens
followed by one paged split-K decode call (decode kernel + split merge
kernel).  Inputs are
resident in HBM before timing starts; the cache is rotated over 4 copies
(> 256 MB Infinity Cache) so that decode reads come from HBM.

Printed: one JSON line with queries/s (B / step time, host clock), the
roofline of the decode call (a second timed region of back-to-back decode
calls between one pair of HIP events on the launch stream),
the oracle's CPU throughput on a bounded sample, and extra lines for the
other paths (tiny decode, 16-head decode, ragged decode at 128 and 16 heads, top-k
sparse decode, the stand-alone LSE merge, the full cache write, prefill),
and the roofline constants re-measured on the part (stream copy and read,
MFMA rate of the two product shapes) beside the vendor figures.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from mla_attention_nvfp4_amd import ops, workloads  # noqa: E402

METRIC = "NVFP4 MLA decode HBM GB/s & % roofline; queries/s at B=64, L=4k, 128 heads"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
ROTATE = 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(inp, n_tokens_total: int, H: int) -> int:
    """Algorithmic bytes of one decode launch: records read, q read, out and
    lse written, page-table entries and seq_lens read."""
    B = inp.B
    pages = sum(math.ceil(int(L) / inp.page_size) for L in inp.seq_lens)
    return (n_tokens_total * inp.record_bytes + B * H * 576 * 2 + B * H * 512 * 4 + B * H * 4
            + pages * 4 + B * 4)


def decode_flops(n_tokens_total: int, H: int) -> float:
    return 2.0 * H * n_tokens_total * (576 + 512)


class DecodeBench:
    """Device-resident decode workload with a rotated cache."""

    def __init__(self, inp, rotate: int, sparse: bool = False):
        self.inp = inp
        dev = "cuda"
        base = torch.zeros((inp.num_pages, inp.page_size, inp.record_bytes), dtype=torch.uint8, device=dev)
        ops.cache_write(inp.kv_c.to(dev), inp.k_pe.to(dev), inp.slot_mapping.to(dev), base, inp.outer_scale)
        self.caches = [base] + [base.clone() for _ in range(0 if sparse else rotate - 1)]
        self.n_rot = rotate
        q = inp.q.to(dev)
        self.q_nope, self.q_rope = q[..., :512], q[..., 512:]
        self.pt = inp.page_table.to(dev)
        self.seq = inp.seq_lens.to(dev)
        # sparse: rotate index sets instead of caches (valid entries shifted
        # by a per-set offset modulo L, so each set gathers other records)
        self.idx = None
        if sparse:
            L = inp.seq_lens.to(torch.int64)[:, None]
            base_idx = inp.indices.to(torch.int64)
            sets = []
            for k in range(rotate):
                shifted = torch.where(base_idx >= 0, (base_idx + k * 5461) % L, base_idx)
                sets.append(shifted.to(torch.int32).to(dev))
            self.idx = sets
        B, H = inp.B, inp.H
        self.out = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        need = ops.decode_workspace_bytes(B, H, inp.max_splits)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev) if need else None
        # the step's new tokens overwrite the last position of every sequence
        g = torch.Generator().manual_seed(1234)
        self.new_kv = torch.randn((B, 576), generator=g).to(torch.bfloat16).to(dev)
        last = inp.token_offsets[1:] - 1
        self.new_slots = inp.slot_mapping[last].to(dev)
        torch.cuda.synchronize()

    def write(self, r):
        ops.cache_write(self.new_kv[:, :512], self.new_kv[:, 512:], self.new_slots, self.caches[r],
                        self.inp.outer_scale)

    def decode(self, r):
        inp = self.inp
        if self.idx is None:
            ops.decode(self.q_nope, self.q_rope, self.caches[r], self.pt, self.seq, inp.outer_scale,
                       inp.softmax_scale, inp.max_splits, out=self.out, lse=self.lse, workspace=self.ws)
        else:
            ops.sparse_decode(self.q_nope, self.q_rope, self.caches[0], self.pt, self.seq, self.idx[r],
                              inp.outer_scale, inp.softmax_scale, inp.max_splits, out=self.out, lse=self.lse,
                              workspace=self.ws)

    def run(self, steps: int, warmup: int, with_write: bool = True):
        """Returns (ms per step from the host clock, mean decode-call ms from HIP events).

        Two timed regions: `steps` serving steps (cache write + decode call)
        on the host clock, then `steps` decode calls back to back between one
        pair of HIP events on the launch stream, whose mean is the call's
        launch-to-launch duration (kernels and the gap between them, without
        the few microseconds an event pair around every call would add)."""
        stream = torch.cuda.current_stream()
        for i in range(warmup):
            if with_write:
                self.write(i % self.n_rot)
            self.decode(i % self.n_rot)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            r = i % self.n_rot
            if with_write:
                self.write(r)
            self.decode(r)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(steps):
            self.decode(i % self.n_rot)
        ev1.record(stream)
        torch.cuda.synchronize()
        return (t1 - t0) * 1e3 / steps, ev0.elapsed_time(ev1) / steps


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_kernel_B64_H128_L4096_hbm_bytes.md")
DECODE_SOURCES = ("decode.hip", "device_common.hpp", "launch.hpp")


def measured_traffic():
    """HBM bytes per decode call (decode and split-merge kernels) from the
    committed FETCH_SIZE/WRITE_SIZE counter summary, or None when the decode
    kernels' sources have changed since those counters were taken (the
    summary records their sha256)."""
    import hashlib
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    vals = dict(line.split(" = ", 1) for line in text.splitlines() if " = " in line)
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(ROOT, "mla_attention_nvfp4_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    if vals.get("decode_source_sha256", "").strip() != h.hexdigest():
        return None
    return int(vals["traffic_bytes_per_launch"])


def timed(fn, steps: int, warmup: int) -> float:
    """Mean ms of fn() over `steps` back-to-back launches between one pair of
    HIP events on the current stream."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        fn()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def bench_cache_write(inp, steps: int, warmup: int) -> dict:
    """NVFP4 cache write of every token of the decode workload (T = B*L)."""
    dev = "cuda"
    kv, pe = inp.kv_c.to(dev), inp.k_pe.to(dev)
    slots = inp.slot_mapping.to(dev)
    cache = torch.zeros((inp.num_pages, inp.page_size, inp.record_bytes), dtype=torch.uint8, device=dev)
    ms = timed(lambda: ops.cache_write(kv, pe, slots, cache, inp.outer_scale), steps, warmup)
    T = kv.shape[0]
    nbytes = T * (576 * 2 + 8 + inp.record_bytes)
    return {"tokens": T, "kernel_us": ms * 1e3, "gbps": nbytes / (ms * 1e-3) / 1e9,
            "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, "bytes_per_launch": nbytes}


def measure_machine() -> dict:
    """Roofline constants re-measured on this part, next to the vendor
    figures the fractions use: HBM by a plain device copy (read + write) and a
    read-only stream of 4 GiB each (far beyond the 256 MB Infinity Cache),
    and the dense fp16 MFMA rate of the two product shapes the kernels use,
    operands in registers, 8 wavefronts per SIMD (2048 workgroups of 4)."""
    n = 4 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    ms = timed(lambda: ops.roofline_copy(src, dst), 5, 2)
    copy_gbps = 2 * n / (ms * 1e-3) / 1e9
    del dst
    total = torch.zeros(1, dtype=torch.int32, device="cuda")
    ms = timed(lambda: ops.roofline_read(src, total), 5, 2)
    read_gbps = n / (ms * 1e-3) / 1e9
    del src
    blocks, iters = 2048, 2048
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    out = {"hbm_copy_gbps": copy_gbps, "hbm_read_gbps": read_gbps, "hbm_vendor_gbps": PEAK_HBM_GBPS,
           "hbm_copy_frac_of_vendor": copy_gbps / PEAK_HBM_GBPS,
           "hbm_read_frac_of_vendor": read_gbps / PEAK_HBM_GBPS}
    for shape, name, flops in ((0, "mfma_16x16x32_f16", 16384.0), (1, "mfma_32x32x16_f16", 32768.0)):
        ms = timed(lambda: ops.roofline_mfma(shape, blocks, iters, sink), 3, 1)
        tf = blocks * 4 * iters * 8 * flops / (ms * 1e-3) / 1e12
        out[name + "_tflops"] = tf
        out[name + "_frac_of_vendor"] = tf / PEAK_BF16_TFLOPS
    out["mfma_vendor_tflops"] = PEAK_BF16_TFLOPS
    out["note"] = ("roofline fractions in this line use the vendor peaks; both decode kernels use the "
                   "16x16x32 product, whose measured rate bounds them")
    return out


def bench_lse_merge(steps: int, warmup: int) -> dict:
    """mla_lse_merge on the dense decode shape: B=64 sequences, 4 splits, 128
    heads, 512-d fp32 partials (the stand-alone merge entry point), the input
    rotated over 4 copies (268 MB, above the 256 MB Infinity Cache)."""
    B, S, H, D = 64, 4, 128, 512
    g = torch.Generator().manual_seed(4321)
    po = [torch.randn((B, S, H, D), generator=g).cuda() for _ in range(4)]
    pl = [(torch.randn((B, S, H), generator=g) * 3).cuda() for _ in range(4)]
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    it = [0]

    def run():
        r = it[0] % 4
        it[0] += 1
        ops.lse_merge(po[r], pl[r], out=out, lse=lse)

    ms = timed(run, steps, warmup)
    nbytes = B * S * H * (D + 1) * 4 + B * H * (D + 1) * 4
    return {"kernel_us": ms * 1e3, "gbps": nbytes / (ms * 1e-3) / 1e9,
            "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, "bytes_per_launch": nbytes,
            "note": "input rotated over 4 copies (268 MB)"}


def bench_prefill(steps: int, warmup: int, flags: int | None = None) -> dict:
    """Varlen causal prefill, 8 sequences of 2k-8k tokens, 128 heads, all four
    operand quantizers (NVFP4, or the given flags: FP8 formats, 2:4
    sparsity), NVFP4 output with swizzled scales and LSE."""
    inp = workloads.prefill_workload()
    if flags is not None:
        lens = (inp.cu_seqlens[1:] - inp.cu_seqlens[:-1]).tolist()
        inp = workloads.prefill_inputs(workloads.SEED_BASE + 4, lens, 128, flags, name=f"prefill4-{flags}")
    dev = "cuda"
    q, k, v, cu = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.cu_seqlens.to(dev)
    T, H = inp.T, inp.H
    codes = torch.empty((T, H, 64), dtype=torch.uint8, device=dev)
    scales = torch.empty(ops.swizzled_scale_bytes(T, H * 8), dtype=torch.uint8, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, ops.prefill_workspace_bytes(T, H, inp.flags)), dtype=torch.uint8, device=dev)

    def run():
        ops.prefill(q, k, v, cu, inp.max_seqlen, inp.softmax_scale, inp.flags, inp.g_q, inp.g_k, inp.g_v,
                    inp.g_p, inp.g_out, workspace=ws, codes=codes, scales=scales, lse=lse)

    ms = timed(run, steps, warmup)
    lens = (inp.cu_seqlens[1:] - inp.cu_seqlens[:-1]).tolist()
    flops = float(sum(H * 320 * L * (L + 1) for L in lens))
    p_elems = float(sum(H * L * (L + 1) // 2 for L in lens))
    nbytes = T * H * (192 * 2 * 2 + 128 * 2) + T * H * 64 + scales.numel() + T * H * 4
    return {"tokens": T, "flags": inp.flags, "seq_lens": lens, "ms": ms, "tflops": flops / (ms * 1e-3) / 1e12,
            "frac_mfma": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "flops_per_launch": flops,
            "p_elements_per_s": p_elems / (ms * 1e-3), "gbps": nbytes / (ms * 1e-3) / 1e9}


def bench_chunked_prefill(steps: int, warmup: int) -> dict:
    """A chunk of 512 new tokens for each of 8 sequences holding 4096 cached
    tokens (paged NVFP4 cache, 432-byte records), 128 heads, Q/K/P/V NVFP4:
    gather of the 32,768 context tokens to bf16, context attention and causal
    new-token attention (fp32 rows + LSE into one [T, 2, H, 128] buffer), LSE
    merge, NVFP4 quantization of the merged rows.  The projection of the
    gathered latent (the model's kv_b_proj) is done once beforehand with torch
    and is not timed; it belongs to the model, not to this path."""
    N, C, Tn, H = 8, 4096, 512, 128
    d = workloads.small_decode(4100, N, 1, [C] * N, page_size=64, rec=432, outer=1.3)
    dev = "cuda"
    cache = torch.zeros((d.num_pages, d.page_size, d.record_bytes), dtype=torch.uint8, device=dev)
    ops.cache_write(d.kv_c.to(dev), d.k_pe.to(dev), d.slot_mapping.to(dev), cache, d.outer_scale)
    pt = d.page_table.to(dev)
    cu_ctx = torch.arange(0, (N + 1) * C, C, dtype=torch.int32, device=dev)
    kv, pe = ops.cache_gather(cache, pt, cu_ctx, C, d.outer_scale)
    g = torch.Generator().manual_seed(4101)
    w_uk = (torch.randn((512, H * 128), generator=g) / 512 ** 0.5).to(torch.bfloat16).to(dev)
    w_uv = (torch.randn((512, H * 128), generator=g) / 512 ** 0.5).to(torch.bfloat16).to(dev)
    Tc = N * C
    ctx_k = torch.cat([(kv.float() @ w_uk.float()).to(torch.bfloat16).view(Tc, H, 128),
                       pe.view(Tc, 1, 64).expand(Tc, H, 64)], dim=2).contiguous()
    ctx_v = (kv.float() @ w_uv.float()).to(torch.bfloat16).view(Tc, H, 128).contiguous()
    inp = workloads.prefill_inputs(4102, [Tn] * N, H, 15)
    q, k, v, cu_q = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.cu_seqlens.to(dev)
    T = inp.T
    part_o = torch.empty((T, 2, H, 128), dtype=torch.float32, device=dev)
    part_l = torch.empty((T, 2, H), dtype=torch.float32, device=dev)
    out = torch.empty((T, H, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws_c = torch.empty(ops.prefill_workspace_bytes(Tc, H, 15), dtype=torch.uint8, device=dev)
    ws_n = torch.empty(ops.prefill_workspace_bytes(T, H, 15), dtype=torch.uint8, device=dev)
    a = (inp.softmax_scale, 15, inp.g_q, inp.g_k, inp.g_v, inp.g_p)
    stages = {
        "gather": lambda: ops.cache_gather(cache, pt, cu_ctx, C, d.outer_scale, kv_c=kv, k_pe=pe),
        "context_attention": lambda: ops.prefill_attention(q, ctx_k, ctx_v, cu_q, Tn, *a, causal=False,
                                                           cu_seqlens_k=cu_ctx, max_seqlen_k=C, out=part_o[:, 0],
                                                           lse=part_l[:, 0], workspace=ws_c),
        "new_token_attention": lambda: ops.prefill_attention(q, k, v, cu_q, Tn, *a, causal=True, out=part_o[:, 1],
                                                             lse=part_l[:, 1], workspace=ws_n),
        "merge": lambda: ops.lse_merge(part_o, part_l, out=out, lse=lse),
        "quantize": lambda: ops.quantize_rows(out.view(T, H * 128), inp.g_v),
    }
    res = {name: timed(fn, steps, warmup) * 1e3 for name, fn in stages.items()}

    def chain():
        for fn in stages.values():
            fn()

    ms = timed(chain, steps, warmup)
    f_ctx = 2.0 * H * Tn * C * (192 + 128) * N
    f_new = float(N * H * 320 * Tn * (Tn + 1))
    return {"ms": ms, "stage_us": res, "sequences": N, "context_tokens": C, "new_tokens": Tn, "heads": H,
            "attention_tflops": (f_ctx + f_new) / (ms * 1e-3) / 1e12,
            "context_attention_frac_mfma": f_ctx / (res["context_attention"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
            "gather_gbps": Tc * (432 + 1152) / (res["gather"] * 1e-6) / 1e9}


def bench_decode_qdq(steps: int, warmup: int) -> dict:
    """Decode with quantized operands on the dense decode shape (B=64, H=128,
    L=4096, 4 splits): NVFP4 cache with Q and P NVFP4; raw bf16 cache
    (1152-byte records, rotated over 2 copies) with Q/K/P/V NVFP4 and with
    all four per-tensor FP8."""
    inp = workloads.decode_workload(1)
    dev = "cuda"
    H, B = inp.H, inp.B
    ntok = int(inp.seq_lens.sum())
    q = inp.q.to(dev)
    qn, qr = q[..., :512], q[..., 512:]
    pt, seq = inp.page_table.to(dev), inp.seq_lens.to(dev)
    out = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = torch.empty(ops.decode_workspace_bytes(B, H, inp.max_splits), dtype=torch.uint8, device=dev)
    kv, pe, slots = inp.kv_c.to(dev), inp.k_pe.to(dev), inp.slot_mapping.to(dev)

    def scale(x, fp8):
        return float(np.float32(float(x.abs().max()) / (448.0 if fp8 else 2688.0)))

    res = {}
    nv = torch.zeros((inp.num_pages, inp.page_size, 432), dtype=torch.uint8, device=dev)
    ops.cache_write(kv, pe, slots, nv, inp.outer_scale)
    nvs = [nv, nv.clone(), nv.clone(), nv.clone()]
    raw = torch.zeros((inp.num_pages, inp.page_size, 1152), dtype=torch.uint8, device=dev)
    ops.raw_cache_write(kv, pe, slots, raw)
    raws = [raw, raw.clone()]
    kvpe = torch.cat([inp.kv_c.float(), inp.k_pe.float()], 1)
    for name, caches, flags in (("nvfp4_cache_QP", nvs, 1 | 4), ("raw_cache_QKPV", raws, 15),
                                ("raw_cache_fp8", raws, 255)):
        sc = dict(g_q=scale(inp.q.float(), flags & 16), g_k=scale(kvpe, flags & 32),
                  g_v=scale(inp.kv_c.float(), flags & 128), g_p=float(np.float32(1 / (448 if flags & 64 else 2688))))
        it = [0]

        def run(caches=caches, flags=flags, sc=sc):
            r = it[0] % len(caches)
            it[0] += 1
            ops.decode_qdq(qn, qr, caches[r], pt, seq, inp.outer_scale, inp.softmax_scale, flags,
                           max_splits=inp.max_splits, out=out, lse=lse, workspace=ws, **sc)

        ms = timed(run, steps, warmup)
        rec = caches[0].shape[-1]
        nbytes = ntok * rec + B * H * 576 * 2 + B * H * 513 * 4
        fl = decode_flops(ntok, H)
        res[name] = {"kernel_us": ms * 1e3, "tflops": fl / (ms * 1e-3) / 1e12,
                     "frac_mfma": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "gbps": nbytes / (ms * 1e-3) / 1e9,
                     "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, "flags": flags, "record_bytes": rec}
    return res


def cpu_baseline(inp, budget_s: float = 12.0):
    """The oracle (unchanged) on whole sequences of the same workload, until
    the time budget is used: queries/s on the host cores."""
    from oracle import decode as OD
    from oracle import record as OR
    try:
        import threadpoolctl
        threads = max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = 1
    q = inp.q.float().numpy()
    offs = inp.token_offsets.numpy()
    done = 0
    t0 = time.perf_counter()
    while done < inp.B and (done == 0 or time.perf_counter() - t0 < budget_s):
        b = done
        cache = np.zeros((inp.num_pages, inp.page_size, inp.record_bytes), np.uint8)
        rows = np.arange(offs[b], offs[b + 1])
        kv = inp.kv_c[rows].contiguous().view(torch.int16).numpy().view(np.uint16)
        pe = inp.k_pe[rows].contiguous().view(torch.int16).numpy().view(np.uint16)
        OR.cache_write(cache, kv, pe, inp.slot_mapping.numpy()[rows], inp.outer_scale)
        OD.dense_decode(q[..., :512], q[..., 512:], cache, inp.page_table.numpy(), inp.seq_lens.numpy(),
                        inp.page_size, inp.outer_scale, inp.softmax_scale, batch=[b])
        done += 1
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "queries/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {inp.B} sequences (all {inp.H} heads, L={int(inp.seq_lens[0])}): per query the "
                      f"oracle writes the sequence's {int(inp.seq_lens[0])} tokens into its cache (the GPU step writes "
                      f"one per query) then decodes in fp64, {el:.1f} s; host cpu_count={os.cpu_count()}, "
                      f"affinity={len(os.sched_getaffinity(0))}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the 16-head, sparse, cache-write and prefill measurements")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 3 plain device copies of 256 MiB (reference kernel for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the decode path is measured "
              f"on one GPU's share", flush=True)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", flush=True)
        sys.exit(2)

    log("generating decode workload 1 (B=64, H=128, L=4096)")
    inp = workloads.decode_workload(1)
    H, B = inp.H, inp.B
    ntok = int(inp.seq_lens.sum())
    bench = DecodeBench(inp, ROTATE)
    ms_step, k_ms = bench.run(args.steps, args.warmup)
    flops = decode_flops(ntok, H)
    nbytes = decode_bytes(inp, ntok, H)
    tflops = flops / (k_ms * 1e-3) / 1e12
    gbps = nbytes / (k_ms * 1e-3) / 1e9
    log(f"decode kernel {k_ms * 1e3:.1f} us, step {ms_step * 1e3:.1f} us, {tflops:.1f} TFLOP/s, {gbps:.0f} GB/s")

    result = {
        "metric": METRIC,
        "value": B / (ms_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16/bf16 MFMA on exact NVFP4 operands, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": "dense NVFP4 MLA decode step: B=64, H=128, L=4096, page 64, 432-byte records, "
                               "4 splits + merge kernel, plus NVFP4 cache write of 64 new tokens",
                   "global_batch": B, "seq_len": 4096, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / PEAK_BF16_TFLOPS, "traffic": measured_traffic(),
                     "kernel": "decode_kernel + split_merge_kernel (one decode call)", "kernel_us": k_ms * 1e3,
                     "flops_per_launch": flops, "bytes_per_launch": nbytes},
        "hbm": {"achieved_gbps": gbps, "peak_gbps": PEAK_HBM_GBPS, "frac": gbps / PEAK_HBM_GBPS},
    }
    del bench
    torch.cuda.empty_cache()

    if not args.no_extra:
        paths = {}
        log("tiny decode (workload 0: B=1, H=16, L=256)")
        inp0 = workloads.decode_workload(0)
        b0 = DecodeBench(inp0, 1)
        _, k0 = b0.run(max(10, args.steps // 2), 5, with_write=False)
        paths["tiny_decode"] = {"kernel_us": k0 * 1e3, "note": "launch-latency bound: one decode call, "
                                "back-to-back calls between one event pair"}
        del b0, inp0
        torch.cuda.empty_cache()
        log("16-head decode (workload 1 shape, H=16)")
        inp16 = workloads.decode_workload(1, H=16)
        b16 = DecodeBench(inp16, ROTATE)
        _, k16 = b16.run(max(10, args.steps // 2), 5, with_write=False)
        by = decode_bytes(inp16, ntok, 16)
        paths["decode_H16"] = {"kernel_us": k16 * 1e3, "gbps": by / (k16 * 1e-3) / 1e9,
                               "frac_hbm": by / (k16 * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                               "queries_per_s": inp16.B / (k16 * 1e-3)}
        del b16, inp16
        torch.cuda.empty_cache()
        # Ragged decode: 128 sequences of 1k-32k tokens (2.2 M in all), e4m3
        # RoPE (368-byte records), 1% latent outliers x20, per-sequence split
        # counts; the cache (812 MB) is rotated over 2 copies.  The 16-head
        # case takes the first 16 heads of the same queries.
        log("ragged decode (workload 2: B=128, L in [1k, 32k]), 128 and 16 heads")
        inp2 = workloads.decode_workload(2)
        n2 = int(inp2.seq_lens.sum())
        for H2, key in ((128, "ragged_decode"), (16, "ragged_decode_H16")):
            inpx = inp2 if H2 == inp2.H else dataclasses.replace(inp2, H=H2, q=inp2.q[:, :H2].contiguous())
            bx = DecodeBench(inpx, 2)
            _, kx = bx.run(max(10, args.steps // 2), 3, with_write=False)
            fx, byx = decode_flops(n2, H2), decode_bytes(inpx, n2, H2)
            paths[key] = {"kernel_us": kx * 1e3, "tokens": n2,
                          "tflops": fx / (kx * 1e-3) / 1e12, "frac_mfma": fx / (kx * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                          "gbps": byx / (kx * 1e-3) / 1e9, "frac_hbm": byx / (kx * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                          "queries_per_s": inpx.B / (kx * 1e-3)}
            del bx, inpx
            torch.cuda.empty_cache()
        log("cache write of the ragged workload's 2.2 M tokens (368-byte records, e4m3 RoPE)")
        paths["cache_write_ragged"] = bench_cache_write(inp2, max(10, args.steps // 2), 3)
        torch.cuda.empty_cache()
        del inp2
        log("sparse top-k decode (workload 3)")
        inp3 = workloads.decode_workload(3)
        b3 = DecodeBench(inp3, 12, sparse=True)
        _, k3 = b3.run(max(10, args.steps // 2), 5, with_write=False)
        idx = inp3.indices
        nvalid = int(((idx >= 0) & (idx < inp3.seq_lens[:, None])).sum())
        f3 = decode_flops(nvalid, inp3.H)
        paths["sparse_decode"] = {"kernel_us": k3 * 1e3, "tflops": f3 / (k3 * 1e-3) / 1e12,
                                  "frac_mfma": f3 / (k3 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                  "queries_per_s": inp3.B / (k3 * 1e-3), "valid_indices": nvalid}
        del b3, inp3
        torch.cuda.empty_cache()
        log("stand-alone LSE merge (B=64, 4 splits, 128 heads, fp32 partials)")
        paths["lse_merge"] = bench_lse_merge(max(10, args.steps // 2), 3)
        torch.cuda.empty_cache()
        log("cache write of the decode workload's 262,144 tokens")
        paths["cache_write"] = bench_cache_write(inp, max(10, args.steps // 2), 3)
        paths["cache_write"]["note"] = ("its 113 MB cache fits the 256 MB Infinity Cache, which absorbs the writes; "
                                        "cache_write_ragged is the HBM figure")
        torch.cuda.empty_cache()
        log("prefill (8 sequences of 2k-8k tokens, 128 heads, NVFP4 output)")
        paths["prefill"] = bench_prefill(max(3, args.steps // 10), 1)
        torch.cuda.empty_cache()
        log("prefill with per-tensor FP8 Q/K/P/V")
        paths["prefill_fp8"] = bench_prefill(max(3, args.steps // 10), 1, flags=255)
        torch.cuda.empty_cache()
        log("prefill with NVFP4 Q/K/P/V and 2:4 score sparsity")
        paths["prefill_2_4"] = bench_prefill(max(3, args.steps // 10), 1, flags=15 | 256)
        torch.cuda.empty_cache()
        log("chunked prefill over the NVFP4 cache (8 x 4096 context + 8 x 512 new tokens)")
        paths["chunked_prefill"] = bench_chunked_prefill(max(3, args.steps // 5), 2)
        torch.cuda.empty_cache()
        log("decode with quantized operands (NVFP4 cache Q/P; raw cache Q/K/P/V NVFP4 and FP8)")
        paths["decode_qdq"] = bench_decode_qdq(max(10, args.steps // 2), 3)
        torch.cuda.empty_cache()
        result["paths"] = paths

    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 copies of {n} bytes")
        del src, dst

    log("roofline re-measurement (device copy, MFMA rates)")
    machine = measure_machine()
    result["machine"] = machine
    # The same achieved rates against the re-measured ceilings (the vendor
    # fractions above stay the reported ones): HBM-bound paths against the
    # read-only stream, the 16x16x32 decode kernels against that product's rate.
    result["roofline"]["frac_of_measured_mfma_16x16x32"] = tflops / machine["mfma_16x16x32_f16_tflops"]
    for key in ("decode_H16", "ragged_decode_H16"):
        if key in result.get("paths", {}):
            result["paths"][key]["frac_of_measured_hbm_read"] = result["paths"][key]["gbps"] / machine["hbm_read_gbps"]
    torch.cuda.empty_cache()

    if not args.no_cpu:
        log("oracle CPU baseline")
        result["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
