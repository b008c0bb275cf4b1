"""GPU parity on seeded random shapes, beyond the hand-picked cases: paged
decode (dense and top-k sparse) and the varlen prefill, each compared with the
oracle to the same bars as the other parity tests.

Decode draws: batch 1-4; head counts weighted towards the kernels' edges (1,
15, 16, 17, 64, 127, 128, 129, 255, 256, 300, and uniform 1-300); lengths
including 0, 1 and page/tile boundaries; page sizes 8, 16, 48, 64 with shuffled
page tables; both record widths; split caps 1-64; outer scale U[0.5, 2];
latent outliers in half of the draws; sparse draws with top-k 1-700 (some
entries -1 or past the sequence).  The oracle's work per draw is capped
(B * H * sum(L) <= 6e5) so that the whole sweep runs in about a minute.

Prefill draws: 1-5 sequences of 0-700 tokens, 1-4 heads, and the operand
formats drawn per operand: each of Q, K, P, V quantized or not, a quantized
one as NVFP4 or per-tensor FP8, and 2:4 score sparsity on or off, so that
mixed NVFP4/FP8 calls are covered.  Every draw has T * H >= 600, so that one
valid near-boundary block-scale difference (16 codes) stays within the 0.1%
code bar; the dequantized rel-L2 bar is asserted over all draws pooled.

Context attention draws (new tokens over their sequences' cached context,
fp32 output and LSE): 1-4 sequences, 0-80 new and 0-700 context tokens,
1-3 heads, formats drawn as for the prefill.

Quantized-operand decode draws: a raw bf16 cache with any subset of Q, K, P,
V quantized (each NVFP4 or FP8), or NVFP4 records with Q and P drawn (K and
V are the records' own); 1-3 sequences, 1-160 heads, split caps 1-8.
"""
import numpy as np
import pytest

from gpu_support import compare, gpu_cache, gpu_decode, oracle_cache, oracle_decode
from mla_attention_nvfp4_amd import workloads
import test_gpu_decode_qdq as TD
import test_gpu_prefill as TP
import test_gpu_prefill_ext as TE

pytestmark = pytest.mark.gpu

N_DECODE = 20
N_PREFILL = 8
EDGE_HEADS = [1, 15, 16, 17, 64, 127, 128, 129, 255, 256, 300]
EDGE_LENS = [0, 1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def decode_draw(i):
    r = np.random.default_rng(7000 + i)
    H = int(r.choice(EDGE_HEADS)) if r.random() < 0.6 else int(r.integers(1, 301))
    B = int(r.integers(1, 5))
    budget = max(64, int(6e5 // (B * H)))
    lens = []
    for _ in range(B):
        if r.random() < 0.3:
            lens.append(int(r.choice(EDGE_LENS)))
        else:
            lens.append(int(r.integers(0, min(budget, 2500) + 1)))
    while B * H * sum(lens) > 6e5:
        j = int(np.argmax(lens))
        lens[j] //= 2
    page = int(r.choice([8, 16, 48, 64]))
    rec = int(r.choice([432, 368]))
    splits = int(r.choice([1, 2, 3, 4, 5, 8, 13, 16, 64]))
    outer = float(r.uniform(0.5, 2.0))
    outliers = bool(r.random() < 0.5)
    topk = int(r.choice([0, 0, 1, 31, 32, 33, 200, 700]))
    return dict(seed=7000 + i, B=B, H=H, lens=lens, page=page, rec=rec, splits=splits, outer=outer,
                outliers=outliers, topk=topk, invalid=float(r.uniform(0, 0.3)) if topk else 0.0)


@pytest.mark.parametrize("i", range(N_DECODE), ids=[f"decode-draw{i}" for i in range(N_DECODE)])
def test_decode_random_shape(i):
    d = decode_draw(i)
    print(f"  {d}", flush=True)
    inp = workloads.small_decode(d["seed"], d["B"], d["H"], d["lens"], page_size=d["page"], rec=d["rec"],
                                 outer=d["outer"], max_splits=d["splits"], outliers=d["outliers"],
                                 topk=d["topk"], invalid_frac=d["invalid"])
    cache = gpu_cache(inp)
    out, lse = gpu_decode(inp, cache)
    batch = list(range(d["B"]))
    ref_out, ref_lse = oracle_decode(inp, batch)
    compare(out, lse, ref_out, ref_lse, batch, f"decode-draw{i}")


def prefill_draw(i):
    r = np.random.default_rng(8000 + i)
    H = int(r.integers(1, 5))
    n = int(r.integers(1, 6))
    while True:
        lens = [int(r.choice(EDGE_LENS)) if r.random() < 0.3 else int(r.integers(0, 701)) for _ in range(n)]
        if sum(lens) * H >= 600 and max(lens) >= 64:
            break
    flags = 0
    for bit in (1, 2, 4, 8):           # Q, K, P, V quantized
        if r.random() < 0.7:
            flags |= bit
            if r.random() < 0.35:      # ... as per-tensor FP8
                flags |= bit << 4
    if r.random() < 0.3:
        flags |= 256                   # 2:4 score sparsity
    return dict(seed=8000 + i, lens=lens, H=H, flags=flags)


_PREFILL_ERR = {}


def _run_prefill_draw(i):
    d = prefill_draw(i)
    print(f"  {d}", flush=True)
    inp = workloads.prefill_inputs(d["seed"], d["lens"], d["H"], d["flags"])
    gpu = TP._run_gpu(inp)
    _PREFILL_ERR[i] = TP._compare(inp, gpu, list(range(d["H"])), None, f"prefill-draw{i}")


@pytest.mark.parametrize("i", range(N_PREFILL), ids=[f"prefill-draw{i}" for i in range(N_PREFILL)])
def test_prefill_random_shape(i):
    _run_prefill_draw(i)


def test_prefill_random_shapes_pooled_rel_l2():
    for i in range(N_PREFILL):
        if i not in _PREFILL_ERR:
            _run_prefill_draw(i)
    num = sum(e[0] for e in _PREFILL_ERR.values())
    den = sum(e[1] for e in _PREFILL_ERR.values())
    rel = float(np.sqrt(num / den))
    print(f"  pooled prefill draws: dequantized rel_l2={rel:.3e}", flush=True)
    assert rel <= TP.REL_L2, f"pooled rel L2 {rel:.3e}"


def _formats(r, bits=(1, 2, 4, 8), sparse=True):
    flags = 0
    for bit in bits:
        if r.random() < 0.7:
            flags |= bit
            if r.random() < 0.35:
                flags |= bit << 4
    if sparse and r.random() < 0.3:
        flags |= 256
    return flags


N_CONTEXT = 6


@pytest.mark.parametrize("i", range(N_CONTEXT), ids=[f"context-draw{i}" for i in range(N_CONTEXT)])
def test_context_attention_random_shape(i):
    r = np.random.default_rng(9000 + i)
    n = int(r.integers(1, 5))
    new = [int(r.integers(0, 81)) for _ in range(n)]
    ctx = [int(r.choice(EDGE_LENS)) if r.random() < 0.3 else int(r.integers(0, 701)) for _ in range(n)]
    if sum(new) == 0:
        new[0] = 1
    H = int(r.integers(1, 4))
    flags = _formats(r)
    print(f"  seed={9000 + i} new={new} ctx={ctx} H={H} flags={flags}", flush=True)
    TE._context_case(9000 + i - 400, new, ctx, H, flags)


N_QDQ = 10


@pytest.mark.parametrize("i", range(N_QDQ), ids=[f"qdq-draw{i}" for i in range(N_QDQ)])
def test_decode_qdq_random_shape(i):
    r = np.random.default_rng(9500 + i)
    raw = bool(r.random() < 0.6)
    H = int(r.choice([1, 16, 17, 64, 65, 128, 160])) if r.random() < 0.6 else int(r.integers(1, 161))
    B = int(r.integers(1, 4))
    budget = max(32, int(2e5 // (B * H)))
    lens = [int(r.choice(EDGE_LENS)) if r.random() < 0.3 else int(r.integers(0, min(budget, 1500) + 1))
            for _ in range(B)]
    while B * H * sum(lens) > 2e5:
        j = int(np.argmax(lens))
        lens[j] //= 2
    splits = int(r.choice([1, 2, 3, 4, 8]))
    flags = _formats(r, (1, 2, 4, 8) if raw else (1, 4), sparse=False)
    rec = 432 if raw else int(r.choice([432, 368]))
    print(f"  seed={9500 + i} raw={raw} B={B} H={H} lens={lens} splits={splits} flags={flags} rec={rec}", flush=True)
    inp = workloads.small_decode(9500 + i, B, H, lens, page_size=int(r.choice([16, 64])), rec=rec,
                                 outer=float(r.uniform(0.5, 2.0)), max_splits=splits)
    batch = list(range(B))
    cg, co = TD._raw_caches(inp) if raw else (gpu_cache(inp), oracle_cache(inp, batch))
    sc = TD._scales(inp, flags)
    out, lse, ro, rl, args = TD._run(inp, cg, co, flags, sc, splits, batch)
    TD._check(out, lse, ro, rl, batch, args, flags, f"qdq-draw{i}")
