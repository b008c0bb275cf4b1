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
"""
import numpy as np
import pytest

from gpu_support import compare, gpu_cache, gpu_decode, oracle_decode
from mla_attention_nvfp4_amd import workloads
import test_gpu_prefill as TP

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
