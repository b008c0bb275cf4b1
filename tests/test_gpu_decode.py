"""GPU parity: dense and sparse paged decode and the LSE merge against the
oracle, on small ragged cases, edge cases and the full workload sizes."""
import numpy as np
import pytest
import torch

from gpu_support import compare, gpu_cache, gpu_decode, oracle_decode
from mla_attention_nvfp4_amd import ops, workloads
from oracle import decode as OD

pytestmark = pytest.mark.gpu

SMALL_DENSE = [
    # seed, B, H, lens, page, rec, outer, splits
    (1, 3, 16, [0, 1, 65], 64, 432, 1.0, 1),
    (2, 4, 20, [63, 64, 130, 300], 16, 368, 0.75, 3),
    (3, 2, 128, [1000, 513], 64, 432, 1.7, 4),
    (4, 5, 32, [5, 200, 129, 64, 1], 48, 432, 0.55, 2),
    (5, 2, 64, [2049, 4096], 64, 368, 1.3, 16),
    (6, 1, 1, [77], 8, 432, 1.0, 1),
    (8, 3, 16, [700, 33, 2000], 16, 368, 1.4, 3),     # narrow heads, e4m3 RoPE, outliers
    (9, 2, 7, [300, 1029], 48, 432, 0.6, 2),          # narrow, 7 heads
    (10, 2, 100, [555, 1200], 64, 368, 1.1, 2),       # wide, partial head group
    (16, 2, 256, [700, 1500], 64, 432, 1.2, 3),       # two 128-head groups
    (17, 1, 300, [400], 16, 368, 0.9, 2),             # three head groups, the last partial
    # batches of 8 (the split merge then runs sequence b on XCD b % 8) with
    # head counts that leave the merge's last group of 4 heads partial
    (19, 8, 15, [0, 1, 65, 300, 129, 700, 33, 256], 16, 432, 1.0, 3),
    (20, 8, 130, [64, 700, 1, 300, 0, 257, 900, 40], 64, 368, 0.8, 3),
    (23, 16, 17, [300, 5, 129, 64, 700, 1, 0, 200, 33, 256, 513, 90, 64, 128, 31, 400], 48, 432, 1.1, 2),
]


@pytest.mark.parametrize("case", SMALL_DENSE, ids=[f"dense{c[0]}" for c in SMALL_DENSE])
def test_dense_small(case):
    seed, B, H, lens, page, rec, outer, splits = case
    inp = workloads.small_decode(seed, B, H, lens, page_size=page, rec=rec, outer=outer,
                                 max_splits=splits, outliers=(seed % 2 == 0))
    print(f"  dense seed={seed} B={B} H={H} lens={lens} page={page} rec={rec} splits={splits}", flush=True)
    cache = gpu_cache(inp)
    out, lse = gpu_decode(inp, cache)
    ref_out, ref_lse = oracle_decode(inp, list(range(B)))
    compare(out, lse, ref_out, ref_lse, list(range(B)), f"dense{seed}")


# Latent magnitudes around the single-pass bound of the PV product (|V| near
# 8 at 1.9 sigma): tiles with and without the residual sweep in one
# sequence, for the 128-head and the 16-head kernels.
PV_BOUND = [
    # seed, B, H, lens, page, rec, splits
    (30, 2, 128, [1500, 700], 64, 432, 2),
    (31, 2, 16, [1500, 700], 64, 368, 2),
]


@pytest.mark.parametrize("case", PV_BOUND, ids=[f"pvbound{c[0]}" for c in PV_BOUND])
def test_dense_pv_bound(case):
    seed, B, H, lens, page, rec, splits = case
    inp = workloads.small_decode(seed, B, H, lens, page_size=page, rec=rec, max_splits=splits, kv_gain=1.9)
    print(f"  pv-bound seed={seed} B={B} H={H} lens={lens} max|kv|={float(inp.kv_c.float().abs().max()):.2f}",
          flush=True)
    cache = gpu_cache(inp)
    out, lse = gpu_decode(inp, cache)
    ref_out, ref_lse = oracle_decode(inp, list(range(B)))
    compare(out, lse, ref_out, ref_lse, list(range(B)), f"pvbound{seed}")


@pytest.mark.parametrize("H", [128, 16], ids=["wide", "narrow"])
def test_dense_mixed_partial_formats(H):
    """Outliers only in the first 300 positions of each sequence: the first
    split exceeds the latent bound (fp32 partial), the later ones do not
    (fp16 partials), and the merge sees both formats in one sequence."""
    inp = workloads.small_decode(40 + H, 2, H, [2048, 1500], page_size=64, rec=432, max_splits=4)
    g = torch.Generator().manual_seed(41)
    for b in range(inp.B):
        r0 = int(inp.token_offsets[b])
        blk = inp.kv_c[r0:r0 + 300]
        hit = torch.rand(blk.shape, generator=g) < 0.01
        blk[hit] = (blk[hit].to(torch.float32) * 20).to(torch.bfloat16)
    cache = gpu_cache(inp)
    out, lse = gpu_decode(inp, cache)
    ref_out, ref_lse = oracle_decode(inp, list(range(inp.B)))
    compare(out, lse, ref_out, ref_lse, list(range(inp.B)), f"mixed-formats-H{H}")


@pytest.mark.parametrize("H", [32, 8], ids=["wide", "narrow"])
def test_dense_more_than_64_splits(H):
    """67 splits of one sequence: the merge's path for more splits than lanes."""
    inp = workloads.small_decode(50 + H, 1, H, [17000], page_size=64, rec=368, max_splits=80)
    assert ops.decode_num_splits(17000, 80) == 67
    cache = gpu_cache(inp)
    out, lse = gpu_decode(inp, cache)
    ref_out, ref_lse = oracle_decode(inp, [0])
    compare(out, lse, ref_out, ref_lse, [0], f"67-splits-H{H}")


SMALL_SPARSE = [
    # seed, B, H, lens, topk, invalid_frac, splits
    (11, 3, 16, [100, 0, 700], 96, 0.1, 1),
    (12, 3, 16, [100, 5, 700], 96, 0.1, 2),
    (13, 2, 128, [5000, 3000], 512, 0.1, 4),
    (14, 2, 48, [64, 300], 130, 0.5, 3),
    (18, 2, 256, [3000, 800], 300, 0.1, 2),           # two 128-head groups
    (24, 8, 18, [900, 100, 0, 600, 2000, 64, 300, 1200], 260, 0.1, 3),   # batch of 8, 18 heads
]


@pytest.mark.parametrize("case", SMALL_SPARSE, ids=[f"sparse{c[0]}" for c in SMALL_SPARSE])
def test_sparse_small(case):
    seed, B, H, lens, topk, bad, splits = case
    inp = workloads.small_decode(seed, B, H, lens, page_size=64, rec=432, outer=1.2, max_splits=splits,
                                 topk=topk, invalid_frac=bad)
    print(f"  sparse seed={seed} B={B} H={H} lens={lens} topk={topk} splits={splits}", flush=True)
    cache = gpu_cache(inp)
    out, lse = gpu_decode(inp, cache)
    ref_out, ref_lse = oracle_decode(inp, list(range(B)))
    compare(out, lse, ref_out, ref_lse, list(range(B)), f"sparse{seed}")


def test_sparse_narrow_fp8_rope():
    inp = workloads.small_decode(15, 2, 16, [900, 300], page_size=16, rec=368, outer=0.8, max_splits=3,
                                 topk=200, invalid_frac=0.2)
    cache = gpu_cache(inp)
    out, lse = gpu_decode(inp, cache)
    ref_out, ref_lse = oracle_decode(inp, [0, 1])
    compare(out, lse, ref_out, ref_lse, [0, 1], "sparse15")


def test_sparse_all_masked_and_masked_pages():
    inp = workloads.small_decode(21, 2, 16, [200, 200], page_size=64, rec=432, topk=64)
    inp.indices[0] = -1                       # nothing valid for sequence 0
    cache = gpu_cache(inp)
    out, lse = gpu_decode(inp, cache)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    ref_out, ref_lse = oracle_decode(inp, [1])
    compare(out, lse, ref_out, ref_lse, [1], "sparse-masked")


@pytest.mark.parametrize("H", [16, 128], ids=["narrow", "wide"])
def test_out_of_range_page_ids_are_masked(H):
    """A page id outside the cache masks its tokens instead of being read:
    the result is the oracle's attention over the remaining tokens (its
    sparse decode over every position but those of the masked page)."""
    inp = workloads.small_decode(22, 2, H, [192, 300], page_size=64, rec=432, max_splits=2)
    cache = gpu_cache(inp)
    pt = inp.page_table.clone()
    pt[0, 1] = 10 ** 6
    pt[1, 3] = -5
    q = inp.q.cuda()
    out, lse = ops.decode(q[..., :512], q[..., 512:], cache, pt.cuda(), inp.seq_lens.cuda(),
                          inp.outer_scale, inp.softmax_scale, 2)
    torch.cuda.synchronize()
    keep = [[j for j in range(192) if j // 64 != 1], [j for j in range(300) if j // 64 != 3]]
    idx = np.full((2, 300), -1, np.int64)
    for b in range(2):
        idx[b, :len(keep[b])] = keep[b]
    inp.indices = torch.from_numpy(idx.astype(np.int32))      # the oracle's reference only
    ref_out, ref_lse = oracle_decode(inp, [0, 1])
    compare(out.cpu().double().numpy(), lse.cpu().double().numpy(), ref_out, ref_lse, [0, 1],
            f"masked-pages-H{H}")


def test_split_counts_agree_and_runs_are_deterministic():
    inp = workloads.small_decode(31, 3, 128, [4096, 1500, 300], page_size=64, rec=432, outer=0.9)
    cache = gpu_cache(inp)
    ref_out, ref_lse = oracle_decode(inp, [0, 1, 2])
    base = None
    for splits in (1, 2, 4, 7, 16):
        out, lse = gpu_decode(inp, cache, max_splits=splits)
        compare(out, lse, ref_out, ref_lse, [0, 1, 2], f"splits={splits}")
        out2, lse2 = gpu_decode(inp, cache, max_splits=splits)
        assert np.array_equal(out, out2) and np.array_equal(lse, lse2), "not bitwise deterministic"
        if base is None:
            base = out


def test_lse_merge_kernel():
    rng = np.random.default_rng(40)
    B, S, H, D = 5, 6, 7, 512
    po = rng.standard_normal((B, S, H, D)).astype(np.float32)
    pl = rng.standard_normal((B, S, H)).astype(np.float32) * 3
    pl[0, 2] = -np.inf
    pl[1] = -np.inf                           # all empty
    pl[2, :, 3] = -np.inf
    counts = np.array([6, 6, 3, 0, 1], np.int32)
    out, lse = ops.lse_merge(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(),
                             torch.from_numpy(counts).cuda())
    torch.cuda.synchronize()
    out, lse = out.cpu().double().numpy(), lse.cpu().double().numpy()
    for b in range(B):
        n = counts[b]
        if n == 0:
            ro, rl = np.zeros((H, D)), np.full(H, -np.inf)
        else:
            ro, rl = OD.lse_merge(po[b, :n], pl[b, :n])
        assert np.array_equal(np.isneginf(lse[b]), np.isneginf(rl))
        fin = ~np.isneginf(rl)
        assert np.allclose(out[b], ro, rtol=1e-5, atol=1e-6)
        assert np.allclose(lse[b][fin], rl[fin], rtol=0, atol=1e-5)
    # no count array: all S splits
    out, lse = ops.lse_merge(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda())
    torch.cuda.synchronize()
    ro, rl = OD.lse_merge(po[3], pl[3])
    assert np.allclose(out.cpu().numpy()[3], ro, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("B,S,H,D", [(4, 1, 3, 4), (3, 64, 5, 100), (3, 70, 5, 100), (2, 17, 9, 4096)])
def test_lse_merge_shapes(B, S, H, D):
    """Split counts at and past one wavefront's lanes (64), a single split,
    the smallest and largest rows, ragged per-sequence counts, empty splits."""
    rng = np.random.default_rng(B * 1000 + S * 10 + D)
    po = rng.standard_normal((B, S, H, D)).astype(np.float32)
    pl = (rng.standard_normal((B, S, H)) * 4).astype(np.float32)
    pl[rng.uniform(size=(B, S, H)) < 0.2] = -np.inf
    counts = rng.integers(0, S + 1, B).astype(np.int32)
    counts[0] = S
    out, lse = ops.lse_merge(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(),
                             torch.from_numpy(counts).cuda())
    torch.cuda.synchronize()
    out, lse = out.cpu().double().numpy(), lse.cpu().double().numpy()
    for b in range(B):
        n = counts[b]
        if n == 0:
            ro, rl = np.zeros((H, D)), np.full(H, -np.inf)
        else:
            ro, rl = OD.lse_merge(po[b, :n], pl[b, :n])
        assert np.array_equal(np.isneginf(lse[b]), np.isneginf(rl))
        fin = ~np.isneginf(rl)
        assert np.allclose(out[b], ro, rtol=1e-5, atol=1e-6)
        assert np.allclose(lse[b][fin], rl[fin], rtol=0, atol=1e-5)


FULL = [(0, None), (1, None), (1, 16), (2, None), (2, 16), (3, None)]


@pytest.mark.parametrize("n,H", FULL, ids=[f"workload{n}" + (f"-H{H}" if H else "") for n, H in FULL])
def test_workload_full_size(n, H, decode_workload):
    """Full workload sizes in the launch configuration the benchmark times;
    the oracle checks a subset of sequences (all heads)."""
    inp = decode_workload(n, H)
    cache = gpu_cache(inp)
    out, lse = gpu_decode(inp, cache)
    batch = {0: [0], 1: [0, 1], 2: [0, 1, 2, 3], 3: [0, 1, 2, 3]}[n]
    ref_out, ref_lse = oracle_decode(inp, batch)
    compare(out, lse, ref_out, ref_lse, batch, f"workload{n} H={inp.H}")
    # every sequence, including those the oracle skipped, must be finite
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
