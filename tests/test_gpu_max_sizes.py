"""GPU parity at the largest sizes the decode calls accept: H = 4096 heads (32
groups of 128 heads, the grid's head-group dimension, and 1024 workgroups of 4
heads per sequence in the split merge) and B = 65535 sequences (the grid's
sequence dimension), for the 16-head and the 128-head kernels and the
quantized-operand decode.  At B = 65535 the oracle checks a sample of
sequences one by one, and every row's empty / non-empty pattern is checked."""
import numpy as np
import pytest
import torch

from gpu_support import compare, gpu_cache, oracle_cache
from mla_attention_nvfp4_amd import ops, workloads
from oracle import decode as OD
import test_gpu_decode_qdq as TD

pytestmark = pytest.mark.gpu

MAX_B, MAX_H = 65535, 4096


def _oracle_rows(inp, sample):
    """Oracle out / lse of the sequences in ``sample`` (rows in that order)."""
    cache = oracle_cache(inp, sample)
    q = inp.q[sample].float().numpy()
    pt, sl = inp.page_table.numpy()[sample], inp.seq_lens.numpy()[sample]
    args = (q[..., :512], q[..., 512:], cache, pt, sl, inp.page_size, inp.outer_scale, inp.softmax_scale)
    if inp.indices is None:
        return OD.dense_decode(*args)
    return OD.sparse_decode(*args, inp.indices.numpy()[sample])


def _decode(inp, cache):
    q = inp.q.cuda()
    args = (q[..., :512], q[..., 512:], cache, inp.page_table.cuda(), inp.seq_lens.cuda())
    if inp.indices is None:
        out, lse = ops.decode(*args, inp.outer_scale, inp.softmax_scale, inp.max_splits)
    else:
        out, lse = ops.sparse_decode(*args, inp.indices.cuda(), inp.outer_scale, inp.softmax_scale, inp.max_splits)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("sparse", [False, True], ids=["dense", "sparse"])
def test_decode_4096_heads(sparse):
    inp = workloads.small_decode(93, 2, MAX_H, [300, 65], page_size=64, rec=432, max_splits=3,
                                 topk=200 if sparse else 0)
    print(f"  H={MAX_H} sparse={sparse} lens=[300, 65] splits=3", flush=True)
    out, lse = _decode(inp, gpu_cache(inp))
    ref_o, ref_l = _oracle_rows(inp, [0, 1])
    compare(out.cpu().double().numpy(), lse.cpu().double().numpy(), ref_o, ref_l, [0, 1], f"H{MAX_H}")


@pytest.mark.parametrize("H", [16, 17], ids=["narrow", "wide"])
def test_decode_65535_sequences(H):
    g = torch.Generator().manual_seed(94 + H)
    lens = torch.randint(0, 21, (MAX_B,), generator=g).tolist()
    lens[0], lens[1], lens[-1] = 0, 1, 20
    inp = workloads.small_decode(94 + H, MAX_B, H, lens, page_size=16, rec=432, max_splits=2)
    print(f"  B={MAX_B} H={H} tokens={int(inp.seq_lens.sum())} splits=2", flush=True)
    out, lse = _decode(inp, gpu_cache(inp))
    rng = np.random.default_rng(95 + H)
    sample = sorted({0, 1, MAX_B - 2, MAX_B - 1, *rng.choice(MAX_B, 44, replace=False).tolist()})
    idx = torch.tensor(sample, device="cuda")
    o = out.index_select(0, idx).cpu().double().numpy()
    lo = lse.index_select(0, idx).cpu().double().numpy()
    ref_o, ref_l = _oracle_rows(inp, sample)
    compare(o, lo, ref_o, ref_l, list(range(len(sample))), f"B{MAX_B}-H{H}")
    # every row: empty sequences give out = 0 and lse = -inf, the others finite
    empty = (inp.seq_lens == 0).cuda()
    assert torch.equal(torch.isneginf(lse), empty[:, None].expand(-1, H))
    assert torch.isfinite(out).all() and (out[empty] == 0).all()


def test_decode_qdq_4096_heads():
    flags = 15
    inp = workloads.small_decode(96, 1, MAX_H, [200], page_size=64, rec=432, max_splits=2)
    print(f"  quantized-operand decode, raw cache, H={MAX_H}, flags={flags}", flush=True)
    cg, co = TD._raw_caches(inp)
    sc = TD._scales(inp, flags)
    out, lse, ro, rl, args = TD._run(inp, cg, co, flags, sc, 2, [0])
    TD._check(out, lse, ro, rl, [0], args, flags, f"qdq-H{MAX_H}")
