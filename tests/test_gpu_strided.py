"""Strided operands: the calls take Q (and the prefill's K, V) through their
row and head strides, so views into larger buffers are read in place.  Each
call on such views is compared bit for bit with the same call on contiguous
copies of the same values (the same kernels and arithmetic, other addresses),
and the contiguous result is itself checked against the oracle by the other
parity tests."""
import pytest
import torch

from gpu_support import gpu_cache
from mla_attention_nvfp4_amd import ops, workloads

pytestmark = pytest.mark.gpu


def _q_views(inp):
    """(contiguous Q, Q as a slice of a wider row, Q as every other head)."""
    q = inp.q.cuda()
    B, H, D = q.shape
    wide = torch.zeros((B, H, 2 * D), dtype=q.dtype, device="cuda")
    wide[..., D // 2:D // 2 + D] = q
    heads = torch.zeros((B, 2 * H, D), dtype=q.dtype, device="cuda")
    heads[:, 1::2] = q
    return q, wide[..., D // 2:D // 2 + D], heads[:, 1::2]


@pytest.mark.parametrize("H", [16, 128])
@pytest.mark.parametrize("sparse", [False, True])
def test_decode_strided_q(H, sparse):
    inp = workloads.small_decode(81, 3, H, [700, 65, 1300], page_size=64, rec=432, max_splits=3,
                                 topk=300 if sparse else 0)
    cache = gpu_cache(inp)
    pt, sl = inp.page_table.cuda(), inp.seq_lens.cuda()
    outs = []
    for q in _q_views(inp):
        assert q.stride(2) == 1
        if sparse:
            o = ops.sparse_decode(q[..., :512], q[..., 512:], cache, pt, sl, inp.indices.cuda(), inp.outer_scale,
                                  inp.softmax_scale, inp.max_splits)
        else:
            o = ops.decode(q[..., :512], q[..., 512:], cache, pt, sl, inp.outer_scale, inp.softmax_scale,
                           inp.max_splits)
        torch.cuda.synchronize()
        outs.append(o)
    print(f"  H={H} sparse={sparse}: strides {[tuple(v.stride()) for v in _q_views(inp)]}", flush=True)
    for o in outs[1:]:
        assert torch.equal(o[0], outs[0][0]) and torch.equal(o[1], outs[0][1])


def test_decode_qdq_raw_cache_strided_q():
    inp = workloads.small_decode(82, 2, 64, [500, 129], page_size=64, rec=432, max_splits=2)
    raw = torch.zeros((inp.num_pages, inp.page_size, 1152), dtype=torch.uint8, device="cuda")
    ops.raw_cache_write(inp.kv_c.cuda(), inp.k_pe.cuda(), inp.slot_mapping.cuda(), raw)
    pt, sl = inp.page_table.cuda(), inp.seq_lens.cuda()
    amax = float(inp.kv_c.float().abs().max())
    sc = dict(g_q=float(inp.q.float().abs().max()) / 2688, g_k=max(amax, float(inp.k_pe.float().abs().max())) / 2688,
              g_v=amax / 2688, g_p=1 / 2688)
    outs = []
    for q in _q_views(inp):
        outs.append(ops.decode_qdq(q[..., :512], q[..., 512:], raw, pt, sl, inp.outer_scale, inp.softmax_scale, 15,
                                   max_splits=2, **sc))
        torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o[0], outs[0][0]) and torch.equal(o[1], outs[0][1])


@pytest.mark.parametrize("flags", [15, 255, 15 | 256])
def test_prefill_packed_qkv(flags):
    """Q, K, V as views into one packed [T, H, 512] buffer (192 + 192 + 128)."""
    inp = workloads.prefill_inputs(83, [300, 129, 1], 3, flags)
    q, k, v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    packed = torch.cat([q, k, v], dim=2)
    pq, pk, pv = packed[..., :192], packed[..., 192:384], packed[..., 384:]
    cu = inp.cu_seqlens.cuda()
    a = (inp.max_seqlen, inp.softmax_scale, flags, inp.g_q, inp.g_k, inp.g_v, inp.g_p, inp.g_out)
    ref = ops.prefill(q, k, v, cu, *a)
    got = ops.prefill(pq, pk, pv, cu, *a)
    torch.cuda.synchronize()
    for x, y in zip(ref, got):
        assert torch.equal(x, y)
    # the fp32-output attention over the same views (causal)
    b = (inp.max_seqlen, inp.softmax_scale, flags & ~256, inp.g_q, inp.g_k, inp.g_v, inp.g_p)
    ro, rl = ops.prefill_attention(q, k, v, cu, *b)
    go, gl = ops.prefill_attention(pq, pk, pv, cu, *b)
    torch.cuda.synchronize()
    assert torch.equal(ro, go) and torch.equal(rl, gl)
