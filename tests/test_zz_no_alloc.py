"""GPU test of the allocation-free decode entry point: its output equals the
workspace entry point's (same kernels, same summation order: bit for bit) and
the oracle's within the decode tolerances, on two calls in a row, the second
with a smaller input, and it refuses a request larger than its scratch."""
import numpy as np
import pytest
import torch

from gpu_support import compare, gpu_cache, oracle_decode
from mla_attention_nvfp4_amd import MlaError, ops, workloads

pytestmark = pytest.mark.gpu


def _both(inp, cache):
    q = inp.q.cuda()
    args = (q[..., :512], q[..., 512:], cache, inp.page_table.cuda(), inp.seq_lens.cuda(), inp.outer_scale,
            inp.softmax_scale, inp.max_splits)
    ref = ops.decode(*args)
    got = ops.decode_noalloc(*args)
    torch.cuda.synchronize()
    return [t.cpu().double().numpy() for t in (*got, *ref)]


def test_noalloc_decode_matches_workspace_decode_twice():
    cases = [
        workloads.small_decode(60, 4, 128, [3000, 4096, 1000, 2500], page_size=64, rec=432, outer=1.3,
                               max_splits=4),
        workloads.small_decode(61, 2, 16, [700, 300], page_size=16, rec=368, outer=0.7, max_splits=3),
    ]
    for n, inp in enumerate(cases):
        print(f"  call {n}: B={inp.B} H={inp.H} lens={inp.seq_lens.tolist()} splits={inp.max_splits}", flush=True)
        cache = gpu_cache(inp)
        out, lse, ref_out, ref_lse = _both(inp, cache)
        assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse), f"call {n}: differs from mla_decode_nvfp4"
        batch = list(range(inp.B))
        o_out, o_lse = oracle_decode(inp, batch)
        compare(out, lse, o_out, o_lse, batch, f"noalloc call {n}")


def test_noalloc_decode_refuses_more_than_its_scratch():
    inp = workloads.small_decode(62, 2, 128, [300, 300], page_size=64, rec=432, max_splits=1)
    cache = gpu_cache(inp)
    q = inp.q.cuda()
    B, H = 600, 128
    need = ops.decode_workspace_bytes(B, H, 8)
    assert need > 128 << 20
    qb = torch.zeros((B, H, 576), dtype=torch.bfloat16, device="cuda")
    pt = torch.zeros((B, 1), dtype=torch.int32, device="cuda")
    sl = torch.zeros(B, dtype=torch.int32, device="cuda")
    with pytest.raises(MlaError) as e:
        ops.decode_noalloc(qb[..., :512], qb[..., 512:], cache, pt, sl, 1.0, 0.04, 8)
    assert e.value.status == -4
    # a request that fits still runs after the refusal
    out, lse = ops.decode_noalloc(q[..., :512], q[..., 512:], cache, inp.page_table.cuda(), inp.seq_lens.cuda(),
                                  inp.outer_scale, inp.softmax_scale, 1)
    torch.cuda.synchronize()
    o_out, o_lse = oracle_decode(inp, [0, 1])
    compare(out.cpu().double().numpy(), lse.cpu().double().numpy(), o_out, o_lse, [0, 1], "noalloc after refusal")
