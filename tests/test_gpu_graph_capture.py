"""HIP graph capture of the library's calls.  A serving step (the NVFP4 cache
write of each sequence's new token, then the paged decode with its split
merge), the allocation-free decode and the varlen prefill are captured into
graphs on a side stream and replayed several times, with new inputs copied
into the captured buffers, other eager calls and synchronizations between the
replays.  Every replay is compared bit for bit with the same call made
eagerly on the same inputs (the kernels are deterministic).  The calls launch
kernels only (no allocation, copy, memset or host synchronization), which is
what capture needs."""
import pytest
import torch

from gpu_support import gpu_cache
from mla_attention_nvfp4_amd import ops, workloads

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _randn_bf16(gen, shape):
    return torch.randn(shape, generator=gen).to(torch.bfloat16).cuda()


def _decode_setup(seed):
    inp = workloads.small_decode(seed, 4, 128, [900, 1500, 64, 2047], page_size=64, rec=432, max_splits=4)
    B, H = inp.B, inp.H
    s = dict(inp=inp, cache=gpu_cache(inp), pt=inp.page_table.cuda(), sl=inp.seq_lens.cuda(),
             q=torch.empty((B, H, 576), dtype=torch.bfloat16, device="cuda"),
             new_kv=torch.empty((B, 576), dtype=torch.bfloat16, device="cuda"),
             slots=inp.slot_mapping[inp.token_offsets[1:] - 1].cuda(),
             out=torch.empty((B, H, 512), dtype=torch.float32, device="cuda"),
             lse=torch.empty((B, H), dtype=torch.float32, device="cuda"))
    s["ws"] = torch.empty(max(1, ops.decode_workspace_bytes(B, H, 4)), dtype=torch.uint8, device="cuda")
    return s


def test_decode_step_graph_replays_match_eager():
    s = _decode_setup(71)
    inp = s["inp"]
    gen = torch.Generator().manual_seed(72)
    inputs = [(_randn_bf16(gen, s["q"].shape), _randn_bf16(gen, s["new_kv"].shape)) for _ in range(REPLAYS)]

    def step():
        ops.cache_write(s["new_kv"][:, :512], s["new_kv"][:, 512:], s["slots"], s["cache"], inp.outer_scale)
        ops.decode(s["q"][..., :512], s["q"][..., 512:], s["cache"], s["pt"], s["sl"], inp.outer_scale,
                   inp.softmax_scale, 4, out=s["out"], lse=s["lse"], workspace=s["ws"])

    ref = []
    for q, kv in inputs:
        s["q"].copy_(q)
        s["new_kv"].copy_(kv)
        step()
        torch.cuda.synchronize()
        ref.append((s["out"].clone(), s["lse"].clone()))
    s["new_kv"].copy_(inputs[0][1])
    s["q"].copy_(inputs[0][0])
    g = _capture(step)
    other = torch.empty_like(s["out"]), torch.empty_like(s["lse"])
    for k, (q, kv) in enumerate(inputs):
        s["q"].copy_(q)
        s["new_kv"].copy_(kv)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"  replay {k}: out and lse equal to the eager step", flush=True)
        assert torch.equal(s["out"], ref[k][0]) and torch.equal(s["lse"], ref[k][1]), f"replay {k}"
        # eager work of the program between replays
        ops.decode(q[..., :512], q[..., 512:], s["cache"], s["pt"], s["sl"], inp.outer_scale, inp.softmax_scale, 2,
                   out=other[0], lse=other[1])
        torch.cuda.synchronize()


def test_noalloc_decode_graph_replays_match_eager():
    s = _decode_setup(73)
    inp = s["inp"]
    gen = torch.Generator().manual_seed(74)
    qs = [_randn_bf16(gen, s["q"].shape) for _ in range(REPLAYS)]

    def call():
        ops.decode_noalloc(s["q"][..., :512], s["q"][..., 512:], s["cache"], s["pt"], s["sl"], inp.outer_scale,
                           inp.softmax_scale, 4, out=s["out"], lse=s["lse"])

    ref = []
    for q in qs:
        s["q"].copy_(q)
        call()
        torch.cuda.synchronize()
        ref.append((s["out"].clone(), s["lse"].clone()))
    s["q"].copy_(qs[0])
    g = _capture(call)
    for k, q in enumerate(qs):
        s["q"].copy_(q)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(s["out"], ref[k][0]) and torch.equal(s["lse"], ref[k][1]), f"replay {k}"
        # an eager call of the same entry point between replays (it shares the scratch)
        ops.decode_noalloc(q[..., :512], q[..., 512:], s["cache"], s["pt"], s["sl"], inp.outer_scale,
                           inp.softmax_scale, 2)
        torch.cuda.synchronize()


def test_prefill_graph_replays_match_eager():
    lens, H, flags = [300, 129, 1], 4, 15
    base = workloads.prefill_inputs(75, lens, H, flags)
    T = base.T
    dev = "cuda"
    q = torch.empty((T, H, 192), dtype=torch.bfloat16, device=dev)
    k = torch.empty_like(q)
    v = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
    cu = base.cu_seqlens.cuda()
    codes = torch.empty((T, H, 64), dtype=torch.uint8, device=dev)
    scales = torch.empty(ops.swizzled_scale_bytes(T, H * 8), dtype=torch.uint8, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, ops.prefill_workspace_bytes(T, H, flags)), dtype=torch.uint8, device=dev)
    gen = torch.Generator().manual_seed(76)
    inputs = [(_randn_bf16(gen, q.shape), _randn_bf16(gen, k.shape), _randn_bf16(gen, v.shape))
              for _ in range(REPLAYS)]

    def call():
        ops.prefill(q, k, v, cu, base.max_seqlen, base.softmax_scale, flags, base.g_q, base.g_k, base.g_v,
                    base.g_p, base.g_out, workspace=ws, codes=codes, scales=scales, lse=lse)

    ref = []
    for x in inputs:
        for dst, src in zip((q, k, v), x):
            dst.copy_(src)
        call()
        torch.cuda.synchronize()
        ref.append((codes.clone(), scales.clone(), lse.clone()))
    for dst, src in zip((q, k, v), inputs[0]):
        dst.copy_(src)
    g = _capture(call)
    for n, x in enumerate(inputs):
        for dst, src in zip((q, k, v), x):
            dst.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(codes, ref[n][0]) and torch.equal(scales, ref[n][1]) and torch.equal(lse, ref[n][2]), \
            f"replay {n}"
