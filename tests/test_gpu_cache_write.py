"""GPU parity: the cache-write kernel against the oracle, bit for bit."""
import numpy as np
import pytest
import torch

from gpu_support import bits, gpu_cache
from mla_attention_nvfp4_amd import ops, workloads
from oracle import record as OR

pytestmark = pytest.mark.gpu


def _check_records(inp, cache, rows):
    flat = cache.view(-1, inp.record_bytes)
    slots = inp.slot_mapping[rows]
    got = flat[slots.cuda()].cpu().numpy()
    want = OR.pack_records(bits(inp.kv_c[rows]), bits(inp.k_pe[rows]), inp.outer_scale, inp.record_bytes)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at (row, byte) {bad[:5].tolist()}"


@pytest.mark.parametrize("rec", [432, 368])
@pytest.mark.parametrize("outer", [1.0, 0.6180339887, 1.9])
def test_small_records_bit_exact(rec, outer):
    inp = workloads.small_decode(100 + rec, 3, 16, [70, 1, 129], page_size=16, rec=rec, outer=outer,
                                 outliers=True)
    cache = gpu_cache(inp, fill=0xAB)
    _check_records(inp, cache, np.arange(inp.kv_c.shape[0]))


def test_skipped_slots_leave_cache_untouched():
    inp = workloads.small_decode(7, 2, 16, [40, 40], page_size=16, rec=432)
    T = inp.kv_c.shape[0]
    slots = inp.slot_mapping.clone()
    slots[3] = -1
    slots[10] = 10 ** 9          # beyond the cache: skipped by the kernel
    slots[11] = -77
    cache = torch.full((inp.num_pages, inp.page_size, inp.record_bytes), 0xAB, dtype=torch.uint8, device="cuda")
    ops.cache_write(inp.kv_c.cuda(), inp.k_pe.cuda(), slots.cuda(), cache, inp.outer_scale)
    flat = cache.view(-1, 432).cpu().numpy()
    want = np.full_like(flat, 0xAB)
    keep = slots >= 0
    keep &= slots < flat.shape[0]
    OR.cache_write(want, bits(inp.kv_c), bits(inp.k_pe), np.where(keep.numpy(), slots.numpy(), -1),
                   inp.outer_scale)
    assert np.array_equal(flat, want)


def test_strided_inputs():
    """kv_c and k_pe as column slices of one [T, 576] tensor."""
    inp = workloads.small_decode(8, 1, 16, [100], page_size=64, rec=368, outer=0.75)
    both = torch.cat([inp.kv_c, inp.k_pe], dim=1).cuda()
    cache = torch.zeros((inp.num_pages, 64, 368), dtype=torch.uint8, device="cuda")
    ops.cache_write(both[:, :512], both[:, 512:], inp.slot_mapping.cuda(), cache, inp.outer_scale)
    _check_records(inp, cache, np.arange(100))


@pytest.mark.parametrize("n", [0, 1, 2, 3])
def test_workload_records_bit_exact(n, decode_workload):
    inp = decode_workload(n)
    cache = gpu_cache(inp)
    T = inp.kv_c.shape[0]
    rows = np.arange(T) if n == 0 else np.random.default_rng(n).choice(T, 1024, replace=False)
    print(f"  workload {n}: T={T}, checking {len(rows)} records", flush=True)
    _check_records(inp, cache, np.sort(rows))


@pytest.mark.parametrize("outer", [float(np.float32(1 / 6)), 0.5])
def test_block_scale_ties_bit_exact(outer):
    """Block maxima at every e4m3 value and every midpoint between
    neighbours, times 6 * outer (exact in bf16 for these two outer scales),
    and their bf16 neighbours: t = amax / (6 outer) lands on the e4m3
    rounding ties, which the kernel resolves by the exact division."""
    from oracle import formats as F
    inp = workloads.small_decode(31, 2, 16, [200, 100], page_size=16, rec=432, outer=outer)
    vals = np.sort(np.unique(F.e4m3_value(np.arange(1, 0x7F)).astype(np.float64)))
    targets = np.concatenate([vals, (vals[:-1] + vals[1:]) / 2]) * (6.0 * np.float32(outer))
    tb = torch.from_numpy(targets.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(tb.float().numpy().astype(np.float64), targets.astype(np.float32).astype(np.float64))
    tbits = tb.view(torch.int16).numpy().view(np.uint16).astype(np.int64)
    allbits = np.concatenate([tbits, tbits + 1, tbits - 1]).astype(np.uint16)
    amax = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).float().numpy()
    T = inp.kv_c.shape[0]
    nb = T * 32
    rng = np.random.default_rng(5)
    a = np.resize(amax, nb).astype(np.float32)
    blocks = (rng.uniform(-1, 1, (nb, 16)) * a[:, None]).astype(np.float32)
    blocks[:, 0] = np.where(rng.uniform(size=nb) < 0.5, a, -a)
    inp.kv_c = torch.from_numpy(blocks.reshape(T, 512)).to(torch.bfloat16)
    cache = gpu_cache(inp, fill=0xAB)
    _check_records(inp, cache, np.arange(T))


def test_fp8_rope_every_finite_bf16_value():
    """The e4m3 RoPE cast over every finite bf16 bit pattern (both signs,
    subnormal e4m3 range, ties, values far above 448), bit-exact."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (pats & 0x7F80) != 0x7F80
    pats = pats[finite]
    T = (pats.size + 63) // 64
    pe = np.zeros(T * 64, dtype=np.uint16)
    pe[:pats.size] = pats
    g = torch.Generator().manual_seed(55)
    kv = torch.randn((T, 512), generator=g).to(torch.bfloat16)
    k_pe = torch.from_numpy(pe.view(np.int16).reshape(T, 64).copy()).view(torch.bfloat16)
    slots = torch.arange(T, dtype=torch.int64)
    cache = torch.full((T, 368), 0xAB, dtype=torch.uint8, device="cuda")
    ops.cache_write(kv.cuda(), k_pe.cuda(), slots.cuda(), cache, 1.0)
    got = cache.cpu().numpy()
    want = OR.pack_records(bits(kv), bits(k_pe), 1.0, 368)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at (row, byte) {bad[:5].tolist()}"
