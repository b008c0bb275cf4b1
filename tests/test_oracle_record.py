"""Pins of the oracle's latent cache record (sizes, byte layout, round trip)."""
import numpy as np
import torch

from oracle import formats as F
from oracle import record as R


def _bf16_bits(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_record_sizes_fixed_by_pages():
    # [B12X], review 1: an NVFP4 record is 432 bytes (bf16 RoPE) or 368 (fp8 RoPE)
    assert R.record_bytes(False) == 432 and R.record_bytes(True) == 368
    for bad in (0, 367, 369, 400, 431, 433, 576, 656):
        try:
            R.rope_is_fp8(bad)
        except ValueError:
            continue
        raise AssertionError(bad)


def test_record_bytes_hand_built():
    kv = np.zeros((1, 512), np.float32)
    kv[0, :4] = [6, 3, -1.5, 0.2]          # block 0: scale 0x38, codes 7 5 B 0
    kv[0, 16] = 6000                        # block 1 saturates: scale 0x7E, code 7
    pe = np.zeros((1, 64), np.float32)
    pe[0, 0], pe[0, 1], pe[0, 63] = 1.0, -3.0, 0.5
    for fp8 in (False, True):
        rec = R.pack_records(_bf16_bits(kv), _bf16_bits(pe), 1.0, R.record_bytes(fp8))[0]
        assert rec[0] == 0x57 and rec[1] == 0x0B and rec[8] == 0x07
        assert rec[256] == 0x38 and rec[257] == 0x7E and not rec[258:288].any()
        if fp8:
            assert rec[288] == 0x38 and rec[289] == 0xC4 and rec[351] == 0x30
            assert not rec[352:368].any()
        else:
            # bf16 1.0 = 0x3F80, -3.0 = 0xC040, 0.5 = 0x3F00, little-endian
            assert list(rec[288:292]) == [0x80, 0x3F, 0x40, 0xC0]
            assert list(rec[414:416]) == [0x00, 0x3F]
            assert not rec[416:432].any()


def test_unpack_of_pack_is_dequantization():
    rng = np.random.default_rng(5)
    kv = rng.standard_normal((37, 512)).astype(np.float32)
    kv[rng.random(kv.shape) < 0.01] *= 20
    kvb = _bf16_bits(kv)
    pe = rng.standard_normal((37, 64)).astype(np.float32)
    peb = _bf16_bits(pe)
    for s_l in (1.0, 0.625, 1.875):
        for fp8 in (False, True):
            recs = R.pack_records(kvb, peb, s_l, R.record_bytes(fp8))
            lat, rope = R.unpack_records(recs, s_l)
            want = F.nvfp4_qdq(F.bf16_to_f32(kvb), s_l)
            assert np.array_equal(lat, want)
            pe32 = F.bf16_to_f32(peb).astype(np.float64)
            if fp8:
                ref = torch.from_numpy(F.bf16_to_f32(peb)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
                assert np.array_equal(rope, ref)
            else:
                assert np.array_equal(rope, pe32)


def test_cache_write_touches_only_mapped_slots():
    rng = np.random.default_rng(6)
    cache = rng.integers(0, 256, (4, 8, 432), dtype=np.uint8)
    before = cache.copy()
    kv = _bf16_bits(rng.standard_normal((5, 512)))
    pe = _bf16_bits(rng.standard_normal((5, 64)))
    slots = np.array([3, -1, 17, 31, -5])
    R.cache_write(cache, kv, pe, slots, 1.0)
    flat, fb = cache.reshape(-1, 432), before.reshape(-1, 432)
    keep = slots >= 0
    recs = R.pack_records(kv[keep], pe[keep], 1.0, 432)
    assert np.array_equal(flat[slots[keep]], recs)
    other = np.setdiff1d(np.arange(32), slots[keep])
    assert np.array_equal(flat[other], fb[other])
