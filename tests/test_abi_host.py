"""Host-side tests of the C ABI: the library loads, exports every symbol the
header declares, and rejects invalid arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

from mla_attention_nvfp4_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mla_nvfp4.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert _declared() == sorted(L.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    for name in _declared():
        assert hasattr(lib, name), name


def test_constants_and_policy():
    assert L.record_bytes(False) == 432 and L.record_bytes(True) == 368
    assert L.decode_num_splits(4096, 4) == 4
    assert L.decode_num_splits(0, 8) == 1 and L.decode_num_splits(1, 8) == 1
    assert L.decode_num_splits(257, 8) == 2
    for n in (1, 63, 64, 65, 300, 1000, 4096, 32768):
        for s in (1, 2, 3, 4, 8, 32):
            k = L.decode_num_splits(n, s)
            tiles = (n + 63) // 64
            assert 1 <= k <= s and k <= tiles
    # fp32 partial rows, fp32 partial LSE, one format byte per row (256-B aligned regions)
    assert L.decode_workspace_bytes(64, 128, 4) == 64 * 4 * 128 * 512 * 4 + 64 * 4 * 128 * 4 + 64 * 4 * 128
    assert L.decode_workspace_bytes(3, 5, 2) == 256 * ((3 * 2 * 5 * 2048 + 255) // 256) + 256 + 256
    assert L.decode_workspace_bytes(64, 128, 1) == 0
    assert L.swizzled_scale_bytes(1, 1) == 128 * 4
    assert L.swizzled_scale_bytes(129, 1024) == 256 * 1024


def test_prefill_p_tile_is_the_oracle_schedule():
    from oracle import prefill as OP
    assert L.prefill_p_tile() == OP.BN_P == 64


def _decode_args(**kw):
    a = dict(q_nope=1 << 20, q_rope=1 << 20, sb=576 * 128, sh=576, cache=1 << 20, num_pages=4,
             rec=432, page=64, pt=1 << 20, maxp=4, seq=1 << 20, B=1, H=16, outer=1.0, scale=0.04,
             splits=1, ws=None, wsb=0, out=1 << 20, lse=1 << 20, stream=None)
    a.update(kw)
    return [a[k] for k in ("q_nope", "q_rope", "sb", "sh", "cache", "num_pages", "rec", "page", "pt", "maxp",
                           "seq", "B", "H", "outer", "scale", "splits", "ws", "wsb", "out", "lse", "stream")]


@pytest.mark.parametrize("kw,code", [
    (dict(rec=400), -2), (dict(rec=0), -2), (dict(rec=431), -2),
    (dict(H=0), -1), (dict(page=0), -1), (dict(splits=0), -1),
    (dict(outer=0.0), -1), (dict(outer=float("inf")), -1), (dict(outer=float("nan")), -1),
    (dict(scale=-1.0), -1), (dict(scale=float("nan")), -1), (dict(sb=576 * 128 + 1), -1),
    (dict(q_nope=None), -1), (dict(num_pages=0), -1),
    (dict(splits=4), -4), (dict(splits=4, ws=1 << 20, wsb=100), -4),
])
def test_decode_rejects_invalid_arguments(kw, code):
    lib = L.lib()
    assert lib.mla_decode_nvfp4(*_decode_args(**kw)) == code
    assert lib.mla_last_error()


def test_other_entry_points_reject_invalid_arguments():
    lib = L.lib()
    # cache write: bad record width, bad scale, misaligned rows
    assert lib.mla_nvfp4_cache_write(1 << 20, 576, 1 << 20, 576, 1 << 20, 5, 1 << 20, 10, 400, 1.0, None) == -2
    assert lib.mla_nvfp4_cache_write(1 << 20, 576, 1 << 20, 576, 1 << 20, 5, 1 << 20, 10, 432, -1.0, None) == -1
    assert lib.mla_nvfp4_cache_write(1 << 20, 577, 1 << 20, 576, 1 << 20, 5, 1 << 20, 10, 432, 1.0, None) == -1
    assert lib.mla_nvfp4_cache_write(None, 576, None, 576, None, 0, None, 0, 432, 1.0, None) == 0  # T = 0
    # sparse: topk must be positive
    args = _decode_args()
    assert lib.mla_sparse_decode_nvfp4(*args[:15], 1 << 20, 0, 1, None, 0, 1 << 20, 1 << 20, None) == -1
    # merge: D must be a multiple of 4
    assert lib.mla_lse_merge(1 << 20, 1 << 20, None, 1, 2, 1, 6, 1 << 20, 1 << 20, None) == -1
    # prefill: unknown flag bits, bad scales
    pf = [1 << 20, 192 * 4, 192, 1 << 20, 192 * 4, 192, 1 << 20, 128 * 4, 128, 1 << 20, 1, 10, 10, 4, 0.07]
    assert lib.mla_prefill_nvfp4_out(*pf, 16, 1., 1., 1., 1., 1., None, 0, 1 << 20, 1 << 20, None, None) == -1
    assert lib.mla_prefill_nvfp4_out(*pf, 15, 1., 0., 1., 1., 1., None, 0, 1 << 20, 1 << 20, None, None) == -1
    assert lib.mla_prefill_nvfp4_out(*pf, 15, 1., 1., 1., 1., 0., None, 0, 1 << 20, 1 << 20, None, None) == -1
    # batch limits: N of the prefill calls and the gather, B and H of the merge
    pf_n = list(pf)
    pf_n[10] = 65536
    assert lib.mla_prefill_nvfp4_out(*pf_n, 15, 1., 1., 1., 1., 1., None, 0, 1 << 20, 1 << 20, None, None) == -1
    assert lib.mla_lse_merge(1 << 20, 1 << 20, None, 65536, 2, 1, 4, 1 << 20, 1 << 20, None) == -1
    assert lib.mla_lse_merge(1 << 20, 1 << 20, None, 1, 2, 65537, 4, 1 << 20, 1 << 20, None) == -1
    assert lib.mla_nvfp4_cache_gather(1 << 20, 16, 432, 64, 1 << 20, 4, 1 << 20, None, 65536, 64, 64, 1.0,
                                      1 << 20, 512, 1 << 20, 64, None) == -1
    # launches beyond 2^32 work-items in a grid dimension: refused as unsupported (-6)
    big = 16 * ((1 << 24) - 1) + 1
    assert lib.mla_nvfp4_cache_write(1 << 20, 576, 1 << 20, 576, 1 << 20, big, 1 << 20, 10, 432, 1.0, None) == -6
    assert lib.mla_raw_cache_write(1 << 20, 576, 1 << 20, 576, 1 << 20, 4 * ((1 << 24) - 1) + 1, 1 << 20, 10,
                                   None) == -6
    pf_t = list(pf)
    pf_t[12] = 1 << 20   # T with H = 4: T * H above 2^28
    pf_t[11] = 16
    pf_t[13] = 1024
    assert lib.mla_prefill_nvfp4_out(*pf_t, 15, 1., 1., 1., 1., 1., None, 0, 1 << 20, 1 << 20, None, None) == -6
    assert lib.mla_nvfp4_quantize_rows(1 << 20, 1 << 30, 4096, 1.0, 1 << 20, 1 << 20, None) == -6
    # quantize_rows: K must be a multiple of 16
    assert lib.mla_nvfp4_quantize_rows(1 << 20, 4, 24, 1.0, 1 << 20, 1 << 20, None) == -1
    assert lib.mla_nvfp4_quantize_rows(1 << 20, 4, 32, 0.0, 1 << 20, 1 << 20, None) == -1


def test_noalloc_decode_refuses_requests_beyond_its_scratch():
    """The allocation-free decode checks its scratch limit on the host first."""
    lib = L.lib()
    args = _decode_args(B=600, H=128, splits=8)
    del args[16:18]                           # no workspace arguments
    assert lib.mla_decode_nvfp4_noalloc(*args) == -4
    assert b"allocation-free" in lib.mla_last_error()
    args = _decode_args(rec=400)
    del args[16:18]
    assert lib.mla_decode_nvfp4_noalloc(*args) == -2


def test_quantized_operand_decode_and_raw_cache_reject_invalid_arguments():
    lib = L.lib()
    a = _decode_args()
    head, tail = a[:15], a[15:]          # ... softmax_scale | max_splits, ws, wsb, out, lse, stream

    def qdq(rec=432, flags=0, g=(1.0, 1.0, 1.0, 1.0)):
        h = list(head)
        h[6] = rec
        return lib.mla_decode_qdq(*h, flags, *g, *tail)
    assert qdq(rec=400) == -2
    assert qdq(rec=432, flags=2) == -1            # K on read needs raw records
    assert qdq(rec=1152, flags=16) == -1          # FP8 bit without its operand
    assert qdq(rec=1152, flags=4, g=(1.0, 1.0, 1.0, 0.0)) == -1
    assert qdq(rec=1152, flags=1 << 9) == -1
    # raw cache write: misaligned rows
    assert lib.mla_raw_cache_write(1 << 20, 513, 1 << 20, 64, 1 << 20, 4, 1 << 20, 8, None) == -1
    assert lib.mla_raw_cache_write(None, 512, None, 64, None, 0, None, 0, None) == 0
