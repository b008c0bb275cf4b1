"""The roofline re-measurement helpers: the stream copy copies every byte, the
stream read sums every word, and the MFMA-rate kernels run and write finite
values (they compute nothing of the method; their timing is reported by
bench.py).  The 128 MiB + 48 byte case reaches the four-loads-per-lane loop of
both stream kernels (their grid is capped at 8192 workgroups of 256 lanes)
and a ragged tail."""
import numpy as np
import pytest
import torch

from mla_attention_nvfp4_amd import ops

pytestmark = pytest.mark.gpu


SIZES = (16, 4096, (3 << 20) + 48, (128 << 20) + 48)


def _bytes(nbytes, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randint(0, 256, (nbytes,), generator=g, dtype=torch.uint8, device="cuda")


def test_roofline_copy_is_exact():
    for nbytes in SIZES:
        src = _bytes(nbytes, 7)
        dst = torch.zeros_like(src)
        ops.roofline_copy(src, dst)
        torch.cuda.synchronize()
        assert torch.equal(src, dst), nbytes


def test_roofline_read_sums_every_word():
    for nbytes in SIZES:
        src = _bytes(nbytes, 11)
        total = torch.zeros(1, dtype=torch.int32, device="cuda")
        ops.roofline_read(src, total)
        ops.roofline_read(src, total)      # adds, so twice the sum
        torch.cuda.synchronize()
        words = src.cpu().numpy().view(np.uint32).astype(np.uint64)
        want = (2 * int(words.sum())) % (1 << 32)
        assert int(total.item()) & 0xFFFFFFFF == want, nbytes


def test_roofline_mfma_runs():
    sink = torch.full((8 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    for shape in (0, 1):
        ops.roofline_mfma(shape, 8, 4, sink)
        torch.cuda.synchronize()
        assert torch.isfinite(sink).all(), shape


def test_roofline_arguments_are_checked():
    sink = torch.empty(256, dtype=torch.float32, device="cuda")
    with pytest.raises(ops.MlaError):
        ops.roofline_mfma(2, 1, 1, sink)
    src = torch.empty(20, dtype=torch.uint8, device="cuda")
    with pytest.raises(ops.MlaError):
        ops.roofline_copy(src, torch.empty_like(src))
    with pytest.raises(ops.MlaError):
        ops.roofline_read(src, torch.zeros(1, dtype=torch.int32, device="cuda"))
