"""ctypes binding of libmla_nvfp4.so (argument marshalling only).

Every computation runs in the library's HIP kernels; this module checks
tensor dtypes, devices and shapes, passes raw device pointers and the current
HIP stream, and turns a negative status into ``MlaError``.  There is no CPU
fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_nvfp4.so")

c_int, c_i64, c_u32, c_f32, c_sz, c_p = (ctypes.c_int, ctypes.c_int64, ctypes.c_uint, ctypes.c_float,
                                         ctypes.c_size_t, ctypes.c_void_p)

# name -> (restype, argtypes); mirrors include/mla_nvfp4.h
SIGNATURES = {
    "mla_last_error": (ctypes.c_char_p, []),
    "mla_nvfp4_record_bytes": (c_int, [c_int]),
    "mla_decode_num_splits": (c_int, [c_int, c_int]),
    "mla_decode_workspace_bytes": (c_sz, [c_int, c_int, c_int]),
    "mla_prefill_p_tile": (c_int, []),
    "mla_nvfp4_swizzled_scale_bytes": (c_sz, [c_i64, c_i64]),
    "mla_nvfp4_cache_write": (c_int, [c_p, c_i64, c_p, c_i64, c_p, c_i64, c_p, c_i64, c_int, c_f32, c_p]),
    "mla_decode_nvfp4": (c_int, [c_p, c_p, c_i64, c_i64, c_p, c_i64, c_int, c_int, c_p, c_int, c_p, c_int,
                                 c_int, c_f32, c_f32, c_int, c_p, c_sz, c_p, c_p, c_p]),
    "mla_decode_nvfp4_noalloc": (c_int, [c_p, c_p, c_i64, c_i64, c_p, c_i64, c_int, c_int, c_p, c_int, c_p,
                                         c_int, c_int, c_f32, c_f32, c_int, c_p, c_p, c_p]),
    "mla_sparse_decode_nvfp4": (c_int, [c_p, c_p, c_i64, c_i64, c_p, c_i64, c_int, c_int, c_p, c_int, c_p,
                                        c_int, c_int, c_f32, c_f32, c_p, c_int, c_int, c_p, c_sz, c_p, c_p,
                                        c_p]),
    "mla_decode_qdq": (c_int, [c_p, c_p, c_i64, c_i64, c_p, c_i64, c_int, c_int, c_p, c_int, c_p, c_int, c_int,
                               c_f32, c_f32, c_u32, c_f32, c_f32, c_f32, c_f32, c_int, c_p, c_sz, c_p, c_p, c_p]),
    "mla_raw_cache_write": (c_int, [c_p, c_i64, c_p, c_i64, c_p, c_i64, c_p, c_i64, c_p]),
    "mla_lse_merge": (c_int, [c_p, c_p, c_p, c_int, c_int, c_int, c_int, c_p, c_p, c_p]),
    "mla_prefill_workspace_bytes": (c_sz, [c_i64, c_int, c_u32]),
    "mla_prefill_nvfp4_out": (c_int, [c_p, c_i64, c_i64, c_p, c_i64, c_i64, c_p, c_i64, c_i64, c_p, c_int,
                                      c_int, c_i64, c_int, c_f32, c_u32, c_f32, c_f32, c_f32, c_f32, c_f32,
                                      c_p, c_sz, c_p, c_p, c_p, c_p]),
    "mla_prefill_attention": (c_int, [c_p, c_i64, c_i64, c_p, c_i64, c_i64, c_p, c_i64, c_i64, c_p, c_p, c_int,
                                      c_int, c_int, c_i64, c_i64, c_int, c_int, c_f32, c_u32, c_f32, c_f32, c_f32,
                                      c_f32, c_p, c_sz, c_p, c_i64, c_i64, c_p, c_i64, c_i64, c_p]),
    "mla_nvfp4_cache_gather": (c_int, [c_p, c_i64, c_int, c_int, c_p, c_int, c_p, c_p, c_int, c_int, c_i64, c_f32,
                                       c_p, c_i64, c_p, c_i64, c_p]),
    "mla_nvfp4_quantize_rows": (c_int, [c_p, c_i64, c_int, c_f32, c_p, c_p, c_p]),
    "mla_roofline_mfma": (c_int, [c_int, c_int, c_int, c_p, c_p]),
    "mla_roofline_copy": (c_int, [c_p, c_p, c_i64, c_p]),
    "mla_roofline_read": (c_int, [c_p, c_i64, c_p, c_p]),
}

MLA_QDQ_Q, MLA_QDQ_K, MLA_QDQ_P, MLA_QDQ_V = 1, 2, 4, 8
MLA_QDQ_FP8_Q, MLA_QDQ_FP8_K, MLA_QDQ_FP8_P, MLA_QDQ_FP8_V = 16, 32, 64, 128
MLA_PREFILL_SPARSE_2_4 = 256


class MlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"mla status {status}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m mla_attention_nvfp4_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def _check(rc: int) -> None:
    if rc != 0:
        raise MlaError(rc, lib().mla_last_error().decode())


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype, name: str) -> None:
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda:
        raise TypeError(f"{name} must be a {dtype} tensor on a GPU")


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


# ---------------------------------------------------------------- helpers --

def record_bytes(rope_fp8: bool) -> int:
    return lib().mla_nvfp4_record_bytes(1 if rope_fp8 else 0)


def decode_num_splits(n: int, max_splits: int) -> int:
    return lib().mla_decode_num_splits(int(n), int(max_splits))


def decode_workspace_bytes(B: int, H: int, max_splits: int) -> int:
    return lib().mla_decode_workspace_bytes(B, H, max_splits)


def prefill_p_tile() -> int:
    """Key-tile width of the prefill's P-quantization schedule, as compiled."""
    return lib().mla_prefill_p_tile()


def swizzled_scale_bytes(rows: int, scale_cols: int) -> int:
    return lib().mla_nvfp4_swizzled_scale_bytes(rows, scale_cols)


def prefill_workspace_bytes(T: int, H: int, flags: int) -> int:
    return lib().mla_prefill_workspace_bytes(T, H, flags)


# ------------------------------------------------------------------ calls --

def cache_write(kv_c, k_pe, slot_mapping, cache, outer_scale: float) -> None:
    """kv_c bf16 [T,512], k_pe bf16 [T,64] (row-strided), slot_mapping int64 [T],
    cache uint8 [..., record_bytes] contiguous."""
    _need(kv_c, torch.bfloat16, "kv_c")
    _need(k_pe, torch.bfloat16, "k_pe")
    _need(slot_mapping, torch.int64, "slot_mapping")
    _need(cache, torch.uint8, "cache")
    if kv_c.dim() != 2 or kv_c.shape[1] != 512 or kv_c.stride(1) != 1:
        raise ValueError("kv_c must be [T, 512] with unit inner stride")
    if k_pe.dim() != 2 or k_pe.shape[1] != 64 or k_pe.stride(1) != 1 or k_pe.shape[0] != kv_c.shape[0]:
        raise ValueError("k_pe must be [T, 64] with unit inner stride")
    if not cache.is_contiguous() or slot_mapping.numel() != kv_c.shape[0]:
        raise ValueError("cache must be contiguous and slot_mapping [T]")
    rec = cache.shape[-1]
    _check(lib().mla_nvfp4_cache_write(kv_c.data_ptr(), kv_c.stride(0), k_pe.data_ptr(), k_pe.stride(0),
                                       slot_mapping.data_ptr(), kv_c.shape[0], cache.data_ptr(),
                                       cache.numel() // rec, rec, float(outer_scale), _stream(cache)))


def _decode_common(q_nope, q_rope, cache, page_table, seq_lens):
    for t, n, d in ((q_nope, "q_nope", torch.bfloat16), (q_rope, "q_rope", torch.bfloat16),
                    (cache, "cache", torch.uint8), (page_table, "page_table", torch.int32),
                    (seq_lens, "seq_lens", torch.int32)):
        _need(t, d, n)
    if q_nope.dim() != 3 or q_nope.shape[2] != 512 or q_rope.shape[:2] != q_nope.shape[:2] \
            or q_rope.shape[2] != 64 or q_nope.stride() != q_rope.stride() or q_nope.stride(2) != 1:
        raise ValueError("q_nope [B,H,512] and q_rope [B,H,64] must share strides with unit inner stride")
    if cache.dim() != 3 or not cache.is_contiguous():
        raise ValueError("cache must be contiguous [num_pages, page_size, record_bytes]")
    if not page_table.is_contiguous() or page_table.dim() != 2 or page_table.shape[0] != q_nope.shape[0]:
        raise ValueError("page_table must be contiguous [B, max_pages]")
    if seq_lens.numel() != q_nope.shape[0]:
        raise ValueError("seq_lens must be [B]")


def _workspace(B, H, max_splits, like, workspace):
    need = decode_workspace_bytes(B, H, max_splits)
    if need == 0:
        return None
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=like.device)
    return workspace


def decode(q_nope, q_rope, cache, page_table, seq_lens, outer_scale, softmax_scale, max_splits=1,
           out=None, lse=None, workspace=None):
    """Dense paged decode.  Returns (out fp32 [B,H,512], lse fp32 [B,H])."""
    _decode_common(q_nope, q_rope, cache, page_table, seq_lens)
    B, H = q_nope.shape[:2]
    out = torch.empty((B, H, 512), dtype=torch.float32, device=q_nope.device) if out is None else out
    lse = torch.empty((B, H), dtype=torch.float32, device=q_nope.device) if lse is None else lse
    ws = _workspace(B, H, max_splits, q_nope, workspace)
    _check(lib().mla_decode_nvfp4(
        q_nope.data_ptr(), q_rope.data_ptr(), q_nope.stride(0), q_nope.stride(1), cache.data_ptr(),
        cache.shape[0], cache.shape[2], cache.shape[1], page_table.data_ptr(), page_table.shape[1],
        seq_lens.data_ptr(), B, H, float(outer_scale), float(softmax_scale), int(max_splits), _ptr(ws),
        0 if ws is None else ws.numel(), out.data_ptr(), lse.data_ptr(), _stream(q_nope)))
    return out, lse


def decode_noalloc(q_nope, q_rope, cache, page_table, seq_lens, outer_scale, softmax_scale, max_splits=1,
                   out=None, lse=None):
    """Dense paged decode through the allocation-free entry point: the split
    partials use the library's per-device scratch (no workspace argument).
    ``out`` and ``lse`` are allocated here only when not given."""
    _decode_common(q_nope, q_rope, cache, page_table, seq_lens)
    B, H = q_nope.shape[:2]
    out = torch.empty((B, H, 512), dtype=torch.float32, device=q_nope.device) if out is None else out
    lse = torch.empty((B, H), dtype=torch.float32, device=q_nope.device) if lse is None else lse
    _check(lib().mla_decode_nvfp4_noalloc(
        q_nope.data_ptr(), q_rope.data_ptr(), q_nope.stride(0), q_nope.stride(1), cache.data_ptr(),
        cache.shape[0], cache.shape[2], cache.shape[1], page_table.data_ptr(), page_table.shape[1],
        seq_lens.data_ptr(), B, H, float(outer_scale), float(softmax_scale), int(max_splits), out.data_ptr(),
        lse.data_ptr(), _stream(q_nope)))
    return out, lse


def sparse_decode(q_nope, q_rope, cache, page_table, seq_lens, indices, outer_scale, softmax_scale,
                  max_splits=1, out=None, lse=None, workspace=None):
    """Top-k sparse paged decode.  indices int32 [B, topk]."""
    _decode_common(q_nope, q_rope, cache, page_table, seq_lens)
    _need(indices, torch.int32, "indices")
    B, H = q_nope.shape[:2]
    if not indices.is_contiguous() or indices.dim() != 2 or indices.shape[0] != B:
        raise ValueError("indices must be contiguous [B, topk]")
    out = torch.empty((B, H, 512), dtype=torch.float32, device=q_nope.device) if out is None else out
    lse = torch.empty((B, H), dtype=torch.float32, device=q_nope.device) if lse is None else lse
    ws = _workspace(B, H, max_splits, q_nope, workspace)
    _check(lib().mla_sparse_decode_nvfp4(
        q_nope.data_ptr(), q_rope.data_ptr(), q_nope.stride(0), q_nope.stride(1), cache.data_ptr(),
        cache.shape[0], cache.shape[2], cache.shape[1], page_table.data_ptr(), page_table.shape[1],
        seq_lens.data_ptr(), B, H, float(outer_scale), float(softmax_scale), indices.data_ptr(),
        indices.shape[1], int(max_splits), _ptr(ws), 0 if ws is None else ws.numel(), out.data_ptr(),
        lse.data_ptr(), _stream(q_nope)))
    return out, lse


RAW_RECORD_BYTES = 1152


def raw_cache_write(kv_c, k_pe, slot_mapping, cache) -> None:
    """kv_c bf16 [T,512], k_pe bf16 [T,64] (row-strided), slot_mapping int64 [T],
    cache uint8 [..., 1152] contiguous (raw records)."""
    _need(kv_c, torch.bfloat16, "kv_c")
    _need(k_pe, torch.bfloat16, "k_pe")
    _need(slot_mapping, torch.int64, "slot_mapping")
    _need(cache, torch.uint8, "cache")
    if kv_c.dim() != 2 or kv_c.shape[1] != 512 or kv_c.stride(1) != 1 or k_pe.dim() != 2 or k_pe.shape[1] != 64 \
            or k_pe.stride(1) != 1 or k_pe.shape[0] != kv_c.shape[0]:
        raise ValueError("kv_c [T, 512] and k_pe [T, 64] with unit inner stride")
    if not cache.is_contiguous() or cache.shape[-1] != RAW_RECORD_BYTES or slot_mapping.numel() != kv_c.shape[0]:
        raise ValueError("cache must be contiguous [..., 1152] and slot_mapping [T]")
    _check(lib().mla_raw_cache_write(kv_c.data_ptr(), kv_c.stride(0), k_pe.data_ptr(), k_pe.stride(0),
                                     slot_mapping.data_ptr(), kv_c.shape[0], cache.data_ptr(), cache.numel() // 1152,
                                     _stream(cache)))


def decode_qdq(q_nope, q_rope, cache, page_table, seq_lens, outer_scale, softmax_scale, flags, g_q=1.0, g_k=1.0,
               g_v=1.0, g_p=1.0, max_splits=1, out=None, lse=None, workspace=None):
    """Dense paged decode with quantized operands (NVFP4 or raw records)."""
    _decode_common(q_nope, q_rope, cache, page_table, seq_lens)
    B, H = q_nope.shape[:2]
    out = torch.empty((B, H, 512), dtype=torch.float32, device=q_nope.device) if out is None else out
    lse = torch.empty((B, H), dtype=torch.float32, device=q_nope.device) if lse is None else lse
    ws = _workspace(B, H, max_splits, q_nope, workspace)
    _check(lib().mla_decode_qdq(
        q_nope.data_ptr(), q_rope.data_ptr(), q_nope.stride(0), q_nope.stride(1), cache.data_ptr(),
        cache.shape[0], cache.shape[2], cache.shape[1], page_table.data_ptr(), page_table.shape[1],
        seq_lens.data_ptr(), B, H, float(outer_scale), float(softmax_scale), int(flags), float(g_q), float(g_k),
        float(g_v), float(g_p), int(max_splits), _ptr(ws), 0 if ws is None else ws.numel(), out.data_ptr(),
        lse.data_ptr(), _stream(q_nope)))
    return out, lse


def lse_merge(partial_out, partial_lse, splits_per_seq=None, out=None, lse=None):
    """partial_out fp32 [B,S,H,D], partial_lse fp32 [B,S,H] -> (out [B,H,D], lse [B,H])."""
    _need(partial_out, torch.float32, "partial_out")
    _need(partial_lse, torch.float32, "partial_lse")
    if not partial_out.is_contiguous() or not partial_lse.is_contiguous():
        raise ValueError("partials must be contiguous")
    B, S, H, D = partial_out.shape
    if tuple(partial_lse.shape) != (B, S, H):
        raise ValueError("partial_lse must be [B, S, H]")
    if splits_per_seq is not None:
        _need(splits_per_seq, torch.int32, "splits_per_seq")
    out = torch.empty((B, H, D), dtype=torch.float32, device=partial_out.device) if out is None else out
    lse = torch.empty((B, H), dtype=torch.float32, device=partial_out.device) if lse is None else lse
    _check(lib().mla_lse_merge(partial_out.data_ptr(), partial_lse.data_ptr(), _ptr(splits_per_seq), B, S, H,
                               D, out.data_ptr(), lse.data_ptr(), _stream(partial_out)))
    return out, lse


def prefill(q, k, v, cu_seqlens, max_seqlen, softmax_scale, flags, g_q, g_k, g_v, g_p, out_global_scale,
            with_lse=True, workspace=None, codes=None, scales=None, lse=None):
    """Varlen causal prefill with NVFP4 output.  Returns (codes uint8 [T,H,64],
    swizzled scales uint8, lse fp32 [T,H] or None); the three outputs may be
    passed in (then they are filled and returned)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, n)
    _need(cu_seqlens, torch.int32, "cu_seqlens")
    T, H = q.shape[:2]
    if q.shape[2] != 192 or k.shape != q.shape or v.shape != (T, H, 128) \
            or q.stride(2) != 1 or k.stride(2) != 1 or v.stride(2) != 1:
        raise ValueError("q, k [T,H,192] and v [T,H,128] with unit inner stride")
    dev = q.device
    if codes is None:
        codes = torch.empty((T, H, 64), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(max(1, swizzled_scale_bytes(T, H * 8)), dtype=torch.uint8, device=dev)
    if lse is None and with_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    if codes.shape != (T, H, 64) or not codes.is_contiguous() or scales.numel() < swizzled_scale_bytes(T, H * 8):
        raise ValueError("codes must be contiguous [T,H,64] and scales hold the swizzled scale buffer")
    if lse is not None:
        _need(lse, torch.float32, "lse")
        if lse.shape != (T, H) or not lse.is_contiguous():
            raise ValueError("lse must be contiguous [T,H]")
    need = prefill_workspace_bytes(T, H, flags)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib().mla_prefill_nvfp4_out(
        q.data_ptr(), q.stride(0), q.stride(1), k.data_ptr(), k.stride(0), k.stride(1), v.data_ptr(),
        v.stride(0), v.stride(1), cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, int(max_seqlen), T, H,
        float(softmax_scale), int(flags), float(g_q), float(g_k), float(g_v), float(g_p),
        float(out_global_scale), _ptr(workspace), 0 if workspace is None else workspace.numel(),
        codes.data_ptr(), scales.data_ptr(), _ptr(lse), _stream(q)))
    return codes, scales, lse


def _check_qkv(q, k, v):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, n)
    if q.dim() != 3 or q.shape[2] != 192 or k.dim() != 3 or k.shape[1:] != q.shape[1:] or v.dim() != 3 \
            or v.shape[0] != k.shape[0] or v.shape[1] != q.shape[1] or v.shape[2] != 128 \
            or q.stride(2) != 1 or k.stride(2) != 1 or v.stride(2) != 1:
        raise ValueError("q [Tq,H,192], k [Tk,H,192] and v [Tk,H,128] with unit inner stride")


def prefill_attention(q, k, v, cu_seqlens_q, max_seqlen_q, softmax_scale, flags, g_q, g_k, g_v, g_p, causal=True,
                      cu_seqlens_k=None, max_seqlen_k=0, out=None, lse=None, workspace=None):
    """Varlen prefill attention with fp32 output.  causal: keys are the query
    rows (k, v have q's rows); otherwise keys of sequence n are rows
    [cu_seqlens_k[n], cu_seqlens_k[n+1]) of k and v (cached context).
    ``out`` ([Tq,H,128] fp32, or a view with strides multiple of 4) and
    ``lse`` ([Tq,H] fp32 view) may be passed in.  Returns (out, lse)."""
    _check_qkv(q, k, v)
    _need(cu_seqlens_q, torch.int32, "cu_seqlens_q")
    Tq, H = q.shape[:2]
    Tk = Tq if causal else k.shape[0]
    if causal and k.shape[0] != Tq:
        raise ValueError("causal attention: k and v have the query rows")
    if not causal:
        _need(cu_seqlens_k, torch.int32, "cu_seqlens_k")
    dev = q.device
    out = torch.empty((Tq, H, 128), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((Tq, H), dtype=torch.float32, device=dev) if lse is None else lse
    _need(out, torch.float32, "out")
    _need(lse, torch.float32, "lse")
    if out.shape != (Tq, H, 128) or out.stride(2) != 1 or lse.shape != (Tq, H):
        raise ValueError("out must be [Tq,H,128] with unit inner stride and lse [Tq,H]")
    need = prefill_workspace_bytes(Tk, H, flags)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib().mla_prefill_attention(
        q.data_ptr(), q.stride(0), q.stride(1), k.data_ptr(), k.stride(0), k.stride(1), v.data_ptr(), v.stride(0),
        v.stride(1), cu_seqlens_q.data_ptr(), _ptr(cu_seqlens_k), cu_seqlens_q.numel() - 1, int(max_seqlen_q),
        int(max_seqlen_k), Tq, Tk, H, 1 if causal else 0, float(softmax_scale), int(flags), float(g_q),
        float(g_k), float(g_v), float(g_p), _ptr(workspace), 0 if workspace is None else workspace.numel(),
        out.data_ptr(), out.stride(0), out.stride(1), lse.data_ptr(), lse.stride(0), lse.stride(1), _stream(q)))
    return out, lse


def cache_gather(cache, page_table, cu_ctx, max_ctx_len, outer_scale, ctx_start=None, kv_c=None, k_pe=None):
    """Gather cached context rows from the paged NVFP4 cache into bf16
    kv_c [T_ctx,512] and k_pe [T_ctx,64] (allocated unless given)."""
    _need(cache, torch.uint8, "cache")
    _need(page_table, torch.int32, "page_table")
    _need(cu_ctx, torch.int32, "cu_ctx")
    if cache.dim() != 3 or not cache.is_contiguous() or not page_table.is_contiguous() or page_table.dim() != 2:
        raise ValueError("cache [num_pages, page_size, record_bytes] and page_table [N, max_pages], contiguous")
    N = cu_ctx.numel() - 1
    if page_table.shape[0] != N:
        raise ValueError("page_table must have one row per sequence")
    if ctx_start is not None:
        _need(ctx_start, torch.int32, "ctx_start")
    T = int(cu_ctx[-1].item()) if kv_c is None else kv_c.shape[0]
    dev = cache.device
    kv_c = torch.empty((T, 512), dtype=torch.bfloat16, device=dev) if kv_c is None else kv_c
    k_pe = torch.empty((T, 64), dtype=torch.bfloat16, device=dev) if k_pe is None else k_pe
    _check(lib().mla_nvfp4_cache_gather(
        cache.data_ptr(), cache.shape[0], cache.shape[2], cache.shape[1], page_table.data_ptr(), page_table.shape[1],
        cu_ctx.data_ptr(), _ptr(ctx_start), N, int(max_ctx_len), T, float(outer_scale), kv_c.data_ptr(),
        kv_c.stride(0), k_pe.data_ptr(), k_pe.stride(0), _stream(cache)))
    return kv_c, k_pe


def quantize_rows(x, global_scale):
    """x fp32 [M,K] contiguous -> (codes uint8 [M,K/2], swizzled scales uint8)."""
    _need(x, torch.float32, "x")
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be contiguous [M, K]")
    M, K = x.shape
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty(max(1, swizzled_scale_bytes(M, K // 16)), dtype=torch.uint8, device=x.device)
    _check(lib().mla_nvfp4_quantize_rows(x.data_ptr(), M, K, float(global_scale), codes.data_ptr(),
                                         scales.data_ptr(), _stream(x)))
    return codes, scales


# ---------------------------------------------------------------- roofline --

def roofline_mfma(shape: int, blocks: int, iters: int, sink: torch.Tensor) -> None:
    """Launch the MFMA-rate kernel (shape 0: 16x16x32 f16, 1: 32x32x16 f16;
    8 products per wavefront and iteration, 4 wavefronts per workgroup) on
    the current stream; ``sink`` is float32 [blocks * 256] on the device."""
    _need(sink, torch.float32, "sink")
    if sink.numel() < blocks * 256:
        raise ValueError("sink needs blocks * 256 floats")
    _check(lib().mla_roofline_mfma(shape, blocks, iters, _ptr(sink), _stream(sink)))


def roofline_copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    """Plain device copy of src's bytes into dst (same byte size, 16-byte
    aligned, multiple of 16 bytes) on the current stream."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or not src.is_contiguous() or not dst.is_contiguous():
        raise ValueError("src and dst must be contiguous with the same byte size")
    _check(lib().mla_roofline_copy(_ptr(src), _ptr(dst), nbytes, _stream(src)))


def roofline_read(src: torch.Tensor, total: torch.Tensor) -> None:
    """Read-only stream over src's bytes (contiguous, 16-byte aligned,
    multiple of 16 bytes) on the current stream: adds the wrapping 32-bit
    sum of its words to ``total`` (int32 [1] on the device, not zeroed)."""
    _need(total, torch.int32, "total")
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    nbytes = src.numel() * src.element_size()
    _check(lib().mla_roofline_read(_ptr(src), nbytes, _ptr(total), _stream(src)))

