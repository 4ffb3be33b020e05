"""ctypes binding of libmla.so (include/mla.h).

Argument marshalling only: tensors are passed as device pointers, every step of
the decode path runs in the library's HIP kernels.  torch is used for device
memory and for the current stream.  There is no fallback: if libmla.so is
missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_ALIGNMENT, MLA_ERR_WORKSPACE, MLA_ERR_HIP = range(6)
MLA_F32, MLA_BF16, MLA_FP8_E4M3 = 0, 1, 2

EXPORTS = ("mla_status_string", "mla_build_info", "mla_absorb_q", "mla_decode_workspace_size",
           "mla_lse_part_offset", "mla_decode", "mla_merge_splits", "mla_out_proj", "mla_cache_store",
           "mla_cache_append", "mla_query_prep_scratch_size", "mla_query_prep", "mla_partition_host",
           "mla_decode_multi_workspace_size", "mla_decode_multi", "mla_merge_out_proj",
           "mla_decode_multi_out_proj", "mla_validate_cache_host", "mla_decode_noalloc",
           "mla_prefill_workspace_size", "mla_prefill", "mla_cache_store_rope", "mla_cache_append_rope",
           "mla_query_prep_rope", "mla_yarn_attention_factor")


class MlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("d_head", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("d_latent", ctypes.c_int32)]


class Rope(ctypes.Structure):
    """mla_rope_t: RoPE base and YaRN parameters (yarn_scale 1 = plain RoPE)."""
    _fields_ = [("base", ctypes.c_float), ("yarn_scale", ctypes.c_float), ("yarn_alpha", ctypes.c_float),
                ("yarn_beta", ctypes.c_float), ("yarn_orig_ctx", ctypes.c_int32)]


class PagedCache(ctypes.Structure):
    _fields_ = [("kv", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("dtype", ctypes.c_int),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("max_pages_per_seq", ctypes.c_int32),
                ("seq_lens", ctypes.c_void_p)]


class Partition(ctypes.Structure):
    _fields_ = [("split_tokens", ctypes.c_int32), ("num_parts", ctypes.c_int32)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmla.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with `python -m mla_latent_kv_37_amd.build` "
                           "(the MLA decode path has no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    PD, PC, PP = ctypes.POINTER(Dims), ctypes.POINTER(PagedCache), ctypes.POINTER(Partition)
    sig = {
        "mla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "mla_build_info": (ctypes.c_char_p, []),
        "mla_absorb_q": (ctypes.c_int, [PD, I32, P, ctypes.c_int, P, ctypes.c_int, P, ctypes.c_int, P]),
        "mla_decode_workspace_size": (ctypes.c_int, [PD, I32, I32, I32, PP, ctypes.POINTER(SZ), ctypes.POINTER(I32)]),
        "mla_lse_part_offset": (SZ, [PD, I32]),
        "mla_decode": (ctypes.c_int, [PD, I32, P, P, ctypes.c_int, PC, ctypes.c_float, PP, P, SZ, P, ctypes.c_int,
                                      P, P]),
        "mla_merge_splits": (ctypes.c_int, [PD, I32, P, I32, I32, PP, P, SZ, P, ctypes.c_int, P, P]),
        "mla_out_proj": (ctypes.c_int, [PD, I32, P, ctypes.c_int, P, ctypes.c_int, P, ctypes.c_int, P]),
        "mla_merge_out_proj": (ctypes.c_int, [PD, I32, P, I32, I32, PP, P, SZ, P, ctypes.c_int, P, P, ctypes.c_int, P,
                                              ctypes.c_int, P]),
        "mla_cache_store": (ctypes.c_int, [PD, I32, P, ctypes.c_int, P, ctypes.c_float, PC, P]),
        "mla_cache_append": (ctypes.c_int, [PD, I32, I32, P, ctypes.c_int, P, P, ctypes.c_int, P, P, ctypes.c_float,
                                            PC, P]),
        "mla_query_prep_scratch_size": (SZ, [PD, I32, I32]),
        "mla_query_prep": (ctypes.c_int, [PD, I32, I32, I32, P, ctypes.c_int, P, P, P, ctypes.c_int, P,
                                          ctypes.c_float, P, P, ctypes.c_int, P, SZ, P]),
        "mla_partition_host": (ctypes.c_int, [ctypes.POINTER(I32), I32, I32, I32, PP, ctypes.POINTER(I32),
                                              ctypes.POINTER(I32)]),
        "mla_decode_noalloc": (ctypes.c_int, [PD, I32, P, P, ctypes.c_int, PC, ctypes.c_float, PP, P, ctypes.c_int, P,
                                              P]),
        "mla_validate_cache_host": (ctypes.c_int, [ctypes.POINTER(I32), ctypes.POINTER(I32), I32, I32, I32, I32,
                                                   ctypes.POINTER(I32)]),
        "mla_decode_multi_workspace_size": (ctypes.c_int, [PD, I32, I32, I32, I32, PP, ctypes.POINTER(SZ),
                                                           ctypes.POINTER(I32)]),
        "mla_decode_multi": (ctypes.c_int, [PD, I32, I32, P, P, ctypes.c_int, PC, ctypes.c_float, PP, P, SZ, P,
                                            ctypes.c_int, P, P]),
        "mla_decode_multi_out_proj": (ctypes.c_int, [PD, I32, I32, P, P, ctypes.c_int, PC, ctypes.c_float, PP, P, SZ,
                                                     P, ctypes.c_int, P, P, ctypes.c_int, P, ctypes.c_int, P]),
        "mla_prefill_workspace_size": (ctypes.c_int, [PD, I32, ctypes.c_int64, ctypes.POINTER(SZ)]),
        "mla_cache_store_rope": (ctypes.c_int, [PD, I32, P, ctypes.c_int, P, ctypes.POINTER(Rope), PC, P]),
        "mla_cache_append_rope": (ctypes.c_int, [PD, I32, I32, P, ctypes.c_int, P, P, ctypes.c_int, P, P,
                                                 ctypes.POINTER(Rope), PC, P]),
        "mla_query_prep_rope": (ctypes.c_int, [PD, I32, I32, I32, P, ctypes.c_int, P, P, P, ctypes.c_int, P,
                                               ctypes.POINTER(Rope), P, P, ctypes.c_int, P, SZ, P]),
        "mla_yarn_attention_factor": (ctypes.c_float, [ctypes.c_float]),
        "mla_prefill": (ctypes.c_int, [PD, I32, P, I32, I32, P, P, ctypes.c_int, PC, ctypes.c_int64, P, P,
                                       ctypes.c_int, ctypes.c_float, P, SZ, P, ctypes.c_int, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().mla_status_string(int(status)).decode()


def build_info() -> str:
    return load().mla_build_info().decode()


def _check(status: int, what: str):
    if status != MLA_OK:
        raise MlaError(status, what)


# ---------------------------------------------------------------------------
# torch-facing helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return MLA_F32
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MLA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def dims(n_heads: int, d_head: int, d_rope: int, d_latent: int) -> Dims:
    return Dims(n_heads, d_head, d_rope, d_latent)


def partition(split_tokens: int = 0, num_parts: int = 0) -> Partition:
    return Partition(split_tokens, num_parts)


def absorb_q(d: Dims, q_nope, w_uk, q_lat, stream=None):
    """q_lat[b,i,:] = (W^UK_i)^T q_nope[b,i,:]; shapes [B,n_h,d_h], [n_h*d_h, d_c], [B,n_h,d_c]."""
    _check(load().mla_absorb_q(ctypes.byref(d), q_nope.shape[0], _ptr(q_nope), dtype_code(q_nope), _ptr(w_uk),
                               dtype_code(w_uk), _ptr(q_lat), dtype_code(q_lat), _stream(stream)), "mla_absorb_q")
    return q_lat


def workspace_size(d: Dims, batch: int, max_pages: int, page_size: int, part: Partition) -> Tuple[int, int]:
    nbytes = ctypes.c_size_t(0)
    slots = ctypes.c_int32(0)
    _check(load().mla_decode_workspace_size(ctypes.byref(d), batch, max_pages, page_size, ctypes.byref(part),
                                            ctypes.byref(nbytes), ctypes.byref(slots)), "mla_decode_workspace_size")
    return nbytes.value, slots.value


def lse_part_offset(d: Dims, num_slots: int) -> int:
    return load().mla_lse_part_offset(ctypes.byref(d), num_slots)


def make_cache(kv, block_table, seq_lens, page_size: int, scales=None) -> PagedCache:
    """Describe a paged cache held in torch device tensors.

    kv: [num_pages, page, W] (float32 / bfloat16 / uint8-or-float8 codes);
    block_table: [B, max_pages] int32; seq_lens: [B] int32; scales: fp8 only.
    """
    return PagedCache(_ptr(kv), _ptr(scales), dtype_code(kv), page_size, kv.shape[0], _ptr(block_table),
                      block_table.shape[1], _ptr(seq_lens))


def decode(d: Dims, q_lat, q_pe, cache: PagedCache, softmax_scale: float, part: Partition, workspace, o_lat,
           lse=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().mla_decode(ctypes.byref(d), q_lat.shape[0], _ptr(q_lat), _ptr(q_pe), dtype_code(q_lat),
                             ctypes.byref(cache), ctypes.c_float(softmax_scale), ctypes.byref(part), _ptr(workspace),
                             ws_bytes, _ptr(o_lat), dtype_code(o_lat), _ptr(lse), _stream(stream)), "mla_decode")
    return o_lat


def decode_noalloc(d: Dims, q_lat, q_pe, cache: PagedCache, softmax_scale: float, part: Partition, o_lat,
                   lse=None, stream=None):
    """mla_decode + mla_merge_splits with the split partials in the library's own device array."""
    _check(load().mla_decode_noalloc(ctypes.byref(d), q_lat.shape[0], _ptr(q_lat), _ptr(q_pe), dtype_code(q_lat),
                                     ctypes.byref(cache), ctypes.c_float(softmax_scale), ctypes.byref(part),
                                     _ptr(o_lat), dtype_code(o_lat), _ptr(lse), _stream(stream)), "mla_decode_noalloc")
    return o_lat, lse


def merge_splits(d: Dims, seq_lens, page_size: int, max_pages: int, part: Partition, workspace, o_lat, lse=None,
                 stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().mla_merge_splits(ctypes.byref(d), seq_lens.shape[0], _ptr(seq_lens), page_size, max_pages,
                                   ctypes.byref(part), _ptr(workspace), ws_bytes, _ptr(o_lat), dtype_code(o_lat),
                                   _ptr(lse), _stream(stream)), "mla_merge_splits")
    return o_lat


def multi_workspace_size(d: Dims, batch: int, q_len: int, max_pages: int, page_size: int,
                         part: Partition) -> Tuple[int, int]:
    nbytes = ctypes.c_size_t(0)
    slots = ctypes.c_int32(0)
    _check(load().mla_decode_multi_workspace_size(ctypes.byref(d), batch, q_len, max_pages, page_size,
                                                  ctypes.byref(part), ctypes.byref(nbytes), ctypes.byref(slots)),
           "mla_decode_multi_workspace_size")
    return nbytes.value, slots.value


def decode_multi(d: Dims, q_lat, q_pe, cache: PagedCache, softmax_scale: float, part: Partition, workspace, o_lat,
                 lse=None, stream=None):
    """q_len new tokens per sequence, causal within them: q_lat [B, q_len, n_h, d_c], q_pe [B, q_len, n_h, d_r],
    o_lat [B, q_len, n_h, d_c], lse [B, q_len, n_h] (merge included)."""
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().mla_decode_multi(ctypes.byref(d), q_lat.shape[0], q_lat.shape[1], _ptr(q_lat), _ptr(q_pe),
                                   dtype_code(q_lat), ctypes.byref(cache), ctypes.c_float(softmax_scale),
                                   ctypes.byref(part), _ptr(workspace), ws_bytes, _ptr(o_lat), dtype_code(o_lat),
                                   _ptr(lse), _stream(stream)), "mla_decode_multi")
    return o_lat


def decode_multi_out_proj(d: Dims, q_lat, q_pe, cache: PagedCache, softmax_scale: float, part: Partition,
                          workspace, o_lat, w_uv, o_heads, lse=None, stream=None):
    """decode_multi(...) then out_proj over the B * q_len rows, the merge and the
    projection in one launch; o_heads [B, q_len, n_h * d_h]."""
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().mla_decode_multi_out_proj(ctypes.byref(d), q_lat.shape[0], q_lat.shape[1], _ptr(q_lat), _ptr(q_pe),
                                            dtype_code(q_lat), ctypes.byref(cache), ctypes.c_float(softmax_scale),
                                            ctypes.byref(part), _ptr(workspace), ws_bytes, _ptr(o_lat),
                                            dtype_code(o_lat), _ptr(lse), _ptr(w_uv), dtype_code(w_uv), _ptr(o_heads),
                                            dtype_code(o_heads), _stream(stream)), "mla_decode_multi_out_proj")
    return o_heads


def prefill_workspace_size(d: Dims, batch: int, total_kv: int) -> int:
    nbytes = ctypes.c_size_t(0)
    _check(load().mla_prefill_workspace_size(ctypes.byref(d), batch, total_kv, ctypes.byref(nbytes)),
           "mla_prefill_workspace_size")
    return nbytes.value


def prefill(d: Dims, q_offsets, total_q: int, max_q_len: int, q_nope, q_pe, cache: PagedCache, total_kv: int,
            w_uk, w_uv, softmax_scale: float, workspace, o_heads, lse=None, stream=None):
    """Non-absorbed attention of new prompt tokens: q_offsets [B+1] int32 (rows of sequence b's new tokens),
    q_nope [total_q, n_h, d_h], q_pe [total_q, n_h, d_r], o_heads [total_q, n_h, d_h], lse [total_q, n_h]."""
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().mla_prefill(ctypes.byref(d), q_offsets.shape[0] - 1, _ptr(q_offsets), total_q, max_q_len,
                              _ptr(q_nope), _ptr(q_pe), dtype_code(q_nope), ctypes.byref(cache), total_kv,
                              _ptr(w_uk), _ptr(w_uv), dtype_code(w_uk), ctypes.c_float(softmax_scale),
                              _ptr(workspace), ws_bytes, _ptr(o_heads), dtype_code(o_heads), _ptr(lse),
                              _stream(stream)), "mla_prefill")
    return o_heads


def out_proj(d: Dims, o_lat, w_uv, o_heads, stream=None):
    """o_heads[b, i*d_h:(i+1)*d_h] = W^UV_i o_lat[b,i,:]; shapes [B,n_h,d_c], [n_h*d_h, d_c], [B, n_h*d_h]."""
    _check(load().mla_out_proj(ctypes.byref(d), o_lat.shape[0], _ptr(o_lat), dtype_code(o_lat), _ptr(w_uv),
                               dtype_code(w_uv), _ptr(o_heads), dtype_code(o_heads), _stream(stream)), "mla_out_proj")
    return o_heads


def merge_out_proj(d: Dims, seq_lens, page_size: int, max_pages: int, part: Partition, workspace, o_lat, w_uv,
                   o_heads, lse=None, stream=None):
    """merge_splits(...) then out_proj(o_lat, w_uv, o_heads), one launch on the bf16 fast path."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().mla_merge_out_proj(ctypes.byref(d), seq_lens.shape[0], _ptr(seq_lens), page_size, max_pages,
                                     ctypes.byref(part), _ptr(workspace), ws_bytes, _ptr(o_lat), dtype_code(o_lat),
                                     _ptr(lse), _ptr(w_uv), dtype_code(w_uv), _ptr(o_heads), dtype_code(o_heads),
                                     _stream(stream)), "mla_merge_out_proj")
    return o_heads


def rope(base: float, yarn_scale: float = 1.0, yarn_alpha: float = 0.0, yarn_beta: float = 0.0,
         yarn_orig_ctx: int = 0) -> Rope:
    return Rope(base, yarn_scale, yarn_alpha, yarn_beta, yarn_orig_ctx)


def yarn_attention_factor(yarn_scale: float) -> float:
    return load().mla_yarn_attention_factor(ctypes.c_float(yarn_scale))


def cache_store(d: Dims, rows, positions, cache: PagedCache, rope_base: float = 0.0, stream=None, rope=None):
    """Write rows [B, d_c+d_rope] (f32/bf16) at token positions [B] (int32, device) into the cache.
    rope: an mla_rope_t (Rope) instead of rope_base (YaRN frequencies)."""
    if rope is not None:
        _check(load().mla_cache_store_rope(ctypes.byref(d), rows.shape[0], _ptr(rows), dtype_code(rows),
                                           _ptr(positions), ctypes.byref(rope), ctypes.byref(cache), _stream(stream)),
               "mla_cache_store_rope")
        return
    _check(load().mla_cache_store(ctypes.byref(d), rows.shape[0], _ptr(rows), dtype_code(rows), _ptr(positions),
                                  ctypes.c_float(rope_base), ctypes.byref(cache), _stream(stream)), "mla_cache_store")


def cache_append(d: Dims, h, w_dkv, w_kr, rows, positions, cache: PagedCache, rope_base: float, stream=None,
                 rope=None):
    """rows = [W^DKV h ; W^KR h], then cache_store(rows, positions, rope_base).

    rows: fp32 scratch [8, B, d_c+d_rope]; rows[0] holds the projected rows afterwards."""
    if rope is not None:
        _check(load().mla_cache_append_rope(ctypes.byref(d), h.shape[1], h.shape[0], _ptr(h), dtype_code(h),
                                            _ptr(w_dkv), _ptr(w_kr), dtype_code(w_dkv), _ptr(rows), _ptr(positions),
                                            ctypes.byref(rope), ctypes.byref(cache), _stream(stream)),
               "mla_cache_append_rope")
        return
    _check(load().mla_cache_append(ctypes.byref(d), h.shape[1], h.shape[0], _ptr(h), dtype_code(h), _ptr(w_dkv),
                                   _ptr(w_kr), dtype_code(w_dkv), _ptr(rows), _ptr(positions),
                                   ctypes.c_float(rope_base), ctypes.byref(cache), _stream(stream)), "mla_cache_append")


def query_prep_scratch_size(d: Dims, d_qlatent: int, batch: int) -> int:
    return load().mla_query_prep_scratch_size(ctypes.byref(d), d_qlatent, batch)


def query_prep(d: Dims, h, w_dq, w_uq, w_qr, positions, q_nope, q_pe, scratch, rope_base: float = 10000.0,
               stream=None, rope=None):
    """c^Q = W^DQ h, q_nope = W^UQ c^Q, q_pe = RoPE(W^QR c^Q) per head; shapes [B, d], [d_q, d],
    [n_h d_h, d_q], [n_h d_r, d_q], positions [B] int32, outputs [B, n_h, d_h], [B, n_h, d_r]."""
    nbytes = scratch.numel() * scratch.element_size()
    d_qlatent = 0 if w_dq is None else w_dq.shape[0]   # 0: query not compressed (w_uq, w_qr act on h)
    if rope is not None:
        _check(load().mla_query_prep_rope(ctypes.byref(d), h.shape[1], d_qlatent, h.shape[0], _ptr(h), dtype_code(h),
                                          _ptr(w_dq), _ptr(w_uq), _ptr(w_qr), dtype_code(w_uq), _ptr(positions),
                                          ctypes.byref(rope), _ptr(q_nope), _ptr(q_pe), dtype_code(q_nope),
                                          _ptr(scratch), nbytes, _stream(stream)), "mla_query_prep_rope")
        return q_nope, q_pe
    _check(load().mla_query_prep(ctypes.byref(d), h.shape[1], d_qlatent, h.shape[0], _ptr(h), dtype_code(h),
                                 _ptr(w_dq), _ptr(w_uq), _ptr(w_qr), dtype_code(w_uq), _ptr(positions),
                                 ctypes.c_float(rope_base), _ptr(q_nope), _ptr(q_pe), dtype_code(q_nope),
                                 _ptr(scratch), nbytes, _stream(stream)), "mla_query_prep")
    return q_nope, q_pe


def partition_host(seq_lens, page_size: int, max_pages: int, part: Partition):
    """Workspace slots of each sequence's partials: (first[b], count[b]) lists (host only)."""
    import numpy as np
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    b = lens.shape[0]
    first = np.zeros(b, dtype=np.int32)
    count = np.zeros(b, dtype=np.int32)
    I32P = ctypes.POINTER(ctypes.c_int32)
    _check(load().mla_partition_host(lens.ctypes.data_as(I32P), b, page_size, max_pages, ctypes.byref(part),
                                     first.ctypes.data_as(I32P), count.ctypes.data_as(I32P)), "mla_partition_host")
    return first, count


def validate_cache_host(block_table, seq_lens, page_size: int, num_pages: int) -> Tuple[int, int]:
    """Host check of a cache's block table and lengths (numpy or CPU arrays):
    returns (status, first offending sequence or -1)."""
    import numpy as np
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    if bt.ndim != 2 or lens.ndim != 1 or bt.shape[0] != lens.shape[0]:
        raise ValueError("block_table must be [batch, max_pages] and seq_lens [batch]")
    bad = ctypes.c_int32(-1)
    I32P = ctypes.POINTER(ctypes.c_int32)
    st = load().mla_validate_cache_host(bt.ctypes.data_as(I32P), lens.ctypes.data_as(I32P), lens.shape[0],
                                        bt.shape[1], page_size, num_pages, ctypes.byref(bad))
    return int(st), int(bad.value)
