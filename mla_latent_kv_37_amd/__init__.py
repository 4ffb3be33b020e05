"""MLA latent-KV decode on AMD Instinct MI355X (gfx950).

The product is libmla.so (include/mla.h), built from csrc/ by
``python -m mla_latent_kv_37_amd.build``.  This package is a thin binding:
``_lib`` marshals torch tensors into the C ABI, ``DecodeStep`` chains the four
calls of one decode step (absorb -> decode -> merge + out proj) with buffers
allocated once; ``cache_store`` / ``cache_append`` write new tokens into the
cache.  Every arithmetic step runs in the library's HIP kernels.
"""
from __future__ import annotations

from . import _lib
from ._lib import (MLA_BF16, MLA_F32, MLA_FP8_E4M3, MlaError, absorb_q, build_info, cache_append,  # noqa: F401
                   cache_store, decode, decode_multi, decode_noalloc, decode_multi_out_proj, dims, lse_part_offset, make_cache, merge_out_proj,
                   merge_splits, multi_workspace_size, out_proj, partition, partition_host, prefill, prefill_workspace_size,
                   query_prep, query_prep_scratch_size, rope, yarn_attention_factor,
                   status_string, validate_cache_host, workspace_size)

__all__ = ["DecodeStep", "DeviceCache", "upload_cache"]


class DeviceCache:
    """A paged latent cache in device memory plus its C descriptor."""

    def __init__(self, kv, block_table, seq_lens, page_size, scales=None):
        self.kv, self.block_table, self.seq_lens, self.scales = kv, block_table, seq_lens, scales
        self.page_size = page_size
        self.desc = make_cache(kv, block_table, seq_lens, page_size, scales)

    @property
    def batch(self) -> int:
        return self.seq_lens.shape[0]

    @property
    def max_pages(self) -> int:
        return self.block_table.shape[1]


def upload_cache(kv_words, block_table, seq_lens, dtype: str, page_size: int, scales=None, device="cuda"):
    """Copy a host paged cache (storage words as numpy) to the device.

    kv_words: uint32 (f32 bits) / uint16 (bf16 bits) / uint8 (fp8 codes) array.
    """
    import numpy as np
    import torch
    if dtype == "f32":
        kv = torch.from_numpy(np.ascontiguousarray(kv_words).view(np.float32)).to(device)
    elif dtype == "bf16":
        kv = torch.from_numpy(np.ascontiguousarray(kv_words).view(np.int16)).to(device).view(torch.bfloat16)
    elif dtype == "fp8":
        kv = torch.from_numpy(np.ascontiguousarray(kv_words)).to(device)
    else:
        raise ValueError(dtype)
    bt = torch.from_numpy(np.ascontiguousarray(block_table, dtype=np.int32)).to(device)
    sl = torch.from_numpy(np.ascontiguousarray(seq_lens, dtype=np.int32)).to(device)
    sc = None if scales is None else torch.from_numpy(np.ascontiguousarray(scales, dtype=np.float32)).to(device)
    return DeviceCache(kv, bt, sl, page_size, sc)


class DecodeStep:
    """One MLA decode step over a batch: absorb -> decode -> merge -> out projection.

    Buffers (q_lat, o_lat, lse, o_heads, workspace) are allocated once for a
    (batch, max_pages, partition) shape and reused by every call.
    """

    def __init__(self, n_heads, d_head, d_rope, d_latent, batch, max_pages, page_size=64, split_tokens=0,
                 num_parts=0, act_dtype=None, device="cuda"):
        import torch
        self.torch = torch
        self.d = dims(n_heads, d_head, d_rope, d_latent)
        self.part = partition(split_tokens, num_parts)
        self.batch, self.max_pages, self.page_size = batch, max_pages, page_size
        act = torch.bfloat16 if act_dtype is None else act_dtype
        self.q_lat = torch.empty(batch, n_heads, d_latent, dtype=act, device=device)
        self.o_lat = torch.empty(batch, n_heads, d_latent, dtype=act, device=device)
        self.lse = torch.empty(batch, n_heads, dtype=torch.float32, device=device)
        self.o_heads = torch.empty(batch, n_heads * d_head, dtype=act, device=device)
        nbytes, self.num_slots = workspace_size(self.d, batch, max_pages, page_size, self.part)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)

    def partials(self):
        """Views (o_part [slots, n_h, d_c] in the output dtype, lse_part [slots, n_h] fp32) into the workspace."""
        n, h, c = self.num_slots, self.d.n_heads, self.d.d_latent
        if n == 0:
            return None, None
        off = lse_part_offset(self.d, n)
        ws = self.workspace
        odt = self.o_lat.dtype
        o = ws[: n * h * c * odt.itemsize].view(odt).view(n, h, c)
        l = ws[off: off + n * h * 4].view(self.torch.float32).view(n, h)
        return o, l

    def absorb(self, q_nope, w_uk, stream=None):
        return absorb_q(self.d, q_nope, w_uk, self.q_lat, stream)

    def attend(self, q_lat, q_pe, cache: DeviceCache, scale, stream=None):
        decode(self.d, q_lat, q_pe, cache.desc, scale, self.part, self.workspace, self.o_lat, self.lse, stream)
        merge_splits(self.d, cache.seq_lens, cache.page_size, cache.max_pages, self.part, self.workspace, self.o_lat,
                     self.lse, stream)
        return self.o_lat, self.lse

    def project(self, w_uv, stream=None):
        return out_proj(self.d, self.o_lat, w_uv, self.o_heads, stream)

    def attend_project(self, q_lat, q_pe, w_uv, cache: DeviceCache, scale, stream=None):
        """decode, then the split merge and W^UV projection in one call (mla_merge_out_proj)."""
        decode(self.d, q_lat, q_pe, cache.desc, scale, self.part, self.workspace, self.o_lat, self.lse, stream)
        return merge_out_proj(self.d, cache.seq_lens, cache.page_size, cache.max_pages, self.part, self.workspace,
                              self.o_lat, w_uv, self.o_heads, self.lse, stream)

    def __call__(self, q_nope, q_pe, w_uk, w_uv, cache: DeviceCache, scale, stream=None):
        self.absorb(q_nope, w_uk, stream)
        return self.attend_project(self.q_lat, q_pe, w_uv, cache, scale, stream)
