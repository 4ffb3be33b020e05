"""Seeded synthetic inputs for MLA decode.

This module is the only code shared by the float64 oracle (``oracle/``) and the
HIP path (``mla_latent_kv_37_amd``).  It draws random numbers, converts them to
the storage formats the cache uses (bf16 bits, OCP fp8 E4M3 codes with one fp32
scale per 128-channel group of a token row) and scatters token rows into a paged
buffer.  It holds none of the attention arithmetic: no projection, no RoPE, no
softmax, no absorption.  Storage conversions are delegated to torch's CPU casts
(round-to-nearest-even for bf16; round-to-nearest-even with a finite maximum of
448 for ``float8_e4m3fn``).

Workloads follow the DeepSeek-V2 shapes given in the DeepSeek-V2 explainer
(一文通透DeepSeek-V2, §3.1.1 model hyper-parameters): 128 heads of width 128,
latent width 512, query latent 1536, decoupled RoPE width 64, hidden 5120, and
weights drawn with standard deviation 0.006; one workload uses the V2-Lite
shapes of the same page (16 heads, hidden 2048, no query compression).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

PAGE_SIZE = 64
FP8_GROUP = 128
FP8_MAX = 448.0

# Standard deviations of the hot-path inputs when the cache and the queries are
# produced from h ~ N(0, 1) by weights ~ N(0, 0.006) at V2 shapes:
#   c^KV = W^DKV h  -> 0.006 * sqrt(5120)
#   k^R  = RoPE(W^KR h): same marginal (rotations keep isotropic pairs isotropic)
#   c^Q  = W^DQ h   -> 0.006 * sqrt(5120);  q^C = W^UQ c^Q -> 0.006 * sqrt(1536) * sd(c^Q)
V2_SIGMA_W = 0.006
V2_SD_LATENT = V2_SIGMA_W * math.sqrt(5120.0)
V2_SD_QUERY = V2_SIGMA_W * math.sqrt(1536.0) * V2_SD_LATENT


@dataclasses.dataclass(frozen=True)
class Dims:
    n_heads: int      # n_h
    d_head: int       # d_h
    d_rope: int       # d_h^R
    d_latent: int     # d_c
    d_qlatent: int    # d_c'
    d_model: int      # d

    @property
    def row(self) -> int:
        """Width of one cached token row: [c^KV | k^R]."""
        return self.d_latent + self.d_rope


TINY = Dims(n_heads=4, d_head=16, d_rope=8, d_latent=32, d_qlatent=48, d_model=128)
V2 = Dims(n_heads=128, d_head=128, d_rope=64, d_latent=512, d_qlatent=1536, d_model=5120)
# DeepSeek-V2-Lite (V2 explainer, the V2-Lite paragraph): 16 heads of width 128,
# latent 512, RoPE width 64, hidden 2048; the query is not compressed (d_c' = 0).
V2LITE = Dims(n_heads=16, d_head=128, d_rope=64, d_latent=512, d_qlatent=0, d_model=2048)
# With weights ~ N(0, 0.006) and h ~ N(0, 1) at V2-Lite shapes, c^KV = W^DKV h and
# the uncompressed q^C = W^Q h both have standard deviation 0.006 * sqrt(2048).
V2LITE_SD = V2_SIGMA_W * math.sqrt(2048.0)


def rng_for(config_id: int, stream: int, seed: Optional[int] = None) -> np.random.Generator:
    """Independent generator for (workload, stream).  Default entropy 1000+config_id."""
    base = 1000 + config_id if seed is None else seed
    return np.random.default_rng(np.random.SeedSequence(base).spawn(stream + 1)[stream])


# Streams used by the generators below.
S_WEIGHTS, S_H, S_LENS, S_PERM, S_CACHE, S_QUERY, S_OUTLIER = range(7)


# ---------------------------------------------------------------------------
# storage conversions (torch CPU casts)
# ---------------------------------------------------------------------------

def _torch():
    import torch  # local: keeps `import synth` cheap for code that never converts
    return torch


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float array -> uint16 bit patterns of the round-to-nearest-even bf16 value."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_f32(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32)


def fp8_group_quantize(rows: np.ndarray, group: int = FP8_GROUP):
    """Quantise token rows to E4M3 codes with one fp32 scale per token per group.

    rows: [N, W] float.  Groups are [0,128), [128,256), ... along W; the last one
    may be narrower (the 64-wide k^R tail of a 576-wide row).  scale = amax/448
    (an all-zero group gets scale 1).  Returns (codes uint8 [N, W], scales f32
    [N, ceil(W/group)]).
    """
    torch = _torch()
    rows = np.ascontiguousarray(rows, dtype=np.float32)
    n, w = rows.shape
    ng = (w + group - 1) // group
    scales = np.empty((n, ng), dtype=np.float32)
    scaled = np.empty_like(rows)
    for g in range(ng):
        sl = slice(g * group, min((g + 1) * group, w))
        amax = np.abs(rows[:, sl]).max(axis=1)
        s = (amax / np.float32(FP8_MAX)).astype(np.float32)
        s[amax == 0] = 1.0
        scales[:, g] = s
        scaled[:, sl] = rows[:, sl] / s[:, None]
    np.clip(scaled, -FP8_MAX, FP8_MAX, out=scaled)
    codes = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, scales


# ---------------------------------------------------------------------------
# paged layout
# ---------------------------------------------------------------------------

POISON = {"f32": np.uint32(0x7FC00000), "bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F)}


@dataclasses.dataclass
class PagedCache:
    """A paged latent cache as the library reads it.

    kv:          [num_pages, page, W] storage words (uint32 for f32 bits, uint16 for
                 bf16 bits, uint8 for fp8 codes).  Slots past a sequence's length
                 and pages no sequence owns hold NaN patterns.
    scales:      [num_pages, page, ceil(W/128)] float32 (fp8 only) else None.
    block_table: [B, max_pages] int32; entries past a sequence's last page are -1.
    seq_lens:    [B] int32.
    """
    dtype: str
    kv: np.ndarray
    scales: Optional[np.ndarray]
    block_table: np.ndarray
    seq_lens: np.ndarray
    page_size: int = PAGE_SIZE

    @property
    def num_pages(self) -> int:
        return self.kv.shape[0]


def build_paged(rows_per_seq: List[np.ndarray], dtype: str, rng: np.random.Generator,
                page_size: int = PAGE_SIZE, scales_per_seq: Optional[List[np.ndarray]] = None,
                spare_pages: int = 1, max_pages: Optional[int] = None) -> PagedCache:
    """Scatter each sequence's stored rows into pages whose ids are a random permutation.

    rows_per_seq[b]: [T_b, W] array already in storage words (see PagedCache.kv).
    """
    lens = [int(r.shape[0]) for r in rows_per_seq]
    w = rows_per_seq[0].shape[1] if rows_per_seq else 1
    npages = [(t + page_size - 1) // page_size for t in lens]
    total = sum(npages) + spare_pages
    mp = max(max(npages) if npages else 0, 1) if max_pages is None else max_pages
    word = {"f32": np.uint32, "bf16": np.uint16, "fp8": np.uint8}[dtype]
    kv = np.full((total, page_size, w), POISON[dtype], dtype=word)
    scales = None
    if dtype == "fp8":
        ng = (w + FP8_GROUP - 1) // FP8_GROUP
        scales = np.full((total, page_size, ng), np.nan, dtype=np.float32)
    perm = rng.permutation(total).astype(np.int32)
    table = np.full((len(lens), mp), -1, dtype=np.int32)
    nxt = 0
    for b, rows in enumerate(rows_per_seq):
        for p in range(npages[b]):
            pid = int(perm[nxt]); nxt += 1
            table[b, p] = pid
            lo, hi = p * page_size, min((p + 1) * page_size, lens[b])
            kv[pid, : hi - lo] = rows[lo:hi]
            if scales is not None:
                scales[pid, : hi - lo] = scales_per_seq[b][lo:hi]
    return PagedCache(dtype=dtype, kv=kv, scales=scales, block_table=table,
                      seq_lens=np.asarray(lens, dtype=np.int32), page_size=page_size)


def store_rows(rows: np.ndarray, dtype: str):
    """float rows -> (storage words, scales or None) for one sequence."""
    if dtype == "f32":
        return to_f32(rows).view(np.uint32), None
    if dtype == "bf16":
        return to_bf16_bits(rows), None
    if dtype == "fp8":
        return fp8_group_quantize(rows)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def weights(dims: Dims, sigma: float, rng: np.random.Generator, with_wo: bool = True) -> Dict[str, np.ndarray]:
    """The eight MLA matrices, float64, in the pages' shapes (rows = output)."""
    d, nh, dh, dr, dc, dq = (dims.d_model, dims.n_heads, dims.d_head, dims.d_rope,
                             dims.d_latent, dims.d_qlatent)
    shapes = {
        "W_DKV": (dc, d), "W_UK": (nh * dh, dc), "W_UV": (nh * dh, dc), "W_KR": (dr, d),
        "W_DQ": (dq, d), "W_UQ": (nh * dh, dq), "W_QR": (nh * dr, dq),
    }
    if with_wo:
        shapes["W_O"] = (d, nh * dh)
    return {k: rng.normal(0.0, sigma, size=s) for k, s in shapes.items()}


def hidden_states(n_tokens: int, d_model: int, rng: np.random.Generator) -> np.ndarray:
    return rng.normal(0.0, 1.0, size=(n_tokens, d_model))


def ragged_lengths(batch: int, lo: int, hi: int, rng: np.random.Generator) -> np.ndarray:
    """Per-sequence cache lengths, uniform on the integers [lo, hi]."""
    return rng.integers(lo, hi + 1, size=batch).astype(np.int32)


def direct_decode_inputs(dims: Dims, lens, rng_cache: np.random.Generator,
                         rng_query: np.random.Generator, sd_latent: float, sd_query: float,
                         outlier_frac: float = 0.0, outlier_mult: float = 1.0,
                         rng_outlier: Optional[np.random.Generator] = None,
                         rng_weights: Optional[np.random.Generator] = None,
                         sigma_w: float = V2_SIGMA_W):
    """Hot-path inputs drawn directly with the marginals of the full chain.

    Returns dict with q_nope [B,n_h,d_h], q_pe [B,n_h,d_r], W_UK/W_UV [n_h*d_h, d_c]
    (float64) and rows: list of float32 [T_b, d_c+d_r] cache rows [c^KV | k^R].
    A seeded fraction of tokens per sequence has its c^KV part multiplied by
    outlier_mult.
    """
    b = len(lens)
    q_nope = rng_query.normal(0.0, sd_query, size=(b, dims.n_heads, dims.d_head))
    q_pe = rng_query.normal(0.0, sd_query, size=(b, dims.n_heads, dims.d_rope))
    rw = rng_weights if rng_weights is not None else rng_query
    w_uk = rw.normal(0.0, sigma_w, size=(dims.n_heads * dims.d_head, dims.d_latent))
    w_uv = rw.normal(0.0, sigma_w, size=(dims.n_heads * dims.d_head, dims.d_latent))
    rows = []
    for t in lens:
        r = rng_cache.standard_normal(size=(int(t), dims.row), dtype=np.float32)
        r *= np.float32(sd_latent)
        if outlier_frac > 0.0:
            k = int(round(outlier_frac * int(t)))
            idx = rng_outlier.choice(int(t), size=k, replace=False)
            r[idx, : dims.d_latent] *= np.float32(outlier_mult)
        rows.append(r)
    return {"q_nope": q_nope, "q_pe": q_pe, "W_UK": w_uk, "W_UV": w_uv, "rows": rows}


@dataclasses.dataclass
class Workload:
    name: str
    dims: Dims
    lens: List[int]
    cache_dtype: str          # "f32" | "bf16" | "fp8"
    split_tokens: int         # fixed split length, 0 = balanced / none
    from_h: bool              # the cache and query come from h through the pages' chain


WORKLOADS = {
    1: Workload("tiny_fp32_b1_t64", TINY, [64], "f32", 0, True),
    2: Workload("v2_bf16_b1_t4096", V2, [4096], "bf16", 0, True),
    3: Workload("v2_bf16_ragged_b64_t1024-8192", V2, [], "bf16", 0, False),
    4: Workload("v2_bf16_long_b4_t131072_split4096", V2, [131072] * 4, "bf16", 4096, False),
    5: Workload("v2_fp8_b32_t16384", V2, [16384] * 32, "fp8", 0, False),
    # the ragged batch of workload 3 at V2-Lite's 16 heads
    6: Workload("v2lite_bf16_ragged_b64_t1024-8192", V2LITE, [], "bf16", 0, False),
}


def workload(config_id: int, seed: Optional[int] = None) -> Workload:
    w = WORKLOADS[config_id]
    if config_id in (3, 6):
        lens = ragged_lengths(64, 1024, 8192, rng_for(config_id, S_LENS, seed)).tolist()
        w = dataclasses.replace(w, lens=lens)
    return w


def direct_inputs_for(config_id: int, seed: Optional[int] = None, lens=None,
                      query_gain: float = 1.0):
    """Direct-draw hot-path inputs for the V2 workloads 3, 4, 5 (or a resized copy)."""
    w = workload(config_id, seed)
    lens = w.lens if lens is None else lens
    sd_q = V2_SD_QUERY
    if config_id == 4:
        sd_lat, frac, mult = 1.0, 0.01, 8.0
    elif config_id == 6:
        sd_lat, sd_q, frac, mult = V2LITE_SD, V2LITE_SD, 0.0, 1.0
    else:
        sd_lat, frac, mult = V2_SD_LATENT, 0.0, 1.0
    out = direct_decode_inputs(
        w.dims, lens, rng_for(config_id, S_CACHE, seed), rng_for(config_id, S_QUERY, seed),
        sd_latent=sd_lat, sd_query=sd_q * query_gain, outlier_frac=frac,
        outlier_mult=mult, rng_outlier=rng_for(config_id, S_OUTLIER, seed),
        rng_weights=rng_for(config_id, S_WEIGHTS, seed))
    out["workload"] = w
    out["lens"] = list(lens)
    return out
