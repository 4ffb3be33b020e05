"""Oracle side: decoding of the stored cache formats and the paged gather, in float64.

Test infrastructure only (see oracle/__init__.py).

* bf16 is the upper half of an IEEE binary32 word, so its value is exact in float64.
* fp8 is OCP E4M3FN: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
  subnormals at exponent field 0, no infinities, and the all-ones pattern
  (S.1111.111) is NaN, giving a finite maximum of 448.  The cache stores one fp32
  scale per token per 128-channel group (the 1x128 per-token-group activation
  format of the FP8 strategy in the V3 interview notes, Deepseek系列从v3到R易背面经版,
  section F8量化策略); a stored value is code * scale.
* A paged cache stores token t of sequence b in page block_table[b][t // page]
  at slot t % page (the paged KV memory idea the DeepSeek-V2 explainer,
  一文通透DeepSeek-V2 §2.1.1, names as a KV-cache optimisation).
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns -> float64 (exact)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def f32_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """uint8 OCP E4M3FN codes -> float64, from the bit fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = sign * (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & ((c & 0x7) == 7), np.nan, val)


def dequantize_rows(codes: np.ndarray, scales: np.ndarray, group: int = 128) -> np.ndarray:
    """codes [N, W] uint8, scales [N, ceil(W/group)] -> float64 [N, W] = code * scale."""
    vals = e4m3fn_to_f64(codes)
    n, w = vals.shape
    for g in range((w + group - 1) // group):
        sl = slice(g * group, min((g + 1) * group, w))
        vals[:, sl] *= np.asarray(scales[:, g], dtype=np.float64)[:, None]
    return vals


def gather_sequence(kv_pages: np.ndarray, block_row: np.ndarray, seq_len: int,
                    page_size: int) -> np.ndarray:
    """Rows [seq_len, W] of one sequence, one token at a time from the paged buffer."""
    out = np.empty((seq_len,) + kv_pages.shape[2:], dtype=kv_pages.dtype)
    for t in range(seq_len):
        out[t] = kv_pages[int(block_row[t // page_size]), t % page_size]
    return out


def stored_rows_f64(cache, b: int) -> np.ndarray:
    """The float64 values of sequence b's cached rows exactly as the GPU reads them."""
    t = int(cache.seq_lens[b])
    words = gather_sequence(cache.kv, cache.block_table[b], t, cache.page_size)
    if cache.dtype == "f32":
        return f32_bits_to_f64(words)
    if cache.dtype == "bf16":
        return bf16_bits_to_f64(words)
    if cache.dtype == "fp8":
        sc = gather_sequence(cache.scales, cache.block_table[b], t, cache.page_size)
        return dequantize_rows(words, sc)
    raise ValueError(cache.dtype)
