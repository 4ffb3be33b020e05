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
* Encoding (for the cache-store step): bf16 is binary32 rounded to nearest,
  ties to even, at bit 16; E4M3FN takes the nearest representable value, ties to
  the even mantissa.  A group's scale is amax / 448 computed in binary32 (an
  all-zero group gets 1, so that its codes are 0), and each value is divided by
  it in binary32 before rounding: the quotient stays within +-448 up to a
  binary32 rounding error, which rounds back to 448.
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


# ---------------------------------------------------------------------------
# encoders (the store side of the formats above)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """binary32 values -> bf16 bit patterns, round to nearest, ties to even.

    Adding 0x7FFF plus the lowest kept bit and truncating is that rounding on the
    bit pattern; NaN stays a (quiet) NaN.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep) >> np.uint64(16)).astype(np.uint16)
    nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    return np.where(nan, ((u >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16), r)


E4M3_MAX = 448.0


def f64_to_e4m3fn(x: np.ndarray) -> np.ndarray:
    """Values -> OCP E4M3FN codes: the nearest representable value, ties to the
    even mantissa (the 3-bit field), sign kept (also for zero).

    Magnitudes are multiples of the quantum 2**(e-3) of their binade e (e >= -6;
    below 2**-6 the subnormal quantum 2**-9 holds).  A magnitude at or past the
    midpoint 464 between 448 and the next binade step has no finite nearest
    value and becomes NaN (0x7F), as the format has no infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    v = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    e = np.clip(e, -6, 8)
    quantum = np.exp2(e - 3)
    q = np.round(v / quantum) * quantum          # numpy rounds halves to even
    # encode q (its binade may be one higher than v's after rounding up)
    with np.errstate(divide="ignore"):
        eq = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    sub = q < 2.0 ** -6
    exp_field = np.where(sub, 0, eq + 7).astype(np.int64)
    mant = np.where(sub, q / 2.0 ** -9, q / np.exp2(eq - 3) - 8.0)
    mant = np.rint(mant).astype(np.int64)
    code = (exp_field << 3) | mant
    code = np.where(q == 0, 0, code)
    code = np.where(np.signbit(x), code | 0x80, code)
    bad = (v >= 464.0) | np.isnan(x)
    return np.where(bad, 0x7F | np.where(np.signbit(x), 0x80, 0), code).astype(np.uint8)


def quantize_e4m3_groups(rows: np.ndarray, group: int = 128):
    """binary32 rows [N, W] -> (codes uint8 [N, W], scales float32 [N, ceil(W/group)]).

    Per row and group of `group` columns: scale = amax / 448 in binary32 (1 when
    the group is all zero), code = E4M3FN(binary32(x / scale)).
    """
    x = np.asarray(rows, dtype=np.float32)
    n, w = x.shape
    ng = (w + group - 1) // group
    codes = np.zeros((n, w), dtype=np.uint8)
    scales = np.ones((n, ng), dtype=np.float32)
    for g in range(ng):
        sl = slice(g * group, min((g + 1) * group, w))
        amax = np.max(np.abs(x[:, sl]), axis=1)
        sc = np.where(amax > 0, (amax / np.float32(E4M3_MAX)).astype(np.float32), np.float32(1.0)).astype(np.float32)
        scales[:, g] = sc
        codes[:, sl] = f64_to_e4m3fn((x[:, sl] / sc[:, None]).astype(np.float32).astype(np.float64))
    return codes, scales
