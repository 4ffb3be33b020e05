"""Float64 oracle of Multi-head Latent Attention (MLA) decode, non-absorbed form.

Test infrastructure only (see oracle/__init__.py).  Every function follows the
formulas of the pages, written out plainly:

* [V2-explainer] 一文通透DeepSeek-V2(改造Transformer的中文模型)：详解MoE、GRPO、MLA —
  §2.1.2 (MHA and its per-token cache), §2.2.1 (joint KV compression and query
  compression), §2.2.2 (decoupled RoPE, the cached pair c^KV / k^R, per-token
  cache (d_c + d_h^R) l), §3.1.1 (V2 hyper-parameters).
* [Key-tech] deepseek(2)——deepseek 關鍵技術 — §1 Multi-Head Latent Attention:
  the full per-head formula set, including the concatenations [k^C; k^R],
  [q^C; q^R] and the softmax scale 1/sqrt(d_h + d_h^R).

Head i owns rows [i*d_h, (i+1)*d_h) of W^UK, W^UV, W^UQ and rows
[i*d_h^R, (i+1)*d_h^R) of W^QR (the stacked notation [x_1; ...; x_{n_h}] of
[Key-tech] §1).  The decoupled key k^R is one vector shared by all heads.

Weights are (out, in) matrices as on the pages: y = W x.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

ROPE_BASE = 10000.0


def softmax_scale(d_head: int, d_rope: int) -> float:
    """1/sqrt(d_h + d_h^R): the scale of the MLA score in [Key-tech] §1."""
    return 1.0 / math.sqrt(d_head + d_rope)


# ---------------------------------------------------------------------------
# RoPE ([V2-explainer] §2.2.2: a position-m rotation R_m applied to q and k)
# ---------------------------------------------------------------------------

def rope(x: np.ndarray, pos, base: float = ROPE_BASE) -> np.ndarray:
    """Rotate consecutive pairs (x[2k], x[2k+1]) by angle pos * base**(-2k/d).

    x: [..., d] with d even; pos: scalar or array broadcastable to x[..., 0].
    The pages show only R_m; the pair layout and base are the RoFormer ones.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    k = np.arange(d // 2, dtype=np.float64)
    theta = base ** (-2.0 * k / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def yarn_theta(d: int, base: float, scale: float, alpha: float, beta: float, orig_ctx: int) -> np.ndarray:
    """RoPE frequencies after YaRN context extension ([V2-explainer] §3.1.3 gives
    s = 40, alpha = 1, beta = 32 and applies YaRN to the RoPE-carrying key k^R;
    the ramp is the YaRN definition the page refers to): pair k's plain
    frequency theta_k = base^(-2k/d) turns r_k = orig_ctx * theta_k / (2 pi)
    times over the original context; gamma_k = clip((r_k - alpha) / (beta -
    alpha), 0, 1); the new frequency is (1 - gamma_k) theta_k / s + gamma_k theta_k
    (slow pairs interpolated by s, fast pairs unchanged, a linear ramp between).
    scale = 1 gives the plain frequencies."""
    k = np.arange(d // 2, dtype=np.float64)
    theta = base ** (-2.0 * k / d)
    if scale == 1.0:
        return theta
    r = orig_ctx * theta / (2.0 * math.pi)
    gamma = np.clip((r - alpha) / (beta - alpha), 0.0, 1.0)
    return (1.0 - gamma) * theta / scale + gamma * theta


def rope_theta(x: np.ndarray, pos, theta: np.ndarray) -> np.ndarray:
    """Rotate consecutive pairs (x[2k], x[2k+1]) by angle pos * theta[k]."""
    x = np.asarray(x, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def yarn_attention_factor(scale: float) -> float:
    """The softmax-scale multiplier of YaRN in MLA: the page's length factor
    sqrt(t) = 0.0707 ln s + 1, applied to both sides of the dot product, so the
    scores are multiplied by t = (0.0707 ln s + 1)^2 ([V2-explainer] §3.1.3)."""
    f = 0.0707 * math.log(scale) + 1.0 if scale > 1.0 else 1.0
    return f * f


# ---------------------------------------------------------------------------
# projections from the hidden state h
# ---------------------------------------------------------------------------

def project_cache(h: np.ndarray, W: Dict[str, np.ndarray], positions: np.ndarray):
    """c^KV_j = W^DKV h_j and k^R_j = RoPE(W^KR h_j) for every token j.

    [V2-explainer] §2.2.1 (first compression formula) and §2.2.2 (k^R);
    k^R is cached after the rotation.  Returns (c_kv [T, d_c], k_r [T, d_r]).
    """
    h = np.asarray(h, dtype=np.float64)
    c_kv = h @ W["W_DKV"].T
    k_r = rope(h @ W["W_KR"].T, positions)
    return c_kv, k_r


def project_query(h_t: np.ndarray, W: Dict[str, np.ndarray], pos: int, n_heads: int):
    """c^Q = W^DQ h_t, q^C = W^UQ c^Q, q^R = RoPE(W^QR c^Q) per head.

    [V2-explainer] §2.2.1 (query compression) and §2.2.2 (q^R); [Key-tech] §1.
    Returns (q_c [n_h, d_h], q_r [n_h, d_r]).
    """
    c_q = W["W_DQ"] @ np.asarray(h_t, dtype=np.float64)
    q_c = (W["W_UQ"] @ c_q).reshape(n_heads, -1)
    q_r = rope((W["W_QR"] @ c_q).reshape(n_heads, -1), pos)
    return q_c, q_r


# ---------------------------------------------------------------------------
# attention over the cache, non-absorbed
# ---------------------------------------------------------------------------

def head_rows(W: np.ndarray, i: int, width: int) -> np.ndarray:
    return W[i * width:(i + 1) * width]


def attend_head(q_c_i: np.ndarray, q_r_i: np.ndarray, c_kv: np.ndarray, k_r: np.ndarray,
                W_UK: np.ndarray, W_UV: np.ndarray, i: int, scale: float):
    """One head of the decode attention, with keys and values up-projected.

    k^C_{j,i} = W^UK_i c^KV_j, v^C_{j,i} = W^UV_i c^KV_j ([V2-explainer] §2.2.1),
    k_{j,i} = [k^C_{j,i}; k^R_j], q_i = [q^C_i; q^R_i] ([Key-tech] §1),
    s_j = q_i . k_{j,i} * scale, p = softmax over all cached tokens j (the query
    is the newest token, so every cached token is visible), o_i = sum_j p_j v^C_{j,i}.

    Returns dict(o [d_h], p [T], lse (natural log of sum_j exp(s_j)), s [T]).
    """
    d_h = q_c_i.shape[0]
    k_c = c_kv @ head_rows(W_UK, i, d_h).T          # [T, d_h]
    v_c = c_kv @ head_rows(W_UV, i, d_h).T          # [T, d_h]
    k = np.concatenate([k_c, k_r], axis=1)          # [T, d_h + d_r]
    q = np.concatenate([q_c_i, q_r_i])
    s = (k @ q) * scale
    m = s.max()
    e = np.exp(s - m)
    z = e.sum()
    p = e / z
    return {"o": p @ v_c, "p": p, "lse": m + math.log(z), "s": s}


def attend(q_c: np.ndarray, q_r: np.ndarray, c_kv: np.ndarray, k_r: np.ndarray,
           W_UK: np.ndarray, W_UV: np.ndarray, scale: Optional[float] = None,
           heads: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Decode attention of one query token over one sequence's cache, per head.

    q_c [n_h, d_h], q_r [n_h, d_r], c_kv [T, d_c], k_r [T, d_r].
    Returns o_heads [n_h, d_h] (the concatenation [o_1; ...; o_nh] that W^O takes,
    [Key-tech] §1), lse [n_h], p [n_h, T] and the absorbed-form quantities that
    the same softmax weights define:
      q_lat_i = (W^UK_i)^T q^C_i  and  o_lat_i = sum_j p_ij c^KV_j,
    ([V2-explainer] §2.2.2: W^UK can be absorbed on the query side and W^UV on
    the output side).  Rows of heads not listed in `heads` are NaN.
    """
    n_h, d_h = q_c.shape
    T = c_kv.shape[0]
    if scale is None:
        scale = softmax_scale(d_h, q_r.shape[1])
    heads = range(n_h) if heads is None else heads
    out = {
        "o_heads": np.full((n_h, d_h), np.nan), "lse": np.full(n_h, np.nan),
        "p": np.full((n_h, T), np.nan), "q_lat": np.full((n_h, c_kv.shape[1]), np.nan),
        "o_lat": np.full((n_h, c_kv.shape[1]), np.nan),
    }
    for i in heads:
        r = attend_head(q_c[i], q_r[i], c_kv, k_r, W_UK, W_UV, i, scale)
        out["o_heads"][i] = r["o"]
        out["lse"][i] = r["lse"]
        out["p"][i] = r["p"]
        out["q_lat"][i] = head_rows(W_UK, i, d_h).T @ q_c[i]
        out["o_lat"][i] = r["p"] @ c_kv
    return out


def attend_new_tokens(q_c: np.ndarray, q_r: np.ndarray, c_kv: np.ndarray, k_r: np.ndarray,
                      W_UK: np.ndarray, W_UV: np.ndarray, scale: Optional[float] = None,
                      heads: Optional[Sequence[int]] = None) -> List[Dict[str, np.ndarray]]:
    """Attention of a sequence's q_len newest tokens, each at its own position.

    q_c [q_len, n_h, d_h], q_r [q_len, n_h, d_r]; c_kv [T, d_c], k_r [T, d_r] hold
    all T cached tokens, the q_len new ones last.  New token t sits at position
    T - q_len + t, and the single-token formula's sum over the tokens up to and
    including the query's own position ([Key-tech] §1, the attention-output
    formula) applies at that position: token t attends to cache rows
    0 .. T - q_len + t.  Several new tokens per step arise when the multi-token
    prediction modules are kept for decoding ([Key-tech] §2.2, MTP at inference).
    Returns one attend() dict per new token (a token with no visible row, when
    T < q_len, gets lse = -inf and zero outputs).
    """
    q_len = q_c.shape[0]
    T = c_kv.shape[0]
    out = []
    for t in range(q_len):
        n = T - q_len + t + 1
        if n <= 0:
            n_h, d_h = q_c.shape[1:]
            out.append({"o_heads": np.zeros((n_h, d_h)), "lse": np.full(n_h, -np.inf),
                        "o_lat": np.zeros((n_h, c_kv.shape[1]))})
            continue
        out.append(attend(q_c[t], q_r[t], c_kv[:n], k_r[:n], W_UK, W_UV, scale, heads))
    return out


def prefill_head(q_c_i: np.ndarray, q_r_i: np.ndarray, c_kv: np.ndarray, k_r: np.ndarray,
                 W_UK: np.ndarray, W_UV: np.ndarray, i: int, scale: Optional[float] = None):
    """Head i of the attention of a sequence's q_len newest tokens, all at once.

    The same quantity as attend_new_tokens, written as matrices: the keys
    k_{j,i} = [W^UK_i c^KV_j; k^R_j] and values v_{j,i} = W^UV_i c^KV_j of all T
    cached rows are formed once ([V2-explainer] §2.2.1 and §2.2.2), the score
    matrix S[t, j] = [q^C_{t,i}; q^R_{t,i}] . k_{j,i} * scale ([Key-tech] §1)
    keeps, for new token t at position T - q_len + t, the rows j <= T - q_len + t
    (the sum over earlier positions of [Key-tech] §1), each kept row of S is
    soft-maxed and O = P V.  This is the prompt-processing (prefill) shape:
    with q_len = T every cached token is new.
    q_c_i [q_len, d_h], q_r_i [q_len, d_r], c_kv [T, d_c], k_r [T, d_r].
    Returns dict(o [q_len, d_h], lse [q_len]); a token with no visible row gets
    o = 0 and lse = -inf.
    """
    q_len, d_h = q_c_i.shape
    T = c_kv.shape[0]
    if scale is None:
        scale = softmax_scale(d_h, q_r_i.shape[1])
    k = np.concatenate([c_kv @ head_rows(W_UK, i, d_h).T, k_r], axis=1)   # [T, d_h + d_r]
    v = c_kv @ head_rows(W_UV, i, d_h).T                                  # [T, d_h]
    q = np.concatenate([q_c_i, q_r_i], axis=1)                            # [q_len, d_h + d_r]
    s = (q @ k.T) * scale                                                 # [q_len, T]
    visible = np.arange(T)[None, :] <= (T - q_len + np.arange(q_len))[:, None]
    s = np.where(visible, s, -np.inf)
    o = np.zeros((q_len, d_h))
    lse = np.full(q_len, -np.inf)
    for t in range(q_len):
        if not visible[t].any():
            continue
        m = s[t].max()
        e = np.exp(s[t] - m)
        z = e.sum()
        o[t] = (e / z) @ v
        lse[t] = m + math.log(z)
    return {"o": o, "lse": lse}


def chunk_partials(q_c, q_r, c_kv, k_r, W_UK, W_UV, chunk: int, scale=None, heads=None):
    """Attention restricted to each chunk [s*chunk, min((s+1)*chunk, T)) of the cache.

    Chunk s yields its own normalised outputs and log-sum-exp (the quantities a
    split of the sequence produces).  Returns a list of dicts like attend().
    """
    T = c_kv.shape[0]
    parts = []
    for lo in range(0, T, chunk):
        hi = min(lo + chunk, T)
        parts.append(attend(q_c, q_r, c_kv[lo:hi], k_r[lo:hi], W_UK, W_UV, scale, heads))
    return parts


def merge_partials(o_parts: List[np.ndarray], lse_parts: List[np.ndarray]):
    """Combine per-chunk softmax results: lse = log sum_s e^{lse_s}, o = sum_s e^{lse_s-lse} o_s.

    An empty chunk carries lse = -inf and weight 0.  With all chunks empty the
    result is o = 0, lse = -inf.
    """
    lse_s = np.stack([np.asarray(x, dtype=np.float64) for x in lse_parts])   # [S, ...]
    m = lse_s.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lse_s), np.exp(lse_s - m_safe), 0.0)
    z = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(z > 0, z, 1.0)), -np.inf)
    o = sum(w[s][..., None] * np.asarray(o_parts[s], dtype=np.float64) for s in range(len(o_parts)))
    o = np.where(finite[..., None], o / np.where(z > 0, z, 1.0)[..., None], 0.0)
    return o, lse


def out_project(o_heads: np.ndarray, W_O: np.ndarray) -> np.ndarray:
    """u_t = W^O [o_1; ...; o_nh] ([Key-tech] §1, last formula)."""
    return W_O @ np.asarray(o_heads, dtype=np.float64).reshape(-1)


def forward_from_h(h: np.ndarray, W: Dict[str, np.ndarray], n_heads: int, t: Optional[int] = None,
                   scale: Optional[float] = None):
    """The whole MLA attention step for query token t (default: the last row of h).

    Tokens 0..t are cached; positions are the token indices.
    """
    h = np.asarray(h, dtype=np.float64)
    t = h.shape[0] - 1 if t is None else t
    pos = np.arange(t + 1)
    c_kv, k_r = project_cache(h[: t + 1], W, pos)
    q_c, q_r = project_query(h[t], W, t, n_heads)
    r = attend(q_c, q_r, c_kv, k_r, W["W_UK"], W["W_UV"], scale)
    r.update(c_kv=c_kv, k_r=k_r, q_c=q_c, q_r=q_r)
    if "W_O" in W:
        r["u"] = out_project(r["o_heads"], W["W_O"])
    return r


# ---------------------------------------------------------------------------
# per-token cache size ([V2-explainer] §2.1.2 and §2.2.2; GQA/MQA in §2.1.1)
# ---------------------------------------------------------------------------

def cache_elems_mha(n_heads: int, d_head: int, layers: int) -> int:
    return 2 * n_heads * d_head * layers


def cache_elems_gqa(n_groups: int, d_head: int, layers: int) -> int:
    return 2 * n_groups * d_head * layers


def cache_elems_mqa(d_head: int, layers: int) -> int:
    return 2 * d_head * layers


def cache_elems_mla(d_latent: int, d_rope: int, layers: int) -> int:
    return (d_latent + d_rope) * layers


def cache_row_elems(cache_row: np.ndarray) -> int:
    """Elements one cached token row really holds (for checking a built cache)."""
    return int(np.asarray(cache_row).size)
