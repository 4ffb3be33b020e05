"""Test cases: seeded inputs (synth), stored values, oracle references, device upload.

Every expected value comes from the oracle (float64, non-absorbed) evaluated on
exactly the values the GPU reads: bf16-rounded queries/weights and the stored
cache (bf16 bits, or fp8 codes times their group scales).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

import oracle
import synth
from oracle import storage as ostore

TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 3e-2}


def bf16_round(x: np.ndarray) -> np.ndarray:
    return ostore.bf16_bits_to_f64(synth.to_bf16_bits(x))


def f32_round(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


@dataclasses.dataclass
class Case:
    dims: synth.Dims
    cache_dtype: str
    act: str                    # "f32" or "bf16": queries, weights, outputs
    q_nope: np.ndarray          # stored values, float64 [B, n_h, d_h]
    q_pe: np.ndarray            # [B, n_h, d_r]
    W_UK: np.ndarray            # [n_h*d_h, d_c]
    W_UV: np.ndarray
    cache: synth.PagedCache
    W_O: Optional[np.ndarray] = None

    @property
    def lens(self) -> List[int]:
        return [int(t) for t in self.cache.seq_lens]

    @property
    def scale(self) -> float:
        return oracle.softmax_scale(self.dims.d_head, self.dims.d_rope)

    def stored_rows(self, b: int) -> np.ndarray:
        return ostore.stored_rows_f64(self.cache, b)

    def reference(self, b: int, heads=None, chunk: Optional[int] = None):
        """Oracle results for sequence b (memoised: a case is compared under
        several partitions)."""
        key = (b, None if heads is None else tuple(heads), chunk)
        memo = self.__dict__.setdefault("_memo", {})
        if key not in memo:
            memo[key] = self._reference(b, heads, chunk)
        return memo[key]

    def _reference(self, b: int, heads=None, chunk: Optional[int] = None):
        rows = self.stored_rows(b)
        dc = self.dims.d_latent
        args = (self.q_nope[b], self.q_pe[b], rows[:, :dc], rows[:, dc:], self.W_UK, self.W_UV, self.scale, heads)
        if chunk is None:
            return oracle.attend(*args)
        return oracle.chunk_partials(*args[:6], chunk=chunk, scale=self.scale, heads=heads)


def _round(x, act):
    return f32_round(x) if act == "f32" else bf16_round(x)


def case_from_rows(dims, rows: List[np.ndarray], q_nope, q_pe, W_UK, W_UV, cache_dtype: str, act: str,
                   rng_perm: np.random.Generator, W_O=None, spare_pages: int = 2, max_pages=None) -> Case:
    words, scales = [], []
    for r in rows:
        w, s = synth.store_rows(r, cache_dtype)
        words.append(w)
        scales.append(s)
    cache = synth.build_paged(words, cache_dtype, rng_perm, scales_per_seq=scales if cache_dtype == "fp8" else None,
                              spare_pages=spare_pages, max_pages=max_pages)
    return Case(dims, cache_dtype, act, _round(q_nope, act), _round(q_pe, act), _round(W_UK, act),
                _round(W_UV, act), cache, W_O)


def from_h_case(config_id: int) -> Case:
    """Workloads 1 and 2: cache and query through the pages' chain from h (oracle projections)."""
    w = synth.workload(config_id)
    d = w.dims
    sigma = 0.02 if config_id == 1 else synth.V2_SIGMA_W
    W = synth.weights(d, sigma, synth.rng_for(config_id, synth.S_WEIGHTS), with_wo=True)
    T = w.lens[0]
    h = synth.hidden_states(T, d.d_model, synth.rng_for(config_id, synth.S_H))
    c_kv, k_r = oracle.project_cache(h, W, np.arange(T))
    q_c, q_r = oracle.project_query(h[T - 1], W, T - 1, d.n_heads)
    rows = [np.concatenate([c_kv, k_r], axis=1).astype(np.float32)]
    act = "f32" if w.cache_dtype == "f32" else "bf16"
    return case_from_rows(d, rows, q_c[None], q_r[None], W["W_UK"], W["W_UV"], w.cache_dtype, act,
                          synth.rng_for(config_id, synth.S_PERM), W_O=W["W_O"])


def direct_case(config_id: int, lens, query_gain: float = 1.0, cache_dtype: Optional[str] = None,
                max_pages=None, seed=None) -> Case:
    inp = synth.direct_inputs_for(config_id, seed=seed, lens=lens, query_gain=query_gain)
    w = inp["workload"]
    cd = cache_dtype or w.cache_dtype
    return case_from_rows(w.dims, inp["rows"], inp["q_nope"], inp["q_pe"], inp["W_UK"], inp["W_UV"], cd, "bf16",
                          synth.rng_for(config_id, synth.S_PERM, seed), max_pages=max_pages)


# ---------------------------------------------------------------------------
# device side
# ---------------------------------------------------------------------------

def to_device(case: Case):
    import torch
    import mla_latent_kv_37_amd as mk
    tdt = torch.float32 if case.act == "f32" else torch.bfloat16

    def t(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(tdt).contiguous()

    dev = dict(q_nope=t(case.q_nope), q_pe=t(case.q_pe), W_UK=t(case.W_UK), W_UV=t(case.W_UV))
    dev["cache"] = mk.upload_cache(case.cache.kv, case.cache.block_table, case.cache.seq_lens, case.cache_dtype,
                                   case.cache.page_size, case.cache.scales)
    dev["dtype"] = tdt
    return dev


def run_step(case: Case, dev, split_tokens=0, num_parts=0):
    import torch
    import mla_latent_kv_37_amd as mk
    d = case.dims
    step = mk.DecodeStep(d.n_heads, d.d_head, d.d_rope, d.d_latent, len(case.lens), case.cache.block_table.shape[1],
                         case.cache.page_size, split_tokens, num_parts, act_dtype=dev["dtype"])
    check_guards = guard_step(step)
    step(dev["q_nope"], dev["q_pe"], dev["W_UK"], dev["W_UV"], dev["cache"], case.scale)
    torch.cuda.synchronize()
    check_guards()
    return step


# ---------------------------------------------------------------------------
# comparison criteria
# ---------------------------------------------------------------------------
#
# Vectors (q_lat, o_lat, o_heads, partial outputs): max|gpu - ref| <= tol *
# max|ref| with tol = 1e-4 (f32 cache), 1e-2 (bf16), 3e-2 (fp8), evaluated per
# sequence (and per new token), so that one short sequence's error is not
# hidden under a long one's larger values.
#
# lse is an fp32 value and is compared in absolute terms, against a bound
# derived from the arithmetic.  The GPU scores use q_lat rounded to the
# activation dtype (relative error u_q: 2^-9 for bf16 plus the fp32 absorb
# accumulation, (d_h + 1) 2^-24) and, for an fp8 cache, the dequantised rows
# rounded to bf16 (u_k = 2^-9); the 576-term dot product accumulates in fp32
# (gamma = (d_c + d_r) 2^-24 relative to the sum of |terms|).  With
# A_j = sum_d |q_d| |k_jd| (latent and RoPE parts), every score is within
#     E = scale * max_j ((u_q + gamma) A^lat_j + (u_k + gamma) A_j)
# of the oracle's, and lse, being 1-Lipschitz in the max norm of the scores,
# within E as well.  On top of that, a floor of c (1 + |lse|) covers the fp32
# exponentials, sums and logarithm of the online softmax and the merge
# (c = 2e-5 with the hardware exp2/log2 of the MFMA kernels, 2e-6 for the
# generic fp32 kernel).

U16 = 2.0 ** -9
U32 = 2.0 ** -24


def lse_tolerance(case: "Case", q_lat_ref: np.ndarray, q_pe: np.ndarray, rows: np.ndarray,
                  lse_ref: np.ndarray) -> np.ndarray:
    """Per-head absolute bound on |lse_gpu - lse_ref| (see above); q_lat_ref
    [H, d_c], q_pe [H, d_r], rows [T, d_c + d_r] (stored values), lse_ref [H]."""
    d = case.dims
    dc = d.d_latent
    a_lat = np.abs(q_lat_ref) @ np.abs(rows[:, :dc]).T
    a_all = a_lat + np.abs(q_pe) @ np.abs(rows[:, dc:]).T
    u_q = (U16 if case.act == "bf16" else 0.0) + (d.d_head + 1) * U32
    u_k = U16 if case.cache_dtype == "fp8" else 0.0
    gamma = (dc + d.d_rope) * U32
    e = case.scale * np.max((u_q + gamma) * a_lat + (u_k + gamma) * a_all, axis=1)
    floor = (2e-6 if case.cache_dtype == "f32" else 2e-5) * (1.0 + np.abs(lse_ref))
    return e + floor


def check_vec(name: str, got, ref, tol: float) -> float:
    """max|got - ref| <= tol * max|ref| over the finite reference entries; returns the error."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = np.isfinite(ref)
    assert np.all(np.isfinite(got[m])), f"{name}: non-finite output"
    err = rel_err(got, ref)
    assert err <= tol, f"{name}: rel err {err:.3e} > {tol:g}"
    return err


def check_lse(name: str, got, ref, bound) -> float:
    """|got - ref| <= bound elementwise; returns the largest |got - ref| / bound."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite lse"
    err = np.abs(got - ref)
    worst = int(np.argmax(err / bound))
    assert np.all(err <= bound), (f"{name}: |lse err| {err.max():.3e} above its bound "
                                  f"(worst at {worst}: err {err[worst]:.3e}, bound {bound[worst]:.3e})")
    return float(np.max(err / bound))


class Worst:
    """Largest error seen per compared tensor, printed once at the end of a comparison."""

    def __init__(self):
        self.e = {}

    def add(self, k, v):
        self.e[k] = max(self.e.get(k, 0.0), v)

    def report(self, tol):
        for k, v in sorted(self.e.items()):
            what = "|err|/bound" if k.startswith("lse") else f"rel err (tol {tol:g})"
            print(f"  {k}: worst {what} {v:.3e}", flush=True)


def compare_seq(case: "Case", b: int, ref, got: dict, tol: float, heads, worst: Worst, tag: str = "",
                rows: Optional[np.ndarray] = None, q_pe: Optional[np.ndarray] = None):
    """Check one sequence's (or one new token's) outputs against the oracle dict
    `ref`: vectors per sequence, lse against its derived bound.  got maps names
    (q_lat, o_lat, o_heads, lse) to [n_h, ...] arrays."""
    hs = list(range(case.dims.n_heads)) if heads is None else list(heads)
    for k in ("q_lat", "o_lat", "o_heads"):
        if k in got:
            worst.add(k, check_vec(f"{k}[{tag or b}]", got[k][hs], ref[k][hs], tol))
    if "lse" in got:
        rows = case.stored_rows(b) if rows is None else rows
        q_pe = case.q_pe[b] if q_pe is None else q_pe
        bound = lse_tolerance(case, ref["q_lat"][hs], q_pe[hs], rows, ref["lse"][hs])
        worst.add("lse", check_lse(f"lse[{tag or b}]", got["lse"][hs], ref["lse"][hs], bound))


# ---------------------------------------------------------------------------
# guard regions around the outputs
# ---------------------------------------------------------------------------

GUARD_BYTES = 4096
GUARD_BYTE = 0x5A


def guarded_empty(shape, dtype, device="cuda"):
    """A tensor of `shape` inside a larger allocation whose GUARD_BYTES before and
    after it hold GUARD_BYTE; returns (tensor, check) where check() asserts that
    the guards are unchanged."""
    import torch
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    raw = torch.full((GUARD_BYTES + n + GUARD_BYTES,), GUARD_BYTE, dtype=torch.uint8, device=device)
    t = raw[GUARD_BYTES:GUARD_BYTES + n].view(dtype).view(shape)

    def check(name="buffer"):
        h = raw.cpu().numpy()
        assert np.all(h[:GUARD_BYTES] == GUARD_BYTE), f"{name}: bytes before the buffer were written"
        assert np.all(h[GUARD_BYTES + n:] == GUARD_BYTE), f"{name}: bytes after the buffer were written"
    return t, check


def guard_step(step):
    """Replace a DecodeStep's buffers (q_lat, o_lat, lse, o_heads, workspace) by
    guarded ones; returns a function that checks every guard."""
    checks = []
    for name in ("q_lat", "o_lat", "lse", "o_heads", "workspace"):
        old = getattr(step, name)
        t, c = guarded_empty(tuple(old.shape), old.dtype)
        setattr(step, name, t)
        checks.append((name, c))

    def check_all():
        for name, c in checks:
            c(name)
    return check_all


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| over finite reference entries."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = np.isfinite(ref)
    denom = np.abs(ref[m]).max() if m.any() else 1.0
    return float(np.abs(got[m] - ref[m]).max() / max(denom, 1e-300))


def host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)
