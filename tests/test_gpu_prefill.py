"""GPU parity of the non-absorbed prefill (mla_prefill) against the oracle's
prefill_head, which is pinned to the per-token attend_new_tokens and to causal
torch SDPA (tests/test_oracle.py).

Each sequence's cache holds T_b tokens, the q_len_b new ones last; new token t
attends to positions 0 .. T_b - q_len_b + t.  The references use the values the
GPU reads (the stored bf16 / fp8-dequantised rows, bf16 queries and weights).
Per new token: the output over the sampled heads within TOL of its max|ref|, and
lse within a bound derived from the arithmetic (below).
"""
import numpy as np
import pytest

import oracle
from _cases import TOL, direct_case, guarded_empty, host, rel_err, to_device, _round

pytestmark = pytest.mark.gpu

U16 = 2.0 ** -9     # bf16 unit roundoff
U32 = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_37_amd as mk
    mk._lib.load()
    print("libmla:", mk.build_info(), flush=True)


def _queries(case, q_lens, seed, gain):
    import synth
    rng = np.random.default_rng(seed)
    d = case.dims
    n = int(sum(q_lens))
    sd = synth.V2LITE_SD if d.n_heads == 16 else synth.V2_SD_QUERY
    q_c = rng.normal(0.0, sd * gain, size=(n, d.n_heads, d.d_head))
    q_r = rng.normal(0.0, sd * gain, size=(n, d.n_heads, d.d_rope))
    return _round(q_c, "bf16"), _round(q_r, "bf16")


def _run(case, dev, q_lens, q_c, q_r, total_kv=None, max_q_len=None, extra_rows=0):
    import torch
    import mla_latent_kv_37_amd as mk
    d = case.dims
    dd = mk.dims(d.n_heads, d.d_head, d.d_rope, d.d_latent)
    if extra_rows:
        q_c = np.concatenate([q_c, np.zeros((extra_rows,) + q_c.shape[1:])])
        q_r = np.concatenate([q_r, np.zeros((extra_rows,) + q_r.shape[1:])])
    n = q_c.shape[0]
    q_off = torch.tensor(np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32), device="cuda")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(torch.bfloat16)  # noqa: E731
    qn, qp = t(q_c).contiguous(), t(q_r).contiguous()
    total_kv = int(sum(case.lens)) if total_kv is None else total_kv
    max_q_len = int(max(q_lens)) if max_q_len is None else max_q_len
    ws = torch.empty(mk.prefill_workspace_size(dd, len(q_lens), total_kv), dtype=torch.uint8, device="cuda")
    out, chk_out = guarded_empty((n, d.n_heads, d.d_head), torch.bfloat16)
    lse, chk_lse = guarded_empty((n, d.n_heads), torch.float32)
    out.fill_(float("nan"))
    lse.fill_(float("nan"))
    mk.prefill(dd, q_off, n, max_q_len, qn, qp, dev["cache"].desc, total_kv, dev["W_UK"], dev["W_UV"], case.scale,
               ws, out, lse)
    torch.cuda.synchronize()
    chk_out("o_heads")
    chk_lse("lse")
    return host(out), host(lse)


def _lse_bound(case, q_c, q_r, rows, W_UK_i, visible, lse_ref):
    """|lse_gpu - lse_ref| <= max over visible j of the score error bound, plus a
    floor.  Bf16 cache: the keys k^C are the only rounded operand of the scores
    (bf16 from an fp32 product over 512 terms), so the error of s_j is at most
    scale * sum_d |q^C_d| |k^C_{j,d}| (U16 + 600 U32); q and k^R are exact stored
    values, dot products and row sums fp32.  Fp8 cache: the gathered rows are
    code * scale rounded to bf16, which adds scale * (|q^C| |W^UK| |c^KV_j| +
    |q^R| |k^R_j|) U16."""
    d = case.dims
    c_kv, k_r = rows[:, :d.d_latent], rows[:, d.d_latent:]
    a = np.abs(q_c) @ np.abs(c_kv @ W_UK_i.T).T * (U16 + 600 * U32)           # [q_len, T]
    if case.cache_dtype == "fp8":
        a = a + (np.abs(q_c) @ (np.abs(W_UK_i) @ np.abs(c_kv).T) + np.abs(q_r) @ np.abs(k_r).T) * U16
    a = np.where(visible, a, 0.0).max(axis=1)
    return case.scale * a + 2e-5 * (1.0 + np.abs(np.where(np.isfinite(lse_ref), lse_ref, 0.0)))


def _compare(case, q_lens, q_c, q_r, got, tol, heads):
    out, lse = got
    d = case.dims
    worst_o = worst_l = 0.0
    row0 = 0
    for b, (T, ql) in enumerate(zip(case.lens, q_lens)):
        if ql == 0:
            continue
        rows = case.stored_rows(b)
        c_kv, k_r = rows[:, :d.d_latent], rows[:, d.d_latent:]
        qs = slice(row0, row0 + ql)
        visible = np.arange(T)[None, :] <= (T - ql + np.arange(ql))[:, None]
        refs = {i: oracle.prefill_head(q_c[qs, i], q_r[qs, i], c_kv, k_r, case.W_UK, case.W_UV, i, case.scale)
                for i in heads}
        for t in range(ql):
            if not visible[t].any():
                assert np.all(out[row0 + t] == 0) and np.all(np.isneginf(lse[row0 + t])), (b, t)
                continue
            ref_o = np.stack([refs[i]["o"][t] for i in heads])
            e = rel_err(out[row0 + t][heads], ref_o)
            assert np.all(np.isfinite(out[row0 + t][heads])), (b, t)
            assert e <= tol, f"o_heads[b={b},t={t}]: rel err {e:.3e} > {tol:g}"
            worst_o = max(worst_o, e)
        for i in heads:
            ref_l = refs[i]["lse"]
            ok = np.isfinite(ref_l)
            bound = _lse_bound(case, q_c[qs, i], q_r[qs, i], rows, case.W_UK[i * d.d_head:(i + 1) * d.d_head],
                               visible, ref_l)
            err = np.abs(np.where(ok, lse[qs, i], 0.0) - np.where(ok, ref_l, 0.0))
            assert np.all(np.isfinite(lse[qs, i][ok])), (b, i)
            assert np.all(err[ok] <= bound[ok]), (f"lse[b={b},head={i}]: |err| {err[ok].max():.3e} above its bound "
                                                  f"{bound[ok][np.argmax(err[ok] / bound[ok])]:.3e}")
            worst_l = max(worst_l, float(np.max(err[ok] / bound[ok])) if ok.any() else 0.0)
        row0 += ql
    print(f"  o_heads: worst rel err {worst_o:.3e} (tol {tol:g}); lse: worst |err|/bound {worst_l:.3e}", flush=True)


HEADS = [0, 1, 31, 64, 127]


@pytest.fixture(scope="module")
def v2_ragged():
    # a single token, a full 64-token prompt, a chunk after a prefix, a prompt
    # longer than its cache (2 of its tokens see nothing), several 256-token
    # blocks with a ragged tail, and a prompt ending mid-tile
    lens = [1, 64, 300, 2, 700, 517]
    case = direct_case(3, lens, max_pages=12, seed=81)
    return case, to_device(case)


V2_Q_LENS = [1, 64, 45, 4, 700, 300]


def test_prefill_v2_bf16_ragged(v2_ragged):
    case, dev = v2_ragged
    print(f"case: prefill V2 bf16, lens {case.lens}, q_lens {V2_Q_LENS}", flush=True)
    q_c, q_r = _queries(case, V2_Q_LENS, seed=11, gain=1.0)
    _compare(case, V2_Q_LENS, q_c, q_r, _run(case, dev, V2_Q_LENS, q_c, q_r), TOL["bf16"], HEADS)


def test_prefill_deterministic_and_capacity_slack(v2_ragged):
    """Two calls give identical bits; a larger total_kv (spare rows) and a larger
    max_q_len (empty token blocks) change nothing."""
    case, dev = v2_ragged
    q_c, q_r = _queries(case, V2_Q_LENS, seed=12, gain=1.0)
    a = _run(case, dev, V2_Q_LENS, q_c, q_r)
    b = _run(case, dev, V2_Q_LENS, q_c, q_r)
    c = _run(case, dev, V2_Q_LENS, q_c, q_r, total_kv=sum(case.lens) + 1000, max_q_len=1500)
    for x, y in ((a, b), (a, c)):
        np.testing.assert_array_equal(x[0], y[0])
        np.testing.assert_array_equal(x[1], y[1])


def test_prefill_v2_bf16_sharp():
    lens = [96, 400]
    case = direct_case(3, lens, max_pages=8, seed=82)
    dev = to_device(case)
    q_lens = [96, 333]
    print(f"case: prefill V2 bf16 sharp (gain 20), lens {lens}, q_lens {q_lens}", flush=True)
    q_c, q_r = _queries(case, q_lens, seed=13, gain=20.0)
    _compare(case, q_lens, q_c, q_r, _run(case, dev, q_lens, q_c, q_r), TOL["bf16"], HEADS)


def test_prefill_v2_fp8():
    lens = [333, 70]
    case = direct_case(3, lens, cache_dtype="fp8", max_pages=8, seed=83)
    dev = to_device(case)
    q_lens = [300, 70]
    print(f"case: prefill V2 fp8 cache, lens {lens}, q_lens {q_lens}", flush=True)
    q_c, q_r = _queries(case, q_lens, seed=14, gain=1.0)
    _compare(case, q_lens, q_c, q_r, _run(case, dev, q_lens, q_c, q_r), TOL["fp8"], HEADS)


def test_prefill_v2lite_all_heads():
    """16 heads (the V2-Lite shape), every head checked."""
    lens = [200, 37, 512]
    case = direct_case(6, lens, max_pages=9, seed=84)
    dev = to_device(case)
    q_lens = [200, 37, 260]
    print(f"case: prefill V2-Lite bf16, lens {lens}, q_lens {q_lens}", flush=True)
    q_c, q_r = _queries(case, q_lens, seed=15, gain=1.0)
    _compare(case, q_lens, q_c, q_r, _run(case, dev, q_lens, q_c, q_r), TOL["bf16"], list(range(16)))


def test_prefill_v2_long_prompt_sampled():
    """Two 2048-token prompts (8 token blocks, 64 position tiles): sampled heads and tokens."""
    lens = [2048, 1500]
    case = direct_case(3, lens, max_pages=32, seed=85)
    dev = to_device(case)
    q_lens = [2048, 1500]
    print(f"case: prefill V2 bf16 long, lens {lens}, q_lens {q_lens}", flush=True)
    q_c, q_r = _queries(case, q_lens, seed=16, gain=1.0)
    out, lse = _run(case, dev, q_lens, q_c, q_r)
    d = case.dims
    rng = np.random.default_rng(3)
    row0 = 0
    worst = 0.0
    for b, (T, ql) in enumerate(zip(lens, q_lens)):
        rows = case.stored_rows(b)
        toks = np.unique(np.concatenate([[0, 255, 256, ql - 1], rng.integers(0, ql, 12)]))
        for i in (5, 100):
            r = oracle.prefill_head(q_c[row0:row0 + ql, i], q_r[row0:row0 + ql, i], rows[:, :d.d_latent],
                                    rows[:, d.d_latent:], case.W_UK, case.W_UV, i, case.scale)
            for t in toks:
                e = rel_err(out[row0 + t, i], r["o"][t])
                assert e <= TOL["bf16"], (b, i, t, e)
                assert abs(lse[row0 + t, i] - r["lse"][t]) <= 2e-2, (b, i, t)
                worst = max(worst, e)
        row0 += ql
    print(f"  sampled o_heads: worst rel err {worst:.3e}", flush=True)


def test_prefill_bad_page_ids_read_as_zero_rows():
    """A block-table entry outside the cache reads as a page of zero rows (no
    fault): the oracle sees those rows as zeros."""
    import torch
    lens = [150]
    case = direct_case(3, lens, max_pages=4, seed=86)
    dev = to_device(case)
    bt = dev["cache"].block_table
    bt[0, 1] = 1 << 20          # positions 64..127
    q_lens = [150]
    q_c, q_r = _queries(case, q_lens, seed=17, gain=1.0)
    out, lse = _run(case, dev, q_lens, q_c, q_r)
    rows = case.stored_rows(0).copy()
    rows[64:128] = 0.0
    d = case.dims
    for i in (0, 77):
        r = oracle.prefill_head(q_c[:, i], q_r[:, i], rows[:, :d.d_latent], rows[:, d.d_latent:], case.W_UK,
                                case.W_UV, i, case.scale)
        for t in (0, 63, 64, 100, 149):
            assert rel_err(out[t, i], r["o"][t]) <= TOL["bf16"], (i, t)
    torch.cuda.synchronize()


def test_prefill_empty_sequences_and_spare_rows():
    """Sequences with no new tokens, an empty cache, and rows of q / o_heads past
    the last sequence's tokens: the spare rows stay untouched (NaN), the others
    match the oracle."""
    lens = [0, 50, 200, 7, 0]
    q_lens = [0, 50, 0, 7, 0]
    case = direct_case(3, lens, max_pages=4, seed=87)
    dev = to_device(case)
    q_c, q_r = _queries(case, q_lens, seed=18, gain=1.0)
    out, lse = _run(case, dev, q_lens, q_c, q_r, extra_rows=5)
    n = sum(q_lens)
    assert np.all(np.isnan(out[n:])) and np.all(np.isnan(lse[n:]))
    _compare(case, q_lens, q_c, q_r, (out[:n], lse[:n]), TOL["bf16"], HEADS)
