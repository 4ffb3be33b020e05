"""Pins of the float64 oracle against things other than itself (CPU only).

Each test names what fixes the expected value: a brute-force enumeration, a
library routine, a closed form, an invariant or a value printed on the pages
(tests/golden/).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from oracle import mla as omla
from oracle import storage as ostore

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny_problem(seed=0, T=9, n_h=3, d_h=4, d_r=2, d_c=6, scale_q=1.0):
    rng = np.random.default_rng(seed)
    return dict(
        q_c=rng.normal(size=(n_h, d_h)) * scale_q, q_r=rng.normal(size=(n_h, d_r)) * scale_q,
        c_kv=rng.normal(size=(T, d_c)), k_r=rng.normal(size=(T, d_r)),
        W_UK=rng.normal(size=(n_h * d_h, d_c)) * 0.5, W_UV=rng.normal(size=(n_h * d_h, d_c)) * 0.5,
    )


def _brute_force_mha(pr, scale):
    """Enumerate the non-absorbed MLA as textbook MHA with explicit Python loops.

    k_{j,i}[a] = sum_c W_UK[i*d_h + a, c] c_kv[j, c]  (a < d_h), then k^R_j;
    v_{j,i}[a] = sum_c W_UV[i*d_h + a, c] c_kv[j, c].
    """
    q_c, q_r, c_kv, k_r = pr["q_c"], pr["q_r"], pr["c_kv"], pr["k_r"]
    n_h, d_h = q_c.shape
    T, d_c = c_kv.shape
    d_r = k_r.shape[1]
    out = []
    lses = []
    for i in range(n_h):
        scores = []
        vals = []
        for j in range(T):
            key = [sum(pr["W_UK"][i * d_h + a][c] * c_kv[j][c] for c in range(d_c)) for a in range(d_h)]
            key += [k_r[j][r] for r in range(d_r)]
            qry = [q_c[i][a] for a in range(d_h)] + [q_r[i][r] for r in range(d_r)]
            scores.append(sum(x * y for x, y in zip(qry, key)) * scale)
            vals.append([sum(pr["W_UV"][i * d_h + a][c] * c_kv[j][c] for c in range(d_c)) for a in range(d_h)])
        mx = max(scores)
        ex = [math.exp(s - mx) for s in scores]
        z = sum(ex)
        out.append([sum(ex[j] / z * vals[j][a] for j in range(T)) for a in range(d_h)])
        lses.append(mx + math.log(z))
    return np.array(out), np.array(lses)


def test_softmax_scale_golden():
    g = json.load(open(os.path.join(GOLDEN, "softmax_scale.json")))
    for c in g["cases"]:
        assert omla.softmax_scale(c["d_head"], c["d_rope"]) == pytest.approx(c["scale"], rel=1e-15)
    assert omla.softmax_scale(128, 64) != pytest.approx(1 / math.sqrt(128))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_attend_matches_bruteforce(seed):
    pr = _tiny_problem(seed)
    scale = omla.softmax_scale(4, 2)
    ref_o, ref_lse = _brute_force_mha(pr, scale)
    r = oracle.attend(pr["q_c"], pr["q_r"], pr["c_kv"], pr["k_r"], pr["W_UK"], pr["W_UV"])
    np.testing.assert_allclose(r["o_heads"], ref_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["lse"], ref_lse, rtol=1e-12, atol=1e-13)


def test_attend_matches_torch_sdpa_float64():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    pr = _tiny_problem(5, T=37, n_h=5, d_h=8, d_r=4, d_c=16, scale_q=2.0)
    n_h, d_h = pr["q_c"].shape
    scale = 1.0 / math.sqrt(d_h + 4)
    r = oracle.attend(pr["q_c"], pr["q_r"], pr["c_kv"], pr["k_r"], pr["W_UK"], pr["W_UV"])
    c = torch.from_numpy(pr["c_kv"])
    for i in range(n_h):
        wk = torch.from_numpy(pr["W_UK"][i * d_h:(i + 1) * d_h])
        wv = torch.from_numpy(pr["W_UV"][i * d_h:(i + 1) * d_h])
        k = torch.cat([c @ wk.T, torch.from_numpy(pr["k_r"])], dim=1)[None, None]
        v = (c @ wv.T)[None, None]
        q = torch.cat([torch.from_numpy(pr["q_c"][i]), torch.from_numpy(pr["q_r"][i])])[None, None, None]
        o = F.scaled_dot_product_attention(q, k, v, scale=scale)[0, 0, 0].numpy()
        np.testing.assert_allclose(r["o_heads"][i], o, rtol=1e-12, atol=1e-14)


def test_new_tokens_single_token_is_attend():
    """q_len = 1: the one new token is the query of the single-token formula."""
    pr = _tiny_problem(11, T=13)
    r1 = oracle.attend_new_tokens(pr["q_c"][None], pr["q_r"][None], pr["c_kv"], pr["k_r"], pr["W_UK"], pr["W_UV"])
    r0 = oracle.attend(pr["q_c"], pr["q_r"], pr["c_kv"], pr["k_r"], pr["W_UK"], pr["W_UV"])
    assert len(r1) == 1
    np.testing.assert_array_equal(r1[0]["o_heads"], r0["o_heads"])
    np.testing.assert_array_equal(r1[0]["lse"], r0["lse"])


@pytest.mark.parametrize("q_len,T", [(2, 9), (4, 21), (3, 3)])
def test_new_tokens_match_torch_sdpa_causal_mask(q_len, T):
    """The q_len new tokens against torch's scaled_dot_product_attention in float64
    with an explicit boolean mask: new token t sees cache row j iff j <= T - q_len + t
    (the causal mask aligned to the end of the cache)."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(100 + q_len)
    n_h, d_h, d_r, d_c = 3, 4, 2, 6
    q_c = rng.normal(size=(q_len, n_h, d_h)) * 2.0
    q_r = rng.normal(size=(q_len, n_h, d_r)) * 2.0
    c_kv, k_r = rng.normal(size=(T, d_c)), rng.normal(size=(T, d_r))
    W_UK, W_UV = rng.normal(size=(n_h * d_h, d_c)) * 0.5, rng.normal(size=(n_h * d_h, d_c)) * 0.5
    scale = 1.0 / math.sqrt(d_h + d_r)
    res = oracle.attend_new_tokens(q_c, q_r, c_kv, k_r, W_UK, W_UV)
    mask = torch.from_numpy(np.arange(T)[None, :] <= (T - q_len + np.arange(q_len))[:, None])
    c = torch.from_numpy(c_kv)
    for i in range(n_h):
        k = torch.cat([c @ torch.from_numpy(W_UK[i * d_h:(i + 1) * d_h]).T, torch.from_numpy(k_r)], dim=1)
        v = c @ torch.from_numpy(W_UV[i * d_h:(i + 1) * d_h]).T
        q = torch.cat([torch.from_numpy(q_c[:, i]), torch.from_numpy(q_r[:, i])], dim=1)
        o = F.scaled_dot_product_attention(q[None, None], k[None, None], v[None, None], attn_mask=mask,
                                           scale=scale)[0, 0].numpy()
        for t in range(q_len):
            np.testing.assert_allclose(res[t]["o_heads"][i], o[t], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("q_len,T", [(9, 9), (4, 21), (6, 3), (1, 7)])
def test_prefill_head_matches_per_token_attention(q_len, T):
    """The matrix form (prefill_head) against the per-token loop of
    attend_new_tokens, head by head: the same visible rows, outputs and lse,
    with T < q_len included (tokens that see nothing: zeros and -inf)."""
    rng = np.random.default_rng(200 + 10 * q_len + T)
    n_h, d_h, d_r, d_c = 3, 4, 2, 6
    q_c = rng.normal(size=(q_len, n_h, d_h)) * 2.0
    q_r = rng.normal(size=(q_len, n_h, d_r)) * 2.0
    c_kv, k_r = rng.normal(size=(T, d_c)), rng.normal(size=(T, d_r))
    W_UK, W_UV = rng.normal(size=(n_h * d_h, d_c)) * 0.5, rng.normal(size=(n_h * d_h, d_c)) * 0.5
    res = oracle.attend_new_tokens(q_c, q_r, c_kv, k_r, W_UK, W_UV)
    for i in range(n_h):
        r = oracle.prefill_head(q_c[:, i], q_r[:, i], c_kv, k_r, W_UK, W_UV, i)
        for t in range(q_len):
            np.testing.assert_allclose(r["o"][t], res[t]["o_heads"][i], rtol=1e-12, atol=1e-14)
            if np.isneginf(res[t]["lse"][i]):
                assert np.isneginf(r["lse"][t])
            else:
                np.testing.assert_allclose(r["lse"][t], res[t]["lse"][i], rtol=1e-13)


def test_prefill_head_full_prompt_is_causal_sdpa():
    """q_len = T (a whole prompt): torch's scaled_dot_product_attention with
    is_causal=True on the up-projected keys and values, in float64; and the first
    token's output is its own value row (softmax over a single row)."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(7)
    T, n_h, d_h, d_r, d_c = 11, 2, 4, 2, 6
    q_c, q_r = rng.normal(size=(T, n_h, d_h)), rng.normal(size=(T, n_h, d_r))
    c_kv, k_r = rng.normal(size=(T, d_c)), rng.normal(size=(T, d_r))
    W_UK, W_UV = rng.normal(size=(n_h * d_h, d_c)), rng.normal(size=(n_h * d_h, d_c))
    scale = 1.0 / math.sqrt(d_h + d_r)
    c = torch.from_numpy(c_kv)
    for i in range(n_h):
        r = oracle.prefill_head(q_c[:, i], q_r[:, i], c_kv, k_r, W_UK, W_UV, i)
        wk = torch.from_numpy(W_UK[i * d_h:(i + 1) * d_h])
        wv = torch.from_numpy(W_UV[i * d_h:(i + 1) * d_h])
        k = torch.cat([c @ wk.T, torch.from_numpy(k_r)], dim=1)
        v = c @ wv.T
        q = torch.cat([torch.from_numpy(q_c[:, i]), torch.from_numpy(q_r[:, i])], dim=1)
        o = F.scaled_dot_product_attention(q[None, None], k[None, None], v[None, None], is_causal=True,
                                           scale=scale)[0, 0].numpy()
        np.testing.assert_allclose(r["o"], o, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(r["o"][0], v[0].numpy(), rtol=1e-13)
        s00 = float(np.dot(np.concatenate([q_c[0, i], q_r[0, i]]), k[0].numpy())) * scale
        np.testing.assert_allclose(r["lse"][0], s00, rtol=1e-13)


def test_new_tokens_shorter_cache_than_q_len():
    """T < q_len: the first q_len - T new tokens see no row (lse -inf, zero output);
    the others see rows 0 .. T - q_len + t."""
    pr = _tiny_problem(12, T=2)
    q_c = np.stack([pr["q_c"]] * 4)
    q_r = np.stack([pr["q_r"]] * 4)
    res = oracle.attend_new_tokens(q_c, q_r, pr["c_kv"], pr["k_r"], pr["W_UK"], pr["W_UV"])
    for t in (0, 1):
        assert np.all(np.isneginf(res[t]["lse"])) and np.all(res[t]["o_heads"] == 0)
    one = oracle.attend(pr["q_c"], pr["q_r"], pr["c_kv"][:1], pr["k_r"][:1], pr["W_UK"], pr["W_UV"])
    # one visible row: the output is that row's value projection (softmax weight 1)
    np.testing.assert_allclose(res[2]["o_heads"], one["o_heads"], rtol=1e-15)
    v0 = np.stack([pr["W_UV"][i * 4:(i + 1) * 4] @ pr["c_kv"][0] for i in range(3)])
    np.testing.assert_allclose(res[2]["o_heads"], v0, rtol=1e-12)


def test_absorbed_identity():
    """q_{t,i}.k_{j,i} = (W^UK_i^T q^C_i).c^KV_j + q^R_i.k^R_j and o_i = W^UV_i o_lat_i."""
    pr = _tiny_problem(7, T=20, n_h=4, d_h=6, d_r=4, d_c=10)
    n_h, d_h = pr["q_c"].shape
    scale = omla.softmax_scale(d_h, 4)
    r = oracle.attend(pr["q_c"], pr["q_r"], pr["c_kv"], pr["k_r"], pr["W_UK"], pr["W_UV"])
    for i in range(n_h):
        s_abs = (pr["c_kv"] @ r["q_lat"][i] + pr["k_r"] @ pr["q_r"][i]) * scale
        s_ref = omla.attend_head(pr["q_c"][i], pr["q_r"][i], pr["c_kv"], pr["k_r"],
                                 pr["W_UK"], pr["W_UV"], i, scale)["s"]
        np.testing.assert_allclose(s_abs, s_ref, rtol=1e-12, atol=1e-13)
        o_abs = pr["W_UV"][i * d_h:(i + 1) * d_h] @ r["o_lat"][i]
        np.testing.assert_allclose(o_abs, r["o_heads"][i], rtol=1e-12, atol=1e-13)


def test_single_token_returns_its_value():
    pr = _tiny_problem(3, T=1)
    r = oracle.attend(pr["q_c"], pr["q_r"], pr["c_kv"], pr["k_r"], pr["W_UK"], pr["W_UV"])
    d_h = pr["q_c"].shape[1]
    for i in range(pr["q_c"].shape[0]):
        np.testing.assert_allclose(r["o_heads"][i], pr["W_UV"][i * d_h:(i + 1) * d_h] @ pr["c_kv"][0], rtol=1e-13)


def test_zero_query_gives_mean_value():
    pr = _tiny_problem(4, T=11)
    pr["q_c"][:] = 0
    pr["q_r"][:] = 0
    r = oracle.attend(pr["q_c"], pr["q_r"], pr["c_kv"], pr["k_r"], pr["W_UK"], pr["W_UV"])
    d_h = pr["q_c"].shape[1]
    for i in range(pr["q_c"].shape[0]):
        mean_v = (pr["c_kv"] @ pr["W_UV"][i * d_h:(i + 1) * d_h].T).mean(axis=0)
        np.testing.assert_allclose(r["o_heads"][i], mean_v, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(r["lse"][i], math.log(11), rtol=1e-13)


def test_reduces_to_textbook_single_head():
    """n_h=1, d_r=0, W^UK = W^UV = I: softmax(q K^T / sqrt(d_h)) V (the MHA formula, [V2-explainer] §2.1.2)."""
    from scipy.special import softmax
    rng = np.random.default_rng(11)
    T, d = 13, 8
    K = rng.normal(size=(T, d))
    q = rng.normal(size=(1, d))
    eye = np.eye(d)
    r = oracle.attend(q, np.zeros((1, 0)), K, np.zeros((T, 0)), eye, eye)
    ref = softmax(q[0] @ K.T / math.sqrt(d)) @ K
    np.testing.assert_allclose(r["o_heads"][0], ref, rtol=1e-13)


def test_rope_invariants():
    rng = np.random.default_rng(2)
    x, y = rng.normal(size=8), rng.normal(size=8)
    # position 0 is the identity
    np.testing.assert_allclose(oracle.rope(x, 0), x, rtol=0, atol=0)
    # rotations keep norms
    for m in (1, 17, 4095):
        assert np.linalg.norm(oracle.rope(x, m)) == pytest.approx(np.linalg.norm(x), rel=1e-14)
    # <R_m x, R_n y> depends on n - m only
    a = oracle.rope(x, 5) @ oracle.rope(y, 12)
    b = oracle.rope(x, 105) @ oracle.rope(y, 112)
    assert a == pytest.approx(b, rel=1e-12)
    # the first pair turns by exactly m radians: (1, 0) -> (cos m, sin m)
    e = np.zeros(8); e[0] = 1.0
    r = oracle.rope(e, 3)
    assert r[0] == pytest.approx(math.cos(3.0), abs=1e-15) and r[1] == pytest.approx(math.sin(3.0), abs=1e-15)
    # the last pair of a width-8 rotation turns by m * 10000**(-6/8)
    e = np.zeros(8); e[6] = 1.0
    r = oracle.rope(e, 1000)
    ang = 1000 * 10000.0 ** -0.75
    assert r[6] == pytest.approx(math.cos(ang), abs=1e-12) and r[7] == pytest.approx(math.sin(ang), abs=1e-12)


def test_merge_identity():
    pr = _tiny_problem(9, T=50, n_h=3, d_h=4, d_r=2, d_c=6, scale_q=3.0)
    args = (pr["q_c"], pr["q_r"], pr["c_kv"], pr["k_r"], pr["W_UK"], pr["W_UV"])
    full = oracle.attend(*args)
    for chunk in (7, 16, 50, 64):
        parts = oracle.chunk_partials(*args, chunk=chunk)
        o, lse = oracle.merge_partials([p["o_heads"] for p in parts], [p["lse"] for p in parts])
        np.testing.assert_allclose(o, full["o_heads"], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse, full["lse"], rtol=1e-13)
        ol, _ = oracle.merge_partials([p["o_lat"] for p in parts], [p["lse"] for p in parts])
        np.testing.assert_allclose(ol, full["o_lat"], rtol=1e-12, atol=1e-14)
    # an empty chunk (lse = -inf) changes nothing
    o, lse = oracle.merge_partials([full["o_heads"], np.full_like(full["o_heads"], 123.0)],
                                   [full["lse"], np.full_like(full["lse"], -np.inf)])
    np.testing.assert_allclose(o, full["o_heads"], rtol=1e-15)
    np.testing.assert_allclose(lse, full["lse"], rtol=1e-15)
    # all chunks empty: o = 0, lse = -inf
    o, lse = oracle.merge_partials([np.ones((2, 3))], [np.full(2, -np.inf)])
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_cache_size_golden():
    g = json.load(open(os.path.join(GOLDEN, "v2_cache_size.json")))
    nh, dh, dc, dr, l = g["n_heads"], g["d_head"], g["d_latent"], g["d_rope"], g["layers"]
    assert dc == g["d_latent_over_d_head"] * dh and dr == g["d_rope_over_d_head"] * dh
    mla = omla.cache_elems_mla(dc, dr, l)
    assert mla == 34560 and omla.cache_elems_mha(nh, dh, l) == 1966080
    # "equal to GQA with 2.25 groups": (d_c + d_h^R) l == 2 * 2.25 * d_h * l
    assert mla == omla.cache_elems_gqa(g["gqa_equivalent_groups"], dh, l)
    assert omla.cache_elems_mqa(dh, l) * g["gqa_equivalent_groups"] == mla
    # what one built cache row holds: the latent plus the shared RoPE key
    w = synth.V2.row
    assert w == omla.cache_elems_mla(dc, dr, 1) == 576
    assert synth.TINY.row == omla.cache_elems_mla(32, 8, 1) == 40
    assert omla.cache_elems_mha(4, 16, 1) == 128


def test_e4m3_decoder_golden_and_torch():
    torch = pytest.importorskip("torch")
    g = json.load(open(os.path.join(GOLDEN, "e4m3fn_codes.json")))
    for code, val in g["codes"].items():
        got = ostore.e4m3fn_to_f64(np.array([int(code, 16)], dtype=np.uint8))[0]
        assert got == val and math.copysign(1, got) == math.copysign(1, val)
    for code in g["nan_codes"]:
        assert np.isnan(ostore.e4m3fn_to_f64(np.array([int(code, 16)], dtype=np.uint8))[0])
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    got = ostore.e4m3fn_to_f64(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    np.testing.assert_array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])


def test_bf16_decoder_against_torch():
    torch = pytest.importorskip("torch")
    bits = np.random.default_rng(0).integers(0, 65536, size=4096).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # drop inf/nan patterns
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ostore.bf16_bits_to_f64(bits), ref)


def test_fp8_dequant_error_bound():
    """Stored value = code * scale is within half an E4M3 ulp of the original."""
    rng = np.random.default_rng(1)
    rows = rng.normal(size=(64, 576)).astype(np.float32) * np.float32(0.43)
    codes, scales = synth.fp8_group_quantize(rows)
    back = ostore.dequantize_rows(codes, scales)
    x = rows.astype(np.float64)
    for g0 in range(0, 576, 128):
        sl = slice(g0, min(g0 + 128, 576))
        s = scales[:, g0 // 128].astype(np.float64)[:, None]
        amax = np.abs(x[:, sl]).max(axis=1, keepdims=True)
        np.testing.assert_allclose(amax / s, 448.0, rtol=1e-6)
        y = np.abs(x[:, sl]) / s
        # normal range: rel. error <= 2^-4; subnormal range (< 2^-6): abs error <= 2^-10
        tol = np.where(y >= 2.0 ** -6, 2.0 ** -4 * y, 2.0 ** -10) * s + 1e-12
        assert np.all(np.abs(back[:, sl] - x[:, sl]) <= tol)


def test_paged_gather_roundtrip():
    rng = np.random.default_rng(3)
    lens = [1, 63, 64, 65, 200]
    rows = [rng.normal(size=(t, 40)).astype(np.float32) for t in lens]
    words = [synth.store_rows(r, "f32")[0] for r in rows]
    cache = synth.build_paged(words, "f32", rng, spare_pages=3)
    for b, t in enumerate(lens):
        got = ostore.stored_rows_f64(cache, b)
        np.testing.assert_array_equal(got, rows[b].astype(np.float64))
    # page ids are a permutation; slots past each length are NaN
    used = cache.block_table[cache.block_table >= 0]
    assert len(set(used.tolist())) == used.size
    last = cache.block_table[3, 1]
    assert np.all(np.isnan(cache.kv[last, 1:].view(np.float32)))


def test_from_h_chain_against_explicit_matrix_products():
    """The full chain at the tiny workload, re-associated: k^C = (W^UK W^DKV) h, q^C = (W^UQ W^DQ) h."""
    w = synth.workload(1)
    d = w.dims
    W = synth.weights(d, 0.02, synth.rng_for(1, synth.S_WEIGHTS))
    h = synth.hidden_states(64, d.d_model, synth.rng_for(1, synth.S_H))
    r = oracle.forward_from_h(h, W, d.n_heads)
    t = 63
    WK = W["W_UK"] @ W["W_DKV"]
    WV = W["W_UV"] @ W["W_DKV"]
    WQ = W["W_UQ"] @ W["W_DQ"]
    WQR = W["W_QR"] @ W["W_DQ"]
    scale = 1.0 / math.sqrt(d.d_head + d.d_rope)
    heads = []
    for i in range(d.n_heads):
        hs = slice(i * d.d_head, (i + 1) * d.d_head)
        rs = slice(i * d.d_rope, (i + 1) * d.d_rope)
        q = np.concatenate([WQ[hs] @ h[t], oracle.rope(WQR[rs] @ h[t], t)])
        K = np.concatenate([h @ WK[hs].T, oracle.rope(h @ W["W_KR"].T, np.arange(64))], axis=1)
        s = K @ q * scale
        p = np.exp(s - s.max()); p /= p.sum()
        heads.append(p @ (h @ WV[hs].T))
    np.testing.assert_allclose(r["o_heads"], np.array(heads), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(r["u"], W["W_O"] @ np.concatenate(heads), rtol=1e-10, atol=1e-14)


# ---------------------------------------------------------------------------
# encoders of the cache-store step
# ---------------------------------------------------------------------------

def test_e4m3_encoder_roundtrip_ties_and_torch():
    import torch
    codes = np.arange(256, dtype=np.uint8)
    vals = ostore.e4m3fn_to_f64(codes)
    fin = ~np.isnan(vals)
    # every finite code is its own value's encoding (both zeros included)
    assert np.array_equal(ostore.f64_to_e4m3fn(vals[fin]), codes[fin])
    # midpoints between neighbouring positive values go to the even mantissa
    pos = np.sort(np.unique(vals[fin & (vals > 0)]))
    mids = (pos[:-1] + pos[1:]) / 2
    got = ostore.f64_to_e4m3fn(mids)
    lo, hi = ostore.f64_to_e4m3fn(pos[:-1]), ostore.f64_to_e4m3fn(pos[1:])
    want = np.where((lo & 1) == 0, lo, hi)
    assert np.array_equal(got, want)
    # past the last midpoint (464) there is no finite nearest value: NaN
    assert ostore.f64_to_e4m3fn(np.array([464.0, -500.0])).tolist() == [0x7F, 0xFF]
    assert ostore.f64_to_e4m3fn(np.array([463.99]))[0] == 0x7E
    # an independent implementation: torch's float8_e4m3fn cast of binary32 values
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.uniform(-460, 460, 20000), rng.normal(size=20000) * 1e-2,
                        rng.normal(size=5000) * 2.0 ** -8]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ostore.f64_to_e4m3fn(x.astype(np.float64)), ref)


def test_bf16_encoder_against_torch():
    import torch
    rng = np.random.default_rng(12)
    x = (rng.normal(size=50000) * np.exp2(rng.integers(-30, 30, 50000))).astype(np.float32)
    # exact ties (lower half 0x8000) with both parities of the kept bit
    u = rng.integers(0, 2 ** 31, 4000, dtype=np.uint64).astype(np.uint32)
    ties = ((u & np.uint32(0x7F7F0000)) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, np.array([0.0, -0.0, 3.4e38, -1e-40], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ostore.f32_to_bf16_bits(x), ref)


def test_group_quantizer_properties():
    rng = np.random.default_rng(13)
    rows = (rng.normal(size=(64, 576)) * np.exp2(rng.integers(-6, 6, (64, 1)))).astype(np.float32)
    rows[3, 128:256] = 0.0                     # an all-zero group
    rows[5, 512:] *= 1e-3                      # a small RoPE group
    codes, scales = ostore.quantize_e4m3_groups(rows)
    assert codes.shape == (64, 576) and scales.shape == (64, 5) and scales.dtype == np.float32
    assert scales[3, 1] == 1.0 and np.all(codes[3, 128:256] == 0)
    deq = ostore.dequantize_rows(codes, scales)
    for g in range(5):
        sl = slice(128 * g, min(128 * (g + 1), 576))
        x = rows[:, sl].astype(np.float64)
        # binary32 amax / 448 is the scale, so the largest magnitude maps to 448
        amax = np.abs(x).max(axis=1)
        nz = amax > 0
        assert np.allclose(scales[nz, g], amax[nz] / 448.0, rtol=2 ** -23)
        assert np.all(np.abs(ostore.e4m3fn_to_f64(codes[nz][:, sl.start:sl.stop][np.arange(nz.sum()),
                      np.argmax(np.abs(x[nz]), axis=1)])) == 448.0)
        # error bound: half a quantum of 3 mantissa bits, or half the subnormal
        # quantum 2**-9 for magnitudes below 2**-6 (in units of the scale)
        err = np.abs(deq[:, sl] - x)
        bound = np.maximum(np.abs(x) * 2.0 ** -4, scales[:, g:g + 1].astype(np.float64) * 2.0 ** -10) * (1 + 1e-6)
        assert np.all(err <= bound)


# ---------------------------------------------------------------------------
# YaRN-extended RoPE frequencies ([V2-explainer] §3.1.3: s = 40, alpha = 1,
# beta = 32, original context 4K, target 160K)
# ---------------------------------------------------------------------------

def test_yarn_reduces_to_plain_rope_at_scale_one():
    rng = np.random.default_rng(31)
    x = rng.normal(size=(5, 64))
    pos = rng.integers(0, 200000, size=5)
    theta = oracle.yarn_theta(64, 10000.0, 1.0, 1.0, 32.0, 4096)
    np.testing.assert_array_equal(theta, 10000.0 ** (-2.0 * np.arange(32) / 64))
    np.testing.assert_allclose(oracle.rope_theta(x, pos, theta), oracle.rope(x, pos), rtol=0, atol=0)
    assert oracle.yarn_attention_factor(1.0) == 1.0


def test_yarn_slow_pairs_interpolate_fast_pairs_stay():
    """Pairs turning fewer than alpha times over the original context are
    interpolated by s (rotating position m*s equals the plain rotation at m);
    pairs turning more than beta times keep their frequency; the pages' s = 40
    over a 4K context reaches the stated 160K target."""
    d, base, s, a, b, L = 64, 10000.0, 40.0, 1.0, 32.0, 4096
    plain = base ** (-2.0 * np.arange(d // 2) / d)
    theta = oracle.yarn_theta(d, base, s, a, b, L)
    r = L * plain / (2 * math.pi)
    slow, fast = r <= a, r >= b
    assert slow.any() and fast.any() and (~slow & ~fast).any()
    np.testing.assert_allclose(theta[slow], plain[slow] / s, rtol=1e-15)
    np.testing.assert_array_equal(theta[fast], plain[fast])
    mid = ~slow & ~fast
    assert np.all(theta[mid] < plain[mid]) and np.all(theta[mid] > plain[mid] / s)
    assert np.all(np.diff(theta) < 0)          # still strictly decreasing frequencies
    rng = np.random.default_rng(32)
    x = rng.normal(size=(d,))
    m = 1234
    got = oracle.rope_theta(x, m * s, theta)
    ref = oracle.rope(x, m, base)
    for k in np.nonzero(slow)[0]:
        np.testing.assert_allclose(got[2 * k:2 * k + 2], ref[2 * k:2 * k + 2], rtol=1e-9, atol=1e-12)
    assert s * L >= 160 * 1000


def test_yarn_ramp_midpoint_and_attention_factor():
    """A pair placed exactly half-way up the ramp (r = (alpha + beta) / 2) gets
    the mean of the interpolated and plain frequencies; the attention factor
    grows with s from 1 at s = 1."""
    d, base, s, a, b = 64, 10000.0, 40.0, 1.0, 32.0
    plain = base ** (-2.0 * np.arange(d // 2) / d)
    k = 10
    L = 2 * math.pi * ((a + b) / 2) / plain[k]        # r_k = 16.5 exactly
    theta = oracle.yarn_theta(d, base, s, a, b, L)
    np.testing.assert_allclose(theta[k], plain[k] * (1 + 1 / s) / 2, rtol=1e-13)
    f = [oracle.yarn_attention_factor(v) for v in (1.0, 2.0, 40.0, 100.0)]
    assert f[0] == 1.0 and all(u < w for u, w in zip(f, f[1:]))
