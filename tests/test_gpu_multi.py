"""GPU parity of multi-token decode (q_len new tokens per sequence, causal within
them) against the oracle's attend_new_tokens.

The cache holds T_b tokens, the q_len new ones last; new token t attends to
tokens [0, T_b - q_len + t + 1).  The device path is mla_absorb_q over the
B * q_len queries, mla_decode_multi (merge included) and mla_out_proj; the
references are the oracle's non-absorbed attention on the stored cache values,
with the same tolerance rule as single-token decode.  V2-sized cases compare a
sample of heads (the oracle's up-projections cost 2.6e5 flop per head per token).
"""
import numpy as np
import pytest

import oracle
from _cases import TOL, Worst, compare_seq, direct_case, from_h_case, host, rel_err, to_device

pytestmark = pytest.mark.gpu

SAMPLE_HEADS = [0, 1, 31, 32, 63, 64, 100, 127]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_37_amd as mk
    mk._lib.load()
    print("libmla:", mk.build_info(), flush=True)


def _queries(case, q_len, seed, gain):
    """q_len queries per sequence, stored values (bf16 or f32 rounding of the case)."""
    import synth
    from _cases import _round
    rng = np.random.default_rng(seed)
    d = case.dims
    B = len(case.lens)
    sd = np.abs(case.q_nope).std() if case.q_nope.size else synth.V2_SD_QUERY
    q_c = rng.normal(0.0, sd * gain, size=(B, q_len, d.n_heads, d.d_head))
    q_r = rng.normal(0.0, sd * gain, size=(B, q_len, d.n_heads, d.d_rope))
    return _round(q_c, case.act), _round(q_r, case.act)


def _run_multi(case, dev, q_c, q_r, part, fused=False):
    import torch
    import mla_latent_kv_37_amd as mk
    d = case.dims
    B, q_len = q_c.shape[:2]
    tdt = dev["dtype"]
    dd = mk.dims(d.n_heads, d.d_head, d.d_rope, d.d_latent)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(tdt).contiguous()  # noqa: E731
    q_nope = t(q_c.reshape(B * q_len, d.n_heads, d.d_head))
    q_pe = t(q_r)
    q_lat = torch.empty((B * q_len, d.n_heads, d.d_latent), dtype=tdt, device="cuda")
    mk.absorb_q(dd, q_nope, dev["W_UK"], q_lat)
    cache = dev["cache"]
    p = mk.partition(*part)
    nbytes, _ = mk.multi_workspace_size(dd, B, q_len, cache.max_pages, cache.page_size, p)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    o_lat = torch.full((B, q_len, d.n_heads, d.d_latent), float("nan"), dtype=tdt, device="cuda")
    lse = torch.full((B, q_len, d.n_heads), float("nan"), dtype=torch.float32, device="cuda")
    o_heads = torch.full((B * q_len, d.n_heads * d.d_head), float("nan"), dtype=tdt, device="cuda")
    if fused:
        mk.decode_multi_out_proj(dd, q_lat.view(B, q_len, d.n_heads, d.d_latent), q_pe, cache.desc, case.scale, p, ws,
                                 o_lat, dev["W_UV"], o_heads, lse)
    else:
        mk.decode_multi(dd, q_lat.view(B, q_len, d.n_heads, d.d_latent), q_pe, cache.desc, case.scale, p, ws, o_lat,
                        lse)
        mk.out_proj(dd, o_lat.view(B * q_len, d.n_heads, d.d_latent), dev["W_UV"], o_heads)
    torch.cuda.synchronize()
    return host(o_lat), host(lse), host(o_heads).reshape(B, q_len, d.n_heads, d.d_head)


def _compare(case, q_c, q_r, got, tol, heads=None):
    """Each (sequence, new token) against the oracle: vectors per token, lse against
    its derived bound over the rows that token sees."""
    o_lat, lse, o_heads = got
    d = case.dims
    q_len = q_c.shape[1]
    worst = Worst()
    for b, T in enumerate(case.lens):
        rows = case.stored_rows(b)
        res = oracle.attend_new_tokens(q_c[b], q_r[b], rows[:, :d.d_latent], rows[:, d.d_latent:], case.W_UK,
                                       case.W_UV, case.scale, heads)
        for t, r in enumerate(res):
            if np.all(np.isneginf(r["lse"])):
                # no visible token: zero output, lse = -inf
                assert np.all(o_lat[b, t] == 0) and np.all(np.isneginf(lse[b, t])), (b, t)
                continue
            compare_seq(case, b, r, {"o_lat": o_lat[b, t], "lse": lse[b, t], "o_heads": o_heads[b, t]}, tol, heads,
                        worst, tag=f"b={b},t={t}", rows=rows[:T - q_len + t + 1], q_pe=q_r[b, t])
    worst.report(tol)


@pytest.fixture(scope="module")
def v2_ragged():
    lens = [1, 2, 3, 64, 65, 700, 2100]
    case = direct_case(3, lens, max_pages=34, seed=71)
    return case, to_device(case)


@pytest.mark.parametrize("part", [(0, 0), (128, 0), (0, 5), (0, 300)])
def test_multi_v2_bf16_ragged(v2_ragged, part):
    case, dev = v2_ragged
    print(f"case: multi-token V2 bf16, lens {case.lens}, q_len 3, partition {part}", flush=True)
    q_c, q_r = _queries(case, 3, seed=5, gain=1.0)
    _compare(case, q_c, q_r, _run_multi(case, dev, q_c, q_r, part), TOL["bf16"], SAMPLE_HEADS)


def test_multi_v2_bf16_sharp_q4():
    lens = [130, 1000, 4]
    case = direct_case(3, lens, max_pages=16, seed=72)
    dev = to_device(case)
    print(f"case: multi-token V2 bf16 sharp (gain 150), lens {lens}, q_len 4", flush=True)
    q_c, q_r = _queries(case, 4, seed=6, gain=150.0)
    _compare(case, q_c, q_r, _run_multi(case, dev, q_c, q_r, (0, 3)), TOL["bf16"], SAMPLE_HEADS)


def test_multi_v2_fp8():
    lens = [300, 1500, 2]
    case = direct_case(3, lens, cache_dtype="fp8", max_pages=24, seed=73)
    dev = to_device(case)
    print(f"case: multi-token V2 fp8, lens {lens}, q_len 2", flush=True)
    q_c, q_r = _queries(case, 2, seed=7, gain=1.0)
    _compare(case, q_c, q_r, _run_multi(case, dev, q_c, q_r, (0, 8)), TOL["fp8"], SAMPLE_HEADS)


@pytest.mark.parametrize("part", [(0, 0), (64, 0), (0, 3)])
def test_multi_tiny_f32(part):
    """Tiny fp32 shapes through the generic decode kernel, all heads."""
    case = from_h_case(1)
    dev = to_device(case)
    print(f"case: multi-token tiny f32, T {case.lens}, q_len 5, partition {part}", flush=True)
    q_c, q_r = _queries(case, 5, seed=8, gain=3.0)
    _compare(case, q_c, q_r, _run_multi(case, dev, q_c, q_r, part), TOL["f32"])


def test_multi_q1_equals_single_token_decode(v2_ragged):
    """q_len = 1 is ordinary decode: same kernels, bit-identical outputs."""
    import torch
    import mla_latent_kv_37_amd as mk
    case, dev = v2_ragged
    d = case.dims
    B = len(case.lens)
    q_c, q_r = _queries(case, 1, seed=9, gain=1.0)
    o_lat_m, lse_m, _ = _run_multi(case, dev, q_c, q_r, (0, 5))
    dd = mk.dims(d.n_heads, d.d_head, d.d_rope, d.d_latent)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(dev["dtype"]).contiguous()  # noqa: E731
    q_lat = torch.empty((B, d.n_heads, d.d_latent), dtype=dev["dtype"], device="cuda")
    mk.absorb_q(dd, t(q_c[:, 0]), dev["W_UK"], q_lat)
    cache = dev["cache"]
    p = mk.partition(0, 5)
    nbytes, _ = mk.workspace_size(dd, B, cache.max_pages, cache.page_size, p)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    o_lat = torch.empty((B, d.n_heads, d.d_latent), dtype=dev["dtype"], device="cuda")
    lse = torch.empty((B, d.n_heads), dtype=torch.float32, device="cuda")
    mk.decode(dd, q_lat, t(q_r[:, 0]), cache.desc, case.scale, p, ws, o_lat, lse)
    mk.merge_splits(dd, cache.seq_lens, cache.page_size, cache.max_pages, p, ws, o_lat, lse)
    torch.cuda.synchronize()
    assert np.array_equal(host(o_lat), o_lat_m[:, 0])
    assert np.array_equal(host(lse), lse_m[:, 0])


@pytest.mark.parametrize("part", [(0, 0), (0, 6), (128, 0)])
def test_multi_v2lite_bf16(part):
    """Two new tokens per sequence at V2-Lite's 16 heads (the 16-head decode
    kernel under the virtual batch), all heads."""
    lens = [2, 70, 900, 129]
    case = direct_case(6, lens, max_pages=16, seed=74)
    dev = to_device(case)
    print(f"case: multi-token V2-Lite bf16, lens {lens}, q_len 2, partition {part}", flush=True)
    q_c, q_r = _queries(case, 2, seed=10, gain=20.0)
    _compare(case, q_c, q_r, _run_multi(case, dev, q_c, q_r, part), TOL["bf16"])


@pytest.mark.parametrize("part", [(0, -1), (128, 0), (0, 0)])
def test_multi_fused_out_proj(v2_ragged, part):
    """mla_decode_multi_out_proj: o_lat / lse the same bits as mla_decode_multi,
    o_heads within one bf16 step of mla_out_proj's, and against the oracle."""
    case, dev = v2_ragged
    print(f"case: multi-token V2 bf16 fused, lens {case.lens}, q_len 3, partition {part}", flush=True)
    q_c, q_r = _queries(case, 3, seed=11, gain=1.0)
    f = _run_multi(case, dev, q_c, q_r, part, fused=True)
    u = _run_multi(case, dev, q_c, q_r, part, fused=False)
    assert np.array_equal(f[0], u[0]), "o_lat differs"
    assert np.array_equal(f[1], u[1]), "lse differs"
    assert np.all(np.isfinite(f[2]))
    err = np.abs(f[2] - u[2]).max() / np.abs(u[2]).max()
    print(f"  o_heads fused vs unfused: {err:.3e} of max", flush=True)
    assert err <= 2.0 ** -7
    _compare(case, q_c, q_r, f, TOL["bf16"], SAMPLE_HEADS)
