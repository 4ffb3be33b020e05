"""mla_merge_out_proj (split merge + W^UV projection in one launch) against the
two calls it replaces, mla_merge_splits then mla_out_proj, on the same decode
output; and, through DecodeStep (which uses it), against the oracle in the
other GPU parity tests.

o_lat and lse must be the same bits (the fused kernel merges with the merge
kernel's operations in the same order).  o_heads differs from mla_out_proj only
in the order of the fp32 additions (four contraction quarters summed at the
end instead of one chain), so after rounding to bf16 the two agree to within
one bf16 step of the largest output: max |fused - unfused| <= 2^-7 max |unfused|.
The fp32 cases take the fallback (the two calls in sequence): bit-identical.
"""
import numpy as np
import pytest

from _cases import TOL, Worst, compare_seq, direct_case, from_h_case, host, rel_err, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_37_amd as mk
    mk._lib.load()
    print("libmla:", mk.build_info(), flush=True)


def _both(case, dev, part):
    """(fused o_lat, lse, o_heads), (unfused o_lat, lse, o_heads) from one decode."""
    import torch
    import mla_latent_kv_37_amd as mk
    d = case.dims
    B = len(case.lens)
    cache = dev["cache"]
    step = mk.DecodeStep(d.n_heads, d.d_head, d.d_rope, d.d_latent, B, cache.max_pages, cache.page_size, *part,
                         act_dtype=dev["dtype"])
    step.absorb(dev["q_nope"], dev["W_UK"])
    mk.decode(step.d, step.q_lat, dev["q_pe"], cache.desc, case.scale, step.part, step.workspace, step.o_lat,
              step.lse)
    # copies of the decode outputs for the unfused calls
    o_lat_u, lse_u = step.o_lat.clone(), step.lse.clone()
    o_heads_u = torch.full_like(step.o_heads, float("nan"))
    step.o_heads.fill_(float("nan"))
    mk.merge_out_proj(step.d, cache.seq_lens, cache.page_size, cache.max_pages, step.part, step.workspace,
                      step.o_lat, dev["W_UV"], step.o_heads, step.lse)
    mk.merge_splits(step.d, cache.seq_lens, cache.page_size, cache.max_pages, step.part, step.workspace, o_lat_u,
                    lse_u)
    mk.out_proj(step.d, o_lat_u, dev["W_UV"], o_heads_u)
    torch.cuda.synchronize()
    return (step.o_lat, step.lse, step.o_heads), (o_lat_u, lse_u, o_heads_u)


def _check(fused, unfused, exact_heads):
    import torch
    (o_f, l_f, h_f), (o_u, l_u, h_u) = fused, unfused
    assert torch.equal(o_f.view(torch.int16) if o_f.dtype == torch.bfloat16 else o_f,
                       o_u.view(torch.int16) if o_u.dtype == torch.bfloat16 else o_u), "o_lat differs"
    lf, lu = l_f.cpu().numpy(), l_u.cpu().numpy()
    assert np.array_equal(lf.view(np.uint32), lu.view(np.uint32)), "lse differs"
    hf, hu = host(h_f), host(h_u)
    assert np.all(np.isfinite(hf)), "o_heads not fully written"
    if exact_heads:
        assert np.array_equal(hf, hu)
    else:
        err = np.abs(hf - hu).max() / np.abs(hu).max()
        print(f"  o_heads fused vs unfused: {err:.3e} of max", flush=True)
        assert err <= 2.0 ** -7


RAGGED = [1, 64, 65, 0, 700, 2100, 3, 129, 0, 1000, 64]


@pytest.fixture(scope="module")
def v2_ragged():
    case = direct_case(3, RAGGED, max_pages=34, seed=81)
    return case, to_device(case)


@pytest.mark.parametrize("part", [(0, -1), (0, 5), (0, 64), (128, 0), (0, 0)])
def test_fused_equals_merge_then_out_proj_v2(v2_ragged, part):
    case, dev = v2_ragged
    print(f"case: V2 bf16 lens {case.lens}, partition {part}", flush=True)
    _check(*_both(case, dev, part), exact_heads=False)


def test_fused_batch_37_with_empty_sequences():
    """two 32-sequence tiles, the second ragged; empty sequences in both"""
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(0, 900, size=37)]
    lens[3] = lens[33] = 0
    case = direct_case(3, lens, max_pages=16, seed=82)
    dev = to_device(case)
    print(f"case: V2 bf16 B=37 lens {lens}", flush=True)
    _check(*_both(case, dev, (0, 9)), exact_heads=False)


def test_fused_more_than_64_splits():
    """79 splits of one sequence (64-token splits of 5000 tokens): the lse values
    beyond the 64 lanes are read per split."""
    lens = [5000, 70, 0, 640]
    case = direct_case(3, lens, max_pages=80, seed=85)
    dev = to_device(case)
    print(f"case: V2 bf16 lens {lens}, split 64", flush=True)
    _check(*_both(case, dev, (64, 0)), exact_heads=False)


def test_fused_one_sequence_64_splits_against_oracle():
    """One sequence in 64 splits (the B = 1 decode): its row is added in four
    parts by four wavefronts; fused against unfused, and against the oracle."""
    lens = [4096]
    case = direct_case(3, lens, max_pages=64, seed=88)
    dev = to_device(case)
    print(f"case: V2 bf16 lens {lens}, split 64", flush=True)
    fused, unfused = _both(case, dev, (64, 0))
    _check(fused, unfused, exact_heads=False)
    o_lat, lse, o_heads = (host(t) for t in fused)
    d = case.dims
    heads = [0, 5, 64, 127]
    worst = Worst()
    compare_seq(case, 0, case.reference(0, heads=heads),
                {"o_lat": o_lat[0], "lse": lse[0], "o_heads": o_heads[0].reshape(d.n_heads, d.d_head)},
                TOL["bf16"], heads, worst)
    worst.report(TOL["bf16"])


def test_fused_v2lite_16_heads():
    lens = [2, 70, 900, 129, 0, 4000]
    case = direct_case(6, lens, max_pages=64, seed=83)
    dev = to_device(case)
    print(f"case: V2-Lite bf16 lens {lens}", flush=True)
    _check(*_both(case, dev, (0, 7)), exact_heads=False)


@pytest.mark.parametrize("part", [(0, 3), (64, 0)])
def test_fallback_f32_equals_two_calls(part):
    case = from_h_case(1)
    dev = to_device(case)
    print(f"case: tiny f32 T {case.lens}, partition {part}", flush=True)
    _check(*_both(case, dev, part), exact_heads=True)


def test_fused_against_oracle_sharp():
    """Sharp softmax (queries x60) split 6 ways: the merged outputs and the
    projection against the oracle."""
    lens = [1500, 260, 3000]
    case = direct_case(3, lens, query_gain=60.0, max_pages=48, seed=84)
    dev = to_device(case)
    fused, _ = _both(case, dev, (0, 6))
    o_lat, lse, o_heads = (host(t) for t in fused)
    d = case.dims
    heads = [0, 1, 63, 64, 127]
    for b in range(len(lens)):
        r = case.reference(b, heads=heads)
        for name, got, ref in (("o_lat", o_lat[b][heads], r["o_lat"][heads]), ("lse", lse[b][heads], r["lse"][heads]),
                               ("o_heads", o_heads[b].reshape(d.n_heads, d.d_head)[heads], r["o_heads"][heads])):
            err = rel_err(got, ref)
            print(f"  b={b} {name}: rel err {err:.3e}", flush=True)
            assert err <= TOL["bf16"], (b, name)


def test_fused_batch_100_and_absorb_second_tile():
    """100 sequences: four 32-row merge tiles (the last ragged) and two 64-row
    absorb tiles (the second ragged); fused against unfused, and the absorbed
    queries and outputs of rows in every tile against the oracle."""
    import torch
    rng = np.random.default_rng(9)
    lens = [int(x) for x in rng.integers(0, 300, size=100)]
    lens[0] = lens[64] = lens[99] = 0
    lens[63], lens[65], lens[98] = 290, 1, 257
    case = direct_case(3, lens, max_pages=5, seed=87)
    dev = to_device(case)
    print(f"case: V2 bf16 B=100 lens {lens}", flush=True)
    fused, unfused = _both(case, dev, (0, -1))
    _check(fused, unfused, exact_heads=False)
    import mla_latent_kv_37_amd as mk
    d = case.dims
    step = mk.DecodeStep(d.n_heads, d.d_head, d.d_rope, d.d_latent, len(lens), dev["cache"].max_pages,
                         dev["cache"].page_size, 0, -1, act_dtype=dev["dtype"])
    step.absorb(dev["q_nope"], dev["W_UK"])
    torch.cuda.synchronize()
    q_lat = host(step.q_lat)
    o_lat, lse, o_heads = (host(t) for t in fused)
    heads = [0, 31, 64, 127]
    for b in (64, 99):   # empty sequences: zero output, lse = -inf
        assert np.all(o_lat[b] == 0) and np.all(np.isneginf(lse[b])), b
    for b in (1, 63, 65, 98):
        r = case.reference(b, heads=heads)
        err = rel_err(q_lat[b][heads], r["q_lat"][heads])
        print(f"  b={b} q_lat: rel err {err:.3e}", flush=True)
        assert err <= TOL["bf16"], b
        for name, got, ref in (("o_lat", o_lat[b][heads], r["o_lat"][heads]),
                               ("o_heads", o_heads[b].reshape(d.n_heads, d.d_head)[heads], r["o_heads"][heads])):
            err = rel_err(got, ref)
            print(f"  b={b} {name}: rel err {err:.3e}", flush=True)
            assert err <= TOL["bf16"], (b, name)
