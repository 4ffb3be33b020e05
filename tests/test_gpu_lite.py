"""GPU parity at DeepSeek-V2-Lite shapes (16 heads, same 576-wide cache row)
against the float64 oracle, through the C ABI (absorb -> decode -> merge ->
out-projection).  Same criterion as the V2 tests: max|gpu - ref| <= 1e-2 *
max|ref| per compared tensor for the bf16 cache.
"""
import numpy as np
import pytest

from _cases import TOL, Worst, check_lse, check_vec, compare_seq, direct_case, host, lse_tolerance, run_step, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_37_amd as mk
    mk._lib.load()
    print("libmla:", mk.build_info(), flush=True)


def check(name, got, ref, tol):
    err = check_vec(name, got, ref, tol)
    print(f"  {name}: rel err {err:.3e} (tol {tol:g})", flush=True)


def compare(case, step, tol, seqs=None, heads=None):
    """Per-sequence vector checks and the derived lse bound (_cases.compare_seq)."""
    q_lat, o_lat, lse, o_heads = host(step.q_lat), host(step.o_lat), host(step.lse), host(step.o_heads)
    d = case.dims
    worst = Worst()
    for b in (range(len(case.lens)) if seqs is None else seqs):
        if case.lens[b] == 0:
            assert np.all(o_lat[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        r = case.reference(b, heads=heads)
        got = {"q_lat": q_lat[b], "o_lat": o_lat[b], "lse": lse[b],
               "o_heads": o_heads[b].reshape(d.n_heads, d.d_head)}
        compare_seq(case, b, r, got, tol, heads, worst)
    worst.report(tol)


RAGGED = [1, 15, 16, 17, 31, 33, 63, 64, 65, 200, 0, 1000, 96, 2, 130]


@pytest.fixture(scope="module")
def lite_ragged():
    case = direct_case(6, RAGGED, max_pages=20)
    assert case.dims.n_heads == 16
    return case, to_device(case)


@pytest.mark.parametrize("part", [(0, 0), (0, 5), (0, 16), (0, 64), (128, 0), (64, 0), (0, -1)])
def test_lite_ragged(lite_ragged, part):
    # tile tails around the 16-token quarter edges, empty quarters of a last page,
    # segments that start mid-item and items that span sequences
    case, dev = lite_ragged
    print(f"case: V2-Lite bf16 ragged lens={RAGGED}, partition {part}", flush=True)
    compare(case, run_step(case, dev, *part), TOL["bf16"])


def test_lite_deterministic(lite_ragged):
    case, dev = lite_ragged
    a = run_step(case, dev, 0, 16)
    b = run_step(case, dev, 0, 16)
    assert np.array_equal(host(a.o_heads), host(b.o_heads))
    assert np.array_equal(host(a.lse), host(b.lse))


def test_lite_sharp_split_partials():
    """Queries x80 (logits spread over several units): the running max is raised inside the
    sequences; fixed 256-token splits also check every partial."""
    lens = [1030, 2048, 300]
    case = direct_case(6, lens, query_gain=80.0, max_pages=32)
    dev = to_device(case)
    print(f"case: V2-Lite sharp lens={lens} split 256", flush=True)
    step = run_step(case, dev, 256, 0)
    compare(case, step, TOL["bf16"])
    spread = max(np.ptp(case.reference(b)["lse"]) for b in range(len(lens)))
    print(f"  lse spread across heads {spread:.2f}", flush=True)
    assert spread > 1.0
    o_part, lse_part = step.partials()
    o_part, lse_part = host(o_part), host(lse_part)
    S = step.num_slots // len(lens)
    worst = Worst()
    for b in range(len(lens)):
        parts = case.reference(b, chunk=256)
        rows = case.stored_rows(b)
        for s, p in enumerate(parts):
            worst.add("o_part", check_vec(f"o_part[b={b},s={s}]", o_part[b * S + s], p["o_lat"], TOL["bf16"]))
            bound = lse_tolerance(case, p["q_lat"], case.q_pe[b], rows[256 * s:256 * (s + 1)], p["lse"])
            worst.add("lse_part", check_lse(f"lse_part[b={b},s={s}]", lse_part[b * S + s], p["lse"], bound))
    worst.report(TOL["bf16"])


def test_lite_fullsize_ragged_b64():
    """The benchmark's V2-Lite workload in its launch configuration (balanced over
    the compute units); sampled sequences against the oracle, properties everywhere."""
    import synth
    w = synth.workload(6)
    print(f"case: V2-Lite full-size ragged B=64 sum T={sum(w.lens)}", flush=True)
    case = direct_case(6, w.lens, max_pages=128)
    step = run_step(case, to_device(case), 0, -1)
    compare(case, step, TOL["bf16"], seqs=[0, 17, 63])
    o_lat, lse = host(step.o_lat), host(step.lse)
    assert np.all(np.isfinite(o_lat)) and np.all(np.isfinite(lse))
    for b in range(len(case.lens)):
        rows = case.stored_rows(b)[:, :case.dims.d_latent]
        slack = 1e-2 * np.abs(rows).max()
        assert np.all(o_lat[b] >= rows.min(axis=0) - slack) and np.all(o_lat[b] <= rows.max(axis=0) + slack)
