"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Criterion per compared tensor: max|gpu - ref| <= tol * max|ref|, tol = 1e-4
(fp32 cache), 1e-2 (bf16 cache), 3e-2 (fp8 cache).  References are computed
on the stored values the GPU reads (see _cases.py).
"""
import math

import numpy as np
import pytest

import oracle
from _cases import TOL, direct_case, from_h_case, host, rel_err, run_step, to_device

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
    err = rel_err(got, ref)
    print(f"  {name}: rel err {err:.3e} (tol {tol:g})", flush=True)
    assert np.all(np.isfinite(np.asarray(got)[np.isfinite(ref)])), f"{name}: non-finite output"
    assert err <= tol, f"{name}: {err:.3e} > {tol:g}"


def compare_all(case, step, tol, heads=None):
    """Compare q_lat, o_lat, lse and o_heads of every sequence with the oracle."""
    q_lat, o_lat, lse, o_heads = host(step.q_lat), host(step.o_lat), host(step.lse), host(step.o_heads)
    d = case.dims
    refs = {"q_lat": [], "o_lat": [], "lse": [], "o_heads": []}
    gots = {"q_lat": [], "o_lat": [], "lse": [], "o_heads": []}
    for b, T in enumerate(case.lens):
        if T == 0:
            assert np.all(o_lat[b] == 0) and np.all(np.isneginf(lse[b])), "empty sequence must give o=0, lse=-inf"
            continue
        r = case.reference(b, heads=heads)
        hs = list(range(d.n_heads)) if heads is None else list(heads)
        refs["q_lat"].append(r["q_lat"][hs]); gots["q_lat"].append(q_lat[b][hs])
        refs["o_lat"].append(r["o_lat"][hs]); gots["o_lat"].append(o_lat[b][hs])
        refs["lse"].append(r["lse"][hs]); gots["lse"].append(lse[b][hs])
        oh = o_heads[b].reshape(d.n_heads, d.d_head)
        refs["o_heads"].append(r["o_heads"][hs]); gots["o_heads"].append(oh[hs])
    for k in refs:
        if refs[k]:
            check(k, np.stack(gots[k]), np.stack(refs[k]), tol)
    return refs


# ---------------------------------------------------------------------------
# workload 1: tiny fp32 through the pages' chain from h (generic kernels)
# ---------------------------------------------------------------------------

def test_tiny_fp32_from_h():
    print("case: tiny fp32 from h, B=1 T=64", flush=True)
    case = from_h_case(1)
    dev = to_device(case)
    step = run_step(case, dev)
    compare_all(case, step, TOL["f32"])
    # u_t = W^O [o_1; ...; o_nh] applied on the host to the GPU's o_heads
    u_gpu = case.W_O @ host(step.o_heads)[0]
    u_ref = oracle.out_project(case.reference(0)["o_heads"], case.W_O)
    check("u", u_gpu, u_ref, TOL["f32"])


@pytest.mark.parametrize("part", [(0, 0), (64, 0), (128, 0), (0, 3), (0, 7)])
def test_tiny_fp32_ragged_partitions(part):
    import synth
    print(f"case: tiny fp32 ragged, partition {part}", flush=True)
    rng = np.random.default_rng(7)
    lens = [1, 63, 64, 65, 130, 0, 257]
    d = synth.TINY
    rows = [rng.normal(0, 0.3, size=(t, d.row)).astype(np.float32) for t in lens]
    from _cases import case_from_rows
    case = case_from_rows(d, rows, rng.normal(0, 1, (len(lens), d.n_heads, d.d_head)),
                          rng.normal(0, 1, (len(lens), d.n_heads, d.d_rope)),
                          rng.normal(0, 0.2, (d.n_heads * d.d_head, d.d_latent)),
                          rng.normal(0, 0.2, (d.n_heads * d.d_head, d.d_latent)), "f32", "f32",
                          np.random.default_rng(8), max_pages=6)
    dev = to_device(case)
    step = run_step(case, dev, *part)
    compare_all(case, step, TOL["f32"])


# ---------------------------------------------------------------------------
# workload 2: V2 shapes from h, bf16 cache (MFMA kernels)
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def v2_from_h():
    case = from_h_case(2)
    return case, to_device(case)


@pytest.mark.parametrize("part", [(0, 0), (0, 8), (512, 0), (0, 256)])
def test_v2_from_h(v2_from_h, part):
    case, dev = v2_from_h
    print(f"case: V2 bf16 from h, B=1 T=4096, partition {part}", flush=True)
    step = run_step(case, dev, *part)
    compare_all(case, step, TOL["bf16"])
    u_gpu = case.W_O @ host(step.o_heads)[0]
    u_ref = oracle.out_project(case.reference(0)["o_heads"], case.W_O)
    check("u", u_gpu, u_ref, TOL["bf16"])


# ---------------------------------------------------------------------------
# ragged batches, partitions, edge lengths (V2 shapes, bf16)
# ---------------------------------------------------------------------------

RAGGED = [1, 31, 32, 33, 63, 64, 65, 200, 0, 1000, 96, 2]


@pytest.fixture(scope="module")
def v2_ragged():
    case = direct_case(3, RAGGED, max_pages=20)
    return case, to_device(case)


@pytest.mark.parametrize("part", [(0, 0), (0, 5), (0, 16), (0, 64), (128, 0), (64, 0), (0, -1)])
def test_v2_ragged(v2_ragged, part):
    case, dev = v2_ragged
    print(f"case: V2 bf16 ragged lens={RAGGED}, partition {part}", flush=True)
    step = run_step(case, dev, *part)
    compare_all(case, step, TOL["bf16"])


SHORT = [64] * 12 + [1] * 5 + [0, 130]


@pytest.mark.parametrize("part", [(0, 17), (0, 20), (0, 29)])
def test_v2_cost_stream_partition_short_sequences(part):
    """Many one-page sequences, about as many parts as pages: the 2 extra cost
    units between sequences leave some work items without any page (20 pages,
    54 units: 2 of 20 items are empty for 20 or more parts)."""
    case = direct_case(3, SHORT, max_pages=4, seed=91)
    print(f"case: V2 bf16 lens={SHORT}, partition {part}", flush=True)
    step = run_step(case, to_device(case), *part)
    compare_all(case, step, TOL["bf16"])


def test_v2_deterministic(v2_ragged):
    case, dev = v2_ragged
    print("case: V2 bf16 ragged, repeat bitwise", flush=True)
    a = run_step(case, dev, 0, 16)
    b = run_step(case, dev, 0, 16)
    assert np.array_equal(host(a.o_heads), host(b.o_heads))
    assert np.array_equal(host(a.lse), host(b.lse))


# ---------------------------------------------------------------------------
# split-K partials and the sharp-softmax variant (V2 shapes, bf16)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("gain", [1.0, 34.0])
def test_v2_split_partials(gain):
    lens = [1030, 2048, 300]
    print(f"case: V2 bf16 long-context recipe lens={lens} split 256 query gain {gain}", flush=True)
    case = direct_case(4, lens, query_gain=gain, max_pages=32)
    dev = to_device(case)
    step = run_step(case, dev, 256, 0)
    compare_all(case, step, TOL["bf16"])
    o_part, lse_part = step.partials()
    o_part, lse_part = host(o_part), host(lse_part)
    S = step.num_slots // len(lens)
    for b, T in enumerate(lens):
        parts = case.reference(b, chunk=256)
        if len(parts) == 1:
            continue
        got_o = np.stack([o_part[b * S + s] for s in range(len(parts))])
        got_l = np.stack([lse_part[b * S + s] for s in range(len(parts))])
        check(f"o_part[b={b}]", got_o, np.stack([p["o_lat"] for p in parts]), TOL["bf16"])
        check(f"lse_part[b={b}]", got_l, np.stack([p["lse"] for p in parts]), TOL["bf16"])
    if gain > 1:
        spread = max(np.ptp(case.reference(b)["lse"]) for b in range(len(lens)))
        print(f"  lse spread across heads {spread:.2f} (sharp softmax exercised)", flush=True)


# ---------------------------------------------------------------------------
# fp8 E4M3 cache with 1x128 group scales
# ---------------------------------------------------------------------------

def test_v2_fp8_small():
    lens = [1, 65, 300, 0, 777]
    print(f"case: V2 fp8 lens={lens}", flush=True)
    case = direct_case(5, lens, max_pages=16)
    dev = to_device(case)
    for part in [(0, 0), (0, 6), (128, 0)]:
        step = run_step(case, dev, *part)
        compare_all(case, step, TOL["fp8"])


FP8_RAGGED = [31, 32, 33, 64, 95, 129, 200, 700, 1100, 5]


@pytest.fixture(scope="module")
def v2_fp8_ragged():
    case = direct_case(5, FP8_RAGGED, max_pages=20)
    return case, to_device(case)


@pytest.mark.parametrize("part", [(0, 0), (0, 3), (0, 16), (64, 0), (0, -1)])
def test_v2_fp8_ragged(v2_fp8_ragged, part):
    # tile tails around the 32-token tile edge, several tiles per item,
    # segments that start mid-item
    case, dev = v2_fp8_ragged
    print(f"case: V2 fp8 lens={FP8_RAGGED} part={part}", flush=True)
    step = run_step(case, dev, *part)
    compare_all(case, step, TOL["fp8"])


def test_v2_fp8_sharp():
    # queries x34: logits spread wide enough that the running max is raised
    # mid-sequence (the rescale path) on the fp8 tiles too
    lens = [700, 1500]
    print(f"case: V2 fp8 sharp lens={lens}", flush=True)
    case = direct_case(5, lens, query_gain=34.0, max_pages=24)
    step = run_step(case, to_device(case), 0, 8)
    compare_all(case, step, TOL["fp8"])


# ---------------------------------------------------------------------------
# full sizes, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------

SAMPLE_HEADS = [0, 37, 64, 127]


def _sampled(case, step, tol, seqs):
    o_lat, lse, o_heads = host(step.o_lat), host(step.lse), host(step.o_heads)
    d = case.dims
    for b in seqs:
        r = case.reference(b, heads=SAMPLE_HEADS)
        check(f"o_lat[b={b}]", o_lat[b][SAMPLE_HEADS], r["o_lat"][SAMPLE_HEADS], tol)
        check(f"lse[b={b}]", lse[b][SAMPLE_HEADS], r["lse"][SAMPLE_HEADS], tol)
        oh = o_heads[b].reshape(d.n_heads, d.d_head)
        check(f"o_heads[b={b}]", oh[SAMPLE_HEADS], r["o_heads"][SAMPLE_HEADS], tol)
    # properties at every (sequence, head): finite, o_lat a convex combination of cached latents
    assert np.all(np.isfinite(o_lat)) and np.all(np.isfinite(lse))
    for b in range(len(case.lens)):
        rows = case.stored_rows(b)[:, : d.d_latent]
        lo, hi = rows.min(axis=0), rows.max(axis=0)
        slack = 1e-2 * np.abs(rows).max()
        assert np.all(o_lat[b] >= lo - slack) and np.all(o_lat[b] <= hi + slack)


def test_fullsize_ragged_b64():
    import synth
    w = synth.workload(3)
    print(f"case: full-size ragged B=64 sum T={sum(w.lens)} balanced over CUs", flush=True)
    case = direct_case(3, w.lens, max_pages=128)
    dev = to_device(case)
    step = run_step(case, dev, 0, -1)
    _sampled(case, step, TOL["bf16"], seqs=[0, 17, 63])


def test_fullsize_long_b4_split4096():
    print("case: full-size long B=4 T=131072 split 4096", flush=True)
    case = direct_case(4, [131072] * 4, max_pages=2048)
    dev = to_device(case)
    step = run_step(case, dev, 4096, 0)
    _sampled(case, step, TOL["bf16"], seqs=[0, 3])


def test_fullsize_fp8_b32():
    print("case: full-size fp8 B=32 T=16384 balanced over CUs", flush=True)
    case = direct_case(5, [16384] * 32, max_pages=256)
    dev = to_device(case)
    step = run_step(case, dev, 0, -1)
    _sampled(case, step, TOL["fp8"], seqs=[0, 31])
