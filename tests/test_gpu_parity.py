"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Criterion per compared tensor: max|gpu - ref| <= tol * max|ref|, tol = 1e-4
(fp32 cache), 1e-2 (bf16 cache), 3e-2 (fp8 cache).  References are computed
on the stored values the GPU reads (see _cases.py).
"""
import math

import numpy as np
import pytest

import oracle
import synth
from _cases import (TOL, Worst, check_lse, check_vec, compare_seq, direct_case, from_h_case, host, lse_tolerance,
                    run_step, to_device)

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


def compare_all(case, step, tol, heads=None, seqs=None):
    """Compare q_lat, o_lat, lse and o_heads of every sequence (or of `seqs`) with
    the oracle: vectors per sequence against tol * max|ref| of that sequence,
    lse against its derived absolute bound (_cases.lse_tolerance)."""
    q_lat, o_lat, lse, o_heads = host(step.q_lat), host(step.o_lat), host(step.lse), host(step.o_heads)
    d = case.dims
    worst = Worst()
    for b in (range(len(case.lens)) if seqs is None else seqs):
        if case.lens[b] == 0:
            assert np.all(o_lat[b] == 0) and np.all(np.isneginf(lse[b])), "empty sequence must give o=0, lse=-inf"
            continue
        r = case.reference(b, heads=heads)
        got = {"q_lat": q_lat[b], "o_lat": o_lat[b], "lse": lse[b],
               "o_heads": o_heads[b].reshape(d.n_heads, d.d_head)}
        compare_seq(case, b, r, got, tol, heads, worst)
    worst.report(tol)


def check_partials(case, step, tol, chunk, lens):
    """Per-split partials (o_s, lse_s) of fixed splits against the oracle's chunks."""
    o_part, lse_part = step.partials()
    o_part, lse_part = host(o_part), host(lse_part)
    S = step.num_slots // len(lens)
    dc = case.dims.d_latent
    worst = Worst()
    for b, T in enumerate(lens):
        parts = case.reference(b, chunk=chunk)
        if len(parts) == 1:
            continue
        rows = case.stored_rows(b)
        for s, p in enumerate(parts):
            worst.add("o_part", check_vec(f"o_part[b={b},s={s}]", o_part[b * S + s], p["o_lat"], tol))
            bound = lse_tolerance(case, p["q_lat"], case.q_pe[b], rows[s * chunk:(s + 1) * chunk], p["lse"])
            worst.add("lse_part", check_lse(f"lse_part[b={b},s={s}]", lse_part[b * S + s], p["lse"], bound))
    worst.report(tol)


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
    check_partials(case, step, TOL["bf16"], 256, lens)
    if gain > 1:
        spread = max(np.ptp(case.reference(b)["lse"]) for b in range(len(lens)))
        print(f"  lse spread across heads {spread:.2f} (sharp softmax exercised)", flush=True)


def test_v2_max_jump_past_reference():
    """A token whose score exceeds every score of its segment's first tile by far
    more than 64 log2 units.  The bf16 kernel fixes each head's reference max at
    a segment's first tile and lets later probabilities exceed 1; past that
    bound it recomputes the segment with the exact maximum.  Row 300 of sequence
    0 and row 40 of sequence 1 are c * sign pattern of head 0's absorbed query
    (latent and RoPE parts), so head 0's softmax is nearly one-hot there; the
    rows sit in the first tile's segment under every partition below."""
    from oracle.mla import head_rows
    from _cases import case_from_rows
    lens = [700, 1500]
    cid = 3
    inp = synth.direct_inputs_for(cid, seed=21, lens=lens)
    w = inp["workload"]
    rows = [r.copy() for r in inp["rows"]]
    base = case_from_rows(w.dims, rows, inp["q_nope"], inp["q_pe"], inp["W_UK"], inp["W_UV"], "bf16", "bf16",
                          synth.rng_for(cid, synth.S_PERM, 21), max_pages=32)
    d = w.dims
    log2e = 1.0 / math.log(2.0)
    for b, t_star in ((0, 300), (1, 40)):
        q_lat0 = head_rows(base.W_UK, 0, d.d_head).T @ base.q_nope[b, 0]
        pattern = np.concatenate([np.sign(q_lat0), np.sign(base.q_pe[b, 0])])
        r0 = oracle.attend_head(base.q_nope[b, 0], base.q_pe[b, 0], base.stored_rows(b)[:32, :d.d_latent],
                                base.stored_rows(b)[:32, d.d_latent:], base.W_UK, base.W_UV, 0, base.scale)
        l1 = np.abs(q_lat0).sum() + np.abs(base.q_pe[b, 0]).sum()
        # smallest power of two that puts the jump past 96 log2 units (exact in bf16)
        need = (96.0 / log2e + r0["s"].max()) / (base.scale * l1)
        c = 2.0 ** math.ceil(math.log2(max(need, 1.0)))
        rows[b][t_star] = (c * pattern).astype(np.float32)
    case = case_from_rows(w.dims, rows, inp["q_nope"], inp["q_pe"], inp["W_UK"], inp["W_UV"], "bf16", "bf16",
                          synth.rng_for(cid, synth.S_PERM, 21), max_pages=32)
    for b, t_star in ((0, 300), (1, 40)):
        r = oracle.attend_head(case.q_nope[b, 0], case.q_pe[b, 0], case.stored_rows(b)[:, :d.d_latent],
                               case.stored_rows(b)[:, d.d_latent:], case.W_UK, case.W_UV, 0, case.scale)
        jump = (r["s"][t_star] - r["s"][:32].max()) * log2e
        print(f"  seq {b}: token {t_star} score jump over the first tile {jump:.1f} log2 units", flush=True)
        assert jump > 64.0 and r["p"][t_star] > 0.99
    dev = to_device(case)
    for part in [(0, 0), (256, 0), (0, -1)]:
        print(f"case: V2 bf16 max jump lens={lens} part={part}", flush=True)
        compare_all(case, run_step(case, dev, *part), TOL["bf16"])


@pytest.mark.parametrize("cfg", [3, 5], ids=["bf16", "fp8"])
def test_v2_bad_page_ids_and_overlong_lengths(cfg):
    """A block-table entry outside [0, num_pages) reads as a page of zero rows
    (score 0 and value 0: those tokens are still attended), and a length above
    max_pages_per_seq * page_size is clamped to it.  Sequence 1's third page id
    is set past the cache; sequence 2 fills its block-table row (11 pages) and its
    length is raised by 100.  References: the oracle on the rows the kernel
    reads (sequence 1 with tokens 128-191 zero; sequence 2 at its true length)."""
    import torch
    lens = [300, 700, 704]
    case = direct_case(cfg, lens, max_pages=11, seed=33)
    dev = to_device(case)
    num_pages = case.cache.kv.shape[0]
    bt = case.cache.block_table.copy()
    bt[1, 2] = num_pages + 5
    sl = case.cache.seq_lens.copy()
    sl[2] += 100
    dev["cache"].block_table.copy_(torch.from_numpy(bt))
    dev["cache"].seq_lens.copy_(torch.from_numpy(sl))
    d = case.dims
    rows1 = case.stored_rows(1).copy()
    rows1[128:192] = 0.0
    ref1 = oracle.attend(case.q_nope[1], case.q_pe[1], rows1[:, :d.d_latent], rows1[:, d.d_latent:], case.W_UK,
                         case.W_UV, case.scale)
    tol = TOL["fp8" if cfg == 5 else "bf16"]
    for part in [(0, 0), (128, 0), (0, -1)]:
        print(f"case: V2 {'fp8' if cfg == 5 else 'bf16'} bad page id / long length lens={lens} part={part}",
              flush=True)
        step = run_step(case, dev, *part)
        q_lat, o_lat, lse, o_heads = host(step.q_lat), host(step.o_lat), host(step.lse), host(step.o_heads)
        worst = Worst()
        for b, ref, rows in ((0, case.reference(0), None), (1, ref1, rows1), (2, case.reference(2), None)):
            got = {"q_lat": q_lat[b], "o_lat": o_lat[b], "lse": lse[b],
                   "o_heads": o_heads[b].reshape(d.n_heads, d.d_head)}
            compare_seq(case, b, ref, got, tol, None, worst, rows=rows)
        worst.report(tol)


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


def test_v2_fp8_short_tails():
    """Sequences of 1-5 and 33-36 tokens: the last row's scales end inside a 16-byte
    load whenever T % 4 != 0; each sequence is checked against its own values."""
    lens = [1, 2, 3, 4, 5, 33, 34, 35, 36]
    print(f"case: V2 fp8 short tails lens={lens}", flush=True)
    case = direct_case(5, lens, max_pages=2, seed=77)
    dev = to_device(case)
    for part in [(0, 0), (0, 3)]:
        compare_all(case, run_step(case, dev, *part), TOL["fp8"])


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

def _sampled(case, step, tol, seqs):
    """All 128 heads of the sampled sequences against the oracle; finite values and
    o_lat inside the convex hull of the cached latents at every (sequence, head)."""
    o_lat, lse = host(step.o_lat), host(step.lse)
    d = case.dims
    compare_all(case, step, tol, seqs=seqs)
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


@pytest.fixture(scope="module")
def long_b4():
    case = direct_case(4, [131072] * 4, max_pages=2048)
    return case, to_device(case)


def test_fullsize_long_b4_split4096(long_b4):
    print("case: full-size long B=4 T=131072 split 4096", flush=True)
    case, dev = long_b4
    _sampled(case, run_step(case, dev, 4096, 0), TOL["bf16"], seqs=[0, 3])


def test_fullsize_long_b4_bench_partition(long_b4):
    """The benchmark's launch configuration for the long workload: one work item
    per compute unit (64 splits of each 131,072-token sequence)."""
    print("case: full-size long B=4 T=131072, one work item per compute unit", flush=True)
    case, dev = long_b4
    _sampled(case, run_step(case, dev, 0, -1), TOL["bf16"], seqs=[0, 3])


def test_fullsize_fp8_b32():
    print("case: full-size fp8 B=32 T=16384 balanced over CUs", flush=True)
    case = direct_case(5, [16384] * 32, max_pages=256)
    dev = to_device(case)
    step = run_step(case, dev, 0, -1)
    _sampled(case, step, TOL["fp8"], seqs=[0, 31])
