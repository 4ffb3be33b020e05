"""GPU tests of the query-side projection entry point against the oracle.

mla_query_prep computes c^Q = W^DQ h, q^C = W^UQ c^Q and q^R = RoPE(W^QR c^Q)
per head; the oracle's project_query is the float64 reference, on the same
inputs (bf16 inputs are rounded to bf16 values before the oracle sees them).
Between the two products the device rounds c^Q to the weights' dtype, so the
bf16 cases are held to the bf16 tolerance of the decode path (1e-2 of the
largest reference magnitude), the fp32 ones to 1e-4.
"""
import numpy as np
import pytest

import oracle
from oracle import storage as ostore
from oracle.mla import ROPE_BASE

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_37_amd as mk
    print(mk.build_info(), flush=True)


def _round(x, kind):
    x = np.asarray(x, dtype=np.float64)
    if kind == "f32":
        return x.astype(np.float32).astype(np.float64)
    return ostore.bf16_bits_to_f64(ostore.f32_to_bf16_bits(x.astype(np.float32)))


def _run(dims, batch, h_kind, w_kind, out_kind, seed, rope_base=10000.0, max_pos=None, sigma=None, yarn=None):
    import torch
    import synth
    import mla_latent_kv_37_amd as mk
    assert rope_base in (0.0, ROPE_BASE), "the oracle's RoPE base is fixed"
    rng = np.random.default_rng(seed)
    sigma = synth.V2_SIGMA_W if sigma is None else sigma
    W = synth.weights(dims, sigma, rng, with_wo=False)
    W = {k: _round(W[k], w_kind) for k in ("W_DQ", "W_UQ", "W_QR")}
    h = _round(rng.normal(size=(batch, dims.d_model)), h_kind)
    pos = rng.integers(0, max_pos or 32768, batch).astype(np.int32)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    dev = lambda x, k: torch.from_numpy(x.astype(np.float32)).cuda().to(tdt[k]).contiguous()  # noqa: E731
    d = mk.dims(dims.n_heads, dims.d_head, dims.d_rope, dims.d_latent)
    nbytes = mk.query_prep_scratch_size(d, dims.d_qlatent, batch)
    scratch = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    q_nope = torch.empty((batch, dims.n_heads, dims.d_head), dtype=tdt[out_kind], device="cuda")
    q_pe = torch.empty((batch, dims.n_heads, dims.d_rope), dtype=tdt[out_kind], device="cuda")
    print(f"case: query prep B={batch} d={dims.d_model} h {h_kind} w {w_kind} out {out_kind} "
          f"base {rope_base} scratch {nbytes}", flush=True)
    rope = None if yarn is None else mk.rope(rope_base, *yarn)
    mk.query_prep(d, dev(h, h_kind), dev(W["W_DQ"], w_kind), dev(W["W_UQ"], w_kind), dev(W["W_QR"], w_kind),
                  torch.from_numpy(pos).cuda(), q_nope, q_pe, scratch, rope_base, rope=rope)
    torch.cuda.synchronize()
    got_c = q_nope.float().cpu().numpy().astype(np.float64)
    got_r = q_pe.float().cpu().numpy().astype(np.float64)
    ref_c = np.empty_like(got_c)
    ref_r = np.empty_like(got_r)
    for b in range(batch):
        qc, qr = oracle.project_query(h[b], W, int(pos[b]), dims.n_heads)
        ref_c[b] = qc
        # rope_base 0 means the device leaves q^R unrotated: position 0 in the oracle
        ref_r[b] = qr if rope_base > 0 else oracle.project_query(h[b], W, 0, dims.n_heads)[1]
        if yarn is not None:
            theta = oracle.yarn_theta(dims.d_rope, rope_base, *yarn)
            ref_r[b] = oracle.rope_theta(oracle.project_query(h[b], W, 0, dims.n_heads)[1], int(pos[b]), theta)
    return got_c, got_r, ref_c, ref_r


def _rel(got, ref):
    return np.abs(got - ref).max() / np.abs(ref).max()


@pytest.mark.parametrize("batch", [64, 37, 100])
def test_query_prep_v2_bf16(batch):
    import synth
    got_c, got_r, ref_c, ref_r = _run(synth.V2, batch, "bf16", "bf16", "bf16", seed=100 + batch)
    ec, er = _rel(got_c, ref_c), _rel(got_r, ref_r)
    print(f"q^C rel err {ec:.3e}  q^R rel err {er:.3e}", flush=True)
    assert ec <= TOL["bf16"] and er <= TOL["bf16"]


def test_query_prep_v2_mixed_f32_out():
    """fp32 h and fp32 outputs around bf16 weights: the first product takes the
    generic path, the second the MFMA one (c^Q is rounded to bf16)."""
    import synth
    got_c, got_r, ref_c, ref_r = _run(synth.V2, 16, "f32", "bf16", "f32", seed=7)
    ec, er = _rel(got_c, ref_c), _rel(got_r, ref_r)
    print(f"q^C rel err {ec:.3e}  q^R rel err {er:.3e}", flush=True)
    assert ec <= TOL["bf16"] and er <= TOL["bf16"]


@pytest.mark.parametrize("batch", [1, 9])
def test_query_prep_tiny_f32(batch):
    import synth
    got_c, got_r, ref_c, ref_r = _run(synth.TINY, batch, "f32", "f32", "f32", seed=200 + batch, sigma=0.05,
                                      max_pos=100000)
    assert _rel(got_c, ref_c) <= TOL["f32"]
    assert _rel(got_r, ref_r) <= TOL["f32"]


def test_query_prep_unrotated():
    import synth
    got_c, got_r, ref_c, ref_r = _run(synth.TINY, 5, "f32", "f32", "f32", seed=3, rope_base=0.0, sigma=0.05)
    assert _rel(got_c, ref_c) <= TOL["f32"]
    assert _rel(got_r, ref_r) <= TOL["f32"]


def test_query_prep_v2_unrotated():
    """The V2 shapes (the second product writes q^C and q^R from its epilogue)
    with the rotation off: q^R is the plain product."""
    import synth
    got_c, got_r, ref_c, ref_r = _run(synth.V2, 8, "bf16", "bf16", "bf16", seed=5, rope_base=0.0)
    assert _rel(got_c, ref_c) <= TOL["bf16"]
    assert _rel(got_r, ref_r) <= TOL["bf16"]


def _fused_weights(W, n_heads, d_head):
    """The offline-fused query weight of the pages' absorption remark: head i's
    block is W^UK_i^T W^UQ_i, so W^UQK c^Q gives every head's q_lat directly."""
    return np.concatenate([oracle.mla.head_rows(W["W_UK"], i, d_head).T @ oracle.mla.head_rows(W["W_UQ"], i, d_head)
                           for i in range(n_heads)], axis=0)


@pytest.mark.parametrize("batch", [64, 37])
def test_query_prep_fused_absorb_v2(batch):
    """q_lat two ways, each against q_lat_i = W^UK_i^T q^C_i from the oracle's q^C:
    (1) query prep then mla_absorb_q; (2) query prep on the fused weight
    [W^UK_i^T W^UQ_i] (d_h replaced by d_c), which writes q_lat itself."""
    import torch
    import synth
    import mla_latent_kv_37_amd as mk
    dims = synth.V2
    nh, dh, dr, dc, dq = dims.n_heads, dims.d_head, dims.d_rope, dims.d_latent, dims.d_qlatent
    rng = np.random.default_rng(500 + batch)
    W = synth.weights(dims, synth.V2_SIGMA_W, rng, with_wo=False)
    W = {k: _round(W[k], "bf16") for k in ("W_DQ", "W_UQ", "W_QR", "W_UK")}
    fused = _round(_fused_weights(W, nh, dh), "bf16")
    h = _round(rng.normal(size=(batch, dims.d_model)), "bf16")
    pos = rng.integers(0, 32768, batch).astype(np.int32)
    bf = lambda x: torch.from_numpy(np.asarray(x, dtype=np.float32)).cuda().to(torch.bfloat16).contiguous()  # noqa: E731
    pos_d = torch.from_numpy(pos).cuda()
    print(f"case: q_lat via absorb and via fused weights, B={batch}", flush=True)
    # (1) unfused
    d = mk.dims(nh, dh, dr, dc)
    scratch = torch.empty(mk.query_prep_scratch_size(d, dq, batch), dtype=torch.uint8, device="cuda")
    q_nope = torch.empty((batch, nh, dh), dtype=torch.bfloat16, device="cuda")
    q_pe = torch.empty((batch, nh, dr), dtype=torch.bfloat16, device="cuda")
    mk.query_prep(d, bf(h), bf(W["W_DQ"]), bf(W["W_UQ"]), bf(W["W_QR"]), pos_d, q_nope, q_pe, scratch, ROPE_BASE)
    q_lat1 = torch.empty((batch, nh, dc), dtype=torch.bfloat16, device="cuda")
    mk.absorb_q(d, q_nope, bf(W["W_UK"]), q_lat1)
    # (2) fused: the same entry point with d_h := d_c and W^UQK in place of W^UQ
    dfu = mk.dims(nh, dc, dr, dc)
    scratch2 = torch.empty(mk.query_prep_scratch_size(dfu, dq, batch), dtype=torch.uint8, device="cuda")
    q_lat2 = torch.empty((batch, nh, dc), dtype=torch.bfloat16, device="cuda")
    q_pe2 = torch.empty((batch, nh, dr), dtype=torch.bfloat16, device="cuda")
    mk.query_prep(dfu, bf(h), bf(W["W_DQ"]), bf(fused), bf(W["W_QR"]), pos_d, q_lat2, q_pe2, scratch2, ROPE_BASE)
    torch.cuda.synchronize()
    ref_lat = np.empty((batch, nh, dc))
    ref_r = np.empty((batch, nh, dr))
    for b in range(batch):
        qc, qr = oracle.project_query(h[b], W, int(pos[b]), nh)
        for i in range(nh):
            ref_lat[b, i] = oracle.mla.head_rows(W["W_UK"], i, dh).T @ qc[i]
        ref_r[b] = qr
    got1 = q_lat1.float().cpu().numpy()
    got2 = q_lat2.float().cpu().numpy()
    e1, e2 = _rel(got1, ref_lat), _rel(got2, ref_lat)
    er1, er2 = _rel(q_pe.float().cpu().numpy(), ref_r), _rel(q_pe2.float().cpu().numpy(), ref_r)
    print(f"q_lat rel err: absorb {e1:.3e}, fused {e2:.3e}; q^R {er1:.3e} / {er2:.3e}", flush=True)
    assert max(e1, e2, er1, er2) <= TOL["bf16"]


def _run_uncompressed(dims, batch, kind, seed, sigma):
    """V2-Lite form (no query compression): q^C = W^UQ h, q^R = RoPE(W^QR h), with
    W^UQ [n_h d_h, d_model], W^QR [n_h d_r, d_model].  The oracle's project_query
    with W^DQ = I computes exactly that."""
    import torch
    import mla_latent_kv_37_amd as mk
    rng = np.random.default_rng(seed)
    nh, dh, dr, dm = dims.n_heads, dims.d_head, dims.d_rope, dims.d_model
    W = {"W_DQ": np.eye(dm), "W_UQ": _round(rng.normal(0.0, sigma, (nh * dh, dm)), kind),
         "W_QR": _round(rng.normal(0.0, sigma, (nh * dr, dm)), kind)}
    h = _round(rng.normal(size=(batch, dm)), kind)
    pos = rng.integers(0, 32768, batch).astype(np.int32)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[kind]
    dev = lambda x: torch.from_numpy(x.astype(np.float32)).cuda().to(tdt).contiguous()  # noqa: E731
    d = mk.dims(nh, dh, dr, dims.d_latent)
    scratch = torch.empty(mk.query_prep_scratch_size(d, 0, batch), dtype=torch.uint8, device="cuda")
    q_nope = torch.empty((batch, nh, dh), dtype=tdt, device="cuda")
    q_pe = torch.empty((batch, nh, dr), dtype=tdt, device="cuda")
    print(f"case: uncompressed query prep B={batch} d={dm} {kind}", flush=True)
    mk.query_prep(d, dev(h), None, dev(W["W_UQ"]), dev(W["W_QR"]), torch.from_numpy(pos).cuda(), q_nope, q_pe,
                  scratch, ROPE_BASE)
    torch.cuda.synchronize()
    ref_c = np.stack([oracle.project_query(h[b], W, int(pos[b]), nh)[0] for b in range(batch)])
    ref_r = np.stack([oracle.project_query(h[b], W, int(pos[b]), nh)[1] for b in range(batch)])
    return q_nope.float().cpu().numpy(), q_pe.float().cpu().numpy(), ref_c, ref_r


@pytest.mark.parametrize("batch", [64, 37])
def test_query_prep_v2lite_uncompressed(batch):
    import synth
    got_c, got_r, ref_c, ref_r = _run_uncompressed(synth.V2LITE, batch, "bf16", 300 + batch, synth.V2_SIGMA_W)
    ec, er = _rel(got_c, ref_c), _rel(got_r, ref_r)
    print(f"q^C rel err {ec:.3e}  q^R rel err {er:.3e}", flush=True)
    assert ec <= TOL["bf16"] and er <= TOL["bf16"]


def test_query_prep_tiny_uncompressed_f32():
    import synth
    got_c, got_r, ref_c, ref_r = _run_uncompressed(synth.TINY, 7, "f32", 11, 0.05)
    assert _rel(got_c, ref_c) <= TOL["f32"] and _rel(got_r, ref_r) <= TOL["f32"]


YARN_V2 = (40.0, 1.0, 32.0, 4096)   # s, alpha, beta, original context ([V2-explainer] §3.1.3)


def test_query_prep_yarn():
    """q^R rotated with the YaRN frequencies (mla_query_prep_rope) at positions
    up to 160K; the plain-RoPE reference differs there, so the check sees the
    frequencies."""
    import synth
    got_c, got_r, ref_c, ref_r = _run(synth.V2, 24, "bf16", "bf16", "f32", seed=61, max_pos=163840, yarn=YARN_V2)
    ec, er = _rel(got_c, ref_c), _rel(got_r, ref_r)
    print(f"q^C rel err {ec:.3e}  q^R rel err {er:.3e}", flush=True)
    assert ec <= TOL["bf16"] and er <= TOL["bf16"]
    _, plain_r, _, _ = _run(synth.V2, 24, "bf16", "bf16", "f32", seed=61, max_pos=163840)
    assert _rel(plain_r, ref_r) > 0.1
