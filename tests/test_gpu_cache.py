"""GPU tests of the cache-store and cache-append entry points against the oracle.

Stores are compared byte for byte: the rows are given (or taken from the GPU's
own fp32 projection), so the rounding decisions (bf16 bits, E4M3 codes, group
scales) are taken from the same binary32 values on both sides and must agree
exactly.  The RoPE columns are compared within a tolerance, since the rotation
is evaluated in float64 on the host and in fp32-in/fp64-math on the device.
Slots not addressed by a call must keep their sentinel bytes.
"""
import zlib

import numpy as np
import pytest

import oracle
from oracle import storage as ostore

pytestmark = pytest.mark.gpu

PAGE = 64
SENTINEL = 0xAB


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_37_amd as mk
    print(mk.build_info(), flush=True)


def _layout(rng, batch, max_pages, num_pages):
    """Random block table (distinct pages) and target positions, with skipped cases."""
    perm = rng.permutation(num_pages)[: batch * max_pages].reshape(batch, max_pages).astype(np.int32)
    pos = rng.integers(0, max_pages * PAGE, batch).astype(np.int32)
    pos[3] = -1                              # skipped: negative position
    pos[5] = max_pages * PAGE                # skipped: past the block table
    perm[7, pos[7] // PAGE] = num_pages      # skipped: page id outside the cache
    return perm, pos


def _targets(rng, pos, max_pages, num_pages):
    """Block table whose entry for each sequence's target position is a page of its
    own (page b); the other entries point anywhere in the cache."""
    perm = rng.integers(0, num_pages, (len(pos), max_pages)).astype(np.int32)
    for b, t in enumerate(pos):
        perm[b, t // PAGE] = b
    return perm


def _rows(rng, batch, width):
    x = rng.normal(size=(batch, width)) * np.exp2(rng.integers(-8, 8, (batch, 1)))
    x[1, : min(128, width)] = 0.0            # an all-zero group
    if width >= 256:
        # E4M3 ties: group 1 of row 2 holds exact midpoints between codes, times a
        # power of two, with its largest magnitude exactly 448 times that power
        codes = np.arange(1, 126, dtype=np.uint8)
        vals = ostore.e4m3fn_to_f64(codes)
        mids = (vals[:-1] + vals[1:]) / 2
        g = np.resize(mids, 128) * 2.0 ** -3
        g[0] = 448.0 * 2.0 ** -3
        x[2, 128:256] = g
    # bf16 ties in row 4: binary32 patterns whose low half is exactly 0x8000
    u = rng.integers(0, 2 ** 31, width, dtype=np.uint64).astype(np.uint32)
    x[4] = ((u & np.uint32(0x3F7F0000)) | np.uint32(0x8000)).view(np.float32)
    return x.astype(np.float32)


def _expected(kind, rows32, perm, pos, num_pages, max_pages, width):
    """Host image of the cache bytes after the store: sentinel except the written rows."""
    ng = (width + 127) // 128
    ebytes = {"f32": 4, "bf16": 2, "fp8": 1}[kind]
    kv = np.full((num_pages * PAGE, width * ebytes), SENTINEL, dtype=np.uint8)
    sc = np.full((num_pages * PAGE, ng), SENTINEL, dtype=np.uint8).repeat(4, axis=1) if kind == "fp8" else None
    for b in range(rows32.shape[0]):
        t = int(pos[b])
        if t < 0 or t >= max_pages * PAGE:
            continue
        page = int(perm[b, t // PAGE])
        if page < 0 or page >= num_pages:
            continue
        r = page * PAGE + t % PAGE
        if kind == "f32":
            kv[r] = rows32[b].view(np.uint8)
        elif kind == "bf16":
            kv[r] = ostore.f32_to_bf16_bits(rows32[b]).view(np.uint8)
        else:
            codes, scales = ostore.quantize_e4m3_groups(rows32[b : b + 1])
            kv[r] = codes[0]
            sc[r] = scales[0].view(np.uint8)
    return kv, sc


def _device_cache(kind, num_pages, width, perm):
    import torch
    import mla_latent_kv_37_amd as mk
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[kind]
    kv = torch.empty((num_pages, PAGE, width), dtype=tdt, device="cuda")
    kv.view(torch.uint8).fill_(SENTINEL)
    scales = None
    if kind == "fp8":
        scales = torch.empty((num_pages, PAGE, (width + 127) // 128), dtype=torch.float32, device="cuda")
        scales.view(torch.uint8).fill_(SENTINEL)
    bt = torch.from_numpy(perm).cuda()
    lens = torch.zeros(perm.shape[0], dtype=torch.int32, device="cuda")
    return kv, scales, bt, mk.make_cache(kv, bt, lens, PAGE, scales)


def _host_bytes(t, rows):
    return t.contiguous().view(-1).view(__import__("torch").uint8).cpu().numpy().reshape(rows, -1)


@pytest.mark.parametrize("kind", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("rows_dt", ["f32", "bf16"])
@pytest.mark.parametrize("shape", ["v2", "tiny"])
def test_cache_store_bit_exact(kind, rows_dt, shape):
    import torch
    import mla_latent_kv_37_amd as mk
    if shape == "v2":
        d, width = mk.dims(128, 128, 64, 512), 576
    else:
        d, width = mk.dims(4, 16, 8, 32), 40
    rng = np.random.default_rng(zlib.crc32(f"{kind}/{rows_dt}/{shape}".encode()))
    batch, max_pages, num_pages = 23, 5, 200
    print(f"case: cache store {shape} rows {rows_dt} -> {kind}, B={batch}", flush=True)
    perm, pos = _layout(rng, batch, max_pages, num_pages)
    rows32 = _rows(rng, batch, width)
    if rows_dt == "bf16":
        rows32 = ostore.bf16_bits_to_f64(ostore.f32_to_bf16_bits(rows32)).astype(np.float32)
    kv, scales, bt, cache = _device_cache(kind, num_pages, width, perm)
    rows = torch.from_numpy(rows32).cuda().to(torch.float32 if rows_dt == "f32" else torch.bfloat16)
    mk.cache_store(d, rows, torch.from_numpy(pos).cuda(), cache, 0.0)
    torch.cuda.synchronize()
    ekv, esc = _expected(kind, rows32, perm, pos, num_pages, max_pages, width)
    got = _host_bytes(kv, num_pages * PAGE)
    assert np.array_equal(got, ekv), f"{np.count_nonzero(got != ekv)} bytes differ"
    if kind == "fp8":
        assert np.array_equal(_host_bytes(scales, num_pages * PAGE), esc)


def _stored_values(kind, kv, scales, perm, pos, num_pages, width):
    """float64 rows as stored at each sequence's target slot (None where skipped)."""
    kvb = _host_bytes(kv, num_pages * PAGE)
    out = []
    for b in range(len(pos)):
        t = int(pos[b])
        page = int(perm[b, t // PAGE]) if 0 <= t < perm.shape[1] * PAGE else -1
        if page < 0 or page >= num_pages:
            out.append(None)
            continue
        r = page * PAGE + t % PAGE
        if kind == "f32":
            out.append(kvb[r].view(np.float32).astype(np.float64))
        elif kind == "bf16":
            out.append(ostore.bf16_bits_to_f64(kvb[r].view(np.uint16)))
        else:
            sc = _host_bytes(scales, num_pages * PAGE)[r].view(np.float32)
            out.append(ostore.dequantize_rows(kvb[r][None], sc[None])[0])
    return out


ROPE_TOL = {"f32": 1e-6, "bf16": 2.0 ** -8, "fp8": 2.0 ** -3}


def _check_rope_part(kind, got_row, ref_row, d_latent):
    ref = ref_row[d_latent:]
    err = np.abs(got_row[d_latent:] - ref)
    assert np.all(err <= ROPE_TOL[kind] * np.abs(ref).max() + 1e-30), f"RoPE part max err {err.max():.3e}"


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_cache_store_rope(kind):
    import torch
    import mla_latent_kv_37_amd as mk
    d, width, dc = mk.dims(128, 128, 64, 512), 576, 512
    rng = np.random.default_rng(21)
    batch, max_pages = 16, 2048
    num_pages = batch + 4
    print(f"case: cache store with RoPE, {kind}, positions up to {max_pages * PAGE - 1}", flush=True)
    pos = np.concatenate([[0, 1, 63, 64, max_pages * PAGE - 1], rng.integers(0, max_pages * PAGE, batch - 5)])
    pos = pos.astype(np.int32)
    perm = _targets(rng, pos, max_pages, num_pages)
    rows32 = (rng.normal(size=(batch, width)) * 0.4).astype(np.float32)
    kv, scales, bt, cache = _device_cache(kind, num_pages, width, perm)
    mk.cache_store(d, torch.from_numpy(rows32).cuda(), torch.from_numpy(pos).cuda(), cache, 10000.0)
    torch.cuda.synchronize()
    got = _stored_values(kind, kv, scales, perm, pos, num_pages, width)
    for b in range(batch):
        ref = np.concatenate([rows32[b, :dc].astype(np.float64), oracle.rope(rows32[b, dc:], pos[b])])
        # c^KV columns: the same rounding decisions as the oracle encoder
        if kind == "bf16":
            want = ostore.bf16_bits_to_f64(ostore.f32_to_bf16_bits(rows32[b, :dc]))
        else:
            c, s = ostore.quantize_e4m3_groups(rows32[b : b + 1, :dc])
            want = ostore.dequantize_rows(c, s)[0]
        assert np.array_equal(got[b][:dc], want)
        _check_rope_part(kind, got[b], ref, dc)


@pytest.mark.parametrize("model,kind", [("V2", "bf16"), ("V2", "fp8"), ("V2LITE", "bf16")])
def test_cache_append_v2(model, kind):
    """Projection from h (d_model 5120 for V2, 2048 for V2-Lite), RoPE, rounding and scatter."""
    import torch
    import synth
    import mla_latent_kv_37_amd as mk
    dims = getattr(synth, model)
    d = mk.dims(dims.n_heads, dims.d_head, dims.d_rope, dims.d_latent)
    dc, width = dims.d_latent, dims.d_latent + dims.d_rope
    rng = np.random.default_rng(31)
    batch, max_pages = 64, 16
    num_pages = batch + 4
    print(f"case: cache append {model} (d_model {dims.d_model}) -> {kind}, B={batch}", flush=True)
    W = synth.weights(dims, 0.006, rng, with_wo=False)
    to_bf16 = lambda x: ostore.bf16_bits_to_f64(ostore.f32_to_bf16_bits(x.astype(np.float32)))  # noqa: E731
    h, w_dkv, w_kr = to_bf16(rng.normal(size=(batch, dims.d_model))), to_bf16(W["W_DKV"]), to_bf16(W["W_KR"])
    pos = rng.integers(0, max_pages * PAGE, batch).astype(np.int32)
    perm = _targets(rng, pos, max_pages, num_pages)
    # skipped sequences: their cache slot is not written, but rows[b] still
    # holds the summed projection
    pos[3] = -1                              # negative position
    perm[7, pos[7] // PAGE] = num_pages      # page id outside the cache
    kv, scales, bt, cache = _device_cache(kind, num_pages, width, perm)
    t = lambda x: torch.from_numpy(x.astype(np.float32)).cuda().to(torch.bfloat16)  # noqa: E731
    rows = torch.empty((8, batch, width), dtype=torch.float32, device="cuda")
    mk.cache_append(d, t(h), t(w_dkv), t(w_kr), rows, torch.from_numpy(pos).cuda(), cache, 10000.0)
    torch.cuda.synchronize()
    rows_gpu = rows[0].cpu().numpy()
    ref_c, ref_r = h @ w_dkv.T, h @ w_kr.T          # the projections, float64
    ref = np.concatenate([ref_c, ref_r], axis=1)
    for b in range(batch):                          # every sequence, the skipped ones included
        err = np.abs(rows_gpu[b] - ref[b]).max() / np.abs(ref[b]).max()
        assert err <= 1e-4, f"rows[{b}] rel err {err:.3e}"
    got = _stored_values(kind, kv, scales, perm, pos, num_pages, width)
    assert got[3] is None and got[7] is None
    # nothing outside the written slots changed (the skipped sequences wrote nothing)
    written = {int(perm[b, pos[b] // PAGE]) * PAGE + int(pos[b]) % PAGE for b in range(batch) if got[b] is not None}
    kvb = _host_bytes(kv, num_pages * PAGE)
    untouched = np.array([r for r in range(num_pages * PAGE) if r not in written])
    assert np.all(kvb[untouched] == SENTINEL)
    for b in range(batch):
        if got[b] is None:
            continue
        if kind == "bf16":
            want = ostore.bf16_bits_to_f64(ostore.f32_to_bf16_bits(rows_gpu[b, :dc]))
        else:
            c, s = ostore.quantize_e4m3_groups(rows_gpu[b : b + 1, :dc])
            want = ostore.dequantize_rows(c, s)[0]
        assert np.array_equal(got[b][:dc], want)
        _check_rope_part(kind, got[b], np.concatenate([ref_c[b], oracle.rope(ref_r[b], pos[b])]), dc)


def test_cache_append_tiny_f32():
    import torch
    import synth
    import mla_latent_kv_37_amd as mk
    dims = synth.TINY
    d = mk.dims(dims.n_heads, dims.d_head, dims.d_rope, dims.d_latent)
    dc, width = dims.d_latent, dims.d_latent + dims.d_rope
    rng = np.random.default_rng(41)
    batch, max_pages, num_pages = 9, 3, 40
    print("case: cache append tiny f32 (generic projection)", flush=True)
    W = synth.weights(dims, 0.02, rng, with_wo=False)
    h = rng.normal(size=(batch, dims.d_model)).astype(np.float32)
    perm = rng.permutation(num_pages)[: batch * max_pages].reshape(batch, max_pages).astype(np.int32)
    pos = rng.integers(0, max_pages * PAGE, batch).astype(np.int32)
    kv, scales, bt, cache = _device_cache("f32", num_pages, width, perm)
    f = lambda x: torch.from_numpy(np.asarray(x, dtype=np.float32)).cuda()  # noqa: E731
    rows = torch.empty((8, batch, width), dtype=torch.float32, device="cuda")
    mk.cache_append(d, f(h), f(W["W_DKV"]), f(W["W_KR"]), rows, torch.from_numpy(pos).cuda(), cache, 10000.0)
    torch.cuda.synchronize()
    hd = h.astype(np.float64)
    wdkv, wkr = W["W_DKV"].astype(np.float32).astype(np.float64), W["W_KR"].astype(np.float32).astype(np.float64)
    c_kv, k_r = oracle.project_cache(hd, {"W_DKV": wdkv, "W_KR": wkr}, pos)
    ref = np.concatenate([hd @ wdkv.T, hd @ wkr.T], axis=1)
    assert np.abs(rows[0].cpu().numpy() - ref).max() <= 1e-4 * np.abs(ref).max()
    got = _stored_values("f32", kv, scales, perm, pos, num_pages, width)
    for b in range(batch):
        full = np.concatenate([c_kv[b], k_r[b]])
        assert np.abs(got[b] - full).max() <= 1e-5 * np.abs(full).max()


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_cache_store_yarn(kind):
    """k^R rotated with the YaRN frequencies of [V2-explainer] §3.1.3 (s = 40,
    alpha = 1, beta = 32, original context 4096) through mla_cache_store_rope,
    at positions up to 160K; the latent part is stored as without RoPE."""
    import torch
    import mla_latent_kv_37_amd as mk
    d, width, dc = mk.dims(128, 128, 64, 512), 576, 512
    rng = np.random.default_rng(22)
    batch, max_pages = 16, 2560
    num_pages = batch + 4
    pos = np.concatenate([[0, 1, 4095, 4096, max_pages * PAGE - 1], rng.integers(0, max_pages * PAGE, batch - 5)])
    pos = pos.astype(np.int32)
    print(f"case: cache store with YaRN RoPE, {kind}, positions up to {max_pages * PAGE - 1}", flush=True)
    perm = _targets(rng, pos, max_pages, num_pages)
    rows32 = (rng.normal(size=(batch, width)) * 0.4).astype(np.float32)
    kv, scales, bt, cache = _device_cache(kind, num_pages, width, perm)
    mk.cache_store(d, torch.from_numpy(rows32).cuda(), torch.from_numpy(pos).cuda(), cache,
                   rope=mk.rope(10000.0, 40.0, 1.0, 32.0, 4096))
    torch.cuda.synchronize()
    got = _stored_values(kind, kv, scales, perm, pos, num_pages, width)
    theta = oracle.yarn_theta(64, 10000.0, 40.0, 1.0, 32.0, 4096)
    differs = 0
    for b in range(batch):
        ref = np.concatenate([rows32[b, :dc].astype(np.float64), oracle.rope_theta(rows32[b, dc:], pos[b], theta)])
        _check_rope_part(kind, got[b], ref, dc)
        plain = oracle.rope(rows32[b, dc:], pos[b])
        differs += np.abs(plain - ref[dc:]).max() > 0.1 * np.abs(ref[dc:]).max()
    assert differs >= batch // 2   # (the YaRN frequencies are what the check sees)
