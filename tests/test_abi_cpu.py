"""C-ABI checks that need no GPU: exports, status strings, validation errors,
workspace sizing and the host partition helper (against a brute-force model)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


@pytest.fixture(scope="module")
def lib():
    from mla_latent_kv_37_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libmla.so not built (run python -m mla_latent_kv_37_amd.build)")
    return _lib


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    fns = declared_functions()
    for name in ("mla_absorb_q", "mla_decode", "mla_merge_splits", "mla_out_proj"):
        assert name in fns


def test_library_exports_every_declared_symbol(lib):
    l = lib.load()
    for name in declared_functions():
        assert hasattr(l, name), name
    assert set(declared_functions()) == set(lib.EXPORTS)


def test_status_strings(lib):
    assert lib.status_string(0) == "MLA_OK"
    for s in range(1, 6):
        assert lib.status_string(s).startswith("MLA_ERR_")
    assert "gfx950" in lib.build_info()


def _v2(lib):
    return lib.dims(128, 128, 64, 512)


def test_workspace_sizes(lib):
    d = _v2(lib)
    assert lib.workspace_size(d, 8, 10, 64, lib.partition(0, 0)) == (0, 0)
    nbytes, slots = lib.workspace_size(d, 4, 2048, 64, lib.partition(4096, 0))
    assert slots == 4 * 32
    lse_off = lib.lse_part_offset(d, slots)
    assert lse_off == slots * 128 * 512 * 4
    assert nbytes == lse_off + slots * 128 * 4
    nbytes, slots = lib.workspace_size(d, 64, 128, 64, lib.partition(0, 256))
    assert slots == 256 + 64
    assert nbytes >= lib.lse_part_offset(d, slots) + slots * 128 * 4 + 2 * 64 * 4


def _raw(lib):
    return lib.load()


def test_validation_errors_before_any_device_access(lib):
    L = _raw(lib)
    d = _v2(lib)
    fake = ctypes.c_void_p(0x10000)        # never dereferenced: every case fails validation first
    odd = ctypes.c_void_p(0x10008)
    cache = lib.PagedCache(0x10000, None, lib.MLA_BF16, 64, 100, 0x20000, 16, 0x30000)
    part = lib.partition(0, 0)
    # null dims / null pointers
    assert L.mla_absorb_q(None, 1, fake, 1, fake, 1, fake, 1, None) == lib.MLA_ERR_INVALID_ARG
    assert L.mla_absorb_q(ctypes.byref(d), 1, None, 1, fake, 1, fake, 1, None) == lib.MLA_ERR_INVALID_ARG
    # fp8 queries are not supported for absorb; misaligned output
    assert L.mla_absorb_q(ctypes.byref(d), 1, fake, 2, fake, 1, fake, 1, None) == lib.MLA_ERR_UNSUPPORTED
    assert L.mla_absorb_q(ctypes.byref(d), 1, fake, 1, fake, 1, odd, 1, None) == lib.MLA_ERR_ALIGNMENT
    # decode: bf16 cache needs bf16 queries
    assert L.mla_decode(ctypes.byref(d), 1, fake, fake, lib.MLA_F32, ctypes.byref(cache), 0.07, ctypes.byref(part),
                        None, 0, fake, 1, None, None) == lib.MLA_ERR_UNSUPPORTED
    # non-positive scale
    assert L.mla_decode(ctypes.byref(d), 1, fake, fake, 1, ctypes.byref(cache), 0.0, ctypes.byref(part),
                        None, 0, fake, 1, None, None) == lib.MLA_ERR_INVALID_ARG
    # split not a multiple of the page size
    bad = lib.partition(100, 0)
    assert L.mla_decode(ctypes.byref(d), 1, fake, fake, 1, ctypes.byref(cache), 0.07, ctypes.byref(bad),
                        None, 0, fake, 1, None, None) == lib.MLA_ERR_INVALID_ARG
    # split partition needs a workspace
    sp = lib.partition(128, 0)
    assert L.mla_decode(ctypes.byref(d), 1, fake, fake, 1, ctypes.byref(cache), 0.07, ctypes.byref(sp),
                        None, 0, fake, 1, None, None) == lib.MLA_ERR_WORKSPACE
    assert L.mla_decode(ctypes.byref(d), 1, fake, fake, 1, ctypes.byref(cache), 0.07, ctypes.byref(sp),
                        fake, 16, fake, 1, None, None) == lib.MLA_ERR_WORKSPACE
    # misaligned cache
    c2 = lib.PagedCache(0x10004, None, lib.MLA_BF16, 64, 100, 0x20000, 16, 0x30000)
    assert L.mla_decode(ctypes.byref(d), 1, fake, fake, 1, ctypes.byref(c2), 0.07, ctypes.byref(part),
                        None, 0, fake, 1, None, None) == lib.MLA_ERR_ALIGNMENT
    # fp8 cache without scales
    c3 = lib.PagedCache(0x10000, None, lib.MLA_FP8_E4M3, 64, 100, 0x20000, 16, 0x30000)
    assert L.mla_decode(ctypes.byref(d), 1, fake, fake, 1, ctypes.byref(c3), 0.07, ctypes.byref(part),
                        None, 0, fake, 1, None, None) == lib.MLA_ERR_INVALID_ARG
    # merge: fp8 output unsupported; out_proj: null weight
    assert L.mla_merge_splits(ctypes.byref(d), 1, fake, 64, 16, ctypes.byref(part), None, 0, fake, 2, None,
                              None) == lib.MLA_ERR_UNSUPPORTED
    assert L.mla_out_proj(ctypes.byref(d), 1, fake, 1, None, 1, fake, 1, None) == lib.MLA_ERR_INVALID_ARG
    # batch 0 is a no-op that touches nothing
    assert L.mla_absorb_q(ctypes.byref(d), 0, fake, 1, fake, 1, fake, 1, None) == lib.MLA_OK
    # cache store / append: fp8 rows unsupported, missing positions, negative RoPE base,
    # odd column counts, misaligned rows, fp8 cache without scales
    cs = L.mla_cache_store
    assert cs(ctypes.byref(d), 1, fake, lib.MLA_FP8_E4M3, fake, 0.0, ctypes.byref(cache), None) == lib.MLA_ERR_UNSUPPORTED
    assert cs(ctypes.byref(d), 1, fake, lib.MLA_F32, None, 0.0, ctypes.byref(cache), None) == lib.MLA_ERR_INVALID_ARG
    assert cs(ctypes.byref(d), 1, fake, lib.MLA_F32, fake, -1.0, ctypes.byref(cache), None) == lib.MLA_ERR_INVALID_ARG
    d_odd = lib.dims(128, 128, 63, 512)
    assert cs(ctypes.byref(d_odd), 1, fake, lib.MLA_F32, fake, 0.0, ctypes.byref(cache), None) == lib.MLA_ERR_UNSUPPORTED
    assert cs(ctypes.byref(d), 1, odd, lib.MLA_F32, fake, 0.0, ctypes.byref(cache), None) == lib.MLA_ERR_ALIGNMENT
    assert cs(ctypes.byref(d), 1, fake, lib.MLA_F32, fake, 0.0, ctypes.byref(c3), None) == lib.MLA_ERR_INVALID_ARG
    assert cs(ctypes.byref(d), 0, fake, lib.MLA_F32, fake, 0.0, ctypes.byref(cache), None) == lib.MLA_OK
    ca = L.mla_cache_append
    assert ca(ctypes.byref(d), 5120, 1, None, 1, fake, fake, 1, fake, fake, 1e4, ctypes.byref(cache),
              None) == lib.MLA_ERR_INVALID_ARG
    assert ca(ctypes.byref(d), 0, 1, fake, 1, fake, fake, 1, fake, fake, 1e4, ctypes.byref(cache),
              None) == lib.MLA_ERR_INVALID_ARG
    assert ca(ctypes.byref(d), 5120, 1, fake, lib.MLA_FP8_E4M3, fake, fake, 1, fake, fake, 1e4, ctypes.byref(cache),
              None) == lib.MLA_ERR_UNSUPPORTED
    # query prep: too-small scratch, fp8 weights, null weight
    qp = L.mla_query_prep
    need = L.mla_query_prep_scratch_size(ctypes.byref(d), 1536, 4)
    assert need >= 4 * 128 * 192 * 4
    assert qp(ctypes.byref(d), 5120, 1536, 4, fake, 1, fake, fake, fake, 1, fake, 1e4, fake, fake, 1, fake, need - 1,
              None) == lib.MLA_ERR_WORKSPACE
    assert qp(ctypes.byref(d), 5120, 1536, 4, fake, 1, fake, fake, fake, lib.MLA_FP8_E4M3, fake, 1e4, fake, fake, 1,
              fake, need, None) == lib.MLA_ERR_UNSUPPORTED
    assert qp(ctypes.byref(d), 5120, 1536, 4, fake, 1, None, fake, fake, 1, fake, 1e4, fake, fake, 1, fake, need,
              None) == lib.MLA_ERR_INVALID_ARG
    # d_qlatent = 0 (query not compressed): no W^DQ needed, single product sized for the largest k-slice plan
    need0 = L.mla_query_prep_scratch_size(ctypes.byref(d), 0, 4)
    assert need0 >= 16 * 4 * 128 * 192 * 4
    assert qp(ctypes.byref(d), 2048, 0, 4, fake, 1, None, fake, fake, 1, fake, 1e4, fake, fake, 1, fake, need0 - 1,
              None) == lib.MLA_ERR_WORKSPACE
    assert qp(ctypes.byref(d), 2048, -1, 4, fake, 1, None, fake, fake, 1, fake, 1e4, fake, fake, 1, fake, need0,
              None) == lib.MLA_ERR_INVALID_ARG


def test_prefill_workspace_and_validation(lib):
    """mla_prefill: workspace = offsets + gathered rows + up-projected keys and
    values, sized by total_kv; every argument error is reported before launch."""
    L = _raw(lib)
    d = _v2(lib)
    cap = ((1000 + 32 + 255) // 256) * 256
    expect = 256 + cap * 576 * 2 + 2 * 128 * cap * 128 * 2
    assert lib.prefill_workspace_size(d, 3, 1000) == expect
    sz = ctypes.c_size_t(0)
    assert L.mla_prefill_workspace_size(ctypes.byref(d), 3, -1, ctypes.byref(sz)) == lib.MLA_ERR_INVALID_ARG
    assert L.mla_prefill_workspace_size(ctypes.byref(d), 3, 1 << 24, ctypes.byref(sz)) == lib.MLA_ERR_UNSUPPORTED
    d_other = lib.dims(16, 192, 64, 512)
    assert L.mla_prefill_workspace_size(ctypes.byref(d_other), 3, 10, ctypes.byref(sz)) == lib.MLA_ERR_UNSUPPORTED
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10008)
    ws = ctypes.c_void_p(0x100000)
    cache = lib.PagedCache(0x10000, None, lib.MLA_BF16, 64, 100, 0x20000, 16, 0x30000)
    pf = L.mla_prefill

    def call(**kw):
        args = dict(dims=ctypes.byref(d), batch=3, qoff=fake, total_q=100, max_q=64, qn=fake, qp=fake, q_dt=1,
                    cache=ctypes.byref(cache), total_kv=1000, wuk=fake, wuv=fake, w_dt=1, scale=0.07, ws=ws,
                    ws_bytes=expect, out=fake, out_dt=1, lse=None)
        args.update(kw)
        return pf(*args.values(), None)

    assert call(ws_bytes=expect - 1) == lib.MLA_ERR_WORKSPACE
    assert call(ws=None) == lib.MLA_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p(0x100010)) == lib.MLA_ERR_ALIGNMENT
    assert call(qoff=None) == lib.MLA_ERR_INVALID_ARG
    assert call(wuv=None) == lib.MLA_ERR_INVALID_ARG
    assert call(scale=0.0) == lib.MLA_ERR_INVALID_ARG
    assert call(total_q=-1) == lib.MLA_ERR_INVALID_ARG
    assert call(q_dt=lib.MLA_F32) == lib.MLA_ERR_UNSUPPORTED
    assert call(out_dt=lib.MLA_F32) == lib.MLA_ERR_UNSUPPORTED
    assert call(out=odd) == lib.MLA_ERR_ALIGNMENT
    c_f32 = lib.PagedCache(0x10000, None, lib.MLA_F32, 64, 100, 0x20000, 16, 0x30000)
    assert call(cache=ctypes.byref(c_f32)) == lib.MLA_ERR_UNSUPPORTED
    c_pg = lib.PagedCache(0x10000, None, lib.MLA_BF16, 32, 100, 0x20000, 16, 0x30000)
    assert call(cache=ctypes.byref(c_pg)) == lib.MLA_ERR_UNSUPPORTED
    c_f8 = lib.PagedCache(0x10000, None, lib.MLA_FP8_E4M3, 64, 100, 0x20000, 16, 0x30000)
    assert call(cache=ctypes.byref(c_f8)) == lib.MLA_ERR_INVALID_ARG
    # nothing to do: no launch, no device access
    assert call(batch=0) == lib.MLA_OK
    assert call(total_q=0) == lib.MLA_OK


def test_multi_decode_workspace_and_validation(lib):
    """mla_decode_multi: the workspace is the decode workspace of the virtual
    batch (virtual lengths are derived from seq_lens in the kernels, and virtual
    sequences read their sequence's block-table row in place); checks fail
    before any device access."""
    L = _raw(lib)
    d = _v2(lib)
    fake = ctypes.c_void_p(0x10000)
    B, q, mp = 8, 3, 10
    nbytes, slots = lib.multi_workspace_size(d, B, q, mp, 64, lib.partition(0, 0))
    assert slots == 0 and nbytes == 0
    dec, dslots = lib.workspace_size(d, B * q, mp, 64, lib.partition(0, 40))
    nbytes, slots = lib.multi_workspace_size(d, B, q, mp, 64, lib.partition(0, 40))
    assert slots == dslots and nbytes == dec > 0
    sz = ctypes.c_size_t(0)
    part = lib.partition(0, 40)
    assert L.mla_decode_multi_workspace_size(ctypes.byref(d), B, 0, mp, 64, ctypes.byref(part), ctypes.byref(sz),
                                             None) == lib.MLA_ERR_INVALID_ARG
    cache = lib.PagedCache(0x10000, None, lib.MLA_BF16, 64, 100, 0x20000, mp, 0x30000)
    need, _ = lib.multi_workspace_size(d, B, q, mp, 64, part)
    dm = L.mla_decode_multi
    # q_len 0, too-small workspace, f32 queries on a bf16 cache, fp8 output, null output
    assert dm(ctypes.byref(d), B, 0, fake, fake, 1, ctypes.byref(cache), 0.07, ctypes.byref(part), fake, need, fake,
              1, None, None) == lib.MLA_ERR_INVALID_ARG
    assert dm(ctypes.byref(d), B, q, fake, fake, 1, ctypes.byref(cache), 0.07, ctypes.byref(part), fake, need - 1,
              fake, 1, None, None) == lib.MLA_ERR_WORKSPACE
    assert dm(ctypes.byref(d), B, q, fake, fake, lib.MLA_F32, ctypes.byref(cache), 0.07, ctypes.byref(part), fake,
              need, fake, 1, None, None) == lib.MLA_ERR_UNSUPPORTED
    assert dm(ctypes.byref(d), B, q, fake, fake, 1, ctypes.byref(cache), 0.07, ctypes.byref(part), fake, need, fake,
              lib.MLA_FP8_E4M3, None, None) == lib.MLA_ERR_UNSUPPORTED
    assert dm(ctypes.byref(d), B, q, fake, fake, 1, ctypes.byref(cache), 0.07, ctypes.byref(part), fake, need, None,
              1, None, None) == lib.MLA_ERR_INVALID_ARG
    assert dm(ctypes.byref(d), 0, q, fake, fake, 1, ctypes.byref(cache), 0.07, ctypes.byref(part), fake, need, fake,
              1, None, None) == lib.MLA_OK


def test_merge_out_proj_validation(lib):
    """mla_merge_out_proj checks the arguments of both calls it replaces before
    anything is enqueued."""
    L = _raw(lib)
    d = _v2(lib)
    fake, odd = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x10008)
    B, mp = 8, 10
    part = lib.partition(0, 40)
    need, _ = lib.workspace_size(d, B, mp, 64, part)
    mo = L.mla_merge_out_proj
    args = lambda **k: dict(dict(batch=B, lens=fake, ws=fake, nb=need, o=fake, odt=1, w=fake, wdt=1, oh=fake,  # noqa: E731
                                 ohdt=1), **k)

    def call(a):
        return mo(ctypes.byref(d), a["batch"], a["lens"], 64, mp, ctypes.byref(part), a["ws"], a["nb"], a["o"],
                  a["odt"], None, a["w"], a["wdt"], a["oh"], a["ohdt"], None)
    assert call(args(lens=None)) == lib.MLA_ERR_INVALID_ARG
    assert call(args(w=None)) == lib.MLA_ERR_INVALID_ARG
    assert call(args(oh=None)) == lib.MLA_ERR_INVALID_ARG
    assert call(args(ohdt=lib.MLA_FP8_E4M3)) == lib.MLA_ERR_UNSUPPORTED
    assert call(args(wdt=7)) == lib.MLA_ERR_INVALID_ARG
    assert call(args(oh=odd)) == lib.MLA_ERR_ALIGNMENT
    assert call(args(nb=need - 1)) == lib.MLA_ERR_WORKSPACE
    assert call(args(batch=0)) == lib.MLA_OK


def test_multi_out_proj_validation(lib):
    """mla_decode_multi_out_proj rejects bad projection arguments before the
    decode is enqueued."""
    L = _raw(lib)
    d = _v2(lib)
    fake, odd = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x10008)
    B, q, mp = 8, 3, 10
    part = lib.partition(0, 0)
    cache = lib.PagedCache(0x10000, None, lib.MLA_BF16, 64, 100, 0x20000, mp, 0x30000)
    need, _ = lib.multi_workspace_size(d, B, q, mp, 64, part)
    f = L.mla_decode_multi_out_proj

    def call(batch=B, w=fake, wdt=1, oh=fake, ohdt=1):
        return f(ctypes.byref(d), batch, q, fake, fake, 1, ctypes.byref(cache), 0.07, ctypes.byref(part), fake, need,
                 fake, 1, None, w, wdt, oh, ohdt, None)
    assert call(w=None) == lib.MLA_ERR_INVALID_ARG
    assert call(oh=None) == lib.MLA_ERR_INVALID_ARG
    assert call(wdt=lib.MLA_FP8_E4M3) == lib.MLA_ERR_UNSUPPORTED
    assert call(oh=odd) == lib.MLA_ERR_ALIGNMENT
    assert call(batch=0) == lib.MLA_OK


SEG_COST = 2   # extra cost units between consecutive non-empty sequences


def _brute_parts(lens, page, W):
    """The cost stream unit by unit: the pages of the non-empty sequences in order,
    SEG_COST units between consecutive ones; C units cut into W' = min(W, P) parts
    [floor(w C / W'), floor((w + 1) C / W')).  -> (first slot, count) per sequence."""
    npg = [(t + page - 1) // page for t in lens]
    P = sum(npg)
    m = sum(1 for n in npg if n > 0)
    C = P + SEG_COST * (m - 1) if m else 0
    Wp = min(W, P)
    owner = []
    for w in range(Wp):
        owner += [w] * ((w + 1) * C // Wp - w * C // Wp)
    assert len(owner) == C
    out, u = [], 0
    for b, n in enumerate(npg):
        if lens[b] == 0:
            out.append((-1, 0))
            continue
        ws = sorted(set(owner[u:u + n]))
        assert ws == list(range(ws[0], ws[-1] + 1))
        out.append((ws[0] + b, len(ws)))
        u += n + SEG_COST
    return out


@pytest.mark.parametrize("seed", range(6))
def test_partition_host_balanced_matches_brute_force(lib, seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    lens = rng.integers(0, 3000, size=B)
    lens[rng.random(B) < 0.2] = 0
    page = 64
    maxp = int(max(1, (lens.max() + page - 1) // page))
    for W in (1, 3, 16, 256, 5000):
        first, count = lib.partition_host(lens, page, maxp, lib.partition(0, W))
        assert list(zip(first.tolist(), count.tolist())) == _brute_parts(lens.tolist(), page, W)


def test_partition_host_balanced_cost_model(lib):
    """One sequence is cut exactly into equal page ranges; between sequences the
    extra units move the cut: two 10-page sequences over 2 parts -> 22 units, 11
    each, so part 0 takes all of sequence 0 (pages 0-9 and one extra unit) and
    part 1 the second sequence (one extra unit and its 10 pages)."""
    first, count = lib.partition_host(np.array([640], dtype=np.int32), 64, 10, lib.partition(0, 10))
    assert (first.tolist(), count.tolist()) == ([0], [10])
    first, count = lib.partition_host(np.array([640, 640], dtype=np.int32), 64, 10, lib.partition(0, 2))
    assert (first.tolist(), count.tolist()) == ([0, 2], [1, 1])
    # 3 parts: the 22 units cut at 7 and 14; sequence 0 (units 0-9) spans parts
    # 0-1, sequence 1 (units 12-21) parts 1-2
    first, count = lib.partition_host(np.array([640, 640], dtype=np.int32), 64, 10, lib.partition(0, 3))
    assert (first.tolist(), count.tolist()) == ([0, 2], [2, 2])


def test_partition_host_fixed_and_whole(lib):
    lens = np.array([0, 1, 4096, 4097, 131072], dtype=np.int32)
    first, count = lib.partition_host(lens, 64, 2048, lib.partition(4096, 0))
    assert count.tolist() == [0, 1, 1, 2, 32]
    assert first.tolist()[1:] == [32, 64, 96, 128]
    first, count = lib.partition_host(lens, 64, 2048, lib.partition(0, 0))
    assert count.tolist() == [0, 1, 1, 1, 1]
    with pytest.raises(lib.MlaError):
        lib.partition_host(np.array([5000], dtype=np.int32), 64, 2, lib.partition(0, 0))


def test_validate_cache_host(lib):
    """Host check of block-table ids and lengths: accepts a consistent cache and
    names the first sequence that breaks a rule."""
    rng = np.random.default_rng(5)
    B, maxp, page, num_pages = 6, 4, 64, 30
    bt = rng.integers(0, num_pages, (B, maxp)).astype(np.int32)
    lens = np.array([0, 1, 64, 65, 255, 256], dtype=np.int32)
    assert lib.validate_cache_host(bt, lens, page, num_pages) == (lib.MLA_OK, -1)
    # entries past a sequence's pages are not read: anything goes there
    bt2 = bt.copy()
    bt2[1, 1:] = -7
    bt2[0, :] = 10 ** 6
    assert lib.validate_cache_host(bt2, lens, page, num_pages) == (lib.MLA_OK, -1)
    # a read entry outside [0, num_pages)
    for bad_id in (-1, num_pages, 2 ** 31 - 1):
        bt3 = bt.copy()
        bt3[3, 1] = bad_id
        assert lib.validate_cache_host(bt3, lens, page, num_pages) == (lib.MLA_ERR_INVALID_ARG, 3)
    # lengths outside [0, max_pages * page]
    for bad_len, b in ((-1, 2), (maxp * page + 1, 4)):
        l2 = lens.copy()
        l2[b] = bad_len
        assert lib.validate_cache_host(bt, l2, page, num_pages) == (lib.MLA_ERR_INVALID_ARG, b)
    # invalid arguments themselves
    assert lib.validate_cache_host(bt, lens, 0, num_pages) == (lib.MLA_ERR_INVALID_ARG, -1)
    assert lib.validate_cache_host(bt, lens, page, 0) == (lib.MLA_ERR_INVALID_ARG, -1)
    assert lib.validate_cache_host(bt[:0], lens[:0], page, num_pages) == (lib.MLA_OK, -1)


def test_noalloc_rejects_before_touching_the_device(lib):
    """mla_decode_noalloc checks the partition's partials against its fixed 48 MiB
    array (and the output dtype) before any device access."""
    import ctypes
    l = lib.load()
    d = _v2(lib)
    fake = ctypes.c_void_p(0x100000)
    cache = lib.PagedCache(fake, None, lib.MLA_BF16, 64, 1000, fake, 40, fake)
    big = lib.partition(0, 4096)     # 4096 + 64 slots of 128 KB bf16 partials
    st = l.mla_decode_noalloc(ctypes.byref(d), 64, fake, fake, lib.MLA_BF16, ctypes.byref(cache),
                              ctypes.c_float(0.07), ctypes.byref(big), fake, lib.MLA_BF16, None, None)
    assert st == lib.MLA_ERR_WORKSPACE
    st = l.mla_decode_noalloc(ctypes.byref(d), 64, fake, fake, lib.MLA_BF16, ctypes.byref(cache),
                              ctypes.c_float(0.07), ctypes.byref(big), fake, lib.MLA_FP8_E4M3, None, None)
    assert st == lib.MLA_ERR_UNSUPPORTED


def test_rope_parameters_validation_and_yarn_factor(lib):
    """mla_rope_t is checked before anything is enqueued; the YaRN attention
    factor matches the oracle's (the page's length factor, squared)."""
    import oracle
    L = _raw(lib)
    d = _v2(lib)
    fake = ctypes.c_void_p(0x10000)
    cache = lib.PagedCache(0x10000, None, lib.MLA_BF16, 64, 100, 0x20000, 16, 0x30000)
    cs = L.mla_cache_store_rope
    ok = lib.rope(10000.0, 40.0, 1.0, 32.0, 4096)
    assert cs(ctypes.byref(d), 0, fake, lib.MLA_F32, fake, ctypes.byref(ok), ctypes.byref(cache), None) == lib.MLA_OK
    for bad in (lib.rope(-1.0), lib.rope(1e4, 0.5), lib.rope(1e4, 40.0, 32.0, 1.0, 4096),
                lib.rope(1e4, 40.0, 1.0, 32.0, 0), lib.rope(float("nan")), lib.rope(1e4, float("inf"), 1.0, 32.0, 4096)):
        assert cs(ctypes.byref(d), 1, fake, lib.MLA_F32, fake, ctypes.byref(bad), ctypes.byref(cache),
                  None) == lib.MLA_ERR_INVALID_ARG
    assert cs(ctypes.byref(d), 1, fake, lib.MLA_F32, fake, None, ctypes.byref(cache), None) == lib.MLA_ERR_INVALID_ARG
    qp = L.mla_query_prep_rope
    need = L.mla_query_prep_scratch_size(ctypes.byref(d), 1536, 4)
    bad = lib.rope(1e4, 40.0, 5.0, 5.0, 4096)
    assert qp(ctypes.byref(d), 5120, 1536, 4, fake, 1, fake, fake, fake, 1, fake, ctypes.byref(bad), fake, fake, 1,
              fake, need, None) == lib.MLA_ERR_INVALID_ARG
    for s in (1.0, 2.0, 40.0, 100.0):
        assert abs(lib.yarn_attention_factor(s) - oracle.yarn_attention_factor(s)) <= 1e-6
