"""mla_decode_noalloc (no caller workspace; split partials in the library's own
device array) against mla_decode + mla_merge_splits with a caller workspace,
through the C ABI: two calls in a row, the second with a smaller input.  The
two routes run the same kernels on the same partition, so their outputs must
be identical bit for bit; each call is also checked against the oracle to the
bf16 bar (per-sequence vectors, derived lse bound)."""
import math

import numpy as np
import pytest

from _cases import TOL, Worst, compare_seq, direct_case, host, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_37_amd as mk
    mk._lib.load()


def _both_routes(case, part):
    import torch
    import mla_latent_kv_37_amd as mk
    dev = to_device(case)
    d = case.dims
    B, maxp = len(case.lens), case.cache.block_table.shape[1]
    step = mk.DecodeStep(d.n_heads, d.d_head, d.d_rope, d.d_latent, B, maxp, 64, *part, act_dtype=dev["dtype"])
    step.absorb(dev["q_nope"], dev["W_UK"])
    cache = dev["cache"]
    p = mk.partition(*part)
    # the existing entry points with a caller workspace
    mk.decode(step.d, step.q_lat, dev["q_pe"], cache.desc, case.scale, p, step.workspace, step.o_lat, step.lse)
    mk.merge_splits(step.d, cache.seq_lens, 64, maxp, p, step.workspace, step.o_lat, step.lse)
    # the no-allocation entry point into fresh NaN-filled outputs
    o2 = torch.full_like(step.o_lat, float("nan"))
    l2 = torch.full_like(step.lse, float("nan"))
    mk.decode_noalloc(step.d, step.q_lat, dev["q_pe"], cache.desc, case.scale, p, o2, l2)
    torch.cuda.synchronize()
    return host(step.q_lat), host(step.o_lat), host(step.lse), host(o2), host(l2)


def _check(case, part):
    q_lat, o_ref, l_ref, o_na, l_na = _both_routes(case, part)
    same_o = np.array_equal(o_na, o_ref, equal_nan=False)
    same_l = np.array_equal(l_na, l_ref) or np.array_equal(np.nan_to_num(l_na, neginf=-1e30),
                                                             np.nan_to_num(l_ref, neginf=-1e30))
    print(f"  B={len(case.lens)} part={part}: o_lat identical {same_o}, lse identical {same_l}", flush=True)
    assert same_o and same_l, "mla_decode_noalloc differs from mla_decode + mla_merge_splits"
    worst = Worst()
    for b, T in enumerate(case.lens):
        if T == 0:
            assert np.all(o_na[b] == 0) and np.all(np.isneginf(l_na[b]))
            continue
        r = case.reference(b)
        compare_seq(case, b, r, {"q_lat": q_lat[b], "o_lat": o_na[b], "lse": l_na[b]}, TOL["bf16"], None, worst)
    worst.report(TOL["bf16"])


def test_noalloc_two_calls_second_smaller():
    big = direct_case(3, [1000, 0, 2100, 65, 1, 777, 3000, 129], max_pages=48, seed=11)
    small = direct_case(3, [300, 64, 0, 31], max_pages=6, seed=12)
    print("case: no-alloc decode, balanced partition over the CUs, then a smaller batch", flush=True)
    _check(big, (0, -1))
    _check(small, (0, -1))


def test_noalloc_fixed_splits_then_whole():
    big = direct_case(4, [4096, 2048, 1], max_pages=64, seed=13)
    small = direct_case(4, [200, 33], max_pages=4, seed=14)
    print("case: no-alloc decode, 256-token splits, then one work item per sequence", flush=True)
    _check(big, (256, 0))
    _check(small, (0, 0))


def test_noalloc_rejects_oversized_partition():
    import torch
    import mla_latent_kv_37_amd as mk
    from mla_latent_kv_37_amd import _lib
    case = direct_case(3, [64, 64], max_pages=1, seed=15)
    dev = to_device(case)
    step = mk.DecodeStep(128, 128, 64, 512, 2, 1, 64, 0, 4096)
    step.absorb(dev["q_nope"], dev["W_UK"])
    # 4096 parts of 2 sequences: 4098 slots x 128 KB of bf16 partials > 48 MiB
    with pytest.raises(_lib.MlaError) as e:
        mk.decode_noalloc(step.d, step.q_lat, dev["q_pe"], dev["cache"].desc, case.scale, mk.partition(0, 4096),
                          step.o_lat, step.lse)
    assert e.value.status == _lib.MLA_ERR_WORKSPACE
    torch.cuda.synchronize()
