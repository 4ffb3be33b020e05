#!/usr/bin/env python3
"""MLA decode benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ragged|long|fp8|v2b1]
    python bench.py --workload append_bf16|append_fp8     (cache append step, reported apart)
    python bench.py --workload prefill_b4_t4096|prefill_b1_t16384|prefill_chunk_b4_t8192_q1024
                                                          (non-absorbed prefill, reported apart)

A step is one full MLA decode step over the batch: mla_absorb_q -> mla_decode ->
mla_merge_splits -> mla_out_proj, every input already resident in HBM.  The
default workload is the ragged batch (B=64, cache lengths uniform in
[1024, 8192], DeepSeek-V2 shapes, bf16 paged cache, pages in random order).
Inputs are rotated over --copies full copies so that successive steps do not
find their cache in the 256 MB Infinity Cache, and W^UK / W^UV over at least
512 MB of copies, so that every step reads its weights from HBM as a layer of a
many-layer model does (--warm-weights reuses them).

Prints one JSON line with the contract fields plus `roofline` (the decode
kernel's algorithmic bytes per launch / its mean launch time, HIP events on the
launch stream) and `cpu_baseline` (the float64 oracle on a bounded sample).

Helper modes for the rocprofv3 summaries kept in profiles/:
    python bench.py --summarize-stats DIR OUT.md      (kernel-trace --stats)
    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR COPY_BYTES OUT.json OUT.md [--workload W]
    python bench.py --summarize-counters DIR OUT.md                (--pmc MfmaUtil ... OccupancyPercent)
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode KV-tokens/s + achieved TB/s & % roofline, 128 heads, d_c=512"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix
N_H, D_H, D_R, D_C = 128, 128, 64, 512
ROW_BYTES_BF16 = (D_C + D_R) * 2
CSRC = os.path.join(ROOT, "mla_latent_kv_37_amd", "csrc")
# the decode kernel of each workload: (source file, name fragment in rocprofv3 output)
DECODE_KERNEL = {"lite": ("decode_lite.hip", "decode_lite")}
DEFAULT_DECODE_KERNEL = ("decode_wide.hip", "decode_wide")   # bf16 and fp8 caches at 128 heads


def traffic_json(workload: str) -> str:
    """Measured HBM traffic of a workload's decode kernel (written by --summarize-pmc)."""
    return os.path.join(ROOT, "profiles", f"decode_traffic_{workload}.json")

WORKLOADS = {
    # name: (synth config id, description, partition (split_tokens, num_parts))
    "ragged": (3, "v2_bf16_ragged_b64_t1024-8192", (0, -1)),
    # one work item per compute unit (64 per sequence); the fixed 4096-token
    # split of the parity cases gives 128 items, half the compute units
    # (--partition 4096 0)
    "long": (4, "v2_bf16_long_b4_t131072", (0, -1)),
    "fp8": (5, "v2_fp8_b32_t16384", (0, -1)),
    "v2b1": (2, "v2_bf16_b1_t4096", (0, -1)),
    # the ragged batch with two new query tokens per sequence (causal within them)
    "mtp2": (3, "v2_bf16_ragged_b64_t1024-8192_qlen2", (0, -1)),
    # the ragged batch at DeepSeek-V2-Lite's 16 heads (same cache row)
    "lite": (6, "v2lite_bf16_ragged_b64_t1024-8192", (0, -1)),
}
Q_LEN = {"mtp2": 2}


def decode_source_hash(workload: str = "ragged") -> str:
    """Hash of the decode kernel's source and the headers it includes (a measured
    traffic record is only reported for the code it was measured on)."""
    src = DECODE_KERNEL.get(workload, DEFAULT_DECODE_KERNEL)[0]
    h = hashlib.sha256()
    for f in (src, "kernels.h", "mla_common.h", "partition.h", "decode_tile.h"):
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# algorithmic bytes / flops (what the method must move / compute)
# ---------------------------------------------------------------------------

def algorithmic(lens, cache_dtype: str, q_len: int = 1, n_h: int = N_H):
    """Bytes and flops of one decode step and of the decode kernel alone.

    Per cached token: the row [c^KV | k^R] (1152 B bf16; 576 B + 5 fp32 scales
    for fp8) and 2*n_h*(d_c+d_r) + 2*n_h*d_c flops.  Per query: q^C, q^R in,
    q_lat/o_lat intermediates excluded, o_heads out; weights W^UK, W^UV once.
    The decode kernel alone: cache rows + its inputs q_lat, q_pe + its output
    o_lat (bf16) and lse; block table and lengths.
    """
    B = len(lens)
    T = sum(lens)
    pages = sum((t + 63) // 64 for t in lens)
    row = ROW_BYTES_BF16 if cache_dtype == "bf16" else (D_C + D_R) + 4 * 5
    cache = T * row
    meta = pages * 4 + B * 4
    Q = B * q_len                      # query tokens: each reads its inputs, writes its outputs
    q_in = Q * n_h * (D_H + D_R) * 2
    weights = 2 * n_h * D_H * D_C * 2
    out = Q * n_h * D_H * 2
    flops_tok = 2 * n_h * (D_C + D_R) + 2 * n_h * D_C
    # new token t of a sequence of T_b tokens attends to T_b - q_len + t + 1 of them
    attended = sum(max(t - q_len + k + 1, 0) for t in lens for k in range(q_len))
    step_flops = attended * flops_tok + 2 * 2 * Q * n_h * D_H * D_C
    decode_bytes = cache + meta + Q * n_h * (D_C + D_R) * 2 + Q * n_h * (D_C * 2 + 4)
    return {
        "step_bytes": cache + meta + q_in + weights + out,
        "step_flops": step_flops,
        "decode_bytes": decode_bytes,
        "decode_flops": attended * flops_tok,
        "cache_bytes": cache,
        "attended_tokens": attended,
    }


# ---------------------------------------------------------------------------
# inputs
# ---------------------------------------------------------------------------

def make_inputs(config_id: int, copies: int, device="cuda", q_len: int = 1):
    import numpy as np
    import torch
    import synth
    import mla_latent_kv_37_amd as mk
    inp = synth.direct_inputs_for(config_id)
    w = inp["workload"]
    lens = inp["lens"]
    words, scales = [], []
    for r in inp["rows"]:
        wd, sc = synth.store_rows(r, w.cache_dtype)
        words.append(wd)
        scales.append(sc)
    del inp["rows"]
    maxp = max((t + 63) // 64 for t in lens)
    if q_len > 1:
        # q_len queries per sequence ([B, q_len, ...] flattened), the first one the workload's own
        rq = synth.rng_for(config_id, synth.S_QUERY + 50)
        B = len(lens)
        extra = lambda x: rq.normal(0.0, synth.V2_SD_QUERY, size=(B, q_len - 1) + x.shape[1:])  # noqa: E731
        inp["q_nope"] = np.concatenate([inp["q_nope"][:, None], extra(inp["q_nope"])], axis=1).reshape(
            (B * q_len,) + inp["q_nope"].shape[1:])
        inp["q_pe"] = np.concatenate([inp["q_pe"][:, None], extra(inp["q_pe"])], axis=1).reshape(
            (B * q_len,) + inp["q_pe"].shape[1:])
    sets = []
    for c in range(copies):
        cache = synth.build_paged(words, w.cache_dtype, synth.rng_for(config_id, synth.S_PERM + 10 * c),
                                  scales_per_seq=scales if w.cache_dtype == "fp8" else None, spare_pages=0,
                                  max_pages=maxp)
        dc = mk.upload_cache(cache.kv, cache.block_table, cache.seq_lens, w.cache_dtype, 64, cache.scales, device)
        del cache

        def t(x):
            return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device).to(torch.bfloat16)

        sets.append(dict(cache=dc, q_nope=t(inp["q_nope"]), q_pe=t(inp["q_pe"]), W_UK=t(inp["W_UK"]),
                         W_UV=t(inp["W_UV"])))
    return w, lens, sets


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def host_cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo ("unknown" where it is not readable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(config_id: int, budget_s: float = 15.0):
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 0) for p in threadpool_info()), default=0)
    except Exception:
        threads = 0
    cores = threads or len(os.sched_getaffinity(0))
    w = synth.workload(config_id)
    tokens = 0
    elapsed = 0.0
    nseq = 0
    for b in range(len(w.lens)):
        inp = synth.direct_inputs_for(config_id, lens=[w.lens[b]])
        rows = inp["rows"][0]
        if w.cache_dtype == "bf16":
            from oracle.storage import bf16_bits_to_f64
            rows = bf16_bits_to_f64(synth.to_bf16_bits(rows))
        else:
            rows = rows.astype(np.float64)
        t0 = time.perf_counter()
        oracle.attend(inp["q_nope"][0], inp["q_pe"][0], rows[:, :D_C], rows[:, D_C:], inp["W_UK"], inp["W_UV"])
        elapsed += time.perf_counter() - t0
        tokens += w.lens[b]
        nseq += 1
        if elapsed >= budget_s:
            break
    return {"value": tokens / elapsed, "unit": "KV-tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": host_cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"oracle.attend (float64, non-absorbed, all {w.dims.n_heads} heads) on the first {nseq} sequences "
                      f"({tokens} cached tokens) of the same workload; {elapsed:.1f} s"}


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def binding_roof(flops: float, nbytes: float):
    """The roof that binds a kernel of `flops` and `nbytes` algorithmic work: the
    larger of its HBM time (8 TB/s) and its bf16 MFMA time (2.5 PFLOP/s)."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    return ("hbm", t_hbm) if t_hbm >= t_mfma else ("mfma", t_mfma)


def run(args, workload=None, partition=None, cpu=True, copy_tbps=None):
    import torch
    import mla_latent_kv_37_amd as mk
    workload = workload or args.workload
    partition = partition if partition is not None else args.partition
    cid, wname, (split, parts) = WORKLOADS[workload]
    if partition is not None:
        split, parts = partition
        wname += f"_part{split}x{parts}"
    q_len = Q_LEN.get(workload, 1)
    torch.cuda.set_device(0)
    mk._lib.load()
    w, lens, sets = make_inputs(cid, args.copies, q_len=q_len)
    maxp = sets[0]["cache"].max_pages
    B = len(lens)
    n_h = w.dims.n_heads
    step = mk.DecodeStep(n_h, D_H, D_R, D_C, B * q_len, maxp, 64, split, parts)
    scale = 1.0 / math.sqrt(D_H + D_R)
    stream = torch.cuda.current_stream()
    if q_len > 1:
        nbytes, _ = mk.multi_workspace_size(step.d, B, q_len, maxp, 64, step.part)
        multi_ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        q_lat_m = step.q_lat.view(B, q_len, N_H, D_C)
        o_lat_m = step.o_lat.view(B, q_len, N_H, D_C)
        lse_m = step.lse.view(B, q_len, N_H)

    # Weight copies rotated apart from the cache copies.  A layer's W^UK and W^UV
    # were last read a whole forward pass earlier in a many-layer model, so by
    # default every step reads its weights from HBM: the rotation holds at least
    # 512 MB of weight copies (twice the 256 MB Infinity Cache).  --warm-weights
    # reuses each input set's own weights instead.
    if args.warm_weights:
        wsets = [(st["W_UK"], st["W_UV"]) for st in sets]
    else:
        per_copy = sets[0]["W_UK"].numel() * 2 + sets[0]["W_UV"].numel() * 2
        n_w = max(len(sets), -(-(512 << 20) // per_copy))
        wsets = [(st["W_UK"], st["W_UV"]) for st in sets]
        while len(wsets) < n_w:
            wsets.append((sets[0]["W_UK"].clone(), sets[0]["W_UV"].clone()))
    weight_rotation_mb = len(wsets) * (sets[0]["W_UK"].numel() + sets[0]["W_UV"].numel()) * 2 / 2**20

    def one(i, ev=None):
        s = sets[i % len(sets)]
        w_uk, w_uv = wsets[i % len(wsets)]
        s = dict(s, W_UK=w_uk, W_UV=w_uv)
        if ev is not None:
            ev[0].record(stream)
        step.absorb(s["q_nope"], s["W_UK"])
        if ev is not None:
            ev[1].record(stream)
        if q_len > 1:
            if args.unfused:
                # decode + merge in one call, then the projection
                mk.decode_multi(step.d, q_lat_m, s["q_pe"].view(B, q_len, N_H, D_R), s["cache"].desc, scale,
                                step.part, multi_ws, o_lat_m, lse_m)
                if ev is not None:
                    ev[2].record(stream)
                step.project(s["W_UV"])
            else:
                # decode, then merge + projection in one launch
                mk.decode_multi_out_proj(step.d, q_lat_m, s["q_pe"].view(B, q_len, N_H, D_R), s["cache"].desc, scale,
                                         step.part, multi_ws, o_lat_m, s["W_UV"], step.o_heads, lse_m)
                if ev is not None:
                    ev[2].record(stream)
            if ev is not None:
                ev[3].record(stream)
        else:
            mk.decode(step.d, step.q_lat, s["q_pe"], s["cache"].desc, scale, step.part, step.workspace, step.o_lat,
                      step.lse)
            if ev is not None:
                ev[2].record(stream)
            if args.unfused:
                mk.merge_splits(step.d, s["cache"].seq_lens, 64, maxp, step.part, step.workspace, step.o_lat, step.lse)
                step.project(s["W_UV"])
            else:
                # split merge + W^UV projection, one launch
                mk.merge_out_proj(step.d, s["cache"].seq_lens, 64, maxp, step.part, step.workspace, step.o_lat,
                                  s["W_UV"], step.o_heads, step.lse)
            if ev is not None:
                ev[3].record(stream)
        if ev is not None:
            ev[4].record(stream)

    # Settle: back-to-back steps for args.settle seconds before the warm-up
    # steps.  The GPU's clocks ramp up over the first few hundred steps after
    # idle (the same step takes ~157 us after 10 steps and ~128 us from ~1000
    # on), and the first pass over the rotated weight copies pays first-touch
    # TLB misses; a decode server runs in the settled state.  Untimed and
    # reported as settle_steps.
    settle_steps = 0
    if args.settle > 0:
        t_end = time.perf_counter() + args.settle
        while time.perf_counter() < t_end:
            for _ in range(25):
                one(settle_steps)
                settle_steps += 1
            torch.cuda.synchronize()
    for i in range(args.warmup):
        one(i)
    torch.cuda.synchronize()
    # timed region: exactly K steps, nothing else on the stream between them
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        one(args.warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    per_kernel = None
    if args.kernel_events:
        # second timed region, same K steps with an event between every two
        # kernels on the launch stream: per-kernel times for the roofline.  The
        # event packets lengthen the step (so this region does not give the
        # headline), and each kernel's time includes its dispatch gap.
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            one(args.warmup + args.steps + i, evs[i])
        torch.cuda.synchronize()
        step_evs = sorted(e[0].elapsed_time(e[4]) for e in evs)
        if q_len > 1:
            names = (["absorb", "decode_multi", "out_proj", "-"] if args.unfused else
                     ["absorb", "decode_multi_out_proj", "-", "-"])
        else:
            names = ["absorb", "decode", "merge + out_proj" if args.unfused else "merge_out_proj", "-"]
        per_kernel = {n: sum(e[k].elapsed_time(e[k + 1]) for e in evs) / args.steps for k, n in enumerate(names)
                      if n != "-"}
        per_kernel_step_ms = sum(e[0].elapsed_time(e[4]) for e in evs) / args.steps
    # warm: the same input copy every step (its cache partly stays in the 256 MB
    # Infinity Cache between steps), K steps, timed like the headline region
    torch.cuda.synchronize()
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for i in range(args.steps):
        one(0)
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / args.steps
    if copy_tbps is None:
        copy_tbps = measured_copy_tbps()
    alg = algorithmic(lens, w.cache_dtype, q_len, n_h)
    T = sum(lens)
    value = T * args.steps / (total_ms * 1e-3)
    metric, unit = METRIC, "KV-tokens/s"
    if n_h != N_H:
        metric = f"MLA decode KV-tokens/s + achieved TB/s & % roofline, {n_h} heads (V2-Lite), d_c=512"
    if q_len > 1:
        metric = f"MLA multi-token decode query-tokens/s ({q_len} new tokens per sequence, causal)"
        unit = "query-tokens/s"
        value = B * q_len * args.steps / (total_ms * 1e-3)
    res = {
        "metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_steps": settle_steps, "settle_s": args.settle,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wname, "batch": len(lens), "sum_cache_tokens": T, "cache_dtype": w.cache_dtype,
                   "heads": n_h, "d_latent": D_C, "d_rope": D_R, "page_size": 64,
                   "partition": {"split_tokens": split, "num_parts": parts}, "input_copies": args.copies,
                   "weights": ("warm: each input set's own W^UK / W^UV" if args.warm_weights else
                               f"cold: {len(wsets)} copies of W^UK / W^UV rotated ({weight_rotation_mb:.0f} MB)"),
                   "parallelism": "single GPU", "q_len": q_len},
    }
    step_s = ms_per_step * 1e-3
    res["query_tokens_per_s"] = B * q_len / step_s
    res["cache_tokens_per_s"] = T / step_s
    if q_len > 1:
        res["attended_kv_tokens_per_s"] = alg["attended_tokens"] / step_s
    res["step_TBps"] = alg["step_bytes"] / step_s / 1e12
    res["step_TFLOPs"] = alg["step_flops"] / step_s / 1e12
    step_bound, step_roof_s = binding_roof(alg["step_flops"], alg["step_bytes"])
    res["step_roofline"] = {
        "hbm_us": alg["step_bytes"] / (HBM_PEAK_GBS * 1e9) * 1e6,
        "mfma_us": alg["step_flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e6,
        "bound": step_bound,
        # the step's time at the binding roof over its measured time
        "frac_of_min_roof": step_roof_s / step_s,
    }
    res["warm_ms_per_step"] = warm_ms
    res["measured_copy_TBps"] = copy_tbps
    if per_kernel:
        res["kernel_ms"] = per_kernel
        res["kernel_events_step_ms"] = per_kernel_step_ms
        n = len(step_evs)
        res["kernel_events_step_ms_p10_p50_p90"] = [step_evs[n // 10], step_evs[n // 2], step_evs[(9 * n) // 10]]
        dec_name = ("decode_multi" if args.unfused else "decode_multi_out_proj") if q_len > 1 else "decode"
        dec_s = per_kernel[dec_name] * 1e-3
        ach = alg["decode_bytes"] / dec_s / 1e9
        traffic = None
        if os.path.exists(traffic_json(workload)):
            tj = json.load(open(traffic_json(workload)))
            if tj.get("decode_source_sha") == decode_source_hash(workload) and tj.get("workload") == wname:
                traffic = tj.get("decode_bytes_per_launch")
        res["decode_frac_of_measured_copy"] = ach / (copy_tbps * 1e3)
        # the decode kernel against its binding roof: HBM for the bf16 cache at one
        # query token (242 flop/B, under the 312 flop/B ridge); bf16 MFMA for the
        # fp8 cache (467 flop/B) and for several new tokens per sequence
        bound, _ = binding_roof(alg["decode_flops"], alg["decode_bytes"])
        if bound == "hbm":
            r_ach, r_peak, r_unit = ach, HBM_PEAK_GBS, "GB/s"
        else:
            r_ach, r_peak, r_unit = alg["decode_flops"] / dec_s / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
        res["roofline"] = {"bound": bound, "achieved": r_ach, "peak": r_peak, "unit": r_unit,
                           "frac": r_ach / r_peak, "traffic": traffic,
                           "hbm_GBps": ach, "hbm_frac": ach / HBM_PEAK_GBS,
                           "kernel": ("decode_wide_kernel<true> (fp8 cache, one wavefront per SIMD)" if cid == 5 else
                                      "decode_lite_kernel (16 heads, bf16 cache)" if n_h == 16 else
                                      "decode_wide_kernel<false> (bf16 cache, one wavefront per SIMD)") +
                                     ((" + merge_kernel (mla_decode_multi)" if args.unfused else
                                       " + merge_proj_kernel (mla_decode_multi_out_proj; the "
                                       "time includes the W^UV projection)") if q_len > 1 else ""),
                           "algorithmic_bytes_per_launch": alg["decode_bytes"],
                           "algorithmic_flops_per_launch": alg["decode_flops"],
                           "mean_launch_ms": per_kernel[dec_name],
                           "mfma_frac": alg["decode_flops"] / dec_s / (MFMA_BF16_PEAK_TFLOPS * 1e12)}
    res["wall_s_timed"] = wall
    if cpu and not args.no_cpu_baseline and q_len == 1:
        res["cpu_baseline"] = cpu_baseline(cid, args.cpu_budget)
    del sets, wsets
    torch.cuda.empty_cache()
    return res


# the other workloads that the default run times as well (sub-objects of the one
# JSON line): (name, workload, partition override)
EXTRA_WORKLOADS = (
    ("v2_bf16_b1_t4096", "v2b1", None),
    ("v2_bf16_long_b4_t131072", "long", None),
    ("v2_bf16_long_b4_t131072_split4096", "long", (4096, 0)),
    ("v2_fp8_b32_t16384", "fp8", None),
)


def summary(r):
    """The per-workload figures kept in the headline line's `other_workloads`."""
    out = {k: r[k] for k in ("value", "unit", "ms_per_step", "query_tokens_per_s", "cache_tokens_per_s",
                             "step_TBps", "step_TFLOPs", "step_roofline", "warm_ms_per_step", "steps", "warmup",
                             "settle_steps") if k in r}
    out["config"] = {k: r["config"][k] for k in ("workload", "batch", "sum_cache_tokens", "cache_dtype",
                                                 "partition")}
    if "roofline" in r:
        out["roofline"] = {k: r["roofline"][k] for k in ("bound", "achieved", "peak", "unit", "frac", "hbm_GBps",
                                                         "mean_launch_ms", "kernel")}
    if "kernel_ms" in r:
        out["kernel_ms"] = r["kernel_ms"]
    return out


# ---------------------------------------------------------------------------
# rocprofv3 summaries
# ---------------------------------------------------------------------------

def _db(d):
    hits = sorted(glob.glob(os.path.join(d, "**", "*results.db"), recursive=True))
    if not hits:
        raise SystemExit(f"no rocprofv3 results database under {d}")
    import sqlite3
    return sqlite3.connect(hits[-1])


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").split("(")[0]
    for pre in ("void ", "mla::"):
        name = name.replace(pre, "")
    return name[:60]


def summarize_stats(d, out_md, cmd=""):
    """Per-kernel call count and duration from a `rocprofv3 --kernel-trace --stats` run."""
    con = _db(d)
    rows = list(con.execute("select name, total_calls, total_duration, average, percentage from top_kernels"))
    mins = {}
    for name, lo, hi in con.execute("select name, min(duration), max(duration) from kernels "
                                    "group by name"):
        mins[name] = (lo, hi)
    lines = ["# Kernel time summary (rocprofv3 --kernel-trace --stats)", "", f"Command: `{cmd}`", "",
             "| kernel | calls | total us | mean us | min us | max us | % |", "|---|---|---|---|---|---|---|"]
    for name, calls, tot, avg, pct in rows:
        lo, hi = mins.get(name, (0, 0))
        lines.append(f"| {_short(name)} | {calls} | {tot:.1f} | {avg:.2f} | {lo / 1e3:.2f} | {hi / 1e3:.2f} | "
                     f"{pct:.1f} |")
    # steady state: the last half of each kernel's calls (the GPU's clocks ramp up
    # over the first few hundred steps), and the idle time before each dispatch
    disp = list(con.execute("select name, start, end, duration from kernels order by start"))
    per, gaps = {}, {}
    prev_end = None
    for name, st, en, dur in disp:
        per.setdefault(name, []).append(dur)
        if prev_end is not None:
            gaps.setdefault(name, []).append(st - prev_end)
        prev_end = en
    lines += ["", "Steady state (last half of each kernel's calls; gap = idle time between the previous "
              "dispatch's end and this one's start):", "",
              "| kernel | calls used | mean us | median us | median gap before us |", "|---|---|---|---|---|"]
    for name, _, _, _, _ in rows:
        d = per.get(name, [])
        if not d:
            continue
        tail = sorted(d[len(d) // 2:])
        g = sorted(gaps.get(name, [0])[len(gaps.get(name, [0])) // 2:])
        lines.append(f"| {_short(name)} | {len(tail)} | {sum(tail) / len(tail) / 1e3:.2f} | "
                     f"{tail[len(tail) // 2] / 1e3:.2f} | {g[len(g) // 2] / 1e3:.2f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _pmc_per_kernel(d, counter):
    con = _db(d)
    vals = {}
    for name, v in con.execute("select kernel_name, value from counters_collection where counter_name = ?",
                               (counter,)):
        vals.setdefault(_short(name), []).append(float(v))
    return vals


COUNTER_METRICS = ("MfmaUtil", "MfmaFlopsBF16", "VALUBusy", "LdsUtil", "LDSBankConflict", "OccupancyPercent")


def summarize_counters(d, out_md, cmd="", workload="ragged"):
    """Median per dispatch of rocprofv3's derived metrics for each kernel of one
    `rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 VALUBusy LdsUtil LDSBankConflict
    OccupancyPercent` run: MFMA busy %, bf16 MFMA flops, VALU busy %, LDS busy %,
    LDS bank-conflict stall % and occupancy % (each over the GPU-active cycles)."""
    import statistics
    con = _db(d)
    vals = {}
    for name, cnt, v in con.execute("select kernel_name, counter_name, value from counters_collection"):
        vals.setdefault(_short(name), {}).setdefault(cnt, []).append(float(v))
    lines = ["# Per-kernel counters (rocprofv3 derived metrics, median per dispatch)", "", f"Command: `{cmd}`", "",
             "MfmaUtil = MFMA busy cycles / (SIMDs x GPU-active cycles); LdsUtil = LDS indexed-op cycles / "
             "(CUs x active cycles); LDSBankConflict = bank-conflict stall cycles / (CUs x active cycles); "
             "OccupancyPercent = resident waves / maximum; VALUBusy = VALU instruction cycles / (CUs x active "
             "cycles); MfmaFlopsBF16 = bf16 MFMA flops per dispatch.", "",
             "| kernel | dispatches | " + " | ".join(COUNTER_METRICS) + " |",
             "|---|---|" + "---|" * len(COUNTER_METRICS)]
    for k in sorted(vals, key=lambda k: -len(vals[k].get(COUNTER_METRICS[0], []))):
        row = vals[k]
        n = max(len(v) for v in row.values())
        cells = []
        for m in COUNTER_METRICS:
            x = row.get(m)
            cells.append("—" if not x else (f"{statistics.median(x):.3g}" if m == "MfmaFlopsBF16" else
                                            f"{statistics.median(x):.1f}"))
        lines.append(f"| {k} | {n} | " + " | ".join(cells) + " |")
    open(out_md, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_pmc(fetch_dir, write_dir, copy_bytes, out_json, out_md, cmd="", workload="ragged"):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of a workload's decode kernel,
    scaled by what the same counters read for a plain device copy of known size."""
    import statistics
    copy_bytes = int(copy_bytes)
    fetch = _pmc_per_kernel(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_kernel(write_dir, "WRITE_SIZE")
    print("kernels seen:", sorted(fetch))

    def pick(vals, key):
        ks = [k for k in vals if key in k]
        return ks[0] if ks else None

    # the calibration copy is the largest dispatch of the runtime copy kernel
    f_copy = max(fetch[pick(fetch, "copyBuffer")]) * 1024 / copy_bytes
    w_copy = max(write[pick(write, "copyBuffer")]) * 1024 / copy_bytes
    src, key = DECODE_KERNEL.get(workload, DEFAULT_DECODE_KERNEL)
    f_dec = statistics.median(fetch[pick(fetch, key)]) * 1024 / f_copy
    w_dec = statistics.median(write[pick(write, key)]) * 1024 / w_copy
    others = {}
    for k in ("merge_kernel", "merge_proj", "absorb_v2", "outproj_v2"):
        kf, kw = pick(fetch, k), pick(write, k)
        if kf and kw:
            others[k] = {"fetch_bytes": statistics.median(fetch[kf]) * 1024 / f_copy,
                         "write_bytes": statistics.median(write[kw]) * 1024 / w_copy}
    res = {"workload": WORKLOADS[workload][1], "decode_source_sha": decode_source_hash(workload),
           "copy_bytes": copy_bytes, "fetch_factor": f_copy, "write_factor": w_copy,
           "decode_fetch_bytes": f_dec, "decode_write_bytes": w_dec, "decode_bytes_per_launch": f_dec + w_dec,
           "other_kernels": others, "command": cmd}
    json.dump(res, open(out_json, "w"), indent=2)
    lines = ["# HBM traffic per dispatch (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)", "",
             f"Commands: `{cmd}`", "",
             f"- calibration: the runtime's device copy of {copy_bytes} B; FETCH_SIZE reads "
             f"{f_copy:.4f} KiB per KiB copied and WRITE_SIZE {w_copy:.4f}; all figures below are divided by "
             "these factors",
             f"- decode kernel ({pick(fetch, key)}, {src}; source sha256[:16] {res['decode_source_sha']}): "
             f"fetched {f_dec / 1e6:.2f} MB, written {w_dec / 1e6:.2f} MB, total {(f_dec + w_dec) / 1e6:.2f} MB "
             "per launch"]
    for k, v in others.items():
        lines.append(f"- {k}: fetched {v['fetch_bytes'] / 1e6:.2f} MB, written {v['write_bytes'] / 1e6:.2f} MB")
    open(out_md, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def measured_copy_tbps(nbytes: int = 1 << 30, reps: int = 5) -> float:
    """HBM bandwidth of a plain device-to-device copy (the runtime's copy kernel) in
    the same job: bytes read + written per second, best of `reps`, in TB/s."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del src, dst
    return 2 * nbytes / (best * 1e-3) / 1e12


def copy_calibration(nbytes: int, reps: int = 3):
    """A plain device-to-device copy of known size (the runtime's copy kernel) whose
    counter readings scale the decode kernel's HBM counters."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").normal_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# cache append (project [W^DKV; W^KR] h, rotate, round, scatter): one new token
# per sequence of the ragged batch, written at position T_b
# ---------------------------------------------------------------------------

APPEND_WORKLOADS = {"append_bf16": "bf16", "append_fp8": "fp8"}
# prefill: (batch, cached tokens per sequence, new tokens per sequence, cache dtype)
PREFILL_WORKLOADS = {
    "prefill_b4_t4096": (4, 4096, 4096, "bf16"),
    "prefill_b1_t16384": (1, 16384, 16384, "bf16"),
    "prefill_chunk_b4_t8192_q1024": (4, 8192, 1024, "bf16"),
    "prefill_fp8_b4_t4096": (4, 4096, 4096, "fp8"),
}
QUERY_WORKLOADS = ("query_prep", "query_lat", "query_lat_fused", "query_lite")
D_MODEL = 5120
D_QLATENT = 1536


def _cold_weight_steps(fn, args):
    """Per-step durations (ms, sorted) of fn on the current stream, HIP events around
    each call.  A 512 MB buffer is read (summed) between steps: that pushes the
    weights out of the 256 MB Infinity Cache, so every step streams them from
    HBM, and leaves no dirty lines behind (a 256 MB copy did, and the timed step
    then paid for their write-back: 8-12% on the query side), as the other
    layers' weight and cache reads between two uses of a layer's weights would."""
    import torch
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    sink = torch.empty(1, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        fn()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        sink.copy_(flush.sum().reshape(1))
        evs[i][0].record(stream)
        fn()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return sorted(e[0].elapsed_time(e[1]) for e in evs)


def run_query(args):
    """Query side of one decode step for the 64-sequence batch, bf16 weights read
    cold each step:
      query_prep      - c^Q = W^DQ h, q^C = W^UQ c^Q, q^R = RoPE(W^QR c^Q) (91 MB of weights);
      query_lat       - the same, then q_lat_i = W^UK_i^T q^C_i (mla_absorb_q; +16.8 MB);
      query_lat_fused - one product on the offline-fused W^UK_i^T W^UQ_i (201 MB) writes q_lat."""
    import numpy as np
    import torch
    import synth
    import mla_latent_kv_37_amd as mk
    variant = args.workload
    torch.cuda.set_device(0)
    mk._lib.load()
    if variant == "query_lite":
        return run_query_lite(args)
    w = synth.workload(3)
    lens = np.asarray(w.lens, dtype=np.int32)
    B = len(lens)
    W = synth.weights(synth.V2, 0.006, synth.rng_for(3, synth.S_WEIGHTS), with_wo=False)
    bf = lambda x: torch.from_numpy(np.asarray(x, dtype=np.float32)).cuda().to(torch.bfloat16)  # noqa: E731
    h = bf(synth.hidden_states(B, D_MODEL, synth.rng_for(3, synth.S_H)))
    pos = torch.from_numpy(lens).cuda()
    w_dq, w_qr = bf(W["W_DQ"]), bf(W["W_QR"])
    q_pe = torch.empty((B, N_H, D_R), dtype=torch.bfloat16, device="cuda")
    d = mk.dims(N_H, D_H, D_R, D_C)
    if variant == "query_lat_fused":
        # offline weight preparation (host, float32): head i's block is W^UK_i^T W^UQ_i
        wuk = W["W_UK"].astype(np.float32).reshape(N_H, D_H, D_C)
        wuq = W["W_UQ"].astype(np.float32).reshape(N_H, D_H, D_QLATENT)
        w_uq = bf(np.matmul(wuk.transpose(0, 2, 1), wuq).reshape(N_H * D_C, D_QLATENT))
        dq = mk.dims(N_H, D_C, D_R, D_C)
        q_out = torch.empty((B, N_H, D_C), dtype=torch.bfloat16, device="cuda")
        w_bytes = 2 * (D_QLATENT * D_MODEL + N_H * (D_C + D_R) * D_QLATENT)
        out_bytes = B * N_H * (D_C + D_R) * 2
    else:
        w_uq = bf(W["W_UQ"])
        dq = d
        q_out = torch.empty((B, N_H, D_H), dtype=torch.bfloat16, device="cuda")
        w_bytes = 2 * (D_QLATENT * D_MODEL + N_H * (D_H + D_R) * D_QLATENT)
        out_bytes = B * N_H * (D_H + D_R) * 2
    scratch = torch.empty(mk.query_prep_scratch_size(dq, D_QLATENT, B), dtype=torch.uint8, device="cuda")
    if variant == "query_lat":
        w_uk = bf(W["W_UK"])
        q_lat = torch.empty((B, N_H, D_C), dtype=torch.bfloat16, device="cuda")
        w_bytes += 2 * N_H * D_H * D_C
        out_bytes = B * N_H * (D_C + D_R) * 2

        def fn():
            mk.query_prep(d, h, w_dq, w_uq, w_qr, pos, q_out, q_pe, scratch, 10000.0)
            mk.absorb_q(d, q_out, w_uk, q_lat)
    else:
        def fn():
            mk.query_prep(dq, h, w_dq, w_uq, w_qr, pos, q_out, q_pe, scratch, 10000.0)
    times = _cold_weight_steps(fn, args)
    ms = times[len(times) // 2]
    alg_bytes = w_bytes + B * D_MODEL * 2 + out_bytes + B * 4
    ach = alg_bytes / (ms * 1e-3) / 1e9
    kernels = "gemm_ws_mfma_kernel x2 + reduce_cast_kernel + query_finish_kernel"
    if variant == "query_lat":
        kernels += " + absorb_v2_kernel"
    outputs = "q^C, q^R" if variant == "query_prep" else "q_lat, q^R"
    return {
        "metric": f"MLA query-side projections, sequences/s (h -> {outputs})",
        "value": B / (ms * 1e-3), "unit": "sequences/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"v2_{variant}_b{B}", "batch": B, "d_model": D_MODEL, "d_qlatent": D_QLATENT,
                   "weight_bytes": w_bytes, "weights": "cold (512 MB read between steps)",
                   "timing": "median of per-step HIP events"},
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "traffic": None, "kernel": kernels,
                     "algorithmic_bytes_per_launch": alg_bytes, "mean_launch_ms": sum(times) / len(times)},
    }


def run_query_lite(args):
    """V2-Lite query side for the 64-sequence batch: no query compression, so one
    product [W^Q ; W^QR] h (16 heads, d_model 2048; 12.6 MB of bf16 weights read
    cold each step), then the per-head RoPE."""
    import numpy as np
    import torch
    import synth
    import mla_latent_kv_37_amd as mk
    dims = synth.V2LITE
    nh, dh, dr, dm = dims.n_heads, dims.d_head, dims.d_rope, dims.d_model
    w = synth.workload(6)
    lens = np.asarray(w.lens, dtype=np.int32)
    B = len(lens)
    rng = synth.rng_for(6, synth.S_WEIGHTS)
    bf = lambda x: torch.from_numpy(np.asarray(x, dtype=np.float32)).cuda().to(torch.bfloat16)  # noqa: E731
    w_q, w_qr = bf(rng.normal(0.0, synth.V2_SIGMA_W, (nh * dh, dm))), bf(rng.normal(0.0, synth.V2_SIGMA_W, (nh * dr, dm)))
    h = bf(synth.hidden_states(B, dm, synth.rng_for(6, synth.S_H)))
    pos = torch.from_numpy(lens).cuda()
    d = mk.dims(nh, dh, dr, dims.d_latent)
    scratch = torch.empty(mk.query_prep_scratch_size(d, 0, B), dtype=torch.uint8, device="cuda")
    q_nope = torch.empty((B, nh, dh), dtype=torch.bfloat16, device="cuda")
    q_pe = torch.empty((B, nh, dr), dtype=torch.bfloat16, device="cuda")
    times = _cold_weight_steps(lambda: mk.query_prep(d, h, None, w_q, w_qr, pos, q_nope, q_pe, scratch, 10000.0), args)
    ms = times[len(times) // 2]
    w_bytes = 2 * nh * (dh + dr) * dm
    alg_bytes = w_bytes + B * dm * 2 + B * nh * (dh + dr) * 2 + B * 4
    ach = alg_bytes / (ms * 1e-3) / 1e9
    return {
        "metric": "MLA query-side projection, V2-Lite (no query compression), sequences/s (h -> q^C, q^R)",
        "value": B / (ms * 1e-3), "unit": "sequences/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"v2lite_query_prep_b{B}", "batch": B, "d_model": dm, "heads": nh,
                   "weight_bytes": w_bytes, "weights": "cold (512 MB read between steps)",
                   "timing": "median of per-step HIP events"},
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "traffic": None, "kernel": "gemm_ws_mfma_kernel + query_finish_kernel",
                     "algorithmic_bytes_per_launch": alg_bytes, "mean_launch_ms": sum(times) / len(times)},
    }


def prefill_flops(batch: int, T: int, q_len: int, n_h: int = N_H):
    """Algorithmic flops of one mla_prefill call: the up-projection of every
    cached row (2 x 512 x 2 n_h d_h) and, per head, the score and output
    products over the visible positions (2 x (192 + 128) per query-position
    pair; new token t of a sequence sees T - q_len + t + 1 positions)."""
    visible = batch * (q_len * (T - q_len) + q_len * (q_len + 1) // 2)
    return 2.0 * batch * T * D_C * 2 * n_h * D_H + 2.0 * n_h * visible * (D_H + D_R + D_H)


def run_prefill(args, name=None):
    """mla_prefill over synthetic V2-shaped inputs: B sequences of T cached
    tokens whose last q_len are new (prompt processing; q_len < T is a chunk
    after a cached prefix), pages in random order.  The call is timed whole
    (HIP events around each call on its stream: scan, gather, up-projection
    and attention); the roofline is MFMA-bound on the algorithmic flops."""
    import numpy as np
    import torch
    import synth
    import mla_latent_kv_37_amd as mk
    name = name or args.workload
    B, T, Q, cdt = PREFILL_WORKLOADS[name]
    torch.cuda.set_device(0)
    mk._lib.load()
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    pages = (T + 63) // 64
    rows = torch.randn(B * pages, 64, D_C + D_R, device="cuda", generator=g) * synth.V2_SD_LATENT
    if cdt == "bf16":
        kv, scales = rows.to(torch.bfloat16), None
    else:
        # 1 x 128 groups: scale = max|x| / 448 per token and group, codes = x / scale in E4M3
        r = torch.nn.functional.pad(rows, (0, 640 - (D_C + D_R))).view(B * pages, 64, 5, 128)
        scales = (r.abs().amax(dim=-1) / 448.0).clamp_min(1e-12).contiguous()
        kv = (r / scales[..., None]).view(B * pages, 64, 640)[..., : D_C + D_R].to(torch.float8_e4m3fn).contiguous()
    bt = torch.randperm(B * pages, device="cuda", generator=g).to(torch.int32).view(B, pages)
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    cache = mk.make_cache(kv, bt, lens, 64, scales)
    q_off = torch.arange(B + 1, dtype=torch.int32, device="cuda") * Q
    n = B * Q
    sdq = synth.V2_SD_QUERY
    qn = (torch.randn(n, N_H, D_H, device="cuda", generator=g) * sdq).to(torch.bfloat16)
    qp = (torch.randn(n, N_H, D_R, device="cuda", generator=g) * sdq).to(torch.bfloat16)
    wuk = (torch.randn(N_H * D_H, D_C, device="cuda", generator=g) * synth.V2_SIGMA_W).to(torch.bfloat16)
    wuv = (torch.randn(N_H * D_H, D_C, device="cuda", generator=g) * synth.V2_SIGMA_W).to(torch.bfloat16)
    d = mk.dims(N_H, D_H, D_R, D_C)
    total_kv = B * T
    ws = torch.empty(mk.prefill_workspace_size(d, B, total_kv), dtype=torch.uint8, device="cuda")
    out = torch.empty(n, N_H, D_H, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(n, N_H, dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(D_H + D_R)

    def fn():
        mk.prefill(d, q_off, n, Q, qn, qp, cache, total_kv, wuk, wuv, scale, ws, out, lse)
    steps, warm = max(1, min(args.steps, 50)), max(1, min(args.warmup, 10))
    for _ in range(warm):
        fn()
    stream = torch.cuda.current_stream()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        evs[i][0].record(stream)
        fn()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    times = sorted(e[0].elapsed_time(e[1]) for e in evs)
    ms = times[len(times) // 2]
    fl = prefill_flops(B, T, Q)
    ach = fl / (ms * 1e-3) / 1e12
    return {
        "metric": "MLA prefill new tokens/s (non-absorbed, causal, 128 heads)",
        "value": n / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "batch": B, "cached_tokens_per_seq": T, "new_tokens_per_seq": Q,
                   "cache_dtype": cdt, "timing": "median of per-call HIP events"},
        "roofline": {"bound": "mfma", "achieved": ach, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": ach / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                     "kernel": "mla_prefill (scan + gather + prefill_kv_kernel + prefill_attn_kernel), whole call",
                     "algorithmic_flops_per_launch": fl, "mean_launch_ms": sum(times) / len(times)},
    }


def run_append(args):
    import numpy as np
    import torch
    import synth
    import mla_latent_kv_37_amd as mk
    kind = APPEND_WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    mk._lib.load()
    w = synth.workload(3)
    lens = np.asarray(w.lens, dtype=np.int32)
    B = len(lens)
    rng = synth.rng_for(3, synth.S_WEIGHTS)
    W = synth.weights(synth.V2, 0.006, rng, with_wo=False)
    bf = lambda x: torch.from_numpy(np.asarray(x, dtype=np.float32)).cuda().to(torch.bfloat16)  # noqa: E731
    w_dkv, w_kr = bf(W["W_DKV"]), bf(W["W_KR"])
    h = bf(synth.hidden_states(B, D_MODEL, synth.rng_for(3, synth.S_H)))
    # one page of its own per sequence for the new token's slot
    max_pages = int((lens.max() + 64) // 64) + 1
    bt = np.zeros((B, max_pages), dtype=np.int32)
    bt[np.arange(B), lens // 64] = np.arange(B)
    width = D_C + D_R
    tdt = torch.bfloat16 if kind == "bf16" else torch.uint8
    kv = torch.zeros((B, 64, width), dtype=tdt, device="cuda")
    scales = torch.zeros((B, 64, 5), dtype=torch.float32, device="cuda") if kind == "fp8" else None
    cache = mk.make_cache(kv, torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(), 64, scales)
    pos = torch.from_numpy(lens).cuda()
    rows = torch.empty((8, B, width), dtype=torch.float32, device="cuda")
    d = mk.dims(N_H, D_H, D_R, D_C)
    times = _cold_weight_steps(lambda: mk.cache_append(d, h, w_dkv, w_kr, rows, pos, cache, 10000.0), args)
    ms = times[len(times) // 2]
    elem = 2 if kind == "bf16" else 1
    alg_bytes = (width * D_MODEL * 2 + B * D_MODEL * 2 + B * width * elem + (B * 5 * 4 if kind == "fp8" else 0)
                 + B * 4 * 2)
    ach = alg_bytes / (ms * 1e-3) / 1e9
    return {
        "metric": "MLA cache append new tokens/s (project [W^DKV; W^KR] h, RoPE, round, scatter)",
        "value": B / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"v2_cache_append_b{B}_{kind}", "batch": B, "d_model": D_MODEL, "cache_dtype": kind,
                   "weights": "cold (512 MB read between steps)", "timing": "median of per-step HIP events"},
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "traffic": None, "kernel": "gemm_ws_mfma_kernel + cache_store_kernel",
                     "algorithmic_bytes_per_launch": alg_bytes, "mean_launch_ms": sum(times) / len(times)},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU's clocks ramp up over the first few hundred steps (~130 us each):
    # 1000 warmup steps reach the steady state that a serving loop runs at
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="ragged",
                    choices=sorted(WORKLOADS) + sorted(APPEND_WORKLOADS) + sorted(QUERY_WORKLOADS) + sorted(PREFILL_WORKLOADS))
    ap.add_argument("--copies", type=int, default=2)
    ap.add_argument("--warm-weights", action="store_true",
                    help="reuse each input set's W^UK / W^UV (they may stay cached between steps)")
    ap.add_argument("--partition", type=int, nargs=2, metavar=("SPLIT_TOKENS", "NUM_PARTS"), default=None,
                    help="override the workload's partition (split_tokens, num_parts; -1 parts = one per compute unit)")
    ap.add_argument("--no-kernel-events", dest="kernel_events", action="store_false")
    ap.add_argument("--unfused", action="store_true",
                    help="run mla_merge_splits + mla_out_proj (mla_decode_multi + mla_out_proj) instead of "
                         "mla_merge_out_proj (mla_decode_multi_out_proj), for comparison")
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed back-to-back steps before the warm-up steps (clock ramp, TLB warm-up)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time the ragged workload alone (no other decode workloads first)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("DIR", "OUT_MD"))
    ap.add_argument("--summarize-pmc", nargs=5, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_BYTES", "OUT_JSON", "OUT_MD"))
    ap.add_argument("--summarize-counters", nargs=2, metavar=("DIR", "OUT_MD"))
    ap.add_argument("--cmd", default="")
    args = ap.parse_args()
    if args.summarize_stats:
        return summarize_stats(*args.summarize_stats, cmd=args.cmd)
    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc, cmd=args.cmd, workload=args.workload)
    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters, cmd=args.cmd, workload=args.workload)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the MLA decode path here is single-GPU (no sharding, no "
              "collectives); use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
    if args.workload in APPEND_WORKLOADS:
        res = run_append(args)
    elif args.workload in PREFILL_WORKLOADS:
        res = run_prefill(args)
    elif args.workload in QUERY_WORKLOADS:
        res = run_query(args)
    elif args.workload == "ragged" and args.partition is None and not args.headline_only:
        # The default run: the other decode workloads first (each with its own
        # warm-up and K timed steps), then the headline ragged batch, so that the
        # headline is timed at the clocks a GPU that has been decoding holds.
        copy_tbps = measured_copy_tbps()
        others = {}
        for name, wl, part in EXTRA_WORKLOADS:
            r = run(args, wl, part, cpu=False, copy_tbps=copy_tbps)
            others[name] = summary(r)
            print(f"# {name}: {r['ms_per_step'] * 1e3:.1f} us/step, {r['value'] / 1e9:.3f} G {r['unit']}", flush=True)
        pf = run_prefill(args, "prefill_b4_t4096")
        others["prefill_b4_t4096"] = {k: pf[k] for k in ("metric", "value", "unit", "ms_per_step", "steps", "warmup",
                                                         "config", "roofline")}
        print(f"# prefill_b4_t4096: {pf['ms_per_step'] * 1e3:.1f} us/call, {pf['value'] / 1e6:.3f} M tokens/s, "
              f"{pf['roofline']['achieved']:.0f} TFLOP/s", flush=True)
        res = run(args, copy_tbps=copy_tbps)
        res["other_workloads"] = others
    else:
        res = run(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
