#!/usr/bin/env python3
"""Benchmark of the FP4 decode hot path on one MI355X.

Workload (the 128K long-context decode): batch 1, Qwen3-4B shapes (32 query
/ 8 KV heads, head_dim 128), 131,072-token context paged at block_size 128
through a permuted block table, 16-token BF16 sink, no tail; 36 layers with
independent seeded K/V/Q/key means (seed = layer); bitdecoding-nvfp4 recipe
(Hadamard rotation, key centering, K four_six, V/Q amax6, two-term query,
P amax2_or_amax6, c = 8, tau = 1.0). Inputs are synthetic, drawn on the
device, and every layer's pages are written by the HIP page writer before
timing; all inputs are resident in HBM when the timed region starts.

A step is one decode token through all 36 layers: 36 launches of
bdfp4_decode_attention (each: two-term query quantization, QK^T over the FP4
pages, partition softmax, P quantization, PV, BF16 sink partition and the
split-K merge). The MXFP4 and BF16-KV arms, a batch of 16 sequences of
2K..16K tokens, the page writer (131,072
tokens x 8 heads prefill write) and the decode-time append (batch 1 and 64 x 8
KV heads, inside a page and at the token that freezes one) and the key-mean
calibration over the prefill keys are timed the same way and reported beside
it.

Prints one JSON line; run `python bench.py --help` for options.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "FP4 decode-attention µs/step + achieved HBM GB/s (% of peak) at 128K ctx"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=36)
    ap.add_argument("--context", type=int, default=131072)
    ap.add_argument("--ppp", type=int, default=0, help="pages per partition (0 = library plan)")
    ap.add_argument("--arms", default="nvfp4,mxfp4,bf16")
    ap.add_argument("--no-writer", action="store_true")
    ap.add_argument("--no-append", action="store_true")
    ap.add_argument("--no-calibration", action="store_true")
    ap.add_argument("--no-batched", action="store_true")
    ap.add_argument("--no-small", action="store_true", help="skip the tiny 2K and the 32K single-layer decodes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="replay each step as a captured HIP graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for counter calibration) and exit")
    return ap.parse_args()


# ----------------------------------------------------------------- algorithmic bytes

def decode_bytes(seq_len: int, hq: int, hkv: int, sink: int, mx: bool) -> int:
    """Bytes one decode launch must move: FP4 K/V codes + scales of tokens
    [sink, 128 n), BF16 sink/tail tokens, query, key means, block table, output."""
    n_full = seq_len // 128
    fp4_tok = max(0, 128 * n_full - sink) if n_full else 0
    bf16_tok = min(sink, seq_len) + max(0, seq_len - max(sink, 128 * n_full))
    per_tok = 2 * (64 + (4 if mx else 8))
    return (fp4_tok * hkv * per_tok + bf16_tok * hkv * 512 + hq * 256 + hkv * 512 + 4 * n_full + hq * 512)


def bf16_decode_bytes(seq_len: int, hq: int, hkv: int) -> int:
    return seq_len * hkv * 512 + hq * 256 + 4 * (-(-seq_len // 128)) + hq * 512


def writer_bytes(tokens: int, hkv: int, mx: bool) -> int:
    read = tokens * hkv * 128 * 2 * 2 + hkv * 512 + 4 * (tokens // 128)
    write = tokens * hkv * 2 * (64 + (4 if mx else 8))
    return read + write


# ----------------------------------------------------------------- timing

LAST_PERCENTILES = {"p10": None, "p90": None, "n": 0}   # of the per-launch durations of the last time_launches
PERCENTILE_LAUNCHES = 100      # launches timed one by one for the per-launch statistics
ROTATE_BYTES = 2 << 30         # buffer copies cycled through per measurement, so none stays in the 256 MB MALL


# Untimed launches before a bulk kernel (page writer, key means, page errors)
# is timed. The page writer's launch time falls by about 15 % over its first
# ~150 back-to-back launches on the same buffers (197 -> 167 us measured in
# blocks of 40 launches), then holds: a prefill of many layers runs in that
# steady state.
BULK_WARMUP = 200


def time_launches(fns, steps: int, warmup: int, graph: bool = False):
    """Run `warmup` untimed steps, then exactly `steps` timed steps of the
    launches in `fns` on the current stream. Returns (ms per step, mean ms per
    launch from per-launch events in a second pass over the same launches)."""
    import torch

    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    g = None
    if graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for f in fns:
                f()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in fns:
                f()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        if g is not None:
            g.replay()
        else:
            for f in fns:
                f()
    end.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ms_step = start.elapsed_time(end) / steps
    # per-launch durations: events around each launch, same stream, over at
    # least PERCENTILE_LAUNCHES launches
    n_ev = max(1, -(-PERCENTILE_LAUNCHES // len(fns)))
    evs = []
    torch.cuda.synchronize()
    for _ in range(n_ev):
        for f in fns:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            evs.append((a, b))
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in evs]
    LAST_PERCENTILES["p10"], LAST_PERCENTILES["p90"] = (float(v) for v in np.percentile(per, [10, 90]))
    LAST_PERCENTILES["n"] = len(per)
    return ms_step, float(np.mean(per)), wall, float(np.median(per))


# ----------------------------------------------------------------- setup

def build_layers(args, arms):
    import torch

    import fp4_kv_cache_nvfp4_amd as bd
    from fp4_kv_cache_nvfp4_amd import synth

    rec = {"nvfp4": bd.recipe_default_nvfp4(tau=1.0), "mxfp4": bd.recipe_default_mxfp4(tau=1.0)}
    L = args.context
    ppp, parts = bd.decode_plan(1, 8, L, args.ppp)
    # the BF16-KV arm in its own automatic plan (about 512 workgroups)
    ppp_arm = {a: bd.bf16_decode_plan(1, 8, L, 0)[0] if a == "bf16" else ppp for a in arms}
    layers = {a: [] for a in arms}
    ws = {a: bd.alloc_workspace(bd.decode_workspace_size(1, 32, 8, L, ppp_arm[a])) for a in arms}
    outs = {a: torch.empty((1, 32, 128), dtype=torch.float32, device="cuda") for a in arms}
    for layer in range(args.layers):
        d = synth.torch_decode_layer(layer, seq_len=L)
        for a in arms:
            if a in rec:
                r = rec[a]
                cache = bd.PagedCache.allocate(r, d["num_pages"], 8)
                bd.quantize_pages(r, cache, d["k"], d["v"], d["page_ids"], d["key_shift"])
                call = bd.DecodeCall(r, cache, d["q"], d["block_tables"], d["seq_lens"], L, d["sink_k"],
                                     d["sink_v"], d["tail_k"], d["tail_v"], d["key_shift"], d["sigma"], ppp,
                                     ws[a], outs[a])
            else:
                kp = synth.bf16_pages_from_tokens(d["k"], d["block_tables"], d["num_pages"])
                vp = synth.bf16_pages_from_tokens(d["v"], d["block_tables"], d["num_pages"])
                call = bd.Bf16DecodeCall(d["q"], kp, vp, d["block_tables"], d["seq_lens"], L, d["sigma"],
                                         ppp_arm[a], ws[a], outs[a])
            layers[a].append(call)
        del d
        torch.cuda.synchronize()
    return layers, outs, ppp, parts


def bench_batched(args):
    """NVFP4 decode of 16 sequences with lengths drawn from 2K..16K (seeded)
    over one shuffled pool (32 query / 8 KV heads), the library's plan for
    the batch: one launch per call, cycled over buffer copies. Bytes = the
    sum of every sequence's decode bytes."""
    from fp4_kv_cache_nvfp4_amd import synth

    return bench_workload(args, synth.batched(0),
                          "16 sequences, L ~ U{2048..16384} (seed 0), shared shuffled pool")


def bench_small_configs(args):
    """The two single-layer decode shapes beside the 128K one: the tiny 2K
    single-KV-head case (4 query heads; launch-bound, so its µs is the
    figure, measured on one resident buffer set) and the Qwen3-4B-shaped 32K
    layer (256 full pages in a permuted pool plus a 77-token BF16 tail),
    cycled over copies of its buffers, each with the library's plan."""
    from fp4_kv_cache_nvfp4_amd import synth

    return {"tiny_2k_1kv": bench_workload(args, synth.tiny(0), "1 sequence, L = 2048, 1 KV head / 4 query heads",
                                          rotate=False),
            "qwen3_4b_32k_layer": bench_workload(args, synth.qwen_32k(0),
                                                 "1 sequence, L = 32,845 (256 pages + 77-token tail), 8 KV / 32 query heads")}


def bench_workload(args, wl, what: str, rotate: bool = True):
    """NVFP4 decode of a seeded numpy workload: pages written by the HIP
    writer, one launch per call, the library's plan. With rotate, every
    buffer the decode reads (cache, query, tables, sink, tail, key means) is
    copied until the copies hold at least ROTATE_BYTES, and the timed steps
    cycle through them, so that the figure is an HBM figure and not one of
    the 256 MB last-level cache; without it one buffer set is re-read and the
    result says cache_resident."""
    import torch

    import fp4_kv_cache_nvfp4_amd as bd

    r = bd.recipe_default_nvfp4(tau=1.0)
    B, msl = wl.batch, int(wl.seq_lens.max())
    hq, hkv = int(wl.q.shape[1]), int(wl.num_kv_heads)
    ppp, parts = bd.decode_plan(B, hkv, msl, 0)
    nbytes = sum(decode_bytes(int(L), hq, hkv, 16, False) for L in wl.seq_lens)
    copies = max(1, -(-ROTATE_BYTES // nbytes)) if rotate else 1
    t16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    k, v, ids = wl.writer_inputs()
    kd, vd, idd = t16(k), t16(v), t(ids)
    sk, sv, tk, tv = wl.sink_tail()
    ws = bd.alloc_workspace(bd.decode_workspace_size(B, hq, hkv, msl, ppp))
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    calls = []
    for _ in range(copies):
        cache = bd.PagedCache.allocate(r, wl.num_pages, hkv)
        mu = t(wl.key_shift)
        bd.quantize_pages(r, cache, kd, vd, idd, mu)
        calls.append(bd.DecodeCall(r, cache, t16(wl.q), t(wl.block_tables), t(wl.seq_lens), msl, t16(sk), t16(sv),
                                   t16(tk), t16(tv), mu, wl.sigma, ppp, ws, out))
    del kd, vd
    torch.cuda.synchronize()
    ms, per, _, med = time_launches(calls, max(args.steps, 20), args.warmup)
    if not torch.isfinite(out).all():
        raise RuntimeError(f"{what}: non-finite decode output")
    us = ms * 1e3 / len(calls)
    res = {"workload": what, "tokens": int(wl.seq_lens.sum()), "pages_per_partition": ppp,
           "max_partitions": parts, "us": round(us, 3), "us_kernel_events_mean": round(per * 1e3, 3),
           "us_kernel_events_median": round(med * 1e3, 3),
           "us_kernel_events_p10": round(LAST_PERCENTILES["p10"] * 1e3, 3),
           "us_kernel_events_p90": round(LAST_PERCENTILES["p90"] * 1e3, 3),
           "kernel_events_n": LAST_PERCENTILES["n"],
           "bytes": nbytes, "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
           "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
           "buffer_copies": copies, "bytes_cycled": nbytes * copies, "cache_resident": not rotate}
    del calls
    torch.cuda.empty_cache()
    return res


def bench_writer(args, mx: bool):
    import torch

    import fp4_kv_cache_nvfp4_amd as bd
    from fp4_kv_cache_nvfp4_amd import synth

    w = synth.torch_write_rows(0)
    r = bd.recipe_default_mxfp4(tau=1.0) if mx else bd.recipe_default_nvfp4(tau=1.0)
    cache = bd.PagedCache.allocate(r, w["num_pages"], 8)
    fn = lambda: bd.quantize_pages(r, cache, w["k"], w["v"], w["page_ids"], w["key_shift"])
    ms, per, _, med = time_launches([fn], max(args.steps, 10), BULK_WARMUP)
    nbytes = writer_bytes(w["tokens"], 8, mx)
    del w, cache
    torch.cuda.empty_cache()
    return {"us": ms * 1e3, "us_kernel_events": per * 1e3, "bytes": nbytes, "GBps": nbytes / (ms * 1e-3) / 1e9,
            "frac_of_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


def append_bytes(batch: int, hkv: int, fill: bool, mx: bool) -> int:
    """Algorithmic HBM bytes of one append call: the new K and V rows read,
    written to the tail (256 B each); a fill also reads the other 127 tail
    rows and writes the page's codes and scales."""
    b = batch * hkv * 2 * (256 + 256)
    if fill:
        b += batch * hkv * 2 * (127 * 256 + 8192 + (512 if mx else 1024))
    return b


def bench_append(args, batch: int):
    """One decode-time append per call for `batch` sequences x 8 KV heads:
    at a position inside a page (tail write only) and at the last slot of a
    page (tail write plus freezing the page)."""
    import torch

    import fp4_kv_cache_nvfp4_amd as bd

    hkv = 8
    r = bd.recipe_default_nvfp4(tau=1.0)
    g = torch.Generator(device="cuda").manual_seed(7)
    rows = lambda *s: torch.randn(*s, device="cuda", generator=g).to(torch.bfloat16)
    cache = bd.PagedCache.allocate(r, batch * 4, hkv)
    bt = torch.arange(batch * 4, device="cuda", dtype=torch.int32).reshape(batch, 4)
    tk, tv = rows(batch, hkv, 128, 128), rows(batch, hkv, 128, 128)
    sk, sv = rows(batch, hkv, 16, 128), rows(batch, hkv, 16, 128)
    kn, vn = rows(batch, hkv, 128), rows(batch, hkv, 128)
    mu = torch.randn(hkv, 128, device="cuda", generator=g)
    out = {}
    for name, p in (("tail", 200), ("fill", 255)):
        pos = torch.full((batch,), p, device="cuda", dtype=torch.int32)
        fn = lambda: bd.append_tokens(r, cache, kn, vn, pos, bt, sk, sv, tk, tv, mu)
        # 20 calls captured in one graph per step, so the host's per-call
        # cost (argument marshalling) stays out of the device time; repeated
        # appends at one position rewrite the same bytes
        reps = 20
        ms, per, _, med = time_launches([fn] * reps, max(args.steps, 20), 5, graph=True)
        us = ms * 1e3 / reps
        nb = append_bytes(batch, hkv, name == "fill", False)
        out[name] = {"us": round(us, 3), "bytes": nb, "GBps": round(nb / (us * 1e-6) / 1e9, 1)}
    return out


def bench_key_means(args):
    """Key-mean calibration over the 131,072-token x 8-head prefill keys
    (the writer's input): bytes = the bf16 keys read once."""
    import torch

    import fp4_kv_cache_nvfp4_amd as bd
    from fp4_kv_cache_nvfp4_amd import synth

    w = synth.torch_write_rows(0)
    k = w["k"]
    tokens = int(k.shape[0])
    need = bd.key_means_workspace_size(tokens, 8)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    mu = torch.empty((8, 128), dtype=torch.float32, device="cuda")
    fn = lambda: bd.key_means_into(k, 8, ws, mu)
    ms, per, _, med = time_launches([fn], max(args.steps, 10), BULK_WARMUP)
    nbytes = tokens * 8 * 128 * 2
    res = {"key_means_131072x8": {"us": round(ms * 1e3, 3), "bytes": nbytes,
                                  "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                  "frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}}
    # diagnostics: page errors of the whole prefill (reads the bf16 K/V rows
    # and the written pages)
    r = bd.recipe_default_nvfp4(tau=1.0)
    cache = bd.PagedCache.allocate(r, w["num_pages"], 8)
    bd.quantize_pages(r, cache, w["k"], w["v"], w["page_ids"], w["key_shift"])
    fn = lambda: bd.page_errors(r, cache, w["k"], w["v"], w["page_ids"], w["key_shift"])
    ms, per, _, med = time_launches([fn], max(args.steps, 10), BULK_WARMUP)
    nbytes = writer_bytes(tokens, 8, False)
    res["page_errors_131072x8"] = {"us": round(ms * 1e3, 3), "bytes": nbytes,
                                   "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    del w, k, cache
    torch.cuda.empty_cache()
    return res


def cpu_baseline(args):
    """The oracle (numpy) decode on a bounded sample of the same workload:
    one layer, 2 of the 8 KV heads (8 query heads), the full 131,072-token
    context, pages quantized by the oracle writer beforehand (untimed); the
    decode is repeated until at least 10 s of CPU time have passed."""
    from fp4_kv_cache_nvfp4_amd import synth
    from oracle import decode as OD
    from oracle import recipe as RC
    from oracle import writer as W

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    L = args.context
    wl = synth.decode_workload("qwen3_4b_128k_sample", 0, [L], 8, 2, "qwen")
    r = RC.nvfp4_default().with_(tau=1.0)
    cache = W.empty_cache(wl.num_pages, 2, r)
    k, v, ids = wl.writer_inputs()
    W.write_pages(r, cache, k, v, ids, wl.key_shift)
    sk, sv, tk, tv = wl.sink_tail()
    ppp = 4
    reps, dt = 0, 0.0
    while dt < 10.0 and reps < 50:
        t0 = time.perf_counter()
        OD.decode(r, cache, wl.q, wl.block_tables, wl.seq_lens, sk, sv, tk, tv, wl.key_shift, wl.sigma, ppp)
        dt += time.perf_counter() - t0
        reps += 1
    nbytes = decode_bytes(L, 8, 2, 16, False)
    cores = len(os.sched_getaffinity(0))
    return {"value": round(nbytes * reps / dt / 1e9, 4), "unit": "GB/s", "cores": blas_threads or cores,
            "kind": "oracle",
            "sample": f"{reps} runs of the oracle float64 decode of 1 layer x 2 of 8 KV heads (8 query heads) over "
                      f"the full {L}-token context on oracle-written NVFP4 pages ({nbytes} algorithmic bytes per "
                      f"run), {dt:.1f} s; {cores} host cores visible, BLAS threads {blas_threads}",
            "seconds": round(dt, 2), "us_per_layer_equiv": round(dt / reps * 4 * 1e6, 1)}


def _cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return None


def _repeat(fn, min_seconds: float, max_reps: int = 1000):
    reps, dt = 0, 0.0
    while dt < min_seconds and reps < max_reps:
        t0 = time.perf_counter()
        fn()
        dt += time.perf_counter() - t0
        reps += 1
    return reps, dt


def cpu_baseline_decode(wl, ppp: int, what: str, min_seconds: float = 10.0):
    """The oracle decode of a bounded sample of a decode workload (the same
    recipe and shapes per KV head, fewer KV heads), on pages the oracle writer
    quantized beforehand (untimed), repeated until min_seconds of CPU time."""
    from oracle import decode as OD
    from oracle import recipe as RC
    from oracle import writer as W

    r = RC.nvfp4_default().with_(tau=1.0)
    cache = W.empty_cache(wl.num_pages, wl.num_kv_heads, r)
    k, v, ids = wl.writer_inputs()
    W.write_pages(r, cache, k, v, ids, wl.key_shift)
    sk, sv, tk, tv = wl.sink_tail()
    reps, dt = _repeat(lambda: OD.decode(r, cache, wl.q, wl.block_tables, wl.seq_lens, sk, sv, tk, tv,
                                         wl.key_shift, wl.sigma, ppp), min_seconds)
    hq, hkv = int(wl.q.shape[1]), int(wl.num_kv_heads)
    nbytes = sum(decode_bytes(int(L), hq, hkv, 16, False) for L in wl.seq_lens)
    cores = len(os.sched_getaffinity(0))
    threads = _cpu_threads()
    return {"value": round(nbytes * reps / dt / 1e9, 4), "unit": "GB/s", "cores": threads or cores, "kind": "oracle",
            "us_per_decode": round(dt / reps * 1e6, 1),
            "sample": f"{reps} runs of the oracle float64 decode of {what} ({nbytes} algorithmic bytes per run, "
                      f"pages_per_partition {ppp}), {dt:.1f} s; {cores} host cores visible, BLAS threads {threads}"}


def cpu_baseline_writer(min_seconds: float = 10.0, pages: int = 32):
    """The oracle page writer (NVFP4: K four_six with rotation and centering,
    V amax6) on a bounded sample of the prefill write: `pages` pages x 8 KV
    heads of the same recipe of keys and values, repeated until min_seconds."""
    from fp4_kv_cache_nvfp4_amd import synth
    from oracle import recipe as RC
    from oracle import writer as W

    r = RC.nvfp4_default().with_(tau=1.0)
    w = synth.write_workload(0, tokens=pages * 128, num_kv_heads=8)
    cache = W.empty_cache(w.num_pages, 8, r)
    reps, dt = _repeat(lambda: W.write_pages(r, cache, w.k_rows, w.v_rows, w.page_ids, w.key_shift), min_seconds)
    nbytes = writer_bytes(pages * 128, 8, False)
    cores = len(os.sched_getaffinity(0))
    threads = _cpu_threads()
    return {"value": round(nbytes * reps / dt / 1e9, 4), "unit": "GB/s", "cores": threads or cores, "kind": "oracle",
            "tokens_per_s": round(pages * 128 * reps / dt, 1),
            "sample": f"{reps} runs of the oracle NVFP4 page writer over {pages} pages x 8 KV heads "
                      f"({pages * 128} tokens, {nbytes} algorithmic bytes per run), {dt:.1f} s; {cores} host cores "
                      f"visible, BLAS threads {threads}"}


def _plan(batch: int, hkv: int, max_seq_len: int):
    """The library's split plan for these sizes (host call, no GPU), so the
    oracle decodes with the partitioning the GPU arm uses."""
    import fp4_kv_cache_nvfp4_amd as bd

    return bd.decode_plan(batch, hkv, max_seq_len, 0)


def cpu_baselines_beside():
    """Oracle timings beside the configurations other than the headline."""
    from fp4_kv_cache_nvfp4_amd import synth

    out = {"writer_131072x8_sample": cpu_baseline_writer()}
    out["tiny_2k_1kv"] = cpu_baseline_decode(synth.tiny(0), _plan(1, 1, 2048)[0],
                                             "the tiny 2K single-KV-head workload (whole)")
    out["qwen3_4b_32k_layer"] = cpu_baseline_decode(
        synth.decode_workload("qwen3_4b_32k_sample", 0, [32845], 4, 1, "qwen"), _plan(1, 8, 32845)[0],
        "1 of the 8 KV heads (4 query heads) of the 32,845-token layer")
    bwl = synth.batched(0, num_kv_heads=1)
    bppp, _ = _plan(bwl.batch, 8, int(bwl.seq_lens.max()))
    out["batched_16x_2k_16k"] = cpu_baseline_decode(
        bwl, bppp, "1 of the 8 KV heads (4 query heads) of the 16 sequences of 2K..16K tokens")
    return out


# ----------------------------------------------------------------- counter traffic

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_nvfp4_128k_traffic.txt")
KERNEL_SOURCES = ["decode.hip", "codec.hpp", "merge.hpp", "launch.hpp"]


def kernel_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "fp4_kv_cache_nvfp4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_traffic():
    """HBM bytes per decode launch from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by the factor a plain
    copy of known size gives), or None when the summary is missing or the
    decode sources changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, "no counter summary"
    kv = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if "=" in line and not line.lstrip().startswith("#"):
                key, val = line.split("=", 1)
                kv[key.strip()] = val.strip()
    if kv.get("source_sha256") != kernel_source_hash():
        return None, "decode sources changed since the counters were taken"
    return int(float(kv["traffic_bytes_per_launch"])), "counters"


def read_ceiling(nbytes: int, slices: int = 8, rounds: int = 10, workgroups: int = 512):
    """The practical HBM read ceiling for one decode layer's byte count: the
    library's plain streaming read (bdfp4_stream_read) over `slices` distinct
    buffers of that size in turn, so no slice is still in the last-level
    cache when it is read again."""
    import torch

    import fp4_kv_cache_nvfp4_amd as bd

    n = (nbytes + 15) // 16 * 16
    buf = torch.empty(n * slices, dtype=torch.uint8, device="cuda")
    buf.fill_(3)
    sink = torch.empty(workgroups * 256, dtype=torch.int32, device="cuda")
    views = [buf[i * n:(i + 1) * n] for i in range(slices)]
    for v in views:
        bd.stream_read(v, sink, workgroups)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(rounds):
        for v in views:
            bd.stream_read(v, sink, workgroups)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (rounds * slices)
    del buf
    return {"bytes": n, "us": round(us, 3), "GBps": round(n / (us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(n / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), "workgroups": workgroups,
            "kernel": "bdfp4_stream_read (plain coalesced read, 4 x 16 B in flight per thread)"}


def copy_calibration():
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": ms, "GBps_rw": 2 * n / (ms * 1e-3) / 1e9}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding of the decode is not built.", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    arms = [a for a in args.arms.split(",") if a]
    assert arms and arms[0] == "nvfp4", "the first arm is the headline NVFP4 decode"
    print(f"[bench] building {args.layers} layers x {args.context} tokens, arms {arms}", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    layers, outs, ppp, parts = build_layers(args, arms)
    print(f"[bench] setup {time.perf_counter() - t0:.1f} s; pages/partition {ppp}, partitions {parts}",
          file=sys.stderr, flush=True)
    res = {}
    for a in arms:
        ms, per, wall, med = time_launches(layers[a], args.steps, args.warmup, graph=args.graph)
        if not torch.isfinite(outs[a]).all():
            raise RuntimeError(f"{a}: non-finite decode output")
        nb = (bf16_decode_bytes(args.context, 32, 8) if a == "bf16"
              else decode_bytes(args.context, 32, 8, 16, a == "mxfp4"))
        res[a] = {"ms_per_step": ms, "us_per_layer": ms * 1e3 / args.layers, "us_kernel_events": per * 1e3,
                  "us_kernel_events_median": med * 1e3, "us_kernel_events_p10": LAST_PERCENTILES["p10"] * 1e3,
                  "us_kernel_events_p90": LAST_PERCENTILES["p90"] * 1e3, "wall_ms_per_step": wall,
                  "bytes_per_layer": nb, "GBps": nb * args.layers / (ms * 1e-3) / 1e9,
                  "kernel_GBps": nb / (per * 1e-3) / 1e9}
        if a == "bf16":
            import fp4_kv_cache_nvfp4_amd as bd
            res[a]["pages_per_partition"] = bd.bf16_decode_plan(1, 8, args.context, 0)[0]
        print(f"[bench] {a}: {ms * 1e3:.1f} us/step, {res[a]['GBps']:.0f} GB/s, kernel "
              f"{per * 1e3:.2f} us ({res[a]['kernel_GBps']:.0f} GB/s)", file=sys.stderr, flush=True)
    del layers
    torch.cuda.empty_cache()
    ceiling = read_ceiling(res["nvfp4"]["bytes_per_layer"])
    print(f"[bench] plain read of {ceiling['bytes']} B: {ceiling['us']:.2f} us ({ceiling['GBps']:.0f} GB/s)",
          file=sys.stderr, flush=True)
    writer = {}
    if not args.no_writer:
        for mx in (False, True):
            writer["mxfp4" if mx else "nvfp4"] = bench_writer(args, mx)
            print(f"[bench] writer {'mxfp4' if mx else 'nvfp4'}: {writer['mxfp4' if mx else 'nvfp4']['us']:.1f} us",
                  file=sys.stderr, flush=True)
    batched = None
    if not args.no_batched:
        batched = bench_batched(args)
        print(f"[bench] batched: {batched}", file=sys.stderr, flush=True)
    small = {}
    if not args.no_small:
        small = bench_small_configs(args)
        for k, v in small.items():
            print(f"[bench] {k}: {v['us']:.2f} us, {v['GBps']:.0f} GB/s", file=sys.stderr, flush=True)
    append = {}
    if not args.no_append:
        for batch in (1, 64):
            append[f"batch{batch}"] = bench_append(args, batch)
            print(f"[bench] append batch {batch}: {append[f'batch{batch}']}", file=sys.stderr, flush=True)
    calibration = None
    if not args.no_calibration:
        calibration = bench_key_means(args)
        print(f"[bench] key means: {calibration}", file=sys.stderr, flush=True)
    cpu, cpu_beside = None, None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args)
        print("[bench] cpu baselines beside the other configurations (oracle)", file=sys.stderr, flush=True)
        cpu_beside = cpu_baselines_beside()
        if writer:
            writer["cpu_baseline"] = cpu_beside["writer_131072x8_sample"]
        for k in ("tiny_2k_1kv", "qwen3_4b_32k_layer"):
            if k in small:
                small[k]["cpu_baseline"] = cpu_beside[k]
        if batched is not None:
            batched["cpu_baseline"] = cpu_beside["batched_16x_2k_16k"]
    traffic, traffic_src = counter_traffic()
    h = res["nvfp4"]
    # average launch duration over the timed region: the start/end events of
    # the timed steps on the launch stream, divided by the launches in them
    us_launch = h["ms_per_step"] * 1e3 / args.layers
    achieved = h["bytes_per_layer"] / (us_launch * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": round(h["GBps"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["ms_per_step"], 4),
        "us_per_step": round(h["ms_per_step"] * 1e3, 1),
        "frac_of_hbm_peak": round(h["GBps"] / PEAK_HBM_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e2m1 codes, f16 MFMA operands, fp32 accumulate",
        "data": "synthetic (seeded, drawn on device; no model weights)",
        "config": {"workload": "qwen3_4b_shapes_128k_ctx_36_layer_nvfp4_decode", "batch": 1,
                   "context": args.context, "layers": args.layers, "q_heads": 32, "kv_heads": 8, "head_dim": 128,
                   "block_size": 128, "sink_tokens": 16, "recipe": "bitdecoding-nvfp4 (tau=1.0, c=8)",
                   "pages_per_partition": ppp, "partitions": parts, "graph": bool(args.graph)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic, "traffic_source": traffic_src,
                     "kernel": "bdfp4::decode_kernel<false,2,true,false,4,false>",
                     "bytes_per_launch": h["bytes_per_layer"], "us_per_launch": round(us_launch, 3),
                     "us_per_launch_single_events": round(h["us_kernel_events"], 3),
                     "read_ceiling": ceiling,
                     "frac_of_read_ceiling": round(ceiling["us"] / us_launch, 4)},
        "cpu_baseline": cpu,
        "arms": {a: {k: (round(v, 3) if isinstance(v, float) else v) for k, v in res[a].items()} for a in res},
        "writer_131072x8": writer,
        "batched_16x_2k_16k": batched,
        "single_layer_configs": small,
        "append_x8_heads": append,
        "calibration_diagnostics": calibration,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
