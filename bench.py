#!/usr/bin/env python3
"""Benchmark of the fused relation-aware attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

One step is one call of relattn_fwd over one batch of the workload (every step
of the method runs inside that call).  The timed region is K back-to-back
steps on one HIP stream, bracketed by HIP events, after W untimed steps.  The
steps cycle through several copies of the inputs whose total size exceeds the
256 MB last-level cache, so each step reads its operands from HBM as a
stream of fresh batches would.

Prints ONE JSON line: TFLOP/s of the headline workload (Transformer-big
decoder causal self-attention with key and value tables), its fraction of the
bf16 MFMA peak, the HBM roofline of the kernel, the fp64 oracle timed on the
host cores, the same figures for the other Transformer shapes, and those of
incremental decoding, of the offset-bias (ALiBi) arm, of the backward, of
Transformer-XL relative logits and of the 2-D window (Swin) bias.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "rel-attention fwd TFLOP/s at 1 GPU (+% MFMA peak, HBM GB/s), base/big shapes"
HEADLINE = "big_causal_kv"
OTHER = ["base", "big_causal_k", "long", "t5"]
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense MFMA, MI355X
PEAK_HBM_GBS = 8000.0
LLC_BYTES = 256 << 20
CSRC = os.path.join(ROOT, "relative_position_encoding_amd", "csrc")
KERNEL_SRC = os.path.join(CSRC, "relattn_kernels.hip")
LEAN_SRC = os.path.join(CSRC, "relattn_fwd_bf16.hip")
DECODE_SRC = os.path.join(CSRC, "relattn_decode.hip")
BWD_SRC = os.path.join(CSRC, "relattn_backward.hip")
WINDOW_SRC = os.path.join(CSRC, "relattn_window.hip")
# headers every kernel source includes (tile layout, device helpers, parameters)
SHARED_HEADERS = [os.path.join(CSRC, h) for h in
                  ("relattn_device.h", "relattn_internal.h", "relattn_tiles.h")]
# the kernel source each measured arm runs: the lean bf16 kernel serves the Shaw
# tables at d = 64, the small-window kernel the 7 x 7 windows, the general
# kernel the other forward arms
TRAFFIC_SRC = {"base": LEAN_SRC, "big_causal_k": LEAN_SRC, "big_causal_kv": LEAN_SRC,
               "long": KERNEL_SRC, "t5": KERNEL_SRC, "alibi": KERNEL_SRC, "xl": KERNEL_SRC,
               "swin": WINDOW_SRC, "edge": KERNEL_SRC, "edge_kv": KERNEL_SRC,
               "xl128": KERNEL_SRC,
               "decode": DECODE_SRC, "decode_xl": DECODE_SRC}


# ---------------------------------------------------------------------------
# algorithmic work per call
# ---------------------------------------------------------------------------

def work(w, key_lens):
    """(flops, bytes, dense_flops) the method must do for one call.

    flops: 4*d per visible (query, key) pair (content logits and P.V) plus
    2*d*n*R per relative table (the Q.(w^K)^T product and the bucketed
    alpha.w^V product), R = reachable clipped offsets.  bytes: q and out once,
    k and v rows up to the key length once, plus the tables.
    """
    import numpy as np
    B, H, n, d = w.batch, w.heads, w.n, w.d
    esz = w.dtype.itemsize
    lens = [n] * B if key_lens is None else [int(x) for x in key_lens]
    pairs = 0
    for L in lens:
        i = np.arange(n)
        vis = np.minimum(i + 1, L) if w.causal else np.full(n, L)
        pairs += int(vis.sum())
    flops = 4.0 * d * pairs * H
    tables = 0
    if w.t5 is None:
        R = min(w.clip + 1, n) if w.causal else min(2 * w.clip + 1, 2 * n - 1)
        ntab = int(w.use_key_table) + int(w.use_value_table)
        flops += 2.0 * d * n * R * ntab * B * H
        tables = ntab * H * (2 * w.clip + 1) * d * esz
    else:
        tables = w.t5["num_buckets"] * H * 4
    kv_rows = sum(lens)
    nbytes = H * (2 * B * n * d + 2 * kv_rows * d) * esz + tables
    dense = 4.0 * B * H * n * n * d
    return flops, float(nbytes), dense


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def _prepare(ra, w, copies, stream_ptr):
    """Device copies of the inputs and pre-marshalled ctypes arguments."""
    import torch
    import workloads
    x = workloads.make_inputs(w)
    calls = []
    keep = []
    for _ in range(copies):
        g = {k: (t.to("cuda").clone() if t is not None else None) for k, t in x.items()}
        out = torch.empty_like(g["q"])
        if w.t5 is None:
            args, kp = ra._args(g["q"], g["k"], g["v"], g["key_table"], g["value_table"], None,
                                w.clip, w.causal, g["key_lens"], 32, 128, True, None, out)
        else:
            args, kp = ra._args(g["q"], g["k"], g["v"], None, None, g["t5_bias"], 0, w.causal,
                                g["key_lens"], w.t5["num_buckets"], w.t5["max_distance"],
                                w.t5["bidirectional"], None, out)
        calls.append(args + [ctypes.c_void_p(stream_ptr)])
        keep += [g, out, kp]
    return x, calls, keep


def time_gpu(ra, w, steps, warmup, hot=False, reps=1):
    """Time ``steps`` back-to-back calls on one stream, ``reps`` times.

    Cold (default): the calls cycle through enough input copies to exceed twice
    the last-level cache, so operands come from HBM.  Hot: one set of inputs
    for every call, so they stay cache-resident.  ms_per_step is the median
    over the repetitions (the single timed region when reps == 1).
    """
    import statistics
    import torch
    lib = ra._load()
    stream = torch.cuda.Stream()  # default priority
    flops, nbytes, dense = work(w, None)
    copies = 1 if hot else max(1, min(16, int(2 * LLC_BYTES // max(nbytes, 1)) + 1))
    x, calls, keep = _prepare(ra, w, copies, stream.cuda_stream)
    flops, nbytes, dense = work(w, x["key_lens"])
    fwd = lib.relattn_fwd
    times = []
    with torch.cuda.stream(stream):
        for s in range(warmup):
            st = fwd(*calls[s % copies])
            if st != 0:
                raise RuntimeError(lib.relattn_last_error().decode())
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        for r in range(reps):
            wall0 = time.perf_counter()
            t0.record(stream)
            for s in range(steps):
                fwd(*calls[s % copies])
            t1.record(stream)
            wall_submit = time.perf_counter() - wall0
            torch.cuda.synchronize()
            times.append(t0.elapsed_time(t1) / steps)
    ms = statistics.median(times)
    del keep
    sec = ms * 1e-3
    dt = "bf16" if w.dtype.itemsize == 2 else "f32"
    res = {
        "ms_per_step": ms,
        "tflops": flops / sec / 1e12,
        "mfma_peak_frac": flops / sec / 1e12 / PEAK_TFLOPS[dt],
        "dense_equiv_tflops": dense / sec / 1e12,
        "hbm_gbs": nbytes / sec / 1e9,
        "alg_gflop": flops / 1e9,
        "alg_mbytes": nbytes / 1e6,
        "input_copies": copies,
        "host_submit_us_per_step": wall_submit / steps * 1e6,
        "dtype": dt,
        "roofline_frac": flops / sec / 1e12 / ceiling_tflops(flops, nbytes, dt),
        "ms_reps": times,
    }
    return res


def time_gpu_graph(ra, w, steps, warmup, reps=5):
    """The same K back-to-back calls captured once into a HIP graph and replayed:
    the kernels and their inputs are those of time_gpu (cold input copies); the
    host submits one graph launch instead of K kernel launches.  Returns ms per
    call (median over the replays) and the host time per call of a replay."""
    import statistics
    import torch
    lib = ra._load()
    stream = torch.cuda.Stream()  # default priority
    flops, nbytes, dense = work(w, None)
    copies = max(1, min(16, int(2 * LLC_BYTES // max(nbytes, 1)) + 1))
    x, calls, keep = _prepare(ra, w, copies, stream.cuda_stream)
    fwd = lib.relattn_fwd
    with torch.cuda.stream(stream):
        for s in range(warmup):
            if fwd(*calls[s % copies]) != 0:
                raise RuntimeError(lib.relattn_last_error().decode())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for s in range(steps):
            if fwd(*calls[s % copies]) != 0:
                raise RuntimeError(lib.relattn_last_error().decode())
    torch.cuda.synchronize()
    times, submit = [], []
    with torch.cuda.stream(stream):
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        for r in range(reps):
            t0.record(stream)
            w0 = time.perf_counter()
            g.replay()
            submit.append((time.perf_counter() - w0) / steps * 1e6)
            t1.record(stream)
            torch.cuda.synchronize()
            times.append(t0.elapsed_time(t1) / steps)
    del g, keep
    return {"ms_per_step": statistics.median(times), "host_submit_us_per_step":
            statistics.median(submit), "steps": steps, "reps": reps, "input_copies": copies}


def ceiling_tflops(flops, nbytes, dt):
    """Roofline ceiling min(MFMA peak, arithmetic intensity x HBM peak), TFLOP/s."""
    return min(PEAK_TFLOPS[dt], flops / nbytes * PEAK_HBM_GBS / 1e3)


# ---------------------------------------------------------------------------
# incremental decoding (the newest position of each sequence over its cache)
# ---------------------------------------------------------------------------

def time_calls(lib, fn, calls, steps, warmup, reps, stream):
    """Median over ``reps`` timed regions of the time per call (ms) of ``steps``
    back-to-back calls of the C entry point ``fn``, cycling through the argument
    lists ``calls``, on ``stream`` between two HIP events, after ``warmup``
    untimed calls."""
    import statistics
    import torch
    times = []
    with torch.cuda.stream(stream):
        for s_ in range(warmup):
            if fn(*calls[s_ % len(calls)]) != 0:
                raise RuntimeError(lib.relattn_last_error().decode())
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        for _ in range(reps):
            t0.record(stream)
            for s_ in range(steps):
                fn(*calls[s_ % len(calls)])
            t1.record(stream)
            torch.cuda.synchronize()
            times.append(t0.elapsed_time(t1) / steps)
    return statistics.median(times)


def decode_work(w, cache_lens):
    """(flops, bytes) one decoding step must do: q.k and p.v for every visible
    key (4*d per key), the relative key term for the labels (2*d*(k+1)) and
    the value term (2*d*(k+1)) per query; bytes: every visible cache row of k
    and v once, q and out once, the tables once."""
    esz = w.dtype.itemsize
    keys = sum(int(x) for x in cache_lens) * w.heads * w.tq
    rows = w.batch * w.heads * w.tq
    flops = 4.0 * w.d * keys + 2 * 2.0 * w.d * (w.clip + 1) * rows
    cache_bytes = 2.0 * sum(int(x) for x in cache_lens) * w.heads * w.d * esz
    nbytes = cache_bytes + 2.0 * rows * w.d * esz + 2 * w.heads * (2 * w.clip + 1) * w.d * esz
    return flops, nbytes


def time_decode(ra, w, steps, warmup, hot=False, reps=1):
    """Time ``steps`` back-to-back decoding steps (median of ``reps`` timed
    regions).  Cold: the steps cycle through enough cache copies to exceed
    twice the last-level cache; hot: one cache, reused by every step."""
    import torch
    import workloads
    lib = ra._load()
    stream = torch.cuda.Stream()  # default priority
    x = workloads.make_decode_inputs(w)
    flops, nbytes = decode_work(w, x["cache_lens"].tolist())
    copies = 1 if hot else max(1, min(16, int(2 * LLC_BYTES // nbytes) + 1))
    calls, keep = [], []
    for _ in range(copies):
        g = {k: v.to("cuda").clone() for k, v in x.items()}
        out = torch.empty_like(g["q"])
        need = ra.decode_workspace_size(g["q"], g["k"], g["v"], g["key_table"], g["value_table"],
                                        clip=w.clip, out=out)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        args, kp = ra._dec_args(g["q"], g["k"], g["v"], g["key_table"], g["value_table"], None,
                                w.clip, 32, 128, True, None)
        outv = ra._view(out)
        calls.append(args + [ctypes.c_void_p(g["cache_lens"].data_ptr()), ctypes.byref(outv),
                             ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(need),
                             ctypes.c_void_p(stream.cuda_stream)])
        keep += [g, out, ws, kp, outv]
    fn = lib.relattn_decode
    ms = time_calls(lib, fn, calls, steps, warmup, reps, stream)
    del keep
    return {"ms_per_step": ms, "gbs": nbytes / (ms * 1e-3) / 1e9,
            "tflops": flops / (ms * 1e-3) / 1e12, "alg_mbytes": nbytes / 1e6,
            "alg_gflop": flops / 1e9, "input_copies": copies,
            "tokens_per_s": w.batch * w.tq / (ms * 1e-3)}


def decode_report(ra, steps):
    """The decode workload's figures for the JSON line (not the headline)."""
    import workloads
    w = workloads.DECODE_WORKLOADS["decode"]
    cold = time_decode(ra, w, steps, 20, reps=5)
    hot = time_decode(ra, w, steps, 20, hot=True, reps=5)
    tr = traffic_per_launch("decode")
    sec = cold["ms_per_step"] * 1e-3
    return {
        "workload": w.description, "ms_per_step": round(cold["ms_per_step"], 5),
        "tokens_per_s": round(cold["tokens_per_s"], 1),
        "roofline": {"bound": "hbm", "achieved": round(cold["gbs"], 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(cold["gbs"] / PEAK_HBM_GBS, 4),
                     "traffic": None if tr is None else round(tr)},
        "tflops": round(cold["tflops"], 3), "alg_mbytes_per_step": round(cold["alg_mbytes"], 3),
        "hot_ms_per_step": round(hot["ms_per_step"], 5), "input_copies": cold["input_copies"],
        "steps_per_rep": steps,
        "kernels": "decode_partial_kernel (streams the cache) + decode_combine_kernel",
    }


XL_DECODE_SEED = 20260011


def time_decode_xl(ra, w, steps, warmup, hot=False, reps=1):
    """The decode workload's caches and queries with Transformer-XL logits: a
    position table over every distance of the cache (window L - 1) and per-head
    u and v, seeded.  flops: 4*d per visible key (q.k, p.v) + 2*d ((q + v).R);
    bytes: every visible cache row of k and v once, q and out once, the table
    rows the longest row reaches once, u and v."""
    import torch
    import workloads
    lib = ra._load()
    stream = torch.cuda.Stream()  # default priority
    x = workloads.make_decode_inputs(w)
    lens = x["cache_lens"].tolist()
    W = w.cache - 1
    g0 = torch.Generator().manual_seed(XL_DECODE_SEED)
    R = (torch.randn(w.heads, 2 * W + 1, w.d, generator=g0) * 0.5).to(w.dtype)
    u = (torch.randn(w.heads, w.d, generator=g0) * 0.5).to(w.dtype)
    vb = (torch.randn(w.heads, w.d, generator=g0) * 0.5).to(w.dtype)
    esz = w.dtype.itemsize
    keys = sum(int(n) for n in lens) * w.heads * w.tq
    flops = 6.0 * w.d * keys
    nbytes = (2.0 * sum(int(n) for n in lens) * w.heads * w.d * esz
              + 2.0 * w.batch * w.heads * w.tq * w.d * esz
              + w.heads * max(int(n) for n in lens) * w.d * esz + 2 * w.heads * w.d * esz)
    copies = 1 if hot else max(1, min(16, int(2 * LLC_BYTES // nbytes) + 1))
    calls, keep = [], []
    for _ in range(copies):
        g = {k: t.to("cuda").clone() for k, t in x.items()}
        t5 = [R.to("cuda"), u.to("cuda"), vb.to("cuda")]
        out = torch.empty_like(g["q"])
        need = ra.decode_xl_workspace_size(g["q"], g["k"], g["v"], *t5, W, out=out)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        views = [ra._view(t) for t in (g["q"], g["k"], g["v"], *t5)]
        outv = ra._view(out)
        calls.append([ctypes.byref(vw) for vw in views] +
                     [ctypes.c_int32(W), ctypes.c_float(0.0),
                      ctypes.c_void_p(g["cache_lens"].data_ptr()), ctypes.byref(outv),
                      ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(max(need, 16)),
                      ctypes.c_void_p(stream.cuda_stream)])
        keep += [g, t5, out, ws, views, outv]
    fn = lib.relattn_decode_xl
    ms = time_calls(lib, fn, calls, steps, warmup, reps, stream)
    del keep
    return {"ms_per_step": ms, "gbs": nbytes / (ms * 1e-3) / 1e9,
            "tflops": flops / (ms * 1e-3) / 1e12, "alg_mbytes": nbytes / 1e6,
            "input_copies": copies, "tokens_per_s": w.batch * w.tq / (ms * 1e-3)}


def decode_xl_report(ra, steps):
    import workloads
    w = workloads.DECODE_WORKLOADS["decode"]
    cold = time_decode_xl(ra, w, steps, 20, reps=5)
    hot = time_decode_xl(ra, w, steps, 20, hot=True, reps=5)
    tr = traffic_per_launch("decode_xl")
    return {
        "workload": w.description.replace("clip 16, key+value tables",
                                          "Transformer-XL logits, position table over every "
                                          "distance (window 1023), per-head u and v"),
        "ms_per_step": round(cold["ms_per_step"], 5),
        "tokens_per_s": round(cold["tokens_per_s"], 1),
        "roofline": {"bound": "hbm", "achieved": round(cold["gbs"], 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(cold["gbs"] / PEAK_HBM_GBS, 4),
                     "traffic": None if tr is None else round(tr)},
        "tflops": round(cold["tflops"], 3), "alg_mbytes_per_step": round(cold["alg_mbytes"], 3),
        "hot_ms_per_step": round(hot["ms_per_step"], 5), "input_copies": cold["input_copies"],
        "steps_per_rep": steps,
    }


# ---------------------------------------------------------------------------
# scalar bias by clipped offset: causal ALiBi on the T5 shape
# ---------------------------------------------------------------------------

ALIBI = {"name": "alibi", "batch": 8, "heads": 12, "n": 1024, "d": 64, "seed": 20260007,
         "description": "causal ALiBi (-m_h |j - i|, slopes 2^(-8(h+1)/H), window n-1) as a "
                        "table by offset: B8 H12 n1024 d64, bf16"}


def alibi_inputs():
    import torch
    a = ALIBI
    g = torch.Generator().manual_seed(a["seed"])
    q, k, v = (torch.randn(a["batch"], a["heads"], a["n"], a["d"], generator=g).to(torch.bfloat16)
               for _ in range(3))
    W, H = a["n"] - 1, a["heads"]
    slopes = [2.0 ** (-8.0 * (h + 1) / H) for h in range(H)]
    bias = torch.tensor([[-m * abs(x) for x in range(-W, W + 1)] for m in slopes],
                        dtype=torch.float32)
    return q, k, v, bias, W


def time_alibi(ra, steps, warmup, hot=False, reps=5):
    import torch
    lib = ra._load()
    stream = torch.cuda.Stream()
    q, k, v, bias, W = alibi_inputs()
    a = ALIBI
    B, H, n, d = a["batch"], a["heads"], a["n"], a["d"]
    pairs = B * H * n * (n + 1) // 2
    flops = 4.0 * d * pairs
    nbytes = 4.0 * B * H * n * d * 2 + bias.numel() * 4
    copies = 1 if hot else max(1, min(16, int(2 * LLC_BYTES // nbytes) + 1))
    calls, keep = [], []
    for _ in range(copies):
        g = [x.to("cuda").clone() for x in (q, k, v, bias)]
        out = torch.empty_like(g[0])
        args, kp = ra._ob_args(g[0], g[1], g[2], g[3], W, True, None, None, out)
        calls.append(args + [ctypes.c_void_p(stream.cuda_stream)])
        keep += [g, out, kp]
    fn = lib.relattn_fwd_offset_bias
    ms = time_calls(lib, fn, calls, steps, warmup, reps, stream)
    del keep
    sec = ms * 1e-3
    return {"ms_per_step": ms, "tflops": flops / sec / 1e12, "hbm_gbs": nbytes / sec / 1e9,
            "alg_gflop": flops / 1e9, "alg_mbytes": nbytes / 1e6, "input_copies": copies}


def alibi_report(ra, steps):
    cold = time_alibi(ra, steps, 10)
    hot = time_alibi(ra, steps, 10, hot=True)
    ceil = ceiling_tflops(cold["alg_gflop"] * 1e9, cold["alg_mbytes"] * 1e6, "bf16")
    flops, nbytes = cold["alg_gflop"] * 1e9, cold["alg_mbytes"] * 1e6
    bound = bound_of(flops, nbytes, "bf16")
    sec = cold["ms_per_step"] * 1e-3
    if bound == "hbm":
        ach, peak, unit = nbytes / sec / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        ach, peak, unit = flops / sec / 1e12, PEAK_TFLOPS["bf16"], "TFLOP/s"
    tr = traffic_per_launch("alibi")
    return {"workload": ALIBI["description"], "ms_per_step": round(cold["ms_per_step"], 5),
            "tflops": round(cold["tflops"], 3),
            "roofline": {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                         "frac": round(ach / peak, 4),
                         "traffic": None if tr is None else round(tr)},
            "mfma_peak_frac": round(cold["tflops"] / PEAK_TFLOPS["bf16"], 4),
            "roofline_frac": round(cold["tflops"] / ceil, 4),
            "bound": bound_of(cold["alg_gflop"] * 1e9, cold["alg_mbytes"] * 1e6, "bf16"),
            "hbm_gbs": round(cold["hbm_gbs"], 1), "hot_ms_per_step": round(hot["ms_per_step"], 5),
            "alg_gflop_per_step": round(cold["alg_gflop"], 4), "steps_per_rep": steps}


# ---------------------------------------------------------------------------
# backward (relattn_bwd: dq/dk/dv kernels and the table-gradient reduction)
# ---------------------------------------------------------------------------



def bwd_work(w, key_lens):
    """(flops, bytes) one backward call must do.

    flops: 10*d per visible pair (the logits again, dP = dz.v, and the dV,
    dK and dQ products) plus, per query row and reachable label, 2*d for each
    of: the relative logit q.w^K (again), dQ's G w^K term and dw^K's q G term
    (key table); dz.w^V and dw^V's dz W term (value table).  bytes: q, k, v,
    the output z and dz read once; dq, dk, dv written once; the tables read
    and their gradients (fp32) written once; the row log-sum-exp read once.
    """
    import numpy as np
    B, H, n, d = w.batch, w.heads, w.n, w.d
    esz = w.dtype.itemsize
    lens = [n] * B if key_lens is None else [int(x) for x in key_lens]
    pairs = 0
    for L in lens:
        i = np.arange(n)
        pairs += int((np.minimum(i + 1, L) if w.causal else np.full(n, L)).sum())
    flops = 10.0 * d * pairs * H
    tab_bytes = 0.0
    if w.t5 is None:
        R = min(w.clip + 1, n) if w.causal else min(2 * w.clip + 1, 2 * n - 1)
        per = 3 * int(w.use_key_table) + 2 * int(w.use_value_table)
        flops += 2.0 * d * n * R * per * B * H
        ntab = int(w.use_key_table) + int(w.use_value_table)
        tab_bytes = ntab * H * (2 * w.clip + 1) * d * (esz + 4)
    else:
        tab_bytes = 2 * w.t5["num_buckets"] * H * 4
    nbytes = 8.0 * B * H * n * d * esz + 4.0 * B * H * n + tab_bytes
    return flops, nbytes


def time_bwd(ra, w, steps, warmup, hot=False, reps=5):
    """Time ``steps`` back-to-back relattn_bwd calls (median of ``reps``
    timed regions); cold: the calls cycle through enough input copies to
    exceed twice the last-level cache; hot: one input set."""
    import torch
    import workloads
    lib = ra._load()
    stream = torch.cuda.Stream()  # default priority
    x = workloads.make_inputs(w)
    flops, nbytes = bwd_work(w, x["key_lens"])
    copies = 1 if hot else max(1, min(16, int(2 * LLC_BYTES // nbytes) + 1))
    g0 = torch.Generator().manual_seed(20260009)
    dz_cpu = torch.randn(x["q"].shape, generator=g0).to(x["q"].dtype)
    calls, keep = [], []
    t5 = w.t5 or {}
    for _ in range(copies):
        g = {k: (t.to("cuda").clone() if t is not None else None) for k, t in x.items()}
        dz = dz_cpu.to("cuda")
        kw = dict(clip=w.clip, causal=w.causal, key_lens=g["key_lens"])
        if w.t5 is not None:
            kw.update(t5_bias=g["t5_bias"], **t5)
        out, lse = ra.fwd_lse(g["q"], g["k"], g["v"], g["key_table"], g["value_table"], **kw)
        grads = ra._bwd_outputs(g["q"], g["key_table"], g["value_table"], g["t5_bias"], None,
                                None, None, None, None, None, True, True, True)
        args, kp = ra._bwd_args(g["q"], g["k"], g["v"], g["key_table"], g["value_table"],
                                g["t5_bias"], w.clip, w.causal, g["key_lens"],
                                t5.get("num_buckets", 32), t5.get("max_distance", 128),
                                t5.get("bidirectional", True), None, out, dz, lse, grads)
        need = ctypes.c_size_t(0)
        if lib.relattn_bwd_workspace_size(*args, ctypes.byref(need)) != 0:
            raise RuntimeError(lib.relattn_last_error().decode())
        ws = torch.empty(max(need.value, 1), dtype=torch.uint8, device="cuda")
        calls.append(args + [ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(need.value),
                             ctypes.c_void_p(stream.cuda_stream)])
        keep += [g, dz, out, lse, grads, kp, ws]
    torch.cuda.synchronize()
    fn = lib.relattn_bwd
    ms = time_calls(lib, fn, calls, steps, warmup, reps, stream)
    del keep
    sec = ms * 1e-3
    return {"ms_per_step": ms, "tflops": flops / sec / 1e12, "hbm_gbs": nbytes / sec / 1e9,
            "alg_gflop": flops / 1e9, "alg_mbytes": nbytes / 1e6, "input_copies": copies,
            "workspace_mbytes": need.value / 1e6}


def bwd_report(ra, steps, name=HEADLINE):
    """The backward's figures on a workload (the headline's by default)."""
    import workloads
    w = workloads.WORKLOADS[name]
    cold = time_bwd(ra, w, steps, 10)
    hot = time_bwd(ra, w, steps, 10, hot=True)
    flops, nbytes = cold["alg_gflop"] * 1e9, cold["alg_mbytes"] * 1e6
    bound = bound_of(flops, nbytes, "bf16" if w.dtype.itemsize == 2 else "f32")
    sec = cold["ms_per_step"] * 1e-3
    dt = "bf16" if w.dtype.itemsize == 2 else "f32"
    if bound == "hbm":
        ach, peak, unit = nbytes / sec / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        ach, peak, unit = flops / sec / 1e12, PEAK_TFLOPS[dt], "TFLOP/s"
    tr = traffic_per_launch("bwd_" + name)
    return {"workload": w.description, "ms_per_step": round(cold["ms_per_step"], 5),
            "tflops": round(cold["tflops"], 3),
            "mfma_peak_frac": round(cold["tflops"] / PEAK_TFLOPS[dt], 4),
            "roofline": {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                         "frac": round(ach / peak, 4),
                         "traffic": None if tr is None else round(tr)},
            "roofline_frac": round(cold["tflops"] / ceiling_tflops(flops, nbytes, dt), 4),
            "hbm_gbs": round(cold["hbm_gbs"], 1), "hot_ms_per_step": round(hot["ms_per_step"], 5),
            "alg_gflop_per_step": round(cold["alg_gflop"], 4),
            "alg_mbytes_per_step": round(cold["alg_mbytes"], 3),
            "workspace_mbytes": round(cold["workspace_mbytes"], 3),
            "input_copies": cold["input_copies"], "steps_per_rep": steps,
            "kernels": "bwd_q_kernel (dq, label sums, table partials) + bwd_kv_kernel (dk, dv, "
                       "then the table-gradient sums)"}



def bwd_arms_report(ra, steps):
    """The backward passes of the other arms on their workloads: ms per call
    (HIP events over back-to-back calls after a warm-up, one input set, so the
    operands may sit in the last-level cache), beside the forward-with-lse call
    that produces their lse.  No roofline: these passes are built for coverage
    (one workgroup shape per mode, per-pair label and entry gathers)."""
    import torch
    import workloads
    torch.manual_seed(20260011)
    dev = "cuda"

    def ms(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(n):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n

    out = {}
    x = workloads.make_grid_inputs("swin")
    q, k, v, bias = (x[t].to(dev) for t in ("q", "k", "v", "bias"))
    M = workloads.GRID_WORKLOADS["swin"].side
    dz = torch.randn_like(q)
    o, lse = ra.fwd_grid_bias_lse(q, k, v, bias, M)
    out["grid_bias"] = {
        "workload": workloads.GRID_WORKLOADS["swin"].description,
        "fwd_lse_ms": round(ms(lambda: ra.fwd_grid_bias_lse(q, k, v, bias, M, out=o, lse=lse), steps), 5),
        "bwd_ms": round(ms(lambda: ra.bwd_grid_bias(q, k, v, bias, M, out=o, dout=dz, lse=lse), steps), 5)}
    for name, key in (("edge", "edge_bias"), ("edge_kv", "edge_tables")):
        w = workloads.EDGE_WORKLOADS[name]
        x = workloads.make_edge_inputs(name)
        q, k, v = (x[t].to(dev) for t in ("q", "k", "v"))
        lab = ra.edge_label_buffer(q.shape[0], q.shape[2], dev)
        lab.copy_(x["labels"].to(torch.uint8))
        dz = torch.randn_like(q)
        if w.tables:
            wK, wV = x["wK"].to(dev), x["wV"].to(dev)
            o, lse = ra.fwd_edge_tables_lse(q, k, v, lab, wK, wV)
            f = lambda: ra.fwd_edge_tables_lse(q, k, v, lab, wK, wV, out=o, lse=lse)
            b = lambda: ra.bwd_edge_tables(q, k, v, lab, wK, wV, out=o, dout=dz, lse=lse)
        else:
            bias = x["bias"].to(dev)
            o, lse = ra.fwd_edge_bias_lse(q, k, v, lab, bias)
            f = lambda: ra.fwd_edge_bias_lse(q, k, v, lab, bias, out=o, lse=lse)
            b = lambda: ra.bwd_edge_bias(q, k, v, lab, bias, out=o, dout=dz, lse=lse)
        out[key] = {"workload": w.description, "fwd_lse_ms": round(ms(f, steps), 5),
                    "bwd_ms": round(ms(b, steps), 5)}
    x = workloads.make_xl_inputs("xl")
    q, k, v, R, u, vb = (x[t].to(dev) for t in ("q", "k", "v", "R", "u", "vb"))
    W = x["window"]
    dz = torch.randn_like(q)
    o, lse = ra.fwd_xl_lse(q, k, v, R, u, vb, W, causal=True)
    out["xl"] = {
        "workload": workloads.XL_WORKLOADS["xl"].description,
        "fwd_lse_ms": round(ms(lambda: ra.fwd_xl_lse(q, k, v, R, u, vb, W, causal=True, out=o,
                                                      lse=lse), steps), 5),
        "bwd_ms": round(ms(lambda: ra.bwd_xl(q, k, v, R, u, vb, W, out=o, dout=dz, lse=lse,
                                              causal=True), max(5, steps // 10)), 5)}
    return out

# ---------------------------------------------------------------------------
# Transformer-XL relative logits (relattn_fwd_xl)
# ---------------------------------------------------------------------------

def xl_work(w):
    """(flops, bytes) of one call: 6*d per visible pair (terms (a) and (b) of the
    score, and P.V; terms (c) and (d) are the query shifts, O(n d)); bytes: q,
    k, v, out once, the position table and the biases once."""
    B, H, n, d = w.batch, w.heads, w.n, w.d
    esz = w.dtype.itemsize
    pairs = B * H * (n * (n + 1) // 2 if w.causal else n * n)
    W = min(w.window, n - 1)
    flops = 6.0 * d * pairs
    nbytes = 4.0 * B * H * n * d * esz + H * (2 * W + 1 + 2) * d * esz
    return flops, nbytes


def time_xl(ra, steps, warmup, hot=False, reps=5, name="xl"):
    import torch
    import workloads
    lib = ra._load()
    stream = torch.cuda.Stream()
    w = workloads.XL_WORKLOADS[name]
    x = workloads.make_xl_inputs(w)
    flops, nbytes = xl_work(w)
    copies = 1 if hot else max(1, min(16, int(2 * LLC_BYTES // nbytes) + 1))
    calls, keep = [], []
    for _ in range(copies):
        g = {k: (t.to("cuda").clone() if isinstance(t, torch.Tensor) else t) for k, t in x.items()}
        out = torch.empty_like(g["q"])
        args, kp = ra._xl_args(g["q"], g["k"], g["v"], g["R"], g["u"], g["vb"], g["window"],
                               w.causal, None, None, out)
        calls.append(args + [ctypes.c_void_p(stream.cuda_stream)])
        keep += [g, out, kp]
    fn = lib.relattn_fwd_xl
    ms = time_calls(lib, fn, calls, steps, warmup, reps, stream)
    del keep
    sec = ms * 1e-3
    return {"ms_per_step": ms, "tflops": flops / sec / 1e12, "hbm_gbs": nbytes / sec / 1e9,
            "alg_gflop": flops / 1e9, "alg_mbytes": nbytes / 1e6, "input_copies": copies}


def xl_report(ra, steps, name="xl"):
    import workloads
    w = workloads.XL_WORKLOADS[name]
    cold = time_xl(ra, steps, 10, name=name)
    hot = time_xl(ra, steps, 10, hot=True, name=name)
    flops, nbytes = cold["alg_gflop"] * 1e9, cold["alg_mbytes"] * 1e6
    bound = bound_of(flops, nbytes, "bf16")
    sec = cold["ms_per_step"] * 1e-3
    if bound == "hbm":
        ach, peak, unit = nbytes / sec / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        ach, peak, unit = flops / sec / 1e12, PEAK_TFLOPS["bf16"], "TFLOP/s"
    tr = traffic_per_launch(name)
    return {"workload": w.description, "ms_per_step": round(cold["ms_per_step"], 5),
            "tflops": round(cold["tflops"], 3),
            "mfma_peak_frac": round(cold["tflops"] / PEAK_TFLOPS["bf16"], 4),
            "roofline": {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                         "frac": round(ach / peak, 4),
                         "traffic": None if tr is None else round(tr)},
            "hbm_gbs": round(cold["hbm_gbs"], 1), "hot_ms_per_step": round(hot["ms_per_step"], 5),
            "alg_gflop_per_step": round(cold["alg_gflop"], 4),
            "alg_mbytes_per_step": round(cold["alg_mbytes"], 3),
            "input_copies": cold["input_copies"], "steps_per_rep": steps}


# ---------------------------------------------------------------------------
# 2-D window bias (relattn_fwd_grid_bias)
# ---------------------------------------------------------------------------

def grid_work(w):
    """(flops, bytes) of one call: 4*d per pair (every key of a window is
    visible); bytes: q, k, v, out once and the table once."""
    n = w.side * w.side
    pairs = w.batch * w.heads * n * n
    return 4.0 * w.d * pairs, 4.0 * w.batch * w.heads * n * w.d * w.dtype.itemsize + \
        w.heads * (2 * w.side - 1) ** 2 * 4


def time_grid(ra, steps, warmup, hot=False, reps=5):
    import torch
    import workloads
    lib = ra._load()
    stream = torch.cuda.Stream()
    w = workloads.GRID_WORKLOADS["swin"]
    x = workloads.make_grid_inputs(w)
    flops, nbytes = grid_work(w)
    copies = 1 if hot else max(1, min(16, int(2 * LLC_BYTES // nbytes) + 1))
    calls, keep = [], []
    for _ in range(copies):
        g = {k: t.to("cuda").clone() for k, t in x.items()}
        out = torch.empty_like(g["q"])
        args, kp = ra._ob_args(g["q"], g["k"], g["v"], g["bias"], w.side, False, None, None, out)
        calls.append(args + [ctypes.c_void_p(stream.cuda_stream)])
        keep += [g, out, kp]
    fn = lib.relattn_fwd_grid_bias
    ms = time_calls(lib, fn, calls, steps, warmup, reps, stream)
    del keep
    sec = ms * 1e-3
    return {"ms_per_step": ms, "tflops": flops / sec / 1e12, "hbm_gbs": nbytes / sec / 1e9,
            "alg_gflop": flops / 1e9, "alg_mbytes": nbytes / 1e6, "input_copies": copies}


def grid_report(ra, steps):
    import workloads
    w = workloads.GRID_WORKLOADS["swin"]
    cold = time_grid(ra, steps, 10)
    hot = time_grid(ra, steps, 10, hot=True)
    flops, nbytes = cold["alg_gflop"] * 1e9, cold["alg_mbytes"] * 1e6
    bound = bound_of(flops, nbytes, "bf16")
    sec = cold["ms_per_step"] * 1e-3
    if bound == "hbm":
        ach, peak, unit = nbytes / sec / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        ach, peak, unit = flops / sec / 1e12, PEAK_TFLOPS["bf16"], "TFLOP/s"
    tr = traffic_per_launch("swin")
    return {"workload": w.description, "ms_per_step": round(cold["ms_per_step"], 5),
            "tflops": round(cold["tflops"], 3),
            "roofline": {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                         "frac": round(ach / peak, 4),
                         "traffic": None if tr is None else round(tr)},
            "hbm_gbs": round(cold["hbm_gbs"], 1), "hot_ms_per_step": round(hot["ms_per_step"], 5),
            "alg_gflop_per_step": round(cold["alg_gflop"], 4),
            "alg_mbytes_per_step": round(cold["alg_mbytes"], 3),
            "input_copies": cold["input_copies"], "steps_per_rep": steps}


# ---------------------------------------------------------------------------
# Scalar bias by per-pair edge label (relattn_fwd_edge_bias)
# ---------------------------------------------------------------------------

def edge_work(w):
    """(flops, bytes) of one call: 4*d per pair (no mask: every key visible),
    plus with key and value tables 2*d per (query, label) for q.w^K and for the
    weight sums times W^V; bytes: q, k, v, out once, the table(s) once and the
    label matrix once (one byte per pair of a batch entry, shared by its
    heads)."""
    pairs = w.batch * w.heads * w.n * w.n
    flops = 4.0 * w.d * pairs
    nbytes = 4.0 * w.batch * w.heads * w.n * w.d * w.dtype.itemsize + w.batch * w.n * w.n
    if w.tables:
        flops += 2 * 2.0 * w.d * w.batch * w.heads * w.n * w.labels
        nbytes += 2 * w.heads * w.labels * w.d * w.dtype.itemsize
    else:
        nbytes += w.heads * w.labels * 4
    return flops, nbytes


def time_edge(ra, steps, warmup, hot=False, reps=5, name="edge"):
    import torch
    import workloads
    lib = ra._load()
    stream = torch.cuda.Stream()
    w = workloads.EDGE_WORKLOADS[name]
    x = workloads.make_edge_inputs(w)
    flops, nbytes = edge_work(w)
    copies = 1 if hot else max(1, min(16, int(2 * LLC_BYTES // nbytes) + 1))
    calls, keep = [], []
    for _ in range(copies):
        g = {k: t.to("cuda").clone() for k, t in x.items() if k != "labels"}
        lab = ra.edge_label_buffer(w.batch, w.n, "cuda")
        lab.copy_(x["labels"].to(torch.uint8))
        out = torch.empty_like(g["q"])
        if w.tables:
            args, kp = ra._edge_args(g["q"], g["k"], g["v"], lab, None, w.causal, None, None,
                                     out, (g["wK"], g["wV"]))
        else:
            args, kp = ra._edge_args(g["q"], g["k"], g["v"], lab, g["bias"], w.causal, None,
                                     None, out)
        calls.append(args + [ctypes.c_void_p(stream.cuda_stream)])
        keep += [g, lab, out, kp]
    fn = lib.relattn_fwd_edge_tables if w.tables else lib.relattn_fwd_edge_bias
    ms = time_calls(lib, fn, calls, steps, warmup, reps, stream)
    del keep
    sec = ms * 1e-3
    return {"ms_per_step": ms, "tflops": flops / sec / 1e12, "hbm_gbs": nbytes / sec / 1e9,
            "alg_gflop": flops / 1e9, "alg_mbytes": nbytes / 1e6, "input_copies": copies}


def edge_report(ra, steps, name="edge"):
    import workloads
    w = workloads.EDGE_WORKLOADS[name]
    cold = time_edge(ra, steps, 10, name=name)
    hot = time_edge(ra, steps, 10, hot=True, name=name)
    flops, nbytes = cold["alg_gflop"] * 1e9, cold["alg_mbytes"] * 1e6
    bound = bound_of(flops, nbytes, "bf16")
    sec = cold["ms_per_step"] * 1e-3
    if bound == "hbm":
        ach, peak, unit = nbytes / sec / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        ach, peak, unit = flops / sec / 1e12, PEAK_TFLOPS["bf16"], "TFLOP/s"
    tr = traffic_per_launch(name)
    return {"workload": w.description, "ms_per_step": round(cold["ms_per_step"], 5),
            "tflops": round(cold["tflops"], 3),
            "roofline": {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                         "frac": round(ach / peak, 4),
                         "traffic": None if tr is None else round(tr)},
            "hbm_gbs": round(cold["hbm_gbs"], 1), "hot_ms_per_step": round(hot["ms_per_step"], 5),
            "alg_gflop_per_step": round(cold["alg_gflop"], 4),
            "alg_mbytes_per_step": round(cold["alg_mbytes"], 3),
            "input_copies": cold["input_copies"], "steps_per_rep": steps}


def bound_of(flops, nbytes, dt):
    ridge = PEAK_TFLOPS[dt] * 1e12 / (PEAK_HBM_GBS * 1e9)
    return "hbm" if flops / nbytes < ridge else "mfma"


# ---------------------------------------------------------------------------
# HBM traffic from committed rocprofv3 counter summaries
# ---------------------------------------------------------------------------

def kernel_sha(path=KERNEL_SRC):
    """sha256 over a kernel source and the headers it shares with the others."""
    h = hashlib.sha256()
    for fn in [path] + SHARED_HEADERS:
        with open(fn, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_source(name):
    return BWD_SRC if name.startswith("bwd_") else TRAFFIC_SRC[name]


def traffic_per_launch(name):
    """Measured HBM bytes per launch, or None when the counters are missing or
    were taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_sha256") != kernel_sha(traffic_source(name)):
        return None
    return t["fetch_kib"] * 1024 * t["fetch_scale"] + t["write_kib"] * 1024 * t["write_scale"]


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle as it stands, on the host cores
# ---------------------------------------------------------------------------

def cpu_baseline(w, min_seconds=12.0):
    import oracle
    import workloads
    from threadpoolctl import threadpool_info
    x = workloads.make_inputs(w)
    flops, _, _ = work(w, x["key_lens"])
    reps, t0 = 0, time.perf_counter()
    while True:
        if w.t5 is None:
            oracle.relattn_factored(x["q"], x["k"], x["v"], x["key_table"], x["value_table"],
                                    w.clip, causal=w.causal, key_lens=x["key_lens"])
        else:
            oracle.t5_attention(x["q"], x["k"], x["v"], x["t5_bias"], causal=w.causal,
                                key_lens=x["key_lens"], **w.t5)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    import torch
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops * reps / el / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "cpu": host_cpu_model(), "blas_threads": threads,
            "torch_threads": torch.get_num_threads(),
            "sample": f"whole {w.name} workload, fp64 factored oracle (Eq. 5 form, numpy with "
                      f"{threads} BLAS thread(s)), {reps} run(s) in {el:.1f} s, "
                      f"{len(os.sched_getaffinity(0))} host cores visible"}


def host_cpu_model():
    """Model name of the host CPU (first entry of /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_report(per_workload_s=2.0):
    """Wall time of the fp64 oracle per workload on the host cores.

    Factored oracle (Eq. 5 form; T5: its definition) on whole workloads where a
    call is short, else on a few (b, h) heads, scaled to the whole workload;
    brute force (materialised n x n x d edge tensors) on the tiny and base
    workloads; row-sampled brute force elsewhere, as time per output row.
    """
    import numpy as np
    import oracle
    import workloads
    rng = np.random.default_rng(0)
    rep = {}
    for name in ["tiny", "base", "big_causal_k", "big_causal_kv", "long", "t5"]:
        w = workloads.WORKLOADS[name]
        x = workloads.make_inputs(w)
        B, H = w.batch, w.heads
        lens = x["key_lens"]
        kw = dict(causal=w.causal)

        def head_slice(bs, hs):
            y = {k: x[k] for k in ("q", "k", "v")}
            y = {k: t[bs, hs] for k, t in y.items()}
            kl = None if lens is None else lens[bs]
            return y, kl

        def factored(bs, hs):
            y, kl = head_slice(bs, hs)
            if w.t5 is None:
                kt = None if x["key_table"] is None else x["key_table"][hs]
                vt = None if x["value_table"] is None else x["value_table"][hs]
                oracle.relattn_factored(y["q"], y["k"], y["v"], kt, vt, w.clip,
                                        key_lens=kl, **kw)
            else:
                oracle.t5_attention(y["q"], y["k"], y["v"], x["t5_bias"][:, hs],
                                    key_lens=kl, **kw, **w.t5)

        # factored: grow the sample of heads until it takes about per_workload_s
        nb, nh, el = 1, 1, 0.0
        while True:
            t0 = time.perf_counter()
            factored(slice(0, nb), slice(0, nh))
            el = time.perf_counter() - t0
            if el >= per_workload_s / 4 or (nb == B and nh == H):
                break
            if nh < H:
                nh = min(H, nh * 2)
            else:
                nb = min(B, nb * 2)
        entry = {"factored_s_per_call": el * (B * H) / (nb * nh),
                 "factored_sample_heads": nb * nh}
        if name in ("tiny", "base"):
            t0 = time.perf_counter()
            oracle.relattn_bruteforce(x["q"], x["k"], x["v"], x["key_table"],
                                      x["value_table"], w.clip, key_lens=lens, **kw)
            entry["bruteforce_s_per_call"] = time.perf_counter() - t0
        else:
            nrows = 16
            rows = [(int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(w.n)))
                    for _ in range(nrows)]
            t0 = time.perf_counter()
            if w.t5 is None:
                oracle.relattn_rows(x["q"], x["k"], x["v"], x["key_table"], x["value_table"],
                                    w.clip, key_lens=lens, rows=rows, **kw)
            else:
                oracle.t5_rows(x["q"], x["k"], x["v"], x["t5_bias"], key_lens=lens,
                               rows=rows, **kw, **w.t5)
            entry["bruteforce_s_per_row"] = (time.perf_counter() - t0) / nrows
            entry["bruteforce_rows"] = nrows
        rep[name] = {k: (round(v, 6) if isinstance(v, float) else v) for k, v in entry.items()}
    # decode: per-row brute force (Eq. 3 and Eq. 4 key by key) on 8 rows
    wd = workloads.DECODE_WORKLOADS["decode"]
    xd = workloads.make_decode_inputs(wd)
    lens = xd["cache_lens"].tolist()
    t0 = time.perf_counter()
    for r in range(8):
        b, h = int(rng.integers(wd.batch)), int(rng.integers(wd.heads))
        sl = lambda t: t[b:b + 1, h:h + 1]
        oracle.relattn_decode(sl(xd["q"]), sl(xd["k"]), sl(xd["v"]), xd["key_table"][h:h + 1],
                              xd["value_table"][h:h + 1], wd.clip, cache_lens=[lens[b]])
    el = (time.perf_counter() - t0) / 8
    rep["decode"] = {"bruteforce_s_per_row": round(el, 6), "bruteforce_rows": 8,
                     "bruteforce_s_per_step": round(el * wd.batch * wd.heads * wd.tq, 3)}
    # backward: the chain-rule oracle on 4 heads of the headline workload
    w = workloads.WORKLOADS[HEADLINE]
    x = workloads.make_inputs(w)
    dz = x["q"].float()
    t0 = time.perf_counter()
    for h in range(4):
        sl = lambda t: t[0:1, h:h + 1]
        oracle.relattn_backward(sl(x["q"]), sl(x["k"]), sl(x["v"]), x["key_table"][h:h + 1],
                                x["value_table"][h:h + 1], w.clip, sl(dz), causal=w.causal)
    el = (time.perf_counter() - t0) / 4
    rep["backward_" + HEADLINE] = {"s_per_head": round(el, 6), "sample_heads": 4,
                                   "s_per_call": round(el * w.batch * w.heads, 3)}
    return rep


def gpu_identity():
    """Marketing name, ISA and peak engine clock of the first GPU agent (rocminfo)."""
    import subprocess
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    for agent in txt.split("Agent ")[1:]:
        if "Device Type:             GPU" not in agent:
            continue
        info = {}
        for line in agent.splitlines():
            key, _, val = line.strip().partition(":")
            val = val.strip()
            if key == "Marketing Name" and "name" not in info:
                info["name"] = val
            elif key == "Name" and val.startswith("gfx") and "isa" not in info:
                info["isa"] = val
            elif key == "Max Clock Freq. (MHz)" and "max_clock_mhz" not in info:
                info["max_clock_mhz"] = int(val.split()[0])
            elif key == "Compute Unit" and "compute_units" not in info:
                info["compute_units"] = int(val.split()[0])
        return info
    return None


def copy_calibration(mib=512, reps=5):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    a = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": mib << 20, "reps": reps}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--only", action="store_true",
                    help="time the headline workload only (no per-workload table, no oracle report)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="time the decode workload only and print its figures")
    ap.add_argument("--alibi-only", action="store_true",
                    help="time the offset-bias (ALiBi) workload only and print its figures")
    ap.add_argument("--bwd-only", action="store_true",
                    help="time the backward on --workload only and print its figures")
    ap.add_argument("--xl-only", action="store_true",
                    help="time the Transformer-XL workload only and print its figures")
    ap.add_argument("--xl128-only", action="store_true",
                    help="time the Transformer-XL workload with 128-wide heads only")
    ap.add_argument("--grid-only", action="store_true",
                    help="time the 2-D window (Swin) workload only and print its figures")
    ap.add_argument("--edge-only", action="store_true",
                    help="time the edge-label workload only and print its figures")
    ap.add_argument("--decode-xl-only", action="store_true",
                    help="time the Transformer-XL decode workload only and print its figures")
    ap.add_argument("--edge-tables-only", action="store_true",
                    help="time the edge-label workload with key and value tables only")
    a = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {a.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)

    gpu = None if a.copy_calibration else gpu_identity()  # before this process uses the GPU
    import torch
    import relative_position_encoding_amd as ra
    import workloads
    if not os.path.exists(ra.library_path):
        from relative_position_encoding_amd import build
        build.build()
    if a.copy_calibration:
        copy_calibration()
        return
    if a.decode_only:
        print(json.dumps({"decode": decode_report(ra, max(50, a.steps // 5))}))
        return
    if a.alibi_only:
        print(json.dumps({"offset_bias": alibi_report(ra, max(50, a.steps // 5))}))
        return
    if a.bwd_only:
        print(json.dumps({"backward": bwd_report(ra, max(50, a.steps // 5), a.workload)}))
        return
    if a.xl_only:
        print(json.dumps({"xl": xl_report(ra, max(50, a.steps // 5))}))
        return
    if a.xl128_only:
        print(json.dumps({"xl128": xl_report(ra, max(50, a.steps // 5), "xl128")}))
        return
    if a.grid_only:
        print(json.dumps({"grid_bias": grid_report(ra, max(50, a.steps // 5))}))
        return
    if a.edge_only:
        print(json.dumps({"edge_bias": edge_report(ra, max(50, a.steps // 5))}))
        return
    if a.decode_xl_only:
        print(json.dumps({"decode_xl": decode_xl_report(ra, max(50, a.steps // 5))}))
        return
    if a.edge_tables_only:
        print(json.dumps({"edge_tables": edge_report(ra, max(50, a.steps // 5), "edge_kv")}))
        return

    if gpu is not None and not gpu.get("name"):
        gpu["name"] = torch.cuda.get_device_name(0)
    w = workloads.WORKLOADS[a.workload]
    head = time_gpu(ra, w, a.steps, a.warmup)
    flops = head["alg_gflop"] * 1e9
    nbytes = head["alg_mbytes"] * 1e6
    bound = bound_of(flops, nbytes, head["dtype"])
    sec = head["ms_per_step"] * 1e-3
    if bound == "hbm":
        ach, peak, unit = nbytes / sec / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        ach, peak, unit = flops / sec / 1e12, PEAK_TFLOPS[head["dtype"]], "TFLOP/s"
    traffic = traffic_per_launch(w.name)
    mask = ("causal" if w.causal else "") + ("+key_padding" if w.len_range else "")
    tables = ("t5_bias" if w.t5 else
              "+".join([x for x, u in (("key", w.use_key_table), ("value", w.use_value_table))
                        if u]) or "none")
    line = {
        "metric": METRIC, "value": round(head["tflops"], 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": head["dtype"], "data": "synthetic",
        "config": {"workload": w.description, "name": w.name, "batch": w.batch,
                   "heads": w.heads, "seq_len": w.n, "head_dim": w.d, "clip": w.clip,
                   "mask": mask or "none", "tables": tables,
                   "input_copies": head["input_copies"]},
        "mfma_peak_frac": round(head["mfma_peak_frac"], 4),
        "hbm_gbs": round(head["hbm_gbs"], 1),
        "dense_equiv_tflops": round(head["dense_equiv_tflops"], 3),
        "roofline": {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                     "frac": round(ach / peak, 4),
                     "traffic": None if traffic is None else round(traffic)},
        "alg_gflop_per_step": round(head["alg_gflop"], 4),
        "alg_mbytes_per_step": round(head["alg_mbytes"], 3),
        "host_submit_us_per_step": round(head["host_submit_us_per_step"], 2),
        "gpu": gpu,
    }
    # the same calls captured in one HIP graph and replayed (launch-bound loops)
    gr = time_gpu_graph(ra, w, a.steps, a.warmup)
    line["graph"] = {"ms_per_step": round(gr["ms_per_step"], 5),
                     "host_submit_us_per_step": round(gr["host_submit_us_per_step"], 3),
                     "steps": gr["steps"], "replays": gr["reps"],
                     "note": "the timed calls captured once into a HIP graph, replayed whole"}
    if not a.only:
        # every workload, the headline included: median of 5 timed regions with
        # inputs streamed from HBM (cold) and with one cache-resident input set (hot)
        per = {}
        for name in [w.name] + [x for x in OTHER if x != w.name]:
            wl = workloads.WORKLOADS[name]
            k = max(50, a.steps // 5)
            cold = time_gpu(ra, wl, k, 10, reps=5)
            hot = time_gpu(ra, wl, k, 10, hot=True, reps=5)
            e = {key: round(cold[key], 4) for key in
                 ("ms_per_step", "tflops", "mfma_peak_frac", "hbm_gbs", "dense_equiv_tflops",
                  "roofline_frac")}
            e["bound"] = bound_of(cold["alg_gflop"] * 1e9, cold["alg_mbytes"] * 1e6,
                                  cold["dtype"])
            tr = traffic_per_launch(name)
            e["traffic"] = None if tr is None else round(tr)
            e["hot_ms_per_step"] = round(hot["ms_per_step"], 5)
            e["hot_tflops"] = round(hot["tflops"], 4)
            e["steps_per_rep"] = k
            per[name] = e
        line["workloads"] = per
        line["decode"] = decode_report(ra, max(50, a.steps // 5))
        line["decode_xl"] = decode_xl_report(ra, max(50, a.steps // 5))
        line["offset_bias"] = alibi_report(ra, max(50, a.steps // 5))
        line["backward"] = bwd_report(ra, max(50, a.steps // 5))
        line["xl"] = xl_report(ra, max(50, a.steps // 5))
        line["xl128"] = xl_report(ra, max(50, a.steps // 5), "xl128")
        line["grid_bias"] = grid_report(ra, max(50, a.steps // 5))
        line["edge_bias"] = edge_report(ra, max(50, a.steps // 5))
        line["edge_tables"] = edge_report(ra, max(50, a.steps // 5), "edge_kv")
        line["backward_arms"] = bwd_arms_report(ra, max(20, a.steps // 10))
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
        if not a.only:
            line["oracle_timing"] = oracle_report()
    print(json.dumps(line))


if __name__ == "__main__":
    main()
