#!/usr/bin/env python3
"""Benchmark of one INT8-KV decode step on one MI355X.

A step is the whole hot path for one new token of one sequence:
  kvq_plan (host)  ->  kv_append_decode_splitk (the token's K/V quantized and
  written into the cache, fused with the split-K partials)  ->  kv_decode_reduce
on the long-context workload: batch 1, 16 query / 2 kv heads, head_dim 256,
int8 codes under an fp16 scale per 64-value group, context 131072 (K with 1 % outlier
channels x20). Inputs are seeded synthetic data (workloads.py), resident in HBM
before timing.

The 132 MiB cache fits in the 256 MB Infinity Cache, so the timed steps rotate
over 8 identical copies of the cache (1.1 GB): each step streams a copy that
was not touched for 7 steps and has been evicted.

Timing: the headline step time replays a HIP graph that holds one step per
cache copy (split plan fixed at capture, context lengths read on the device),
so kernels run back to back; per-kernel averages come from graphs of 8
back-to-back launches of that kernel. Eager (per-launch, host-driven) step
time, and the same step as three calls (kv_quant_append, kv_decode_attn_splitk,
kv_decode_reduce), are reported beside it.

Prints one JSON line: value = KV bytes read per step / step time (GB/s), the
roofline of the partial kernel from HIP events over the timed region, and the
CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
COPIES = 8
TOL = 2e-3


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


Q4_SOURCES = ("kvq_decode_q4.hip", "kvq_q4_tile.h", "kvq_q4.h", "kvq_tile.h", "kvq_device.h")


def _code_only(text: str) -> str:
    """C++/HIP source with its comments removed and whitespace runs collapsed:
    what the compiler sees, so that a comment edit does not count as a kernel
    change (none of these sources has a comment marker inside a string)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_digest(files=("kvq_decode.hip", "kvq_tile.h", "kvq_device.h")) -> str:
    """Digest of the code (comments excluded) of the sources a kernel is built from."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "int8_quantized_kv_quant_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(digest: str, plan, name: str = "partial_long_128k_traffic.json", kernel: str | None = None):
    """HBM bytes per partial launch measured with rocprofv3 counters, if they
    were taken on the current kernel source and with the same split plan
    (n_splits, chunk); else None."""
    p = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if kernel is not None:
        d = d.get("kernels", {}).get(kernel, {})
    if d.get("kernel_src_sha") != digest or d.get("plan") != [plan.n_splits, plan.chunk]:
        return None
    return d.get("hbm_bytes_per_launch")


def oracle_seq(w, b, L, q_b):
    """fp64 oracle output [n_q][d] of sequence b of workload w at context L
    (w's window and store types), from the workload's own rows."""
    from oracle import kvq_oracle as orc
    import workloads as wl
    lo = max(0, L - w.window) if w.window else 0
    c = orc.Cache(1, L, w.n_kv_heads, w.head_dim, w.scale_group, w.k_dtype, w.v_dtype)
    c.append(wl.kv_rows(w, "k", b, lo, L - lo)[None], wl.kv_rows(w, "v", b, lo, L - lo)[None], [lo])
    return orc.attend(np.asarray(q_b)[None], c, [L], w.window, 1.0 / math.sqrt(w.head_dim))[0]


def codes_match(kvq_setup, lay, cache, w, b, positions):
    """True if the cache rows (b, positions) of every kv head hold exactly the
    oracle's quantization of the workload's rows: int8 codes and fp16 scales,
    Q4_0 bytes and block scales, or the fp16 values widened for an fp32 store."""
    from oracle import kvq_oracle as orc
    import workloads as wl
    positions = np.asarray(positions)
    ok = True
    for s, dt in (("k", w.k_dtype), ("v", w.v_dtype)):
        rows = np.concatenate([wl.kv_rows(w, s, b, int(p), 1) for p in positions])
        for h in range(w.n_kv_heads):
            if dt == "int8":
                want_c, want_s = orc.quantize_rows(rows[:, h], w.scale_group)
                got_c = kvq_setup.rows_of(lay, cache[s], b, positions, h)
                got_s = kvq_setup.scales_of(lay, cache[s + "_scales"], b, positions, h)
                ok &= bool(np.array_equal(got_c, want_c) and np.array_equal(got_s.view(np.uint16), want_s.view(np.uint16)))
            elif dt == "q4":
                codes, want_s = orc.quantize_q4_0(orc.rotate_f32(rows[:, h]))
                got = kvq_setup.q4_rows_of(lay, cache[s], b, positions, h)
                got_s = kvq_setup.scales_of(lay, cache[s + "_scales"], b, positions, h, n=w.head_dim // 32)
                ok &= bool(np.array_equal(got, orc.pack_q4(codes)) and
                           np.array_equal(got_s.view(np.uint16), want_s.view(np.uint16)))
            else:
                got = kvq_setup.rows_of(lay, cache[s], b, positions, h)
                ok &= bool(np.array_equal(got.view(np.uint32), rows[:, h].astype(np.float32).view(np.uint32)))
    return ok


def cpu_info():
    """Host cores and CPU model (for the CPU-baseline record)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"os_cpu_count": os.cpu_count(), "cpu_model": model,
            "sched_affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def cpu_quantize_baseline(seconds=3.0):
    """The oracle's quantize leg timed on the host: orc.quantize_rows of the
    mixed workload's 2048-token chunk (both kv heads, K and V as int8 group-64
    rows of head_dim 256), repeated for about `seconds`, with the BLAS threads
    it has by default. Returns values quantized per second and the repeats."""
    from oracle import kvq_oracle as orc
    import workloads as wl
    w = wl.WORKLOADS["mixed_k8v32"]
    rows = [wl.kv_rows(w, s, 0, w.prefill, w.append) for s in ("k", "v")]
    n_vals = sum(r.size for r in rows)
    reps, t0 = 0, time.perf_counter()
    while True:
        for r in rows:
            orc.quantize_rows(r, w.scale_group)
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    return {"values_per_s": round(n_vals / dt, 1), "seconds_per_chunk": round(dt, 4), "repeats": reps,
            "sample": f"quantize_rows of the {w.append}-token chunk of the mixed workload: K and V, "
                      f"{w.n_kv_heads} kv heads x {w.head_dim} values per row ({n_vals} values), group-64 scales"}


def cpu_baseline(w, lens, q, sm):
    """The oracle as it stands, timed on the host: decode attention of the full
    step (both kv heads, 131072 positions) over the dequantized cache in fp64,
    repeated for about 10 s with the BLAS threads it has by default, then for
    about 10 s on one thread. Returns (output, seconds per step, threads,
    repetitions, seconds per step on one thread, its repetitions, the oracle's
    cache)."""
    from oracle import kvq_oracle as orc
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        cores = os.cpu_count() or 1
    L = int(lens[0])
    cache = orc.Cache(1, L, w.n_kv_heads, w.head_dim, w.scale_group, w.k_dtype, w.v_dtype)
    cache.append(wl.kv_rows(w, "k", 0, 0, L)[None], wl.kv_rows(w, "v", 0, 0, L)[None], [0])

    def timed():
        reps, t0 = 0, time.perf_counter()
        while True:  # repeat the step until about 10 s of host work have been timed
            out = orc.attend(q, cache, lens, 0, sm)
            reps += 1
            if time.perf_counter() - t0 >= 10.0:
                return out, (time.perf_counter() - t0) / reps, reps

    want, dt, reps = timed()
    dt1, reps1 = None, None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            _, dt1, reps1 = timed()
    return want, dt, cores, reps, dt1, reps1, cache


def stream_reference(kvq, n_cu):
    """Bytes per second of kvq_stream_read (a read-only kernel of contiguous
    per-workgroup slices, non-temporal 128-bit loads) over 4 GiB: median and
    best of 20 timed launches after 3 warm-ups, in GB/s."""
    import torch
    n = 1 << 32
    buf = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    for _ in range(3):
        kvq.kvq_stream_read(buf, n, sink, n_cu)
    torch.cuda.synchronize()
    ts = []
    for _ in range(20):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        kvq.kvq_stream_read(buf, n, sink, n_cu)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    del buf
    torch.cuda.empty_cache()
    return n / float(np.median(ts)) / 1e9, n / float(np.min(ts)) / 1e9, n


def stream_at(kvq, n_cu, nbytes, copies=COPIES):
    """What one launch of the read-only streaming kernel takes for exactly
    `nbytes`: kvq_stream_read over `copies` rotating buffers of that size
    (each last read `copies - 1` launches earlier, so not served by the
    Infinity Cache), graphs of back-to-back launches as the decode steps are
    timed; median over 5 timings of 2 graph replays. Returns us and GB/s."""
    import torch
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda:0") for _ in range(copies)]
    for b in bufs:
        kvq.kvq_stream_read(b, nbytes, sink, n_cu)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for b in bufs:
            kvq.kvq_stream_read(b, nbytes, sink, n_cu)
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / (2 * copies))
    del bufs, g
    torch.cuda.empty_cache()
    us = float(np.median(ts))
    return {"us": round(us, 2), "GB_s": round(nbytes / us / 1e3, 1),
            "pct_hbm_peak": round(100 * nbytes / us / 1e3 / HBM_PEAK_GBS, 2)}


def secondary_workloads(kvq, kvq_setup, wl, n_cu, steps):
    """The decode step (kv_append_decode_splitk + kv_decode_reduce, graph-replayed)
    on the other two shapes the metric is quoted on, and the chunk attention of
    a prompt chunk (chunk_workload):
      gemma_4k  -- 8 query / 1 kv head, head_dim 256 in a 512-wide slot, one scale
                   per (position, kv head), context 4096 with a 512-key window;
      batched   -- 64 sequences of lengths U[1024, 32768], 32 query / 8 kv heads,
                   head_dim 128, group-64 scales (2.2 GB of KV per step);
      mixed     -- k8v32 and k32v8 stores (16 query / 2 kv heads, head_dim 256):
                   the 2048-token append at 30000, then the step at 32048.
    Gemma rows come from workloads.py; the batched cache (1.1 G values) is filled
    through kv_quant_append from rows drawn on the device with a seeded
    torch.Generator (timing only: its parity is covered by the GPU tests)."""
    import torch
    dev = torch.device("cuda:0")
    res = {}

    def timed(w, lens, lay, caches, k_new, v_new, parity=None, one_call=False):
        """Graph-replayed decode steps over the cache copies; parity(out, q)
        -> dict of checks on the output of the last step (every copy holds the
        same rows, so every step's output is the same). one_call: the step is
        one kv_decode_attn call (one kernel launch for plans of at most 8
        splits over int8 stores), else kv_append_decode_splitk +
        kv_decode_reduce."""
        B = w.batch
        qd = torch.from_numpy(wl.queries(w)).to(dev)
        ld = torch.from_numpy(lens.astype(np.int32)).to(dev)
        sm = 1.0 / math.sqrt(w.head_dim)
        plan = kvq.kvq_plan(lay, B, w.n_q_heads, w.max_ctx, w.window, n_cu)
        ws = torch.zeros(plan.ws_bytes, dtype=torch.uint8, device=dev)
        out = torch.empty((B, w.n_q_heads, w.head_dim), dtype=torch.float16, device=dev)
        arrive = torch.zeros(kvq.arrive_count(lay, B, w.n_q_heads), dtype=torch.int32, device=dev)

        def step(c):
            if one_call:
                kvq.kv_decode_attn(lay, c["k"], c["v"], c["k_scales"], c["v_scales"], k_new, v_new, qd, B,
                                   w.n_q_heads, ld, w.window, sm, plan, ws, ws.numel(), arrive, out)
                return
            kvq.kv_append_decode_splitk(lay, c["k"], c["v"], c["k_scales"], c["v_scales"], k_new, v_new, qd, B,
                                        w.n_q_heads, ld, w.window, sm, plan, ws, ws.numel())
            kvq.kv_decode_reduce(lay, ws, ws.numel(), ld, B, w.n_q_heads, w.window, plan, out)

        for c in caches:
            step(c)
        torch.cuda.synchronize()
        # COPIES steps per graph (cycling over the cache copies), so that one
        # graph launch covers several steps
        rounds = max(1, COPIES // len(caches))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(rounds):
                for c in caches:
                    step(c)
        g.replay()
        torch.cuda.synchronize()
        per_graph = rounds * len(caches)
        reps = max(2, steps // per_graph)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * per_graph)
        kvb = wl.kv_bytes_per_step(w, lens)
        res = {"us_per_step": round(us, 2), "kv_bytes_per_step": int(kvb), "GB_s": round(kvb / us / 1e3, 1),
               "pct_hbm_peak": round(100 * kvb / us / 1e3 / HBM_PEAK_GBS, 2), "n_splits": plan.n_splits,
               "chunk": plan.chunk, "steps": reps * per_graph, "steps_per_graph": per_graph}
        if one_call:
            res["launches"] = kvq.kvq_decode_launches(lay, B, w.n_q_heads, plan)
            res["arrive_left_zero"] = int(torch.count_nonzero(arrive)) == 0
        if parity is not None:
            res.update(parity(out.float().cpu().numpy().astype(np.float64), wl.queries(w)))
        return res

    def single_parity(w, L, lay, cache, extra_positions=()):
        """max abs error of sequence 0 against the oracle at context L, and the
        codes of the appended row and of sampled rows bit-exact."""
        def check(got, q):
            err = float(np.abs(got[0] - oracle_seq(w, 0, L, q[0])).max())
            rng = np.random.default_rng(5)
            pos = np.unique(np.concatenate([rng.integers(0, L, 64), [L - 1], np.asarray(extra_positions, dtype=np.int64)]))
            return {"max_abs_err": err, "codes_bitexact": codes_match(kvq_setup, lay, cache, w, 0, pos),
                    "tol": TOL}
        return check

    for key, name in (("tiny", "tiny"), ("gemma_4k", "gemma")):
        w = wl.WORKLOADS[name]
        L = w.contexts[-1]
        lens = np.array([L], dtype=np.int32)
        lay, c0 = kvq_setup.fill_cache(w, lens, upto=np.array([L - 1]))
        caches = [c0] + [{k: (None if t is None else t.clone()) for k, t in c0.items()} for _ in range(COPIES - 1)]
        k_new = torch.from_numpy(wl.kv_rows(w, "k", 0, L - 1, 1)).to(dev)
        v_new = torch.from_numpy(wl.kv_rows(w, "v", 0, L - 1, 1)).to(dev)
        two = timed(w, lens, lay, caches, k_new, v_new)
        res[key] = {"context": L, "window": w.window, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                    "head_dim": w.head_dim, "cache_copies": COPIES,
                    "step": "kv_decode_attn (append, partials and the combine in one launch: plans of <= 8 "
                            "splits over int8 stores, query heads in units of <= 512 / head_dim)",
                    **timed(w, lens, lay, caches, k_new, v_new, single_parity(w, L, lay, caches[-1]), one_call=True),
                    "two_call_us_per_step": two["us_per_step"],
                    "two_call_step": "kv_append_decode_splitk + kv_decode_reduce"}
        del caches, c0

    res["prefill_chunk"] = chunk_workload(kvq, kvq_setup, wl, n_cu)
    res["prefill_chunk_q4"] = chunk_workload(kvq, kvq_setup, wl, n_cu, "long_q4")

    # Mixed stores: positions [0, 30000) prefilled, the 2048-token chunk
    # quantize-appended at 30000 (timed on its own: it rewrites the same rows,
    # so the cache is unchanged, which is checked), then the decode step at
    # context 32048 over 8 cache copies.
    for name in ("mixed_k8v32", "mixed_k32v8"):
        w = wl.WORKLOADS[name]
        L = w.prefill + w.append
        lens = np.array([L], dtype=np.int32)
        lay, c0 = kvq_setup.fill_cache(w, lens)
        kr = torch.from_numpy(wl.kv_rows(w, "k", 0, w.prefill, w.append)).to(dev)
        vr = torch.from_numpy(wl.kv_rows(w, "v", 0, w.prefill, w.append)).to(dev)
        app = append_chunk_timing(kvq, wl, w, lay, c0)
        caches = [c0] + [{k: (None if t is None else t.clone()) for k, t in c0.items()} for _ in range(COPIES - 1)]
        k_new = torch.from_numpy(wl.kv_rows(w, "k", 0, L - 1, 1)).to(dev)
        v_new = torch.from_numpy(wl.kv_rows(w, "v", 0, L - 1, 1)).to(dev)
        chunk_rows = np.arange(w.prefill, w.prefill + w.append, 97)
        res[name] = {"k_store": w.k_dtype, "v_store": w.v_dtype, "context": L, "cache_copies": COPIES,
                     **app, **timed(w, lens, lay, caches, k_new, v_new,
                                    single_parity(w, L, lay, caches[-1], extra_positions=chunk_rows))}
        del caches, c0
        torch.cuda.empty_cache()

    w = wl.WORKLOADS["batched"]
    lens = wl.seq_lens(w)
    lay = kvq_setup.layout_for(w)
    cache = kvq.alloc_cache(lay, w.batch, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    # Four sampled sequences (the shortest, the longest and two others) hold
    # the workload's own rows and are checked against the oracle; the other 60
    # are filled from rows drawn on the device (1.1 G host-drawn values would
    # dominate the run).
    sampled = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 7, 40})
    for b in range(w.batch):
        p, n_fill = 0, int(lens[b]) - 1
        while p < n_fill:
            n = min(16384, n_fill - p)
            if b in sampled:
                kvq_setup.append_rows(lay, cache, b, p, wl.kv_rows(w, "k", b, p, n), wl.kv_rows(w, "v", b, p, n))
            else:
                rows = torch.randn((2, n, w.n_kv_heads, w.head_dim), generator=gen, device=dev).half()
                kvq_setup.append_rows_device(lay, cache, b, p, rows[0], rows[1])
            p += n
    new = torch.randn((2, w.batch, w.n_kv_heads, w.head_dim), generator=gen, device=dev).half()
    for b in sampled:
        Lb = int(lens[b])
        new[0, b] = torch.from_numpy(wl.kv_rows(w, "k", b, Lb - 1, 1)[0]).to(dev)
        new[1, b] = torch.from_numpy(wl.kv_rows(w, "v", b, Lb - 1, 1)[0]).to(dev)

    def batched_parity(got, q):
        err = max(float(np.abs(got[b] - oracle_seq(w, b, int(lens[b]), q[b])).max()) for b in sampled)
        rng = np.random.default_rng(6)
        ok = all(codes_match(kvq_setup, lay, cache, w, b,
                             np.unique(np.concatenate([rng.integers(0, int(lens[b]), 32), [int(lens[b]) - 1]])))
                 for b in sampled)
        return {"max_abs_err": err, "codes_bitexact": ok, "tol": TOL,
                "parity_sequences": [int(b) for b in sampled]}

    res["batched"] = {"batch": w.batch, "contexts": "U[1024, 32768]", "total_positions": int(lens.sum()),
                      **timed(w, lens, lay, [cache], new[0].contiguous(), new[1].contiguous(), batched_parity)}
    del cache
    torch.cuda.empty_cache()
    return res


def append_chunk_timing(kvq, wl, w, lay, c0, reps=25):
    """kv_quant_append of the mixed workload's chunk (w.append tokens at
    position w.prefill, both kv heads) into the cache c0, which already holds
    those rows: the rewrite must leave it bit-identical (checked). Timed as
    graphs of COPIES back-to-back appends (one graph launch per COPIES kernels,
    so the host's launch rate does not bound the figure)."""
    import torch
    dev = c0["k"].device
    kr = torch.from_numpy(wl.kv_rows(w, "k", 0, w.prefill, w.append)).to(dev)
    vr = torch.from_numpy(wl.kv_rows(w, "v", 0, w.prefill, w.append)).to(dev)
    sp = torch.tensor([w.prefill], dtype=torch.int32, device=dev)
    before = {k: (None if t is None else t.clone()) for k, t in c0.items()}

    def append():
        kvq.kv_quant_append(lay, c0["k"], c0["v"], c0["k_scales"], c0["v_scales"], kr, vr, sp, 1, w.append)

    append()
    torch.cuda.synchronize()
    same = all(t is None or torch.equal(t.view(torch.uint8), c0[k].view(torch.uint8)) for k, t in before.items())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(COPIES):
            append()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    app_us = e0.elapsed_time(e1) * 1e3 / (reps * COPIES)
    same = same and all(t is None or torch.equal(t.view(torch.uint8), c0[k].view(torch.uint8))
                        for k, t in before.items())
    # fp16 rows in; per store int8 codes + fp16 scales, or fp32 values, out
    n_rows = w.append * w.n_kv_heads
    out_b = sum(w.head_dim + 2 * w.n_groups if dt == "int8" else 4 * w.head_dim for dt in (w.k_dtype, w.v_dtype))
    app_bytes = n_rows * (2 * 2 * w.head_dim + out_b)
    del g, before
    return {"append_tokens": w.append, "append_at": w.prefill, "append_us": round(app_us, 2),
            "append_bytes": int(app_bytes), "append_GB_s": round(app_bytes / app_us / 1e3, 1),
            "append_frac_hbm": round(app_bytes / app_us / 1e3 / HBM_PEAK_GBS, 4),
            "append_launches_per_graph": COPIES, "append_rewrite_bitexact": bool(same)}


def chunk_workload(kvq, kvq_setup, wl, n_cu, name="long"):
    """kv_chunk_attn (partials + combine) on a 2048-token prompt chunk at
    position 30000 of the long-context layout (16 query / 2 kv heads, head_dim
    256, group-64 scales; keys 0..32047 in the cache, causal inside the chunk;
    name="long_q4": the same over the q4_0 layout). Algorithmic work:
    4 * head_dim flops per (token, query head, attended key) (Q.K and P.V);
    bound by the matrix cores (fp16 MFMA peak 2.5 PFLOP/s). Two sampled tokens
    are checked against the fp64 oracle."""
    import torch
    from oracle import kvq_oracle as orc
    dev = torch.device("cuda:0")
    w = wl.WORKLOADS[name].with_(max_ctx=32768)
    T, start = 2048, 30000
    end = start + T
    lay, cache = kvq_setup.fill_cache(w, np.array([end]))
    qh = wl.chunk_queries(w, T)
    q = torch.from_numpy(qh).to(dev)
    sp = torch.tensor([start], dtype=torch.int32, device=dev)
    sm = 1.0 / math.sqrt(w.head_dim)
    plan = kvq.kvq_plan_chunk(lay, 1, T, w.n_q_heads, end, 0, n_cu)
    ws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((1, T, w.n_q_heads, w.head_dim), dtype=torch.float16, device=dev)

    def call():
        kvq.kv_chunk_attn(lay, cache["k"], cache["v"], cache["k_scales"], cache["v_scales"], q, 1, T, w.n_q_heads,
                          sp, 0, sm, plan, ws, ws.numel(), out)

    call()
    torch.cuda.synchronize()
    reps = 10
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    toks = [(0, 5), (0, T - 1)]
    oc = orc.Cache(1, end, w.n_kv_heads, w.head_dim, w.scale_group, w.k_dtype, w.v_dtype)
    oc.append(wl.kv_rows(w, "k", 0, 0, end)[None], wl.kv_rows(w, "v", 0, 0, end)[None], [0])
    want = orc.attend_chunk(qh, oc, np.array([start]), 0, sm, tokens=toks)
    got = out.cpu().numpy().astype(np.float64)
    err = max(float(np.abs(got[b, t] - want[b, t]).max()) for b, t in toks)
    keys = sum(start + t + 1 for t in range(T))
    flops = keys * w.n_q_heads * 4 * w.head_dim
    del cache
    torch.cuda.empty_cache()
    return {"tokens": T, "start": start, "context_end": end, "us": round(us, 1),
            "tflops": round(flops / us / 1e6, 1), "bound": "mfma", "peak_tflops": 2500.0,
            "frac": round(flops / us / 1e6 / 2500.0, 4), "algorithmic_flops": int(flops),
            "n_splits": plan.n_splits, "chunk": plan.chunk, "max_abs_err_sampled": err,
            "k_store": w.k_dtype, "v_store": w.v_dtype,
            "kernel": ("kvq_chunk_q4_kernel" if w.k_dtype == "q4" or w.v_dtype == "q4" else "kvq_chunk_kernel")
            + " + kvq_reduce_kernel"}


def verify_windows(kvq, wl, w, lay, L, n_cu, time_us, oc=None, sizes=(2, 4, 8)):
    """kv_chunk_attn (partials + combine) of a verify window of T tokens at
    positions L - T .. L - 1 over the 128K caches of a decode workload
    (time_us(fn) runs fn(cache) over all copies, graph-replayed as the steps
    are, and returns microseconds per call; causal inside the window). Up to
    32 (token, head) rows per kv head go through the decode partial kernels
    (chunk rows), more through the chunk kernels. The first and last token of
    each window are checked against the fp64 oracle (its cache oc of
    positions [0, L), built here if not given)."""
    import torch
    from oracle import kvq_oracle as orc
    dev = torch.device("cuda:0")
    sm = 1.0 / math.sqrt(w.head_dim)
    if oc is None:
        oc = orc.Cache(1, L, w.n_kv_heads, w.head_dim, w.scale_group, w.k_dtype, w.v_dtype)
        oc.append(wl.kv_rows(w, "k", 0, 0, L)[None], wl.kv_rows(w, "v", 0, 0, L)[None], [0])
    kvb = wl.kv_bytes_per_step(w, np.array([L]))
    res = []
    for T in sizes:
        start = L - T
        qh = wl.chunk_queries(w, T)
        q = torch.from_numpy(qh).to(dev)
        sp = torch.tensor([start], dtype=torch.int32, device=dev)
        plan = kvq.kvq_plan_chunk(lay, 1, T, w.n_q_heads, L, 0, n_cu)
        ws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device=dev)
        o = torch.empty((1, T, w.n_q_heads, w.head_dim), dtype=torch.float16, device=dev)

        def call(c):
            kvq.kv_chunk_attn(lay, c["k"], c["v"], c["k_scales"], c["v_scales"], q, 1, T, w.n_q_heads, sp, 0, sm,
                              plan, ws, ws.numel(), o)

        ms = time_us(call) * 1e-3
        got = o.float().cpu().numpy().astype(np.float64)
        toks = [(0, 0), (0, T - 1)]
        want = orc.attend_chunk(qh, oc, np.array([start]), 0, sm, tokens=toks)
        err = max(float(np.abs(got[b, t] - want[b, t]).max()) for b, t in toks)
        rows = T * (w.n_q_heads // w.n_kv_heads)
        res.append({"tokens": T, "start": start, "rows_per_kv_head": rows, "us": round(ms * 1e3, 2),
                    "kv_bytes_once": int(kvb), "GB_s_once": round(kvb / ms / 1e6, 1),
                    "n_splits": plan.n_splits, "chunk": plan.chunk, "max_abs_err_sampled": err, "tol": TOL})
        del ws
    return res


def q4_workloads(kvq, kvq_setup, wl, n_cu, steps):
    """The decode step over the 4-bit stores at the long-context shape (Strata
    PR 2698, "Not in this PR": q4_0 for K and V, k8v4 for V only, Hadamard-
    rotated Q4_0 blocks at head_dim 256), and verify windows of 2 and 4 tokens
    over the same caches: kv_append_decode_splitk (the new
    token's rotation and quantization fused into the partials) +
    kv_decode_reduce, graph-replayed over COPIES caches of 131072 positions;
    the unfused three-call step beside it. The caches hold the workload's own
    rows (kv_quant_append); the step's output is checked against the oracle and
    sampled rows' Q4_0 bytes against the oracle's quantizer. The partial kernel
    is also timed alone (its roofline: algorithmic bytes / launch time)."""
    import torch
    from oracle import kvq_oracle as orc
    dev = torch.device("cuda:0")
    res = {}
    for name in ("long_q4", "long_k8v4"):
        w = wl.WORKLOADS[name]
        L = w.contexts[-1]
        lens = np.array([L], dtype=np.int32)
        lay, c0 = kvq_setup.fill_cache(w, lens, upto=np.array([L - 1]))
        caches = [c0] + [{k: (None if t is None else t.clone()) for k, t in c0.items()} for _ in range(COPIES - 1)]
        new = torch.stack([torch.from_numpy(wl.kv_rows(w, s, 0, L - 1, 1)) for s in ("k", "v")])[:, None].to(dev)
        qd = torch.from_numpy(wl.queries(w)).to(dev)
        ld = torch.from_numpy(lens).to(dev)
        sp = torch.tensor([L - 1], dtype=torch.int32, device=dev)
        sm = 1.0 / math.sqrt(w.head_dim)
        plan = kvq.kvq_plan(lay, 1, w.n_q_heads, w.max_ctx, w.window, n_cu)
        ws = torch.zeros(plan.ws_bytes, dtype=torch.uint8, device=dev)
        out = torch.empty((1, w.n_q_heads, w.head_dim), dtype=torch.float16, device=dev)

        def append(c):
            kvq.kv_quant_append(lay, c["k"], c["v"], c["k_scales"], c["v_scales"], new[0], new[1], sp, 1, 1)

        def fused(c):
            kvq.kv_append_decode_splitk(lay, c["k"], c["v"], c["k_scales"], c["v_scales"], new[0, 0], new[1, 0], qd,
                                        1, w.n_q_heads, ld, w.window, sm, plan, ws, ws.numel())

        def partial(c):
            kvq.kv_decode_attn_splitk(lay, c["k"], c["v"], c["k_scales"], c["v_scales"], qd, 1, w.n_q_heads, ld,
                                      w.window, sm, plan, ws, ws.numel())

        def reduce():
            kvq.kv_decode_reduce(lay, ws, ws.numel(), ld, 1, w.n_q_heads, w.window, plan, out)

        def graph_us(fn):
            for c in caches:
                fn(c)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for c in caches:
                    fn(c)
            g.replay()
            torch.cuda.synchronize()
            reps = max(2, steps // len(caches))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / (reps * len(caches))

        us = graph_us(lambda c: (fused(c), reduce()))
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        # the oracle's cache of positions [0, L) (the step's own row included),
        # for the step and for the verify windows below
        oc = orc.Cache(1, L, w.n_kv_heads, w.head_dim, w.scale_group, w.k_dtype, w.v_dtype)
        oc.append(wl.kv_rows(w, "k", 0, 0, L)[None], wl.kv_rows(w, "v", 0, 0, L)[None], [0])
        err = float(np.abs(got[0] - orc.attend(wl.queries(w)[:1], oc, [L], w.window, sm)[0]).max())
        rng = np.random.default_rng(7)
        codes_ok = codes_match(kvq_setup, lay, caches[-1], w, 0,
                               np.unique(np.concatenate([rng.integers(0, L, 64), [L - 1]])))
        unfused_us = graph_us(lambda c: (append(c), partial(c), reduce()))
        part_us = graph_us(partial)
        fpart_us = graph_us(fused)
        kvb = wl.kv_bytes_per_step(w, lens)
        verify = verify_windows(kvq, wl, w, lay, L, n_cu, graph_us, oc, sizes=(2, 4))
        del oc
        res[name + "_128k"] = {
            "k_store": w.k_dtype, "v_store": w.v_dtype, "context": L, "cache_copies": COPIES,
            "step": "kv_append_decode_splitk + kv_decode_reduce (rotation and quantize-append fused)",
            "us_per_step": round(us, 2), "kv_bytes_per_step": int(kvb), "GB_s": round(kvb / us / 1e3, 1),
            "pct_hbm_peak": round(100 * kvb / us / 1e3 / HBM_PEAK_GBS, 2),
            "unfused_step_us": round(unfused_us, 2),
            "fused_partial_us": round(fpart_us, 2), "fused_partial_frac_hbm": round(kvb / fpart_us / 1e3 / HBM_PEAK_GBS, 4),
            "partial_us": round(part_us, 2), "partial_GB_s": round(kvb / part_us / 1e3, 1),
            "partial_frac_hbm": round(kvb / part_us / 1e3 / HBM_PEAK_GBS, 4),
            "partial_traffic": traffic_from_profiles(kernel_source_digest(Q4_SOURCES), plan,
                                                     "partial_q4_long_128k_traffic.json", name),
            "n_splits": plan.n_splits, "chunk": plan.chunk,
            "max_abs_err": err, "codes_bitexact": codes_ok, "tol": TOL,
            "verify_windows": verify}
        del caches, c0
        torch.cuda.empty_cache()
    return res


def blob_workload(kvq, lay, cache, L):
    """kv_cache_pack / kv_cache_unpack of all L positions of the 128K cache
    (codes with their scales: 138.4 MB of payload). Each direction reads and
    writes the payload once: bound by HBM at 2 x payload bytes per call. The
    unpacked copy is checked bit-identical to the original."""
    import torch
    size = kvq.kvq_blob_size(lay, L)
    blob = torch.empty(size, dtype=torch.uint8, device="cuda:0")
    other = {k: (None if t is None else torch.zeros_like(t)) for k, t in cache.items()}
    hdr = kvq.kv_cache_pack(lay, cache["k"], cache["v"], cache["k_scales"], cache["v_scales"], 0, 0, L, blob, size)
    kvq.kv_cache_unpack(lay, other["k"], other["v"], other["k_scales"], other["v_scales"], 0, 0, hdr, blob, size)
    torch.cuda.synchronize()
    same = all(torch.equal(cache[k], other[k]) for k in cache if cache[k] is not None)
    res = {"payload_bytes": size, "roundtrip_bitexact": same}
    for name, f in (("pack", lambda: kvq.kv_cache_pack(lay, cache["k"], cache["v"], cache["k_scales"],
                                                        cache["v_scales"], 0, 0, L, blob, size)),
                    ("unpack", lambda: kvq.kv_cache_unpack(lay, other["k"], other["v"], other["k_scales"],
                                                            other["v_scales"], 0, 0, hdr, blob, size))):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            f()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 10
        res[name] = {"us": round(us, 1), "GB_s": round(2 * size / us / 1e3, 1),
                     "frac_hbm": round(2 * size / us / 1e3 / HBM_PEAK_GBS, 3)}
    del other, blob
    torch.cuda.empty_cache()
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--order", choices=("pos", "head"), default="pos",
                    help="cache layout: positions major (default) or heads major")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the Gemma 4K and batched-serving timings (profiling runs of the 128K step)")
    ap.add_argument("--only", choices=("append2048",),
                    help="run one sub-benchmark alone (profiling runs): append2048 = the 2048-token "
                         "quantize-append of the mixed-store workloads (k8v32, k32v8)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy three times (the reference for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters of a rocprofv3 --pmc run to bytes)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = 512 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 3}), flush=True)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this decode path has no multi-GPU mode "
              "(one GPU's share of a sharded step is this same kernel at its shape); use --gpus 1", file=sys.stderr)
        return 2

    import torch
    import int8_quantized_kv_quant_amd as kvq
    import kvq_setup
    import workloads as wl
    from oracle import kvq_oracle as orc

    kvq.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n_cu = kvq_setup.n_cu()
    if args.only == "append2048":
        res = {}
        for name in ("mixed_k8v32", "mixed_k32v8"):
            w = wl.WORKLOADS[name]
            log(f"{name}: filling {w.prefill + w.append} positions")
            lay, c0 = kvq_setup.fill_cache(w, np.array([w.prefill + w.append]))
            res[name] = append_chunk_timing(kvq, wl, w, lay, c0)
            del c0
            torch.cuda.empty_cache()
        print(json.dumps({"only": "append2048", **res}), flush=True)
        return 0 if all(r["append_rewrite_bitexact"] for r in res.values()) else 1
    w = wl.WORKLOADS["long"]
    L = w.contexts[-1]
    lens = np.array([L], dtype=np.int32)
    sm = 1.0 / math.sqrt(w.head_dim)

    log(f"filling the {L}-position cache (quantize-append of {L - 1} tokens)")
    lay, cache0 = kvq_setup.fill_cache(w, lens, upto=np.array([L - 1]), order=args.order)
    k_new = torch.from_numpy(wl.kv_rows(w, "k", 0, L - 1, 1)).to(dev)
    v_new = torch.from_numpy(wl.kv_rows(w, "v", 0, L - 1, 1)).to(dev)
    start = torch.tensor([L - 1], dtype=torch.int32, device=dev)
    q = wl.queries(w)
    qd = torch.from_numpy(q).to(dev)
    ld = torch.from_numpy(lens).to(dev)
    caches = [cache0] + [{k: (None if t is None else t.clone()) for k, t in cache0.items()}
                         for _ in range(COPIES - 1)]
    plan0 = kvq.kvq_plan(lay, 1, w.n_q_heads, L, 0, n_cu)
    ws = torch.zeros(plan0.ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((1, w.n_q_heads, w.head_dim), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream()

    # The timed step: the new token's quantize-append fused into the split-K
    # partials, then the reduce. The plan is made on the host every step.
    def fused_partial(c, plan):
        kvq.kv_append_decode_splitk(lay, c["k"], c["v"], c["k_scales"], c["v_scales"], k_new, v_new, qd, 1,
                                    w.n_q_heads, ld, 0, sm, plan, ws, ws.numel())

    def reduce(plan):
        kvq.kv_decode_reduce(lay, ws, ws.numel(), ld, 1, w.n_q_heads, 0, plan, out)

    def step(c):
        plan = kvq.kvq_plan(lay, 1, w.n_q_heads, L, 0, n_cu)
        fused_partial(c, plan)
        reduce(plan)

    # The same step as three calls (append, partials, reduce), reported beside it.
    def append(c):
        kvq.kv_quant_append(lay, c["k"], c["v"], c["k_scales"], c["v_scales"], k_new, v_new, start, 1, 1)

    def partial(c, plan):
        kvq.kv_decode_attn_splitk(lay, c["k"], c["v"], c["k_scales"], c["v_scales"], qd, 1, w.n_q_heads,
                                  ld, 0, sm, plan, ws, ws.numel())

    log(f"plan: n_splits={plan0.n_splits} chunk={plan0.chunk}; warmup {args.warmup} steps")
    for c in caches:  # every copy holds the new token before anything is checked or timed
        step(c)
    for i in range(args.warmup):
        step(caches[i % COPIES])
    torch.cuda.synchronize()

    # Parity of the state being timed: codes/scales of sampled rows bit-exact
    # (the last row is the one the fused step wrote), and one step's output
    # against the fp64 oracle.
    log("checking codes and output against the oracle")
    rng = np.random.default_rng(11)
    pos = np.unique(np.concatenate([rng.integers(0, L, 2048), [L - 1]]))
    codes_ok = True
    for kind in ("k", "v"):
        rows = wl.kv_rows(w, kind, 0, 0, L)
        for h in range(w.n_kv_heads):
            want_c, want_s = orc.quantize_rows(rows[pos, h], w.scale_group)
            got_c = kvq_setup.rows_of(lay, caches[3][kind], 0, pos, h)
            got_s = kvq_setup.scales_of(lay, caches[3][kind + "_scales"], 0, pos, h)
            codes_ok &= bool(np.array_equal(got_c, want_c) and
                             np.array_equal(got_s.view(np.uint16), want_s.view(np.uint16)))
    step(caches[0])
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)

    cpu = None
    oracle_cache = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the full step")
        want, cpu_s, cores, cpu_reps, cpu_s1, cpu_reps1, oracle_cache = cpu_baseline(w, lens, q, sm)
        max_err = float(np.abs(got - want).max())
        kv_bytes = wl.kv_bytes_per_step(w, lens)
        cpu = {"value": round(kv_bytes / cpu_s / 1e9, 4), "unit": "GB/s", "cores": int(cores),
               "kind": "oracle", "seconds": round(cpu_s, 3),
               "value_1core": None if cpu_s1 is None else round(kv_bytes / cpu_s1 / 1e9, 4),
               "seconds_1core": None if cpu_s1 is None else round(cpu_s1, 3),
               "sample": f"full step repeated {cpu_reps}x (~10 s) on {int(cores)} BLAS threads, then "
                         f"{cpu_reps1}x (~10 s) on one: numpy fp64 decode attention of 16 query heads over "
                         "the dequantized 131072-position cache (both kv heads); cache set-up not timed",
               "quantize": cpu_quantize_baseline(), **cpu_info()}
    else:
        max_err = None

    log(f"timing {args.steps} eager steps over {COPIES} cache copies")
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(caches[i % COPIES])
    t_end.record(stream)
    torch.cuda.synchronize()
    eager_ms = t_start.elapsed_time(t_end) / args.steps

    # Graph-captured decode: one graph holds one step per cache copy (the split
    # plan is fixed at capture; context lengths are read from device memory),
    # so the kernels run back to back without host launch gaps.
    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in caches:
                fn(c)
        return g

    def replay_ms(g, reps):
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * COPIES)

    plan_g = plan0
    reps = max(1, -(-args.steps // COPIES))
    g_step = capture(lambda c: (fused_partial(c, plan_g), reduce(plan_g)))
    log(f"timing {reps * COPIES} graph-replayed steps")
    ms_per_step = replay_ms(g_step, reps)
    # The spread: each replay (one step per cache copy) timed on its own.
    per_replay = []
    for _ in range(50):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g_step.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        per_replay.append(e0.elapsed_time(e1) * 1e3 / COPIES)
    # Hot cache: the same step repeated on one copy (132 MiB stays in the
    # 256 MB Infinity Cache) -- labelled as such, not the headline.
    g_hot = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_hot):
        for _ in range(COPIES):
            fused_partial(caches[0], plan_g)
            reduce(plan_g)
    hot_ms = replay_ms(g_hot, reps)
    graph_out = out.clone()
    step(caches[COPIES - 1])  # eager step on the copy the graph ended with
    torch.cuda.synchronize()
    graph_matches_eager = bool(torch.equal(graph_out, out))
    # Per-kernel graphs (8 back-to-back launches each) for the breakdown and the
    # roofline of the partial kernel; then the unfused three-call step.
    fpart_ms = replay_ms(capture(lambda c: fused_partial(c, plan_g)), reps)
    red_ms = replay_ms(capture(lambda c: reduce(plan_g)), reps)
    unfused_ms = replay_ms(capture(lambda c: (append(c), partial(c, plan_g), reduce(plan_g))), reps)
    app_ms = replay_ms(capture(append), reps)
    part_ms = replay_ms(capture(lambda c: partial(c, plan_g)), reps)

    # The same step at 32K and 64K context on the same caches (rows [0, L - 1)
    # are the workload's; the fused append rewrites row L - 1 with the same
    # values), each with its own plan.
    sweep = []
    for Lc in (32768, 65536):
        ldc = torch.tensor([Lc], dtype=torch.int32, device=dev)
        plan_c = kvq.kvq_plan(lay, 1, w.n_q_heads, Lc, 0, n_cu)
        ws_c = torch.zeros(plan_c.ws_bytes, dtype=torch.uint8, device=dev)
        kn = torch.from_numpy(wl.kv_rows(w, "k", 0, Lc - 1, 1)).to(dev)
        vn = torch.from_numpy(wl.kv_rows(w, "v", 0, Lc - 1, 1)).to(dev)

        def step_c(c):
            kvq.kv_append_decode_splitk(lay, c["k"], c["v"], c["k_scales"], c["v_scales"], kn, vn, qd, 1,
                                        w.n_q_heads, ldc, 0, sm, plan_c, ws_c, ws_c.numel())
            kvq.kv_decode_reduce(lay, ws_c, ws_c.numel(), ldc, 1, w.n_q_heads, 0, plan_c, out)

        ms_c = replay_ms(capture(step_c), reps)
        got_c = out.float().cpu().numpy().astype(np.float64)
        kvb_c = wl.kv_bytes_per_step(w, np.array([Lc]))
        err_c = float(np.abs(got_c[0] - oracle_seq(w, 0, Lc, q[0])).max())
        sweep.append({"context": Lc, "us_per_step": round(ms_c * 1e3, 2), "kv_bytes_per_step": int(kvb_c),
                      "GB_s": round(kvb_c / ms_c / 1e6, 1), "pct_hbm_peak": round(100 * kvb_c / ms_c / 1e6 / HBM_PEAK_GBS, 2),
                      "n_splits": plan_c.n_splits, "chunk": plan_c.chunk, "max_abs_err": err_c, "tol": TOL,
                      "codes_bitexact": codes_match(kvq_setup, lay, caches[-1], w, 0, [Lc - 1, Lc - 2, 7])})
        del ws_c
    log("context sweep: " + ", ".join(f"{d['context']}: {d['us_per_step']} us" for d in sweep))
    log("timing verify windows of 2, 4 and 8 tokens at the end of the 128K context")
    verify = verify_windows(kvq, wl, w, lay, L, n_cu, lambda fn: replay_ms(capture(fn), reps) * 1e3, oracle_cache)
    del oracle_cache
    log("verify windows: " + ", ".join(f"T={d['tokens']}: {d['us']} us" for d in verify))

    others = None
    if not args.no_other_workloads:
        log("timing the cache blob (pack / unpack of the 128K cache)")
        blob = blob_workload(kvq, lay, caches[0], L)
        log("timing the decode step on the Gemma 4K and batched-serving workloads")
        del caches, cache0
        torch.cuda.empty_cache()
        others = secondary_workloads(kvq, kvq_setup, wl, n_cu, args.steps)
        others["cache_blob"] = blob
        log("timing the decode step over the 4-bit stores (q4_0, k8v4) at 128K")
        others.update(q4_workloads(kvq, kvq_setup, wl, n_cu, args.steps))

    log("timing the read-only streaming reference (4 GiB, and at each context's KV bytes)")
    stream_gbs, stream_best, stream_bytes = stream_reference(kvq, n_cu)
    for d in sweep:
        d["stream_at_size"] = stream_at(kvq, n_cu, d["kv_bytes_per_step"])
        d["step_pct_of_stream_at_size"] = round(100 * d["stream_at_size"]["us"] / d["us_per_step"], 2)
    stream_128k = stream_at(kvq, n_cu, wl.kv_bytes_per_step(w, lens))

    kv_bytes = wl.kv_bytes_per_step(w, lens)
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = kv_bytes / (fpart_ms * 1e-3) / 1e9
    digest = kernel_source_digest()
    traffic = traffic_from_profiles(digest, plan0)

    res = {
        # value, ms_per_step, us_per_step: the 128K step; the 4K step's figure is
        # us_per_step_4k (other_workloads.gemma_4k)
        "metric": "int8-KV decode-attention HBM GB/s (% of peak) and \u00b5s/step at 4K and 128K ctx",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "us_per_step_4k": (others or {}).get("gemma_4k", {}).get("us_per_step"),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "stream_reference": {"kernel": "kvq_stream_read (non-temporal 128-bit loads, read only)",
                             "bytes": stream_bytes, "GB_s": round(stream_gbs, 1), "GB_s_best": round(stream_best, 1),
                             "pct_hbm_peak": round(100 * stream_gbs / HBM_PEAK_GBS, 2),
                             "step_pct_of_stream": round(100 * value / stream_gbs, 2),
                             "partial_pct_of_stream": round(100 * achieved / stream_gbs, 2),
                             "at_step_size": stream_128k,
                             "step_pct_of_stream_at_size": round(100 * stream_128k["us"] / (ms_per_step * 1e3), 2),
                             "partial_pct_of_stream_at_size": round(100 * stream_128k["us"] / (fpart_ms * 1e3), 2),
                             "note": "at_step_size: one launch of the read-only kernel over exactly the step's "
                                     "KV bytes, back to back in a graph as the steps are"},
        "step_us_percentiles": {"p10": round(float(np.percentile(per_replay, 10)), 2),
                                "median": round(float(np.median(per_replay)), 2),
                                "p90": round(float(np.percentile(per_replay, 90)), 2),
                                "replays": len(per_replay), "steps_per_replay": COPIES,
                                "note": "50 graph replays timed one by one, beside the --steps timed ones"},
        "hot_cache_us_per_step": round(hot_ms * 1e3, 2),
        "context_sweep": sweep,
        "verify_windows": verify,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 codes, fp16 MFMA operands, fp32 accumulate",
        "data": "synthetic (seeded N(0,1) fp16, K outlier channels x20)",
        "config": {"workload": "long_128k", "batch": 1, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "scale_group": w.scale_group, "context": L,
                   "k_store": w.k_dtype, "v_store": w.v_dtype, "n_splits": plan0.n_splits,
                   "chunk": plan0.chunk, "kv_bytes_per_step": kv_bytes, "cache_copies": COPIES,
                   "layout": "positions-major" if args.order == "pos" else "heads-major"},
        "step": "kv_append_decode_splitk + kv_decode_reduce (quantize-append fused into the partials)",
        "breakdown_us": {"append_and_partial": round(fpart_ms * 1e3, 2), "reduce": round(red_ms * 1e3, 2)},
        "unfused_step_us": {"step": round(unfused_ms * 1e3, 2), "append": round(app_ms * 1e3, 2),
                            "partial": round(part_ms * 1e3, 2), "reduce": round(red_ms * 1e3, 2)},
        "eager_us_per_step": round(eager_ms * 1e3, 2),
        "graph": {"steps_per_graph": COPIES, "replays": reps, "matches_eager_bitwise": graph_matches_eager},
        "roofline": {"bound": "hbm", "kernel": "kvq_partial_kernel (with the fused append)",
                     "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": kv_bytes,
                     "avg_launch_us": round(fpart_ms * 1e3, 3), "kernel_src_sha": digest},
        "parity": {"codes_scales_bitexact_sampled": codes_ok, "max_abs_err_vs_oracle": max_err,
                   "tol": TOL},
        "cpu_baseline": cpu,
        "other_workloads": others,
    }
    print(json.dumps(res), flush=True)
    ok = codes_ok and graph_matches_eager and (max_err is None or max_err <= TOL)
    ok = ok and all(d["max_abs_err_sampled"] <= TOL for d in verify)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
