#!/usr/bin/env python3
"""Benchmark of the GQA attention hot path on one MI355X.

Prints ONE JSON line.  The headline `value` is decode KV-read bandwidth
(GB/s, 1 GB = 1e9 B) of the split-KV decode (split kernel + LSE-combine
kernel) on the Llama3-70B-shaped workload B=1, H_q=64, H_kv=8, d=128,
S_kv=8192, bf16; one step = one decode call.  The `prefill` object reports
causal-prefill TFLOP/s on T_q=S_kv=8192 with the same heads.

Timing: inputs are resident in HBM before the timed region.  Decode K/V are
replicated into >= 512 MiB of rotating copies so each call reads HBM, not the
256 MB Infinity Cache.  The timed decode steps are replayed from a captured
HIP graph (the calls are microseconds long; the graph removes host launch
overhead, every kernel still runs).  HIP events on the launch stream bracket
the K timed steps, with torch.cuda.synchronize() on both sides.

Roofline objects give, for the dominant kernel of each path, algorithmic
bytes (decode: K+V bytes) or flops (prefill: 4 d H_q per visible
query-key pair) per launch divided by that kernel's average duration, timed
alone the same way, against MI355X peaks (HBM 8 TB/s, bf16 MFMA 2.5 PFLOP/s).
`cpu_baseline` times the fp64 CPU oracle on this host (test infrastructure,
never the product path).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode KV-read GB/s (% HBM peak); causal prefill TFLOP/s (% MFMA bf16 peak)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 512 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_tensor(arr, dtype="bf16"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


WARM_MS = 200.0


def warm(fn, min_ms=WARM_MS):
    """Call fn back to back until the GPU has been busy with it for about
    min_ms.  The shader clock ramps up over the first tens of milliseconds
    of sustained load (8k causal prefill: 1.10 ms per call in the first ten
    calls after an idle GPU, 0.95 ms from about the 30th call on); every
    figure here is steady-state throughput."""
    import torch
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        fn()
        torch.cuda.synchronize()


def time_graph(fn_list, reps=1):
    """Capture the calls in fn_list into one graph, replay it `reps` times
    between HIP events after warm-up replays; returns elapsed ms per call."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in fn_list:
            fn()
    warm(g.replay)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / (reps * len(fn_list))


def graph_samples(fn_list, n):
    """Capture fn_list into one graph and time n replays separately; returns
    the elapsed ms per call of each replay (for median and minimum)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in fn_list:
            fn()
    warm(g.replay)
    out = []
    for _ in range(n):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        g.replay()
        end.record()
        torch.cuda.synchronize()
        out.append(start.elapsed_time(end) / len(fn_list))
    return out


def decode_algorithmic_bytes(w, kv_len):
    return int(np.sum(kv_len, dtype=np.int64)) * w.H_kv * w.d * 2 * 2


def prefill_algorithmic_flops(w):
    t = np.arange(w.T_q, dtype=np.float64)
    vis = np.minimum(w.q_offset + t + 1, w.S_kv) if w.causal else np.full(w.T_q, w.S_kv)
    if w.window > 0:     # sinks + local window: min(sink, p+1) + keys in (max(sink, p-window), p]
        p = w.q_offset + t
        sinks = np.minimum(w.sink, p + 1)
        vis = sinks + np.maximum(0.0, p - np.maximum(w.sink, p - w.window + 1) + 1)
    return float(4.0 * w.d * w.H_q * w.B * vis.sum())


def ring_walk_lengths(w, kv_len):
    """Keys a ring-buffer decode reads per sequence (resident sinks + window)."""
    n = np.asarray(kv_len, np.int64)
    s_end = np.minimum(w.sink, n)
    w_lo = np.maximum(s_end, n - w.T_q - w.window + 1)
    return s_end + (n - w_lo)


def bench_decode(name, steps, warmup):
    import torch
    import gqa_attention_flashattention_amd as gq
    from gqa_attention_flashattention_amd import inputs as gin
    inp = gin.make(name)
    w = inp.workload
    kv_bytes = decode_algorithmic_bytes(w, inp.kv_len)
    q = dev_tensor(inp.q_store)
    k0 = dev_tensor(inp.k_store)
    v0 = dev_tensor(inp.v_store)
    n_copies = max(1, min(64, math.ceil(ROTATE_BYTES / kv_bytes)))
    ks = [k0] + [k0.clone() for _ in range(n_copies - 1)]
    vs = [v0] + [v0.clone() for _ in range(n_copies - 1)]
    B, Hq, d = q.shape
    plan = gq.decode_plan(B, Hq, w.H_kv, d, inp.kv_len)
    ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")

    def call(i):
        def f():
            gq.decode_split(q, ks[i % n_copies], vs[i % n_copies], inp.kv_len, ws)
            gq.decode_combine(ws, inp.kv_len, H_q=Hq, H_kv=w.H_kv, d=d, out=out, lse=lse)
        return f

    def split_only(i):
        return lambda: gq.decode_split(q, ks[i % n_copies], vs[i % n_copies], inp.kv_len, ws)

    for i in range(max(warmup, 1)):
        call(i)()
    gq.decode(q, ks[0], vs[0], inp.kv_len, out=out)
    torch.cuda.synchronize()
    ms_call = time_graph([call(i) for i in range(steps)])
    ms_split = time_graph([split_only(i) for i in range(steps)])
    ms_hot = time_graph([lambda: (gq.decode_split(q, k0, v0, inp.kv_len, ws),
                                  gq.decode_combine(ws, inp.kv_len, H_q=Hq, H_kv=w.H_kv, d=d,
                                                    out=out, lse=lse))] * min(steps, 200))
    # after the K timed steps: 20 more replays of 100 calls each, for the
    # median and the minimum of the per-call time
    call_samples = graph_samples([call(i) for i in range(min(steps, 100))], 20)
    o_gpu = out.float().cpu().numpy().astype(np.float64)
    lse_gpu = lse.cpu().numpy().astype(np.float64)
    return dict(inp=inp, kv_bytes=kv_bytes, ms_call=ms_call, ms_split=ms_split, ms_hot=ms_hot,
                n_copies=n_copies, plan=plan, o_gpu=o_gpu, lse_gpu=lse_gpu,
                call_samples=call_samples)


def bench_gqa_reuse(groups, steps, S=32768, H_kv=8, d=128):
    """Decode of one S-key sequence with H_kv = 8 and H_q = G * H_kv for each
    G in `groups`: the same K/V bytes serve G query heads per KV head.  Under
    rocprofv3 --pmc FETCH_SIZE the split kernel's fetched bytes show whether
    K/V are read once for all G heads (the count must not grow with G)."""
    import torch
    import gqa_attention_flashattention_amd as gq
    from gqa_attention_flashattention_amd import inputs as gin
    out = []
    n_copies = 4
    kv_len = np.array([S], np.int32)
    kv_bytes = S * H_kv * d * 2 * 2
    for G in groups:
        inp = gin.random_case("decode", "bf16", B=1, H_q=G * H_kv, H_kv=H_kv, d=d, kv_len=[S],
                              seed=G)
        q = dev_tensor(inp.q_store)
        k0, v0 = dev_tensor(inp.k_store), dev_tensor(inp.v_store)
        ks = [k0] + [k0.clone() for _ in range(n_copies - 1)]
        vs = [v0] + [v0.clone() for _ in range(n_copies - 1)]
        plan = gq.decode_plan(1, G * H_kv, H_kv, d, kv_len)
        ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device="cuda")
        fns = [lambda i=i: gq.decode_split(q, ks[i % n_copies], vs[i % n_copies], kv_len, ws)
               for i in range(steps)]
        for f in fns[:3]:
            f()
        torch.cuda.synchronize()
        ms = time_graph(fns)
        out.append({"G": G, "H_q": G * H_kv, "H_kv": H_kv, "S_kv": S, "kv_bytes": kv_bytes,
                    "splits": int(plan["total_splits"]), "split_us": round(ms * 1e3, 3),
                    "GBps": round(kv_bytes / (ms * 1e-3) / 1e9, 1)})
        del ks, vs, ws
        torch.cuda.empty_cache()
    return out


def bench_decode_multi(name, steps, warmup):
    """Multi-token decode (T_q new tokens per sequence) through the one-call
    entry point, timed by graph replay over rotated K/V copies."""
    import torch
    import gqa_attention_flashattention_amd as gq
    from gqa_attention_flashattention_amd import inputs as gin
    inp = gin.make(name)
    w = inp.workload
    kv_bytes = decode_algorithmic_bytes(w, inp.kv_len)
    q = dev_tensor(inp.q_store)
    k0 = dev_tensor(inp.k_store)
    v0 = dev_tensor(inp.v_store)
    n_copies = max(1, min(64, math.ceil(ROTATE_BYTES / kv_bytes)))
    ks = [k0] + [k0.clone() for _ in range(n_copies - 1)]
    vs = [v0] + [v0.clone() for _ in range(n_copies - 1)]
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")

    def call(i):
        return lambda: gq.decode_multi(q, ks[i % n_copies], vs[i % n_copies], inp.kv_len,
                                       out=out, lse=lse)

    for i in range(max(warmup, 1)):       # also sizes the library workspace before capture
        call(i)()
    torch.cuda.synchronize()
    ms = time_graph([call(i) for i in range(steps)])
    # score/value flops of the visible (token, key) pairs: token t of a
    # sequence of n keys sees n - T_q + t + 1 keys
    pairs = sum(w.T_q * (n - w.T_q) + w.T_q * (w.T_q + 1) // 2
                for n in np.asarray(inp.kv_len, np.int64).tolist())
    flops = 4.0 * w.d * w.H_q * pairs
    res = dict(inp=inp, kv_bytes=kv_bytes, flops=flops, ms=ms, n_copies=n_copies,
               o_gpu=out.float().cpu().numpy().astype(np.float64),
               lse_gpu=lse.cpu().numpy().astype(np.float64))
    del ks, vs, k0, v0
    torch.cuda.empty_cache()
    return res


def bench_prefill(name, steps, warmup):
    import torch
    import gqa_attention_flashattention_amd as gq
    from gqa_attention_flashattention_amd import inputs as gin
    inp = gin.make(name)
    w = inp.workload
    q, k, v = (dev_tensor(x) for x in (inp.q_store, inp.k_store, inp.v_store))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    for _ in range(max(warmup, 1)):
        gq.prefill(q, k, v, causal=w.causal, q_offset=w.q_offset, out=o, lse=lse)
    warm(lambda: gq.prefill(q, k, v, causal=w.causal, q_offset=w.q_offset, out=o, lse=lse))
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        gq.prefill(q, k, v, causal=w.causal, q_offset=w.q_offset, out=o, lse=lse)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    # after the timed calls: each of `steps` more calls between its own events
    # (median and minimum)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        e0.record()
        gq.prefill(q, k, v, causal=w.causal, q_offset=w.q_offset, out=o, lse=lse)
        e1.record()
    torch.cuda.synchronize()
    call_samples = [e0.elapsed_time(e1) for e0, e1 in evs]
    flops = prefill_algorithmic_flops(w)
    rng = np.random.default_rng(0)
    # rows: the CPU baseline's timing sample; wg_rows: one row of every
    # work-group (parity)
    rows = np.unique(np.concatenate([[0, w.B * w.T_q * w.H_q - 1],
                                     rng.integers(0, w.B * w.T_q * w.H_q, 62)]))
    wg_rows = gin.rows_per_workgroup(w.B, w.T_q, w.H_q, w.H_kv, seed=1)
    o_all = o.float().cpu().numpy().reshape(-1, w.d)
    lse_all = lse.cpu().numpy().reshape(-1)
    return dict(inp=inp, ms=ms, flops=flops, rows=rows, wg_rows=wg_rows,
                o_rows=o_all[rows].astype(np.float64), lse_rows=lse_all[rows].astype(np.float64),
                o_wg=o_all[wg_rows].astype(np.float64), lse_wg=lse_all[wg_rows].astype(np.float64),
                call_samples=call_samples)


def bench_prefill_kvsplit(name, steps):
    """KV-parallel prefill (key ranges on separate work-groups + combine)
    beside the plain prefill kernel on the same chunk."""
    import torch
    import gqa_attention_flashattention_amd as gq
    from gqa_attention_flashattention_amd import inputs as gin
    inp = gin.make(name)
    w = inp.workload
    q, k, v = (dev_tensor(x) for x in (inp.q_store, inp.k_store, inp.v_store))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    split = lambda: gq.prefill_kvsplit(q, k, v, causal=w.causal, q_offset=w.q_offset, out=o,
                                       lse=lse)
    plain = lambda: gq.prefill(q, k, v, causal=w.causal, q_offset=w.q_offset, out=o, lse=lse)
    res = {}
    for tag, fn in (("plain", plain), ("kvsplit", split)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        res[tag] = time_graph([fn] * steps)
    o_split = o.float().cpu().numpy()    # the kvsplit result (timed last)
    ns = gq.prefill_kvsplit_count(w.B, w.T_q, w.S_kv, w.H_q, w.H_kv, w.d, causal=w.causal,
                                  q_offset=w.q_offset)
    return dict(inp=inp, ms=res["kvsplit"], ms_plain=res["plain"], n_split=ns,
                flops=prefill_algorithmic_flops(w), o_gpu=o_split,
                lse_gpu=lse.cpu().numpy())


def bench_prefill_window(name, steps):
    import torch
    import gqa_attention_flashattention_amd as gq
    from gqa_attention_flashattention_amd import inputs as gin
    inp = gin.make(name)
    w = inp.workload
    q, k, v = (dev_tensor(x) for x in (inp.q_store, inp.k_store, inp.v_store))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    fn = lambda: gq.prefill_window(q, k, v, q_offset=w.q_offset, window=w.window, sink=w.sink,
                                   out=o, lse=lse)
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    ms = time_graph([fn] * steps)
    return dict(inp=inp, ms=ms, flops=prefill_algorithmic_flops(w), o_gpu=o.float().cpu().numpy(),
                lse_gpu=lse.cpu().numpy())


def bench_decode_ring(name, steps):
    """Ring-buffer decode; rotating copies of the cache keep every call cold."""
    import torch
    import gqa_attention_flashattention_amd as gq
    from gqa_attention_flashattention_amd import inputs as gin
    inp = gin.make(name)
    w = inp.workload
    walk = ring_walk_lengths(w, inp.kv_len)
    kv_bytes = int(walk.sum()) * w.H_kv * w.d * 2 * 2
    q = dev_tensor(inp.q_store)
    k0 = dev_tensor(inp.k_store)
    v0 = dev_tensor(inp.v_store)
    n_copies = max(1, min(64, math.ceil(ROTATE_BYTES / kv_bytes)))
    ks = [k0] + [k0.clone() for _ in range(n_copies - 1)]
    vs = [v0] + [v0.clone() for _ in range(n_copies - 1)]
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")

    def call(i):
        return lambda: gq.decode_ring(q, ks[i % n_copies], vs[i % n_copies], inp.kv_len,
                                      window=w.window, sink=w.sink, out=out, lse=lse)

    for i in range(3):
        call(i)()
    torch.cuda.synchronize()
    ms = time_graph([call(i) for i in range(steps)])
    return dict(inp=inp, ms=ms, kv_bytes=kv_bytes, n_copies=n_copies,
                o_gpu=out.float().cpu().numpy(), lse_gpu=lse.cpu().numpy())


def bench_decode_quant(name, steps):
    """Quantised-cache decode over rotated copies of the code tensors."""
    import torch
    import gqa_attention_flashattention_amd as gq
    from gqa_attention_flashattention_amd import inputs as gin
    inp = gin.make_quant(name)
    w = inp.workload
    pack = (lambda c: c) if w.kv_bits == 8 else gin.pack_int4
    k0 = torch.from_numpy(pack(inp.k_codes)).cuda()
    v0 = torch.from_numpy(pack(inp.v_codes)).cuda()
    kv_bytes = 2 * k0.numel()
    n_copies = max(1, min(64, math.ceil(ROTATE_BYTES / kv_bytes)))
    ks = [k0] + [k0.clone() for _ in range(n_copies - 1)]
    vs = [v0] + [v0.clone() for _ in range(n_copies - 1)]
    q = dev_tensor(inp.q_store)
    ksc = torch.from_numpy(inp.k_scale).cuda()
    vsc = torch.from_numpy(inp.v_scale).cuda()
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")

    def call(i):
        return lambda: gq.decode_quant(q, ks[i % n_copies], vs[i % n_copies], ksc, vsc,
                                       inp.kv_len, kv_bits=w.kv_bits, out=out, lse=lse)

    for i in range(3):
        call(i)()
    torch.cuda.synchronize()
    ms = time_graph([call(i) for i in range(steps)])
    return dict(inp=inp, ms=ms, kv_bytes=kv_bytes, n_copies=n_copies,
                o_gpu=out.float().cpu().numpy(), lse_gpu=lse.cpu().numpy())


def bench_decode_ring_quant(name, steps):
    """Quantised ring-buffer decode (the pccx base configuration) over rotated
    copies of the code tensors; bytes = codes of the resident keys read."""
    import torch
    import gqa_attention_flashattention_amd as gq
    from gqa_attention_flashattention_amd import inputs as gin
    inp = gin.make_quant(name)
    w = inp.workload
    pack = (lambda c: c) if w.kv_bits == 8 else gin.pack_int4
    k0 = torch.from_numpy(pack(inp.k_codes)).cuda()
    v0 = torch.from_numpy(pack(inp.v_codes)).cuda()
    walk = ring_walk_lengths(w, inp.kv_len)
    kv_bytes = int(walk.sum()) * w.H_kv * (w.d * w.kv_bits // 8) * 2
    n_copies = max(1, min(64, math.ceil(ROTATE_BYTES / kv_bytes)))
    ks = [k0] + [k0.clone() for _ in range(n_copies - 1)]
    vs = [v0] + [v0.clone() for _ in range(n_copies - 1)]
    q = dev_tensor(inp.q_store)
    ksc = torch.from_numpy(inp.k_scale).cuda()
    vsc = torch.from_numpy(inp.v_scale).cuda()
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")

    def call(i):
        return lambda: gq.decode_ring_quant(q, ks[i % n_copies], vs[i % n_copies], ksc, vsc,
                                            inp.kv_len, kv_bits=w.kv_bits, window=w.window,
                                            sink=w.sink, out=out, lse=lse)

    for i in range(3):
        call(i)()
    torch.cuda.synchronize()
    ms = time_graph([call(i) for i in range(steps)])
    return dict(inp=inp, ms=ms, kv_bytes=kv_bytes, n_copies=n_copies,
                o_gpu=out.float().cpu().numpy(), lse_gpu=lse.cpu().numpy())


def copy_calibration(mib: int):
    """A plain device-to-device copy of `mib` MiB, three times (rocprofv3
    counter runs scale FETCH_SIZE / WRITE_SIZE by what this copy reads)."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def traffic_record(kernel: str, grid: int):
    """HBM bytes per dispatch of `kernel` launched with `grid` threads, from
    profiles/traffic.json, or None when absent or measured on a different
    kernel source."""
    from gqa_attention_flashattention_amd import profile_summary as ps
    path = ps.TRAFFIC_JSON
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{kernel}@{grid}")
    if not rec or rec.get("source_sha256") != ps.source_sha(kernel):
        return None
    return rec["bytes_per_dispatch"]


def mfma_record(kernel: str, grid: int):
    """MFMA utilisation counters of `kernel` launched with `grid` threads
    (busy and co-issue fractions, VALU instructions per MFMA, counted MFMA
    flops and their rate against the peak at the clock the kernel ran at),
    from profiles/mfma.json, or None when absent or measured on a different
    kernel source."""
    from gqa_attention_flashattention_amd import profile_summary as ps
    path = ps.MFMA_JSON
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{kernel}@{grid}")
    if not rec or rec.get("source_sha256") != ps.source_sha(kernel):
        return None
    return {k: (round(v, 4) if isinstance(v, float) and v < 100 else v)
            for k, v in rec.items() if k != "source_sha256"}


# Launch geometry of the two headline kernels (threads per grid), to match
# rocprofv3 records: the decode split kernel runs 256 threads per (split, KV
# head) at G * T_q <= 16; the prefill kernel 512 threads per 256-row block.
PREFILL_KERNEL = "prefill_bf16_kernel<128,1,false,false,1>"
# bf16 splits of at least this many keys run two KV heads per work-group
# (the library's rule; the kernel name and grid of the profiled launch follow it)
DECODE_PAIR_MIN_SPLIT_LEN = 512


def decode_heads_per_wg(plan, w):
    return 2 if (w.H_kv % 2 == 0 and int(plan["split_len"]) >= DECODE_PAIR_MIN_SPLIT_LEN) else 1


# bf16 caches with at most 32 query rows per KV head stream K/V into LDS, one
# KV head per work-group, with two LDS slots per wave above this many keys
# (always with 17-32 rows: two column blocks)
DECODE_STREAM_ONE_SLOT_KEYS = 128


def decode_is_stream(w):
    return w.G * w.T_q <= 32


def decode_split_kernel_name(plan, w):
    if decode_is_stream(w):
        nh = 2 if w.G * w.T_q > 16 else 1
        r = 2 if nh == 2 or int(plan["split_len"]) > DECODE_STREAM_ONE_SLOT_KEYS else 1
        return f"decode_stream_kernel<{w.d},{r},false,{nh}>"
    return f"decode_split_kernel<{w.d},1,false,0,{decode_heads_per_wg(plan, w)}>"


def decode_split_grid(plan, w):
    hp = 1 if decode_is_stream(w) else decode_heads_per_wg(plan, w)
    return int(plan["total_splits"]) * (w.H_kv // hp) * 256


def prefill_grid(w):
    return -(-w.T_q * w.G // 256) * w.B * w.H_kv * 512


def cpu_threads():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline_decode(inp, kv_bytes, min_seconds=10.0):
    import oracle
    threads = oracle.num_threads(cpu_threads())
    reps, t0 = 0, time.perf_counter()
    while True:
        o, lse = oracle.decode(inp.q, inp.k, inp.v, inp.kv_len, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= 1000:
            break
    return dict(value=kv_bytes * reps / el / 1e9, unit="GB/s", cores=threads, kind="oracle",
                sample=f"whole workload (all {inp.workload.B * inp.workload.H_q} query heads, "
                       f"every key), {reps} passes in {el:.1f} s"), o, lse


def cpu_baseline_prefill(inp, rows, min_seconds=10.0):
    import oracle
    w = inp.workload
    threads = oracle.num_threads(cpu_threads())
    t = (rows // w.H_q) % w.T_q
    vis = np.minimum(w.q_offset + t + 1, w.S_kv) if w.causal else np.full(t.shape, w.S_kv)
    flops_rows = float(4.0 * w.d * vis.sum())
    reps, t0 = 0, time.perf_counter()
    while True:
        o, lse = oracle.prefill(inp.q, inp.k, inp.v, causal=w.causal, q_offset=w.q_offset,
                                rows=rows, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= 1000:
            break
    return dict(value=flops_rows * reps / el / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample=f"{rows.size} sampled query rows of the workload, {reps} passes in "
                       f"{el:.1f} s"), o, lse


def parity_prefill_rows(pre, o_sample, lse_sample, tag):
    """Prefill parity over the timing sample's rows (oracle outputs given)
    and over one row of every work-group (oracle run here)."""
    import oracle
    inp = pre["inp"]
    w = inp.workload
    o, l = oracle.prefill(inp.q, inp.k, inp.v, causal=w.causal, q_offset=w.q_offset,
                          rows=pre["wg_rows"])
    do = max(np.abs(pre["o_rows"] - o_sample).max(), np.abs(pre["o_wg"] - o).max())
    dl = max(np.abs(pre["lse_rows"] - lse_sample).max(), np.abs(pre["lse_wg"] - l).max())
    return {f"{tag}_sample_max_abs_dO": float(do), f"{tag}_sample_max_abs_dLSE": float(dl),
            f"{tag}_sample_rows": int(np.union1d(pre["rows"], pre["wg_rows"]).size)}


def parity_decode_multi(mul, seqs=(0, 1), tag="decode_multi"):
    """Oracle check of sequences `seqs` of a multi-token decode result (every
    row of those sequences)."""
    import oracle
    inp = mul["inp"]
    w = inp.workload
    errs_o, errs_l = [], []
    kv_len = np.asarray(inp.kv_len, np.int64)
    off = np.concatenate([[0], np.cumsum(kv_len)])
    for b in seqs:
        n = int(kv_len[b])
        kb, ke = int(off[b]), int(off[b + 1])
        o, l = oracle.prefill(inp.q[b:b + 1], inp.k[None, kb:ke], inp.v[None, kb:ke],
                              causal=True, q_offset=n - w.T_q)
        errs_o.append(np.abs(mul["o_gpu"][b] - o[0]).max())
        errs_l.append(np.abs(mul["lse_gpu"][b] - l[0]).max())
    return {f"{tag}_sample_max_abs_dO": float(max(errs_o)),
            f"{tag}_sample_max_abs_dLSE": float(max(errs_l))}


def parity_prefill_kvsplit(kvs, n_rows=64):
    import oracle
    from gqa_attention_flashattention_amd import inputs as gin
    inp = kvs["inp"]
    w = inp.workload
    rng = np.random.default_rng(0)
    total = w.B * w.T_q * w.H_q
    rows = np.unique(np.concatenate([[0, total - 1], rng.integers(0, total, n_rows - 2)]))
    rows = np.union1d(rows, gin.rows_per_workgroup(w.B, w.T_q, w.H_q, w.H_kv, seed=1))
    o, l = oracle.prefill(inp.q, inp.k, inp.v, causal=w.causal, q_offset=w.q_offset, rows=rows)
    og = kvs["o_gpu"].reshape(-1, w.d)[rows].astype(np.float64)
    lg = kvs["lse_gpu"].reshape(-1)[rows].astype(np.float64)
    return {"prefill_kvsplit_sample_max_abs_dO": float(np.abs(og - o).max()),
            "prefill_kvsplit_sample_max_abs_dLSE": float(np.abs(lg - l).max())}


def parity_prefill_window(pw_, n_rows=64):
    import oracle
    from gqa_attention_flashattention_amd import inputs as gin
    inp = pw_["inp"]
    w = inp.workload
    rng = np.random.default_rng(0)
    total = w.B * w.T_q * w.H_q
    rows = np.unique(np.concatenate([[0, total - 1], rng.integers(0, total, n_rows - 2)]))
    rows = np.union1d(rows, gin.rows_per_workgroup(w.B, w.T_q, w.H_q, w.H_kv, seed=1))
    o, l = oracle.prefill_window(inp.q, inp.k, inp.v, q_offset=w.q_offset, window=w.window,
                                 sink=w.sink, rows=rows)
    og = pw_["o_gpu"].reshape(-1, w.d)[rows].astype(np.float64)
    lg = pw_["lse_gpu"].reshape(-1)[rows].astype(np.float64)
    return {"prefill_window_sample_max_abs_dO": float(np.abs(og - o).max()),
            "prefill_window_sample_max_abs_dLSE": float(np.abs(lg - l).max())}


def parity_decode_ring(dr, n_seq=2):
    """Oracle check of the first n_seq sequences: the logical sequence each
    ring cache holds, rebuilt from the ring rule, through the window oracle."""
    import oracle
    inp = dr["inp"]
    w = inp.workload
    wrap = w.capacity - w.sink
    eo, el = [], []
    for b, n in enumerate(np.asarray(inp.kv_len).tolist()[:n_seq]):
        pos = np.arange(n)
        keep = (pos < w.sink) | (pos >= n - wrap)
        slot = np.where(pos < w.sink, pos, w.sink + (pos - w.sink) % wrap)
        kl = np.zeros((n, w.H_kv, w.d), np.float32)
        vl = np.zeros((n, w.H_kv, w.d), np.float32)
        kl[keep] = inp.k[b, slot[keep]]
        vl[keep] = inp.v[b, slot[keep]]
        o, l = oracle.prefill_window(inp.q[b:b + 1], kl[None], vl[None], q_offset=n - w.T_q,
                                     window=w.window, sink=w.sink)
        eo.append(np.abs(dr["o_gpu"][b] - o[0]).max())
        el.append(np.abs(dr["lse_gpu"][b] - l[0]).max())
    return {"decode_ring_sample_max_abs_dO": float(max(eo)),
            "decode_ring_sample_max_abs_dLSE": float(max(el))}


def parity_decode_ring_quant(dr, n_seq=2):
    """Oracle check of the first n_seq sequences: the dequantised ring cache
    unwrapped by the ring rule, through the window oracle."""
    import oracle
    inp = dr["inp"]
    w = inp.workload
    wrap = w.capacity - w.sink
    eo, el = [], []
    for b, n in enumerate(np.asarray(inp.kv_len).tolist()[:n_seq]):
        kd = oracle.dequantize(inp.k_codes[b], inp.k_scale)
        vd = oracle.dequantize(inp.v_codes[b], inp.v_scale)
        pos = np.arange(n)
        keep = (pos < w.sink) | (pos >= n - wrap)
        slot = np.where(pos < w.sink, pos, w.sink + (pos - w.sink) % wrap)
        kl = np.zeros((n, w.H_kv, w.d), np.float32)
        vl = np.zeros((n, w.H_kv, w.d), np.float32)
        kl[keep] = kd[slot[keep]]
        vl[keep] = vd[slot[keep]]
        o, l = oracle.prefill_window(inp.q[b:b + 1], kl[None], vl[None], q_offset=n - w.T_q,
                                     window=w.window, sink=w.sink)
        eo.append(np.abs(dr["o_gpu"][b] - o[0]).max())
        el.append(np.abs(dr["lse_gpu"][b] - l[0]).max())
    return {"decode_ring_quant_sample_max_abs_dO": float(max(eo)),
            "decode_ring_quant_sample_max_abs_dLSE": float(max(el))}


def parity_decode_quant(dq, n_seq=1):
    """Oracle over the dequantised cache for the first n_seq sequences."""
    import oracle
    inp = dq["inp"]
    w = inp.workload
    n_keys = int(np.asarray(inp.kv_len[:n_seq], np.int64).sum())
    k = oracle.dequantize(inp.k_codes[:n_keys], inp.k_scale)
    v = oracle.dequantize(inp.v_codes[:n_keys], inp.v_scale)
    eo, el = [], []
    off = 0
    for b, n in enumerate(np.asarray(inp.kv_len).tolist()[:n_seq]):
        o, l = oracle.prefill(inp.q[b:b + 1], k[None, off:off + n], v[None, off:off + n],
                              causal=True, q_offset=n - w.T_q)
        eo.append(np.abs(dq["o_gpu"][b] - o[0]).max())
        el.append(np.abs(dq["lse_gpu"][b] - l[0]).max())
        off += n
    tag = w.name
    return {f"{tag}_sample_max_abs_dO": float(max(eo)),
            f"{tag}_sample_max_abs_dLSE": float(max(el))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000, help="timed decode steps")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--decode-workload", default="decode_8k")
    ap.add_argument("--prefill-workload", default="prefill_8k_causal")
    ap.add_argument("--chunk-workload", default="prefill_chunk_64k",
                    help="chunked causal prefill at an offset (reported under prefill_chunk)")
    ap.add_argument("--kvsplit-workload", default="prefill_chunk_256_64k",
                    help="KV-parallel prefill workload (reported under prefill_kvsplit)")
    ap.add_argument("--window-workload", default="prefill_8k_window1k",
                    help="sink + local-window prefill workload (reported under prefill_window)")
    ap.add_argument("--ring-workload", default="decode_ring_8k_b16",
                    help="ring-buffer decode workload (reported under decode_ring)")
    ap.add_argument("--quant-workloads", default="decode_int8_varlen_b16,decode_int4_varlen_b16",
                    help="quantised-cache decode workloads (reported under decode_quant)")
    ap.add_argument("--multi-workload", default="decode_t4_varlen_b16",
                    help="multi-token decode workload (reported under decode_multi)")
    ap.add_argument("--multi-wide-workloads", default="decode_t16_varlen_b16,decode_t32_varlen_b16",
                    help="multi-token decode workloads with 128 / 256 query rows per KV head "
                         "(reported under decode_multi_wide)")
    ap.add_argument("--ring-quant-workload", default="decode_ring_int4_b16",
                    help="quantised ring-buffer decode workload (reported under decode_ring_quant)")
    ap.add_argument("--scale-workloads", default="decode_varlen_b16,decode_128k",
                    help="larger plain-decode workloads (reported under decode_at_scale)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", choices=["decode", "prefill", "prefill_chunk", "gqa_reuse", "decode_multi", "prefill_kvsplit",
                                       "prefill_window", "decode_ring", "decode_quant",
                                       "decode_ring_quant"],
                    default=None,
                    help="run one path only (profiling runs); prints a partial line")
    ap.add_argument("--gqa-groups", default="1,2,4,8",
                    help="--only gqa_reuse: query heads per KV head to run (H_kv = 8)")
    ap.add_argument("--gqa-keys", type=int, default=32768,
                    help="--only gqa_reuse: keys of the one sequence")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this library runs on one GPU only; --gpus must be 1 "
                                   "(multi-GPU sharding is a design note, not built)"}))
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    import gqa_attention_flashattention_amd as gq
    gq.load_library()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)

    if args.only == "gqa_reuse":
        groups = [int(g) for g in args.gqa_groups.split(",")]
        print(json.dumps({"gqa_reuse": bench_gqa_reuse(groups, min(args.steps, 100),
                                                       S=args.gqa_keys)}), flush=True)
        return
    if args.only == "decode_multi":
        for name in [args.multi_workload] + args.multi_wide_workloads.split(","):
            mul = bench_decode_multi(name, min(args.steps, 200), args.warmup)
            log(f"[bench] decode_multi {name} {mul['ms'] * 1e3:.2f} us/call "
                f"{mul['kv_bytes'] / (mul['ms'] * 1e-3) / 1e9:.1f} GB/s "
                f"{mul['flops'] / (mul['ms'] * 1e-3) / 1e12:.1f} TFLOP/s")
        return
    if args.only == "prefill_window":
        pw_ = bench_prefill_window(args.window_workload, args.prefill_steps)
        log(f"[bench] prefill_window {pw_['ms'] * 1e3:.1f} us/call "
            f"{pw_['flops'] / (pw_['ms'] * 1e-3) / 1e12:.1f} TFLOP/s")
        return
    if args.only == "decode_ring":
        dr = bench_decode_ring(args.ring_workload, min(args.steps, 200))
        log(f"[bench] decode_ring {dr['ms'] * 1e3:.1f} us/call "
            f"{dr['kv_bytes'] / (dr['ms'] * 1e-3) / 1e9:.1f} GB/s")
        return
    if args.only == "decode_ring_quant":
        drq = bench_decode_ring_quant(args.ring_quant_workload, min(args.steps, 200))
        log(f"[bench] decode_ring_quant {drq['ms'] * 1e3:.1f} us/call "
            f"{drq['kv_bytes'] / (drq['ms'] * 1e-3) / 1e9:.1f} GB/s")
        return
    if args.only == "decode_quant":
        for name in args.quant_workloads.split(","):
            dq = bench_decode_quant(name, min(args.steps, 200))
            log(f"[bench] {name} {dq['ms'] * 1e3:.1f} us/call "
                f"{dq['kv_bytes'] / (dq['ms'] * 1e-3) / 1e9:.1f} GB/s")
        return
    if args.only == "prefill_kvsplit":
        kvs = bench_prefill_kvsplit(args.kvsplit_workload, args.prefill_steps)
        log(f"[bench] prefill_kvsplit {kvs['ms'] * 1e3:.1f} us/call (plain "
            f"{kvs['ms_plain'] * 1e3:.1f} us), {kvs['n_split']} ranges")
        return
    if args.only in ("prefill", "prefill_chunk"):
        name = args.prefill_workload if args.only == "prefill" else args.chunk_workload
        pre = bench_prefill(name, args.prefill_steps, 2)
        log(f"[bench] {args.only} {pre['ms']:.3f} ms/call "
            f"{pre['flops'] / (pre['ms'] * 1e-3) / 1e12:.1f} TFLOP/s")
        return
    log(f"[bench] decode {args.decode_workload}: warmup {args.warmup}, steps {args.steps}")
    torch.cuda.synchronize()
    dec = bench_decode(args.decode_workload, args.steps, args.warmup)
    torch.cuda.synchronize()
    log(f"[bench] decode {dec['ms_call'] * 1e3:.2f} us/call, split {dec['ms_split'] * 1e3:.2f} us")
    if args.only == "decode":
        return
    log(f"[bench] prefill {args.prefill_workload}: steps {args.prefill_steps}")
    pre = bench_prefill(args.prefill_workload, args.prefill_steps, 2)
    log(f"[bench] prefill {pre['ms']:.3f} ms/call")

    log(f"[bench] prefill_chunk {args.chunk_workload}: steps {max(args.prefill_steps // 4, 3)}")
    chk = bench_prefill(args.chunk_workload, max(args.prefill_steps // 4, 3), 1)
    log(f"[bench] prefill_chunk {chk['ms']:.3f} ms/call")

    log(f"[bench] decode_multi {args.multi_workload}")
    mul = bench_decode_multi(args.multi_workload, min(args.steps, 200), args.warmup)
    log(f"[bench] decode_multi {mul['ms'] * 1e3:.2f} us/call")
    mulw = []
    for name in [n for n in args.multi_wide_workloads.split(",") if n]:
        log(f"[bench] decode_multi_wide {name}")
        mulw.append(bench_decode_multi(name, min(args.steps, 100), args.warmup))
        log(f"[bench] decode_multi_wide {mulw[-1]['ms'] * 1e3:.2f} us/call")

    log(f"[bench] prefill_kvsplit {args.kvsplit_workload}")
    kvs = bench_prefill_kvsplit(args.kvsplit_workload, args.prefill_steps)
    log(f"[bench] prefill_kvsplit {kvs['ms'] * 1e3:.1f} us/call (plain {kvs['ms_plain'] * 1e3:.1f} us)")

    log(f"[bench] prefill_window {args.window_workload}")
    pwin = bench_prefill_window(args.window_workload, args.prefill_steps)
    log(f"[bench] decode_ring {args.ring_workload}")
    dring = bench_decode_ring(args.ring_workload, min(args.steps, 200))

    dquant = []
    for name in args.quant_workloads.split(","):
        log(f"[bench] decode_quant {name}")
        dquant.append(bench_decode_quant(name, min(args.steps, 200)))

    log(f"[bench] decode_ring_quant {args.ring_quant_workload}")
    dringq = bench_decode_ring_quant(args.ring_quant_workload, min(args.steps, 200))

    dscale = []
    for name in filter(None, args.scale_workloads.split(",")):
        log(f"[bench] decode_at_scale {name}")
        dscale.append(bench_decode(name, min(args.steps, 100), 3))
        torch.cuda.empty_cache()

    dw = dec["inp"].workload
    gbs = dec["kv_bytes"] / (dec["ms_call"] * 1e-3) / 1e9
    gbs_split = dec["kv_bytes"] / (dec["ms_split"] * 1e-3) / 1e9
    pw = pre["inp"].workload
    tflops = pre["flops"] / (pre["ms"] * 1e-3) / 1e12

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["ms_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": dw.name, "B": dw.B, "H_q": dw.H_q, "H_kv": dw.H_kv, "d": dw.d,
                   "S_kv": int(dec["inp"].kv_len.max()), "num_splits": "auto",
                   "splits_per_seq": int(dec["plan"]["max_splits"]),
                   "kv_copies_rotated": dec["n_copies"], "timed_via": "hip graph replay"},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "call_ms_spread": {"median": round(float(np.median(dec["call_samples"])), 5),
                           "min": round(float(np.min(dec["call_samples"])), 5),
                           "samples": len(dec["call_samples"]),
                           "how": "20 graph replays of 100 calls after the timed steps"},
        "hot_cache_GBps": round(dec["kv_bytes"] / (dec["ms_hot"] * 1e-3) / 1e9, 2),
        "roofline": {"bound": "hbm", "kernel": decode_split_kernel_name(dec["plan"], dw),
                     "grid_threads": decode_split_grid(dec["plan"], dw),
                     "achieved": round(gbs_split, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs_split / HBM_PEAK_GBS, 4),
                     "traffic": traffic_record(decode_split_kernel_name(dec["plan"], dw),
                                               decode_split_grid(dec["plan"], dw)),
                     "algorithmic_bytes_per_launch": dec["kv_bytes"],
                     "avg_launch_us": round(dec["ms_split"] * 1e3, 3)},
        "prefill": {
            "workload": pw.name, "T_q": pw.T_q, "S_kv": pw.S_kv, "q_offset": pw.q_offset,
            "causal": pw.causal, "ms_per_call": pre["ms"], "value": round(tflops, 2),
            "call_ms_spread": {"median": round(float(np.median(pre["call_samples"])), 5),
                               "min": round(float(np.min(pre["call_samples"])), 5),
                               "samples": len(pre["call_samples"]),
                               "how": "each call between its own events, after the timed calls"},
            "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "kernel": PREFILL_KERNEL,
                         "grid_threads": prefill_grid(pw),
                         "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": traffic_record(PREFILL_KERNEL, prefill_grid(pw)),
                         "mfma_counters": mfma_record(PREFILL_KERNEL, prefill_grid(pw)),
                         "algorithmic_flops_per_launch": pre["flops"],
                         "avg_launch_us": round(pre["ms"] * 1e3, 3)},
        },
    }
    cw = chk["inp"].workload
    tf_chunk = chk["flops"] / (chk["ms"] * 1e-3) / 1e12
    result["prefill_chunk"] = {
        "workload": cw.name, "T_q": cw.T_q, "S_kv": cw.S_kv, "q_offset": cw.q_offset,
        "causal": cw.causal, "ms_per_call": chk["ms"], "value": round(tf_chunk, 2),
        "call_ms_spread": {"median": round(float(np.median(chk["call_samples"])), 5),
                           "min": round(float(np.min(chk["call_samples"])), 5),
                           "samples": len(chk["call_samples"]),
                           "how": "each call between its own events, after the timed calls"},
        "unit": "TFLOP/s",
        "roofline": {"bound": "mfma", "kernel": PREFILL_KERNEL,
                     "grid_threads": prefill_grid(cw),
                     "achieved": round(tf_chunk, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf_chunk / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_record(PREFILL_KERNEL, prefill_grid(cw)),
                     "mfma_counters": mfma_record(PREFILL_KERNEL, prefill_grid(cw)),
                     "algorithmic_flops_per_launch": chk["flops"],
                     "avg_launch_us": round(chk["ms"] * 1e3, 3),
                     "note": "one prefill kernel launch per call"},
    }
    mw = mul["inp"].workload
    gbs_multi = mul["kv_bytes"] / (mul["ms"] * 1e-3) / 1e9
    result["decode_multi"] = {
        "workload": mw.name, "B": mw.B, "T_q": mw.T_q, "H_q": mw.H_q, "H_kv": mw.H_kv, "d": mw.d,
        "kv_len_range": list(mw.kv_len_range) if mw.kv_len_range else None,
        "ms_per_call": mul["ms"], "value": round(gbs_multi, 2), "unit": "GB/s",
        "roofline": {"bound": "hbm", "achieved": round(gbs_multi, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs_multi / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_call": mul["kv_bytes"],
                     "note": "whole call (split + combine kernels)"},
    }
    result["decode_multi_wide"] = []
    for m in mulw:
        mw = m["inp"].workload
        gbs = m["kv_bytes"] / (m["ms"] * 1e-3) / 1e9
        tfs = m["flops"] / (m["ms"] * 1e-3) / 1e12
        result["decode_multi_wide"].append({
            "workload": mw.name, "B": mw.B, "T_q": mw.T_q, "H_q": mw.H_q, "H_kv": mw.H_kv,
            "d": mw.d, "rows_per_kv_head": mw.T_q * mw.H_q // mw.H_kv,
            "kv_len_range": list(mw.kv_len_range) if mw.kv_len_range else None,
            "ms_per_call": m["ms"], "value": round(gbs, 2), "unit": "GB/s",
            "TFLOPs": round(tfs, 2), "mfma_frac": round(tfs / MFMA_BF16_PEAK_TFLOPS, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_call": m["kv_bytes"],
                         "algorithmic_flops_per_call": m["flops"],
                         "note": "whole call (prefill-loop split kernel + combine); at 256 "
                                 "rows per KV head the bf16 MFMA work per byte is near the "
                                 "ridge, so mfma_frac is given beside the HBM fraction"},
        })
    kw = kvs["inp"].workload
    tf_split = kvs["flops"] / (kvs["ms"] * 1e-3) / 1e12
    result["prefill_kvsplit"] = {
        "workload": kw.name, "T_q": kw.T_q, "S_kv": kw.S_kv, "q_offset": kw.q_offset,
        "causal": kw.causal, "key_ranges": kvs["n_split"], "ms_per_call": kvs["ms"],
        "value": round(tf_split, 2), "unit": "TFLOP/s",
        "plain_prefill_ms_per_call": kvs["ms_plain"],
        "plain_prefill_TFLOPs": round(kvs["flops"] / (kvs["ms_plain"] * 1e-3) / 1e12, 2),
        "roofline": {"bound": "mfma", "achieved": round(tf_split, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf_split / MFMA_BF16_PEAK_TFLOPS, 4),
                     "algorithmic_flops_per_call": kvs["flops"],
                     "note": "whole call (split prefill + combine kernels)"},
    }
    ww = pwin["inp"].workload
    tf_win = pwin["flops"] / (pwin["ms"] * 1e-3) / 1e12
    result["prefill_window"] = {
        "workload": ww.name, "T_q": ww.T_q, "S_kv": ww.S_kv, "window": ww.window,
        "sink": ww.sink, "ms_per_call": pwin["ms"], "value": round(tf_win, 2), "unit": "TFLOP/s",
        "roofline": {"bound": "mfma", "achieved": round(tf_win, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf_win / MFMA_BF16_PEAK_TFLOPS, 4),
                     "algorithmic_flops_per_call": pwin["flops"],
                     "note": "visible (sink + window) pairs only"},
    }
    rw = dring["inp"].workload
    gbs_ring = dring["kv_bytes"] / (dring["ms"] * 1e-3) / 1e9
    result["decode_ring"] = {
        "workload": rw.name, "B": rw.B, "T_q": rw.T_q, "capacity": rw.capacity,
        "window": rw.window, "sink": rw.sink, "kv_len_range": list(rw.kv_len_range),
        "ms_per_call": dring["ms"], "value": round(gbs_ring, 2), "unit": "GB/s",
        "kv_copies_rotated": dring["n_copies"],
        "roofline": {"bound": "hbm", "achieved": round(gbs_ring, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs_ring / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_call": dring["kv_bytes"],
                     "note": "whole call (split + combine kernels); bytes = resident keys read"},
    }
    qw = dringq["inp"].workload
    gbs_rq = dringq["kv_bytes"] / (dringq["ms"] * 1e-3) / 1e9
    result["decode_ring_quant"] = {
        "workload": qw.name, "kv_bits": qw.kv_bits, "B": qw.B, "T_q": qw.T_q,
        "capacity": qw.capacity, "window": qw.window, "sink": qw.sink,
        "kv_len_range": list(qw.kv_len_range), "ms_per_call": dringq["ms"],
        "value": round(gbs_rq, 2), "unit": "GB/s", "kv_copies_rotated": dringq["n_copies"],
        "bf16_equivalent_GBps": round(gbs_rq * 16 / qw.kv_bits, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs_rq, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs_rq / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_call": dringq["kv_bytes"],
                     "note": "whole call; bytes = codes of the resident keys read"},
    }
    result["decode_at_scale"] = []
    for ds in dscale:
        sw = ds["inp"].workload
        g_call = ds["kv_bytes"] / (ds["ms_call"] * 1e-3) / 1e9
        g_split = ds["kv_bytes"] / (ds["ms_split"] * 1e-3) / 1e9
        result["decode_at_scale"].append({
            "workload": sw.name, "B": sw.B, "H_q": sw.H_q, "H_kv": sw.H_kv, "d": sw.d,
            "kv_len_range": list(sw.kv_len_range) if sw.kv_len_range else None,
            "S_kv_max": int(ds["inp"].kv_len.max()), "kv_copies_rotated": ds["n_copies"],
            "ms_per_call": ds["ms_call"], "value": round(g_call, 2), "unit": "GB/s",
            "hbm_frac": round(g_call / HBM_PEAK_GBS, 4),
            "roofline": {"bound": "hbm", "kernel": decode_split_kernel_name(ds["plan"], sw),
                         "grid_threads": decode_split_grid(ds["plan"], sw),
                         "achieved": round(g_split, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(g_split / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_launch": ds["kv_bytes"],
                         "avg_launch_us": round(ds["ms_split"] * 1e3, 3),
                         "note": "split kernel alone; value is the whole call (split + combine)"},
        })
    result["decode_quant"] = []
    for dq in dquant:
        qw = dq["inp"].workload
        gbs_q = dq["kv_bytes"] / (dq["ms"] * 1e-3) / 1e9
        result["decode_quant"].append({
            "workload": qw.name, "kv_bits": qw.kv_bits, "B": qw.B, "H_q": qw.H_q,
            "H_kv": qw.H_kv, "d": qw.d, "kv_len_range": list(qw.kv_len_range),
            "ms_per_call": dq["ms"], "value": round(gbs_q, 2), "unit": "GB/s",
            "bf16_equivalent_GBps": round(gbs_q * 16 / qw.kv_bits, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs_q, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs_q / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_call": dq["kv_bytes"],
                         "note": "whole call; bytes = K and V codes read (scales negligible)"},
        })
    log("[bench] measured ceilings (streaming read, MFMA loop)")
    from gqa_attention_flashattention_amd import ceilings
    read_gbs = ceilings.hbm_read_gbps()
    mfma_tf = ceilings.mfma_bf16_tflops()
    result["ceilings"] = {
        "hbm_read_GBps": round(read_gbs, 1), "hbm_read_frac_of_peak": round(read_gbs / HBM_PEAK_GBS, 4),
        "mfma_bf16_TFLOPs": round(mfma_tf, 1),
        "mfma_bf16_frac_of_peak": round(mfma_tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "note": "measured on this GPU: a 4 GiB read with 16-byte non-temporal loads, one "
                "contiguous range per work-group; back-to-back 32x32x16 bf16 MFMAs on register "
                "operands that change at every issue; the rooflines divide by the spec-sheet "
                "peaks"}
    if not args.no_cpu:
        log("[bench] cpu oracle baseline (decode)")
        cb, o_ref, lse_ref = cpu_baseline_decode(dec["inp"], dec["kv_bytes"])
        result["cpu_baseline"] = cb
        result["parity"] = {"decode_max_abs_dO": float(np.abs(dec["o_gpu"] - o_ref).max()),
                            "decode_max_abs_dLSE": float(np.abs(dec["lse_gpu"] - lse_ref).max())}
        log("[bench] cpu oracle baseline (prefill sample)")
        cbp, op, lp = cpu_baseline_prefill(pre["inp"], pre["rows"])
        result["prefill"]["cpu_baseline"] = cbp
        result["parity"].update(parity_prefill_rows(pre, op, lp, "prefill"))
        log("[bench] cpu oracle baseline (prefill_chunk sample)")
        cbc, oc, lc = cpu_baseline_prefill(chk["inp"], chk["rows"])
        result["prefill_chunk"]["cpu_baseline"] = cbc
        result["parity"].update(parity_prefill_rows(chk, oc, lc, "prefill_chunk"))
        log("[bench] oracle check (prefill_kvsplit sample)")
        result["parity"].update(parity_prefill_kvsplit(kvs))
        log("[bench] oracle check (prefill_window sample)")
        result["parity"].update(parity_prefill_window(pwin))
        log("[bench] oracle check (decode_ring sample)")
        result["parity"].update(parity_decode_ring(dring))
        for dq in dquant:
            log(f"[bench] oracle check ({dq['inp'].workload.name} sample)")
            result["parity"].update(parity_decode_quant(dq))
        log("[bench] oracle check (decode_ring_quant sample)")
        result["parity"].update(parity_decode_ring_quant(dringq))
        log("[bench] oracle check (decode_multi sample)")
        result["parity"].update(parity_decode_multi(mul))
        for m in mulw:
            log(f"[bench] oracle check ({m['inp'].workload.name} sample)")
            # the shortest sequence of the batch, every row
            b = int(np.argmin(np.asarray(m["inp"].kv_len)))
            result["parity"].update(parity_decode_multi(m, seqs=(b,),
                                                        tag=m["inp"].workload.name))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
