#!/usr/bin/env python3
"""Benchmark of the hybrid sliding/global attention hot path on one MI355X.

A step is one pass of the prefill path -- descriptor validation, key-RoPE
pass, fused Q-RoPE + flash attention, fp32 epilogue -- over the full-attention
prefill workload (batch 1, 4096 tokens, 8 query / 2 kv heads, head size 512,
causal, separate K and V, RoPE theta 1e6).  Prints ONE JSON line.

The line also carries:
  roofline      the attention kernel's algorithmic FLOPs per launch / its
                average duration (HIP events recorded around that kernel on
                the stream it runs on) against the bf16 dense MFMA peak;
  cpu_baseline  the fp64 oracle timed on this host on a bounded sample of the
                same workload;
  decode        batched decode (64 sequences x 8192 cached tokens, full layer
                head size 512 plus sliding K=V layer head size 256): KV bytes
                per second of the split-K kernel against HBM peak;
  stack         the 35-layer prefill stack (2048 tokens): every layer's call
                in order, with the sliding and full layers also timed apart;
                shared layers reuse their source layer's operand images;
  long_decode   decode of 4 sequences with long, unequal contexts;
  next_rows     the built NEXT rows against their rooflines: a prefill
                chunk at a start position, image spans, a 4-token verify
                step, a ring-cache sliding layer with fused append, E4M3
                caches;
  small_prefill the 64-token sliding layer (latency-bound, reported only);
  hbm_reference torch's own device copy and sum over 2 GiB on this GPU.

Defaults: 100 warm-up and 100 timed steps.  Before its warm-up each leg runs
its own call, untimed, for SETTLE_MS of wall time: the GPU reaches its steady
clock only after 20-30 ms of sustained load, so short runs (--warmup 5) would
otherwise time the clock ramp.  --no-stack,
--no-long-decode, --no-next, --no-small, --no-hbm-reference and --no-cpu-baseline skip
legs; --calibrate-copy runs only the 1 GiB copy the traffic counters are
calibrated on.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill attention TFLOP/s and decode KV GB/s, as % of MI355X peak"
PEAK_BF16_TFLOPS = 2500.0  # dense MFMA bf16
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def measured_traffic(kernel):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) from the committed rocprofv3
    counter summary, or None when it is missing or was taken on a different kernel source."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        with open(os.path.join(ROOT, t["source"]), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != t["source_sha256"]:
                return None
        e = t["kernels"].get(kernel)
        return None if e is None else e.get("bytes_per_launch")
    except (OSError, ValueError, KeyError):
        return None


# After idle the GPU needs 20-30 ms of sustained load to reach its steady
# clock (the headline step runs at 200-220 us over its first ~50 steps and at
# ~172 us from ~150 steps on).  Every timed leg first runs its own call,
# untimed, for this much wall time, and then its warm-up steps.
SETTLE_MS = 60.0


def settle_clock(fn, min_ms=SETTLE_MS):
    """Untimed calls of fn, in batches of 8, until min_ms of wall time has passed; returns the call count."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= min_ms:
            return n


def time_calls(fn, steps, warmup, flush=None):
    """Average time per call (events around each call) and per main kernel
    (events the library records immediately around it).  The two are taken on
    alternating calls, so the call times carry no profiling events of their
    own."""
    import torch
    from hybrid_sliding_global_amd import _lib
    settle_clock(fn)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()

    def events(n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for pair in evs:  # torch creates the HIP event on first record; the library re-records kernel events
            for e in pair:
                e.record()
        torch.cuda.synchronize()
        return evs

    calls, kerns = events(steps), events(steps)
    for (c0, c1), (k0, k1) in zip(calls, kerns):  # interleaved: both see the same clock state
        if flush is not None:
            flush()
        c0.record()
        fn()
        c1.record()
        if flush is not None:
            flush()
        _lib.set_profile_events(k0, k1)
        fn()
        _lib.set_profile_events(None, None)
    torch.cuda.synchronize()
    tot_call = sum(c0.elapsed_time(c1) for c0, c1 in calls)
    tot_kern = sum(k0.elapsed_time(k1) for k0, k1 in kerns)
    return tot_call / steps, tot_kern / steps


def bench_prefill(steps, warmup):
    import torch
    from hybrid_sliding_global_amd import Stack, inputs
    from hybrid_sliding_global_amd import workloads as wl
    w = wl.workloads()[2]
    d = w.layers[0]
    S, Hq, Hkv, D = w.seq_len, d["num_q_heads"], d["num_kv_heads"], d["head_dim"]
    q_h = inputs.normal_bf16([2, 0, inputs.TENSOR_Q], (1, S, Hq, D))
    k_h = inputs.normal_bf16([2, 0, inputs.TENSOR_K], (1, Hkv, S, D))
    v_h = inputs.normal_bf16([2, 0, inputs.TENSOR_V], (1, Hkv, S, D))
    q, k, v = dev(q_h), dev(k_h), dev(v_h)
    st = Stack(w.layers)
    out = torch.empty((1, S, Hq, D), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(st.prefill_workspace_bytes(0, 1, S), dtype=torch.uint8, device="cuda:0")
    flops = wl.prefill_flops(S, Hq, D, 0)

    def step():
        st.prefill(0, q, [k], [v], out=out, workspace=ws)

    # timed region: K steps bracketed by synchronize
    settle = settle_clock(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / steps
    _, kern_ms = time_calls(step, steps, 2)
    return dict(flops=flops, ms_per_step=ms_per_step, wall=wall, kern_ms=kern_ms, q=q_h, k=k_h, v=v_h, w=w,
                settle_steps=settle)


def cpu_baseline(pre, budget_s=15.0):
    """fp64 oracle on a bounded, position-spread sample of the prefill rows."""
    import oracle
    from hybrid_sliding_global_amd import workloads as wl
    oracle.build(force=False)
    w = pre["w"]
    d = w.layers[0]
    S, Hq, D = w.seq_len, d["num_q_heads"], d["head_dim"]
    rng = np.random.default_rng(0)
    # grow the sample of distinct rows until it takes a few seconds
    n = 8
    while True:
        n = min(n, S * Hq)
        rows = np.sort(rng.choice(S * Hq, size=n, replace=False))
        pos = rows // Hq
        t0 = time.perf_counter()
        oracle.prefill(pre["q"], pre["k"], pre["v"], 0, d["rope_theta"], rows=rows)
        dt = time.perf_counter() - t0
        if dt > budget_s / 4 or n == S * Hq:
            break
        n *= 2
    reps = 1
    if n == S * Hq and dt < budget_s * 2 / 3:
        # the whole workload fits the budget: time it several times over
        reps = max(1, int(budget_s * 2 / 3 / max(dt, 1e-3)))
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.prefill(pre["q"], pre["k"], pre["v"], 0, d["rope_theta"], rows=rows)
        dt = (time.perf_counter() - t0) / reps
    flops = float(sum(4 * D * (int(p) + 1) for p in pos))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": "%d distinct query rows (uniform over positions and heads) of the 4096-token full-attention prefill, "
                      "fp64, %.2f s per pass, %d pass(es)" % (n, dt, reps)}


def make_flush():
    """A call that evicts L2 and the 256 MB MALL by reading (not writing) a
    512 MiB buffer, so the next timed kernel starts from HBM and no dirty
    lines of the flush are written back inside it."""
    import torch
    buf = torch.ones(1 << 27, dtype=torch.float32, device="cuda:0")  # 512 MiB
    sink = torch.empty((), dtype=torch.float32, device="cuda:0")

    def flush():
        torch.sum(buf, dim=0, out=sink)

    return flush


def bench_hbm_reference(reps=10):
    """Rates of plain library kernels on this GPU, as context for the decode
    roofline: torch's device copy of 2 GiB (read + write bytes) and torch's sum
    over 2 GiB (read bytes)."""
    import torch
    n = 1 << 31
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    sink = torch.empty((), dtype=torch.float32, device="cuda:0")
    res = {}
    for tag, fn, nbytes in (("copy", lambda: dst.copy_(src), 2 * n), ("read", lambda: torch.sum(src, dim=0, out=sink), n)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[tag + "_GB/s"] = nbytes / (ms * 1e-3) / 1e9
    del src, dst
    return res


def bench_small_prefill(steps, warmup):
    """The single sliding-layer prefill (B=1, S=64, Hq=4, Hkv=1, D=256, W=32,
    K=V): a latency-bound correctness workload, timed per call."""
    import torch
    from hybrid_sliding_global_amd import Stack, inputs
    from hybrid_sliding_global_amd import workloads as wl
    w = wl.workloads()[1]
    d = w.layers[0]
    q = dev(inputs.normal_bf16([1, 0, inputs.TENSOR_Q], (1, 64, 4, 256)))
    k = dev(inputs.normal_bf16([1, 0, inputs.TENSOR_K], (1, 1, 64, 256)))
    st = Stack(w.layers)
    out = torch.empty((1, 64, 4, 256), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(st.prefill_workspace_bytes(0, 1, 64), dtype=torch.uint8, device="cuda:0")

    def step():
        st.prefill(0, q, [k], [None], out=out, workspace=ws)

    call_ms, kern_ms = time_calls(step, steps, warmup)
    flops = wl.prefill_flops(64, 4, 256, d["window"])
    return {"workload": "sliding_prefill_s64", "algorithmic_flops": flops, "ms_per_call": call_ms,
            "kernel_ms": kern_ms, "TFLOP/s": flops / (call_ms * 1e-3) / 1e12,
            "note": "latency-bound: a few microseconds of launch and set-up for 6.4 MFLOP"}


def bench_decode(steps, warmup):
    import torch
    from hybrid_sliding_global_amd import Stack, inputs
    from hybrid_sliding_global_amd import workloads as wl
    w = wl.workloads()[3]
    B, L = w.batch, w.kv_len
    kv = np.full(B, L, np.int32)
    kl = torch.from_numpy(kv).to("cuda:0")
    flush = make_flush()
    res = {}
    total_bytes = 0
    total_ms = 0.0
    for li, d in enumerate(w.layers):
        D, Hq, Hkv = d["head_dim"], d["num_q_heads"], d["num_kv_heads"]
        q = dev(inputs.normal_bf16([3, li, inputs.TENSOR_Q], (B, Hq, D)))
        k = dev(inputs.normal_bf16([3, li, inputs.TENSOR_K], (B, Hkv, L, D)))
        v = None if d["kv_alias"] else dev(inputs.normal_bf16([3, li, inputs.TENSOR_V], (B, Hkv, L, D)))
        st = Stack([d])
        out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda:0")
        ws = torch.empty(st.decode_workspace_bytes(0, B, L), dtype=torch.uint8, device="cuda:0")

        def step():
            st.decode(0, q, [k], [v], kl, L, out=out, workspace=ws)

        call_ms, kern_ms = time_calls(step, steps, warmup, flush=flush)
        nbytes = wl.decode_bytes(kv, Hq, Hkv, D, d["window"], bool(d["kv_alias"]))
        name = "full" if d["kind"] == wl.FULL else "sliding"
        res[name] = {"bytes": nbytes, "ms_per_call": call_ms, "kernel_ms": kern_ms,
                     "GB/s": nbytes / (call_ms * 1e-3) / 1e9, "kernel_GB/s": nbytes / (kern_ms * 1e-3) / 1e9}
        total_bytes += nbytes
        total_ms += call_ms
        del q, k, v
    full = res["full"]
    return {
        "workload": "decode_b64_l8192 (full hd512 Hq8/Hkv2 + sliding hd256 W1024 K=V)",
        "value": total_bytes / (total_ms * 1e-3) / 1e9, "unit": "GB/s", "layers": res,
        "roofline": {"bound": "hbm", "achieved": full["kernel_GB/s"], "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": full["kernel_GB/s"] / PEAK_HBM_GBS,
                     "traffic": measured_traffic("k_decode<512,false,2>")},
    }


def bench_decode_long(steps, warmup):
    """Long-context decode: B=4, per-sequence KV lengths uniform in [1024, 131072]
    (seeded), full layer (D=512, Hq=16, Hkv=2) and sliding layer (D=256, Hq=16,
    Hkv=2, window 1024, K=V); caches flushed from L2/MALL before every call."""
    import torch
    from hybrid_sliding_global_amd import Stack, inputs
    from hybrid_sliding_global_amd import workloads as wl
    w = wl.workloads()[5]
    B, Lmax = w.batch, w.max_len
    kv = inputs.kv_lengths_uniform([5, 0, inputs.TENSOR_LEN], B, w.kv_len_range[0], w.kv_len_range[1])
    kl = torch.from_numpy(kv).to("cuda:0")
    max_kv = int(kv.max())
    flush = make_flush()
    res = {}
    for li, d in enumerate(w.layers):
        D, Hq, Hkv = d["head_dim"], d["num_q_heads"], d["num_kv_heads"]
        q = dev(inputs.normal_bf16([5, li, inputs.TENSOR_Q], (B, Hq, D)))
        k = dev(inputs.normal_bf16([5, li, inputs.TENSOR_K], (B, Hkv, Lmax, D)))
        v = None if d["kv_alias"] else dev(inputs.normal_bf16([5, li, inputs.TENSOR_V], (B, Hkv, Lmax, D)))
        st = Stack([d])
        out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda:0")
        ws = torch.empty(st.decode_workspace_bytes(0, B, max_kv), dtype=torch.uint8, device="cuda:0")

        def step():
            st.decode(0, q, [k], [v], kl, max_kv, out=out, workspace=ws)

        call_ms, kern_ms = time_calls(step, steps, warmup, flush=flush)
        nbytes = wl.decode_bytes(kv, Hq, Hkv, D, d["window"], bool(d["kv_alias"]))
        name = "full" if d["kind"] == wl.FULL else "sliding"
        res[name] = {"bytes": nbytes, "ms_per_call": call_ms, "kernel_ms": kern_ms,
                     "GB/s": nbytes / (call_ms * 1e-3) / 1e9, "kernel_GB/s": nbytes / (kern_ms * 1e-3) / 1e9}
        del q, k, v
    full = res["full"]
    return {
        "workload": "decode_b4_long (KV lengths %s; full hd512 Hq16/Hkv2 + sliding hd256 Hq16/Hkv2 W1024 K=V)"
                    % kv.tolist(),
        "unit": "GB/s", "layers": res,
        "roofline": {"bound": "hbm", "achieved": full["kernel_GB/s"], "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": full["kernel_GB/s"] / PEAK_HBM_GBS},
    }


def bench_next(steps, warmup):
    """The built NEXT rows, each against its roofline: a prefill chunk at a
    start position, prefill with bidirectional image spans, a 4-token verify
    step over a frozen cache, a sliding layer on a window-sized ring cache
    with the new token appended by the call, and E4M3 caches.  Decode caches
    are flushed from L2/MALL before every call, as in the decode legs."""
    import torch
    from hybrid_sliding_global_amd import Stack, inputs
    from hybrid_sliding_global_amd import workloads as wl

    def dev_u8(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")

    def prefill_entry(workload, flops, call_ms, kern_ms):
        t = flops / (kern_ms * 1e-3) / 1e12
        return {"workload": workload, "algorithmic_flops": flops, "ms_per_call": call_ms, "kernel_ms": kern_ms,
                "TFLOP/s": flops / (call_ms * 1e-3) / 1e12,
                "roofline": {"bound": "mfma", "achieved": t, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                             "frac": t / PEAK_BF16_TFLOPS}}

    def decode_entry(workload, nbytes, call_ms, kern_ms):
        g = nbytes / (kern_ms * 1e-3) / 1e9
        return {"workload": workload, "bytes": nbytes, "ms_per_call": call_ms, "kernel_ms": kern_ms,
                "GB/s": nbytes / (call_ms * 1e-3) / 1e9,
                "roofline": {"bound": "hbm", "achieved": g, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": g / PEAK_HBM_GBS}}

    res = {}
    D, Hq, Hkv = 512, 8, 2
    full = wl.layer_desc(wl.FULL, D, Hq, Hkv, wl.THETA_FULL, 0, 0)
    st = Stack([full])

    # chunked prefill: 2048 queries at positions 2048..4095 against a 4096-key cache
    P0, S = 2048, 2048
    q = dev(inputs.normal_bf16([6, 0, inputs.TENSOR_Q], (1, S, Hq, D)))
    k = dev(inputs.normal_bf16([6, 0, inputs.TENSOR_K], (1, Hkv, P0 + S, D)))
    v = dev(inputs.normal_bf16([6, 0, inputs.TENSOR_V], (1, Hkv, P0 + S, D)))
    out = torch.empty((1, S, Hq, D), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(st.prefill_workspace_bytes(0, 1, S, P0), dtype=torch.uint8, device="cuda:0")
    call_ms, kern_ms = time_calls(lambda: st.prefill(0, q, [k], [v], out=out, workspace=ws, start_pos=P0),
                                  steps, warmup)
    res["chunked_prefill"] = prefill_entry(
        "full layer hd512 Hq8/Hkv2, a 2048-token chunk at position 2048 (4096 cached keys)",
        4 * D * Hq * (S * P0 + S * (S + 1) // 2), call_ms, kern_ms)
    del q, k, v, out, ws

    # bidirectional spans: the 4096-token full layer with two image spans
    S = 4096
    spans = [(512, 1535), (2048, 2559)]
    span_end = np.arange(S, dtype=np.int32)
    for a0, a1 in spans:
        span_end[a0:a1 + 1] = a1
    q = dev(inputs.normal_bf16([6, 1, inputs.TENSOR_Q], (1, S, Hq, D)))
    k = dev(inputs.normal_bf16([6, 1, inputs.TENSOR_K], (1, Hkv, S, D)))
    v = dev(inputs.normal_bf16([6, 1, inputs.TENSOR_V], (1, Hkv, S, D)))
    se = torch.from_numpy(span_end.reshape(1, S)).to("cuda:0")
    out = torch.empty((1, S, Hq, D), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(st.prefill_workspace_bytes(0, 1, S), dtype=torch.uint8, device="cuda:0")
    call_ms, kern_ms = time_calls(lambda: st.prefill(0, q, [k], [v], out=out, workspace=ws, span_end=se),
                                  steps, warmup)
    visible = np.minimum(np.maximum(span_end.astype(np.int64), np.arange(S)), S - 1) + 1
    res["bidirectional_spans"] = prefill_entry(
        "full layer hd512 Hq8/Hkv2, 4096 tokens, image spans %s (bidirectional inside a span)" % spans,
        4 * D * Hq * int(visible.sum()), call_ms, kern_ms)
    del q, k, v, se, out, ws

    flush = make_flush()
    B, L, T = 64, 8192, 4
    kv = np.full(B, L, np.int32)
    kl = torch.from_numpy(kv).to("cuda:0")

    # verify: 4 query tokens per sequence over a frozen 8192-token cache
    q = dev(inputs.normal_bf16([7, 0, inputs.TENSOR_Q], (B, T, Hq, D)))
    k = dev(inputs.normal_bf16([7, 0, inputs.TENSOR_K], (B, Hkv, L, D)))
    v = dev(inputs.normal_bf16([7, 0, inputs.TENSOR_V], (B, Hkv, L, D)))
    out = torch.empty((B, T, Hq, D), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(st.decode_workspace_bytes(0, B, L, T), dtype=torch.uint8, device="cuda:0")
    call_ms, kern_ms = time_calls(lambda: st.decode(0, q, [k], [v], kl, L, out=out, workspace=ws),
                                  steps, 2, flush=flush)
    nbytes = B * Hkv * L * D * 2 * 2 + T * B * Hq * D * (2 + 4) + B * 4
    res["verify_decode"] = decode_entry(
        "B=64 full layer hd512 Hq8/Hkv2, 4 query tokens per sequence over a frozen 8192-token cache",
        nbytes, call_ms, kern_ms)
    del q, k, v, out, ws

    # ring: the batched decode's sliding layer on a 1024-row ring, new token appended by the call
    Ds, Hqs, W = 256, 8, 1024
    ring = wl.layer_desc(wl.SLIDING, Ds, Hqs, 1, wl.THETA_SLIDING, W, 1, kv_ring=W)
    st_r = Stack([ring])
    q = dev(inputs.normal_bf16([7, 1, inputs.TENSOR_Q], (B, Hqs, Ds)))
    k = dev(inputs.normal_bf16([7, 1, inputs.TENSOR_K], (B, 1, W, Ds)))
    kn = dev(inputs.normal_bf16([7, 1, inputs.TENSOR_V], (B, 1, Ds)))
    out = torch.empty((B, Hqs, Ds), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(st_r.decode_workspace_bytes(0, B, L), dtype=torch.uint8, device="cuda:0")
    call_ms, kern_ms = time_calls(lambda: st_r.decode(0, q, [k], [None], kl, L, out=out, workspace=ws, k_new=kn),
                                  steps, 2, flush=flush)
    nbytes = B * (W - 1) * Ds * 2 + B * Ds * 2 * 2 + B * Hqs * Ds * (2 + 4) + B * 4  # ring rows + new key in/out
    res["ring_append_decode"] = decode_entry(
        "B=64 sliding layer hd256 Hq8/Hkv1 W=1024 K=V on a 1024-row ring at position 8191, "
        "the new token's key written by the call", nbytes, call_ms, kern_ms)
    del q, k, kn, out, ws

    # E4M3 caches: the batched decode workload with one byte per cache element
    layers = {}
    total_bytes, total_ms = 0, 0.0
    for name, (Dl, Hql, Hkvl, Wl, alias, ks, vs) in (("full", (512, 8, 2, 0, 0, 0.125, 0.25)),
                                                      ("sliding", (256, 8, 1, 1024, 1, 0.125, 0.125))):
        kind = wl.FULL if Wl == 0 else wl.SLIDING
        theta = wl.THETA_FULL if Wl == 0 else wl.THETA_SLIDING
        d8 = wl.layer_desc(kind, Dl, Hql, Hkvl, theta, Wl, alias, kv_dtype=wl.KV_FP8, k_scale=ks, v_scale=vs)
        st8 = Stack([d8])
        q = dev(inputs.normal_bf16([8, Dl, inputs.TENSOR_Q], (B, Hql, Dl)))
        k = dev_u8(inputs.normal_e4m3([8, Dl, inputs.TENSOR_K], (B, Hkvl, L, Dl), ks))
        v = None if alias else dev_u8(inputs.normal_e4m3([8, Dl, inputs.TENSOR_V], (B, Hkvl, L, Dl), vs))
        out = torch.empty((B, Hql, Dl), dtype=torch.float32, device="cuda:0")
        ws = torch.empty(st8.decode_workspace_bytes(0, B, L), dtype=torch.uint8, device="cuda:0")
        call_ms, kern_ms = time_calls(lambda: st8.decode(0, q, [k], [v], kl, L, out=out, workspace=ws),
                                      steps, 2, flush=flush)
        keys = min(L, Wl) if Wl > 0 else L
        nbytes = B * Hkvl * keys * Dl * (1 if alias else 2) + B * Hql * Dl * (2 + 4) + B * 4
        layers[name] = decode_entry("", nbytes, call_ms, kern_ms)
        del layers[name]["workload"]
        total_bytes += nbytes
        total_ms += call_ms
        del q, k, v, out, ws
    res["fp8_decode"] = {
        "workload": "decode_b64_l8192 with E4M3 caches (one byte per element, per-tensor scales)",
        "GB/s": total_bytes / (total_ms * 1e-3) / 1e9, "layers": layers,
        "roofline": layers["full"]["roofline"]}
    return res


def bench_stack(steps):
    """35-layer prefill stack (B=1, S=2048; 28 sliding hd256 W512 K=V + 7 full hd512, 15 owned caches):
    one pass = every layer's prefill call, in order, on one stream.  A layer
    that shares an earlier layer's cache runs in that layer's workspace and
    reuses the key/value operand images it left there (images_ready): the
    same cache rotated with the same theta, so its key pass would rebuild
    them bit for bit."""
    import torch
    from hybrid_sliding_global_amd import Stack, inputs
    from hybrid_sliding_global_amd import workloads as wl
    w = wl.workloads()[4]
    S = w.seq_len
    st = Stack(w.layers)
    qs, ks, vs, outs, wss = [], [], [], [], []
    for i, d in enumerate(w.layers):
        D = d["head_dim"]
        qs.append(dev(inputs.normal_bf16([4, i, inputs.TENSOR_Q], (1, S, d["num_q_heads"], D))))
        own = d["kv_source_layer"] < 0
        ks.append(dev(inputs.normal_bf16([4, i, inputs.TENSOR_K], (1, d["num_kv_heads"], S, D))) if own else None)
        vs.append(dev(inputs.normal_bf16([4, i, inputs.TENSOR_V], (1, d["num_kv_heads"], S, D)))
                  if own and not d["kv_alias"] else None)
        outs.append(torch.empty((1, S, d["num_q_heads"], D), dtype=torch.float32, device="cuda:0"))
        # an owner's workspace also serves the layers sharing its cache
        need = max(st.prefill_workspace_bytes(j, 1, S) for j, e in enumerate(w.layers)
                   if j == i or e["kv_source_layer"] == i)
        wss.append(torch.empty(need, dtype=torch.uint8, device="cuda:0") if own else None)
    flops = sum(wl.prefill_flops(S, d["num_q_heads"], d["head_dim"], d["window"]) for d in w.layers)
    sl_flops = sum(wl.prefill_flops(S, d["num_q_heads"], d["head_dim"], d["window"]) for d in w.layers
                   if d["kind"] == wl.SLIDING)

    def one_pass(which=None):
        for i, d in enumerate(w.layers):
            if which is None or d["kind"] == which:
                src = st.source(i)
                st.prefill(i, qs[i], ks, vs, out=outs[i], workspace=wss[src], images_ready=src != i)

    def timed(fn):
        settle_clock(fn)
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    res = {}
    for tag, which, fl in (("sliding_layers", wl.SLIDING, sl_flops), ("full_layers", wl.FULL, flops - sl_flops)):
        ms = timed(lambda: one_pass(which))
        res[tag] = {"ms_per_pass": ms, "TFLOP/s": fl / (ms * 1e-3) / 1e12, "algorithmic_flops": fl}
    eager_ms = timed(one_pass)
    # the whole stack as one HIP graph (the library records no memset or allocation)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one_pass()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_pass()
    graph_ms = timed(graph.replay)
    # both ways of issuing a pass are timed; the pass rate is the faster one
    # (the graph replay has measured slower than eager launches here, by
    # 1-3 %: its nodes are not issued back to back as a stream's launches are)
    ms = min(graph_ms, eager_ms)
    res["stack"] = {"ms_per_pass": ms, "TFLOP/s": flops / (ms * 1e-3) / 1e12, "algorithmic_flops": flops,
                    "timing": "one HIP graph replay per pass" if graph_ms <= eager_ms else "eager calls, one stream",
                    "graph_ms_per_pass": graph_ms, "eager_ms_per_pass": eager_ms}
    return {"workload": "stack35_prefill_s2048", **res}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # each leg settles the clock first (SETTLE_MS); 100 timed steps are ~17 ms
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--no-long-decode", action="store_true")
    ap.add_argument("--no-small", action="store_true")
    ap.add_argument("--no-hbm-reference", action="store_true")
    ap.add_argument("--no-next", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy three times (scale for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the attention path has no multi-GPU code (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 3}), flush=True)
        return
    log("prefill: full-attention layer B=1 S=4096 Hq=8 Hkv=2 D=512")
    pre = bench_prefill(args.steps, args.warmup)
    tflops = pre["flops"] / (pre["ms_per_step"] * 1e-3) / 1e12
    kern_tflops = pre["flops"] / (pre["kern_ms"] * 1e-3) / 1e12
    log("prefill: %.3f ms/step (%.1f TFLOP/s), attention kernel %.3f ms (%.1f TFLOP/s)" %
        (pre["ms_per_step"], tflops, pre["kern_ms"], kern_tflops))
    line = {
        "metric": METRIC, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": pre["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "clock_settle": {"min_ms": SETTLE_MS, "headline_steps": pre["settle_steps"],
                         "note": "untimed calls before each leg's warm-up, until the GPU clock has left its idle ramp"},
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) bf16)",
        "config": {"workload": "full_prefill_s4096", "batch": 1, "seq_len": 4096, "q_heads": 8, "kv_heads": 2,
                   "head_dim": 512, "window": 0, "rope_theta": 1e6, "kv_alias": False,
                   "algorithmic_flops": pre["flops"]},
        "roofline": {"bound": "mfma", "achieved": kern_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": kern_tflops / PEAK_BF16_TFLOPS, "traffic": measured_traffic("k_prefill<512,32,2,true>")},
    }
    if not args.no_stack:
        log("stack: 35-layer prefill S=2048")
        line["stack"] = bench_stack(max(3, args.steps // 4))
        log("stack: %.3f ms per pass (%.1f TFLOP/s): %.3f ms as one graph, %.3f ms eager" %
            (line["stack"]["stack"]["ms_per_pass"], line["stack"]["stack"]["TFLOP/s"],
             line["stack"]["stack"]["graph_ms_per_pass"], line["stack"]["stack"]["eager_ms_per_pass"]))
    if not args.no_decode:
        log("decode: B=64 L=8192")
        line["decode"] = bench_decode(max(50, args.steps // 2), 2)  # short calls: enough samples for a stable mean
        log("decode: %.1f GB/s (full-layer kernel %.1f GB/s)" %
            (line["decode"]["value"], line["decode"]["layers"]["full"]["kernel_GB/s"]))
    if not args.no_decode and not args.no_long_decode:
        log("decode: B=4, long contexts")
        line["long_decode"] = bench_decode_long(max(50, args.steps // 2), 2)
        log("decode long: full-layer kernel %.1f GB/s, sliding-layer kernel %.1f GB/s" %
            (line["long_decode"]["layers"]["full"]["kernel_GB/s"],
             line["long_decode"]["layers"]["sliding"]["kernel_GB/s"]))
    if not args.no_next:
        log("next rows: chunked prefill, spans, verify, ring append, E4M3 caches")
        line["next_rows"] = bench_next(max(20, args.steps // 4), 5)
        log("next rows: %s" % json.dumps({k: round(v["roofline"]["frac"], 3) for k, v in line["next_rows"].items()}))
    if not args.no_small:
        log("small prefill: S=64 sliding layer")
        line["small_prefill"] = bench_small_prefill(max(10, args.steps), args.warmup)
        log("small prefill: %.1f us per call" % (line["small_prefill"]["ms_per_call"] * 1e3))
    if not args.no_hbm_reference:
        log("hbm reference: torch copy and sum over 2 GiB")
        line["hbm_reference"] = bench_hbm_reference()
        log("hbm reference: %s" % json.dumps(line["hbm_reference"]))
    if not args.no_cpu_baseline:
        log("cpu baseline: fp64 oracle on sampled rows")
        line["cpu_baseline"] = cpu_baseline(pre)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
