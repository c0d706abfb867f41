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
                in order, with the sliding and full layers also timed apart.
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


def time_calls(fn, steps, warmup, flush=None):
    """Average time per call (events around each call) and per main kernel
    (events the library records immediately around it).  The two are taken on
    alternating calls, so the call times carry no profiling events of their
    own."""
    import torch
    from hybrid_sliding_global_amd import _lib
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
    return dict(flops=flops, ms_per_step=ms_per_step, wall=wall, kern_ms=kern_ms, q=q_h, k=k_h, v=v_h, w=w)


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


def bench_decode(steps, warmup):
    import torch
    from hybrid_sliding_global_amd import Stack, inputs
    from hybrid_sliding_global_amd import workloads as wl
    w = wl.workloads()[3]
    B, L = w.batch, w.kv_len
    kv = np.full(B, L, np.int32)
    kl = torch.from_numpy(kv).to("cuda:0")
    flush_buf = torch.empty(1 << 29, dtype=torch.uint8, device="cuda:0")  # 512 MiB > the 256 MB MALL

    def flush():
        flush_buf.fill_(1)

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
    flush_buf = torch.empty(1 << 29, dtype=torch.uint8, device="cuda:0")  # 512 MiB > the 256 MB MALL

    def flush():
        flush_buf.fill_(1)

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


def bench_stack(steps):
    """35-layer prefill stack (B=1, S=2048; 28 sliding hd256 W512 K=V + 7 full hd512, 15 owned caches):
    one pass = every layer's prefill call, in order, on one stream."""
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
        wss.append(torch.empty(st.prefill_workspace_bytes(i, 1, S), dtype=torch.uint8, device="cuda:0"))
    flops = sum(wl.prefill_flops(S, d["num_q_heads"], d["head_dim"], d["window"]) for d in w.layers)
    sl_flops = sum(wl.prefill_flops(S, d["num_q_heads"], d["head_dim"], d["window"]) for d in w.layers
                   if d["kind"] == wl.SLIDING)

    def one_pass(which=None):
        for i, d in enumerate(w.layers):
            if which is None or d["kind"] == which:
                st.prefill(i, qs[i], ks, vs, out=outs[i], workspace=wss[i])

    def timed(fn):
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
    ms = timed(graph.replay)
    res["stack"] = {"ms_per_pass": ms, "TFLOP/s": flops / (ms * 1e-3) / 1e12, "algorithmic_flops": flops,
                    "timing": "one HIP graph replay per pass", "eager_ms_per_pass": eager_ms}
    return {"workload": "stack35_prefill_s2048", **res}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--no-long-decode", action="store_true")
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
        log("stack: %.3f ms per pass as one graph (%.1f TFLOP/s), %.3f ms eager" %
            (line["stack"]["stack"]["ms_per_pass"], line["stack"]["stack"]["TFLOP/s"],
             line["stack"]["stack"]["eager_ms_per_pass"]))
    if not args.no_decode:
        log("decode: B=64 L=8192")
        line["decode"] = bench_decode(max(5, args.steps // 2), 2)
        log("decode: %.1f GB/s (full-layer kernel %.1f GB/s)" %
            (line["decode"]["value"], line["decode"]["layers"]["full"]["kernel_GB/s"]))
    if not args.no_decode and not args.no_long_decode:
        log("decode: B=4, long contexts")
        line["long_decode"] = bench_decode_long(max(5, args.steps // 2), 2)
        log("decode long: full-layer kernel %.1f GB/s, sliding-layer kernel %.1f GB/s" %
            (line["long_decode"]["layers"]["full"]["kernel_GB/s"],
             line["long_decode"]["layers"]["sliding"]["kernel_GB/s"]))
    if not args.no_cpu_baseline:
        log("cpu baseline: fp64 oracle on sampled rows")
        line["cpu_baseline"] = cpu_baseline(pre)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
