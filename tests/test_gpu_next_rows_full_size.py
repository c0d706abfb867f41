"""Parity of the NEXT rows at the sizes and in the launch configuration the
benchmark times them (bench.py, next_rows): a prefill chunk at a start
position, image spans, a 4-token verify step, a ring-cache sliding layer with
the new key appended by the call, and E4M3 caches.  Same shapes and seeds as
the benchmark legs; the fp64 oracle computes sampled output rows one by one."""
import numpy as np
import pytest

import oracle
from hybrid_sliding_global_amd import Stack, inputs
from hybrid_sliding_global_amd import workloads as wl
from gpu_util import check, to_dev

pytestmark = pytest.mark.gpu

D, HQ, HKV = 512, 8, 2
B_DEC, L_DEC = 64, 8192


def _sample(n_total, n, seed, must=()):
    rng = np.random.default_rng(seed)
    rows = set(int(r) for r in rng.choice(n_total, size=n, replace=False))
    rows.update(int(m) for m in must if 0 <= m < n_total)
    return np.array(sorted(rows), np.int64)


def test_chunked_prefill_bench_size():
    """2048 queries at positions 2048..4095 against a 4096-key full-layer cache."""
    import torch
    P0, S = 2048, 2048
    q = inputs.normal_bf16([6, 0, inputs.TENSOR_Q], (1, S, HQ, D))
    k = inputs.normal_bf16([6, 0, inputs.TENSOR_K], (1, HKV, P0 + S, D))
    v = inputs.normal_bf16([6, 0, inputs.TENSOR_V], (1, HKV, P0 + S, D))
    st = Stack([wl.layer_desc(wl.FULL, D, HQ, HKV, wl.THETA_FULL, 0, 0)])
    out = st.prefill(0, to_dev(q), [to_dev(k)], [to_dev(v)], start_pos=P0)
    torch.cuda.synchronize()
    rows = _sample(S * HQ, 96, 1, must=(0, HQ - 1, S * HQ - 1))
    want = oracle.prefill(q, k, v, 0, wl.THETA_FULL, rows=rows, start_pos=P0)
    check(out.cpu().numpy().reshape(-1, D)[rows], want, "chunked prefill S2048 at 2048 (bench size)")


def test_bidirectional_spans_bench_size():
    """The 4096-token full layer with image spans at 512-1535 and 2048-2559."""
    import torch
    S = 4096
    span_end = np.arange(S, dtype=np.int32)
    for a0, a1 in [(512, 1535), (2048, 2559)]:
        span_end[a0:a1 + 1] = a1
    q = inputs.normal_bf16([6, 1, inputs.TENSOR_Q], (1, S, HQ, D))
    k = inputs.normal_bf16([6, 1, inputs.TENSOR_K], (1, HKV, S, D))
    v = inputs.normal_bf16([6, 1, inputs.TENSOR_V], (1, HKV, S, D))
    st = Stack([wl.layer_desc(wl.FULL, D, HQ, HKV, wl.THETA_FULL, 0, 0)])
    se = torch.from_numpy(span_end.reshape(1, S)).to("cuda:0")
    out = st.prefill(0, to_dev(q), [to_dev(k)], [to_dev(v)], span_end=se)
    torch.cuda.synchronize()
    # span starts, interiors and ends, the positions just outside, and the last row
    must = [p * HQ + h for p in (511, 512, 1000, 1535, 1536, 2048, 2559, 2560, S - 1) for h in (0, HQ - 1)]
    rows = _sample(S * HQ, 96, 2, must=must)
    want = oracle.prefill(q, k, v, 0, wl.THETA_FULL, rows=rows, span_end=span_end.reshape(1, S))
    check(out.cpu().numpy().reshape(-1, D)[rows], want, "image spans S4096 (bench size)")


def test_verify_decode_bench_size():
    """4 query tokens per sequence over the batched decode's frozen full-layer cache."""
    import torch
    T = 4
    q = inputs.normal_bf16([7, 0, inputs.TENSOR_Q], (B_DEC, T, HQ, D))
    k = inputs.normal_bf16([7, 0, inputs.TENSOR_K], (B_DEC, HKV, L_DEC, D))
    v = inputs.normal_bf16([7, 0, inputs.TENSOR_V], (B_DEC, HKV, L_DEC, D))
    kv = np.full(B_DEC, L_DEC, np.int32)
    st = Stack([wl.layer_desc(wl.FULL, D, HQ, HKV, wl.THETA_FULL, 0, 0)])
    out = st.decode(0, to_dev(q), [to_dev(k)], [to_dev(v)], torch.from_numpy(kv).to("cuda:0"), L_DEC)
    torch.cuda.synchronize()
    rows = _sample(B_DEC * T * HQ, 64, 3, must=(0, T * HQ - 1, B_DEC * T * HQ - 1))
    want = oracle.decode(q, k, v, kv, 0, wl.THETA_FULL, rows=rows)
    check(out.cpu().numpy().reshape(-1, D)[rows], want, "verify T4 B64 L8192 (bench size)")


def test_ring_append_decode_bench_size():
    """The batched decode's sliding layer on a 1024-row ring at position 8191,
    the new key written by the call: the output matches the oracle over the
    ring with that row in place, and the row holds the key afterwards."""
    import torch
    Ds, Hqs, W = 256, 8, 1024
    q = inputs.normal_bf16([7, 1, inputs.TENSOR_Q], (B_DEC, Hqs, Ds))
    k = inputs.normal_bf16([7, 1, inputs.TENSOR_K], (B_DEC, 1, W, Ds))
    kn = inputs.normal_bf16([7, 1, inputs.TENSOR_V], (B_DEC, 1, Ds))
    kv = np.full(B_DEC, L_DEC, np.int32)
    st = Stack([wl.layer_desc(wl.SLIDING, Ds, Hqs, 1, wl.THETA_SLIDING, W, 1, kv_ring=W)])
    kd = to_dev(k)
    out = st.decode(0, to_dev(q), [kd], [None], torch.from_numpy(kv).to("cuda:0"), L_DEC, k_new=to_dev(kn))
    torch.cuda.synchronize()
    ring = k.copy()
    ring[:, :, (L_DEC - 1) % W] = kn
    assert np.array_equal(kd.cpu().view(torch.int16).numpy().view(np.uint16), ring), "appended key not in its ring row"
    rows = _sample(B_DEC * Hqs, 64, 4, must=(0, B_DEC * Hqs - 1))
    want = oracle.decode(q, ring, None, kv, W, wl.THETA_SLIDING, rows=rows, ring=W)
    check(out.cpu().numpy().reshape(-1, Ds)[rows], want, "ring append B64 W1024 (bench size)")


@pytest.mark.parametrize("Dl,Hql,Hkvl,Wl,alias,ks,vs", [
    (512, 8, 2, 0, 0, 0.125, 0.25),      # full layer, separate E4M3 values
    (256, 8, 1, 1024, 1, 0.125, 0.125),  # sliding layer, K=V
])
def test_fp8_decode_bench_size(Dl, Hql, Hkvl, Wl, alias, ks, vs):
    """The batched decode workload with E4M3 caches (one byte per element)."""
    import torch
    kind = wl.FULL if Wl == 0 else wl.SLIDING
    theta = wl.THETA_FULL if Wl == 0 else wl.THETA_SLIDING
    q = inputs.normal_bf16([8, Dl, inputs.TENSOR_Q], (B_DEC, Hql, Dl))
    k = inputs.normal_e4m3([8, Dl, inputs.TENSOR_K], (B_DEC, Hkvl, L_DEC, Dl), ks)
    v = None if alias else inputs.normal_e4m3([8, Dl, inputs.TENSOR_V], (B_DEC, Hkvl, L_DEC, Dl), vs)
    kv = np.full(B_DEC, L_DEC, np.int32)
    st = Stack([wl.layer_desc(kind, Dl, Hql, Hkvl, theta, Wl, alias, kv_dtype=wl.KV_FP8, k_scale=ks, v_scale=vs)])
    out = st.decode(0, to_dev(q), [to_dev(k)], [None if v is None else to_dev(v)],
                    torch.from_numpy(kv).to("cuda:0"), L_DEC)
    torch.cuda.synchronize()
    rows = _sample(B_DEC * Hql, 64, 5, must=(0, B_DEC * Hql - 1))
    want = oracle.decode(q, k, v, kv, Wl, theta, rows=rows, k_scale=ks, v_scale=vs)
    check(out.cpu().numpy().reshape(-1, Dl)[rows], want, "E4M3 decode D%d B64 L8192 (bench size)" % Dl)
