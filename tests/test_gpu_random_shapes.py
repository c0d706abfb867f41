"""Parity of the HIP path with the fp64 oracle on seeded random shapes.

The hand-picked cases elsewhere cover each kernel variant at its edges; these
draw batch, sequence length, start position, head counts (group sizes
1-8), head size, window, K=V aliasing, padding of the cache, ragged decode
lengths and tokens per decode step from fixed seeds, so that the work split
(pairs, pieces, 64- or 128-row tiles, both head-size-512 schedules, decode
pieces across ragged streams, column groups) meets combinations nobody
listed; the same for window-sized ring caches, the decode call's own
append of its tokens (output and cache bytes), bidirectional spans and
E4M3 caches with random scales.  Each case compares every output element (max |diff| <= 2e-2,
mean |diff| <= 2e-3, relative RMS <= 1e-2).
"""
import numpy as np
import pytest

import oracle
import test_gpu_parity
from gpu_util import check, to_dev
from hybrid_sliding_global_amd import Stack, inputs
from hybrid_sliding_global_amd import workloads as wl
from test_gpu_parity import _decode_case, _prefill_case

pytestmark = pytest.mark.gpu

_setup = test_gpu_parity._setup  # the oracle build / GPU check fixture (autouse)


def _heads(rng, kvs, gs):
    Hkv = int(rng.choice(kvs))
    return int(rng.choice(gs)) * Hkv, Hkv


def _prefill_shapes(n=32, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([256, 512]))
        Hq, Hkv = _heads(rng, [1, 2, 4], [1, 2, 3, 4, 5, 8])
        B = int(rng.integers(1, 4))
        S = int(rng.integers(1, 1300 if D == 256 else 1000))
        W = 0 if rng.random() < 0.4 else int(rng.integers(1, S + 64))
        alias = bool(rng.random() < 0.5)
        Lmax = S + int(rng.choice([0, 0, 7, 64]))
        out.append((i, B, S, Hq, Hkv, D, W, alias, Lmax))
    return out


def _chunk_shapes(n=16, seed=20261206):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([256, 512]))
        Hq, Hkv = _heads(rng, [1, 2], [1, 2, 4, 8])
        B = int(rng.integers(1, 3))
        S = int(rng.integers(1, 500))
        P0 = int(rng.integers(1, 1500))
        W = 0 if rng.random() < 0.5 else int(rng.integers(1, 1200))
        alias = bool(rng.random() < 0.5)
        out.append((i, B, S, P0, Hq, Hkv, D, W, alias))
    return out


def _decode_shapes(n=32, seed=20261205):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([256, 512]))
        Hq, Hkv = _heads(rng, [1, 2], [1, 2, 4, 8])
        B = int(rng.integers(1, 9))
        Lmax = int(rng.integers(16, 5000))
        kv_len = [int(x) for x in rng.integers(1, Lmax + 1, size=B)]
        W = 0 if rng.random() < 0.5 else int(rng.integers(1, 1200))
        alias = bool(rng.random() < 0.5)
        out.append((i, B, Hq, Hkv, D, W, alias, kv_len, Lmax))
    return out


def _multi_token_shapes(n=16, seed=20261207):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([256, 512]))
        Hq, Hkv = _heads(rng, [1, 2], [1, 2, 4, 8])
        B = int(rng.integers(1, 6))
        T = int(rng.integers(2, 8))
        Lmax = int(rng.integers(T + 8, 4000))
        kv_len = [int(x) for x in rng.integers(T, Lmax + 1, size=B)]
        W = 0 if rng.random() < 0.5 else int(rng.integers(1, 1200))
        alias = bool(rng.random() < 0.5)
        out.append((i, B, T, Hq, Hkv, D, W, alias, kv_len, Lmax))
    return out


def _theta(W):
    return wl.THETA_SLIDING if W > 0 else wl.THETA_FULL


def _kind(W):
    return wl.SLIDING if W > 0 else wl.FULL


@pytest.mark.parametrize("i,B,S,Hq,Hkv,D,W,alias,Lmax", _prefill_shapes())
def test_random_prefill_shape(i, B, S, Hq, Hkv, D, W, alias, Lmax):
    _prefill_case("random prefill %d: B%d S%d Hq%d Hkv%d D%d W%d alias%d Lmax%d" % (i, B, S, Hq, Hkv, D, W, alias, Lmax),
                  B, S, Hq, Hkv, D, W, alias, Lmax, seed=300 + i)


@pytest.mark.parametrize("i,B,S,P0,Hq,Hkv,D,W,alias", _chunk_shapes())
def test_random_chunked_prefill_shape(i, B, S, P0, Hq, Hkv, D, W, alias):
    import torch
    Lmax = P0 + S + 5
    q = inputs.normal_bf16([900 + i, P0, 0], (B, S, Hq, D))
    k = inputs.normal_bf16([900 + i, P0, 1], (B, Hkv, Lmax, D))
    v = None if alias else inputs.normal_bf16([900 + i, P0, 2], (B, Hkv, Lmax, D))
    k[:, :, P0 + S:] = inputs.NAN_BF16  # rows past the chunk must never be read
    if v is not None:
        v[:, :, P0 + S:] = inputs.NAN_BF16
    st = Stack([wl.layer_desc(_kind(W), D, Hq, Hkv, _theta(W), W, int(alias))])
    ws = torch.full((st.prefill_workspace_bytes(0, B, S, P0),), 0xFF, dtype=torch.uint8, device="cuda:0")
    out = st.prefill(0, to_dev(q), [to_dev(k)], [None if v is None else to_dev(v)], workspace=ws, start_pos=P0)
    torch.cuda.synchronize()
    check(out.cpu().numpy(), oracle.prefill(q, k, v, W, _theta(W), start_pos=P0),
          "random chunk %d: B%d S%d P0=%d Hq%d Hkv%d D%d W%d alias%d" % (i, B, S, P0, Hq, Hkv, D, W, alias))


@pytest.mark.parametrize("i,B,Hq,Hkv,D,W,alias,kv_len,Lmax", _decode_shapes())
def test_random_decode_shape(i, B, Hq, Hkv, D, W, alias, kv_len, Lmax):
    _decode_case("random decode %d: B%d Hq%d Hkv%d D%d W%d alias%d kv %s" % (i, B, Hq, Hkv, D, W, alias, kv_len),
                 B, Hq, Hkv, D, W, alias, kv_len, Lmax, seed=300 + i)


@pytest.mark.parametrize("i,B,T,Hq,Hkv,D,W,alias,kv_len,Lmax", _multi_token_shapes())
def test_random_multi_token_decode_shape(i, B, T, Hq, Hkv, D, W, alias, kv_len, Lmax):
    import torch
    kv = np.asarray(kv_len, np.int32)
    q = inputs.normal_bf16([950 + i, T, 0], (B, T, Hq, D))
    k = inputs.poison_beyond(inputs.normal_bf16([950 + i, T, 1], (B, Hkv, Lmax, D)), kv)
    v = None if alias else inputs.poison_beyond(inputs.normal_bf16([950 + i, T, 2], (B, Hkv, Lmax, D)), kv)
    st = Stack([wl.layer_desc(_kind(W), D, Hq, Hkv, _theta(W), W, int(alias))])
    ws = torch.full((st.decode_workspace_bytes(0, B, Lmax, T),), 0xFF, dtype=torch.uint8, device="cuda:0")
    out = st.decode(0, to_dev(q), [to_dev(k)], [None if v is None else to_dev(v)], torch.from_numpy(kv).to("cuda:0"),
                    Lmax, workspace=ws)
    torch.cuda.synchronize()
    check(out.cpu().numpy(), oracle.decode(q, k, v, kv, W, _theta(W)),
          "random decode T%d %d: B%d Hq%d Hkv%d D%d W%d alias%d kv %s" % (T, i, B, Hq, Hkv, D, W, alias, kv_len))


# ---------------------------------------------------------- NEXT-row paths --

def _ring_shapes(n=12, seed=20261208):
    """Sliding layers on window-sized rings (C >= W + T - 1), one or more tokens."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([256, 512]))
        Hq, Hkv = _heads(rng, [1, 2], [1, 2, 4, 8])
        B = int(rng.integers(1, 6))
        T = int(rng.choice([1, 1, 2, 3]))
        W = int(rng.integers(8, 1100))
        C = W + T - 1 + int(rng.choice([0, 0, 5, 64]))
        kv_len = [int(x) for x in rng.integers(T, 6000, size=B)]
        alias = bool(rng.random() < 0.5)
        out.append((i, B, T, Hq, Hkv, D, W, C, alias, kv_len))
    return out


@pytest.mark.parametrize("i,B,T,Hq,Hkv,D,W,C,alias,kv_len", _ring_shapes())
def test_random_ring_decode_shape(i, B, T, Hq, Hkv, D, W, C, alias, kv_len):
    import torch
    kv = np.asarray(kv_len, np.int32)
    Lmax = int(kv.max())
    q = inputs.normal_bf16([1000 + i, C, 0], (B, T, Hq, D) if T > 1 else (B, Hq, D))
    k = inputs.normal_bf16([1000 + i, C, 1], (B, Hkv, Lmax, D))
    v = None if alias else inputs.normal_bf16([1000 + i, C, 2], (B, Hkv, Lmax, D))
    spare = C - (W + T - 1)
    kr = test_gpu_parity._ring_from_linear(k, kv, C, spare)
    vr = None if alias else test_gpu_parity._ring_from_linear(v, kv, C, spare)
    st = Stack([wl.layer_desc(wl.SLIDING, D, Hq, Hkv, wl.THETA_SLIDING, W, int(alias), kv_ring=C)])
    out = st.decode(0, to_dev(q), [to_dev(kr)], [None if vr is None else to_dev(vr)],
                    torch.from_numpy(kv).to("cuda:0"), Lmax)
    torch.cuda.synchronize()
    check(out.cpu().numpy(), oracle.decode(q, kr, vr, kv, W, wl.THETA_SLIDING, ring=C),
          "random ring %d: B%d T%d Hq%d Hkv%d D%d W%d C%d alias%d" % (i, B, T, Hq, Hkv, D, W, C, alias))


def _append_shapes(n=12, seed=20261209):
    """The call writes its tokens' keys/values (linear cache or ring) and attends to them."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([256, 512]))
        Hq, Hkv = _heads(rng, [1, 2], [1, 2, 4, 8])
        B = int(rng.integers(1, 5))
        T = int(rng.choice([1, 1, 2, 4]))
        W = 0 if rng.random() < 0.4 else int(rng.integers(8, 1100))
        C = 0 if (W == 0 or rng.random() < 0.5) else W + T - 1 + int(rng.choice([0, 3]))
        Lmax = 0 if C else int(rng.integers(T + 4, 4000))
        kv_len = [int(x) for x in rng.integers(T, (6000 if C else Lmax) + 1, size=B)]
        alias = bool(rng.random() < 0.5)
        out.append((i, B, T, Hq, Hkv, D, W, C, alias, kv_len, Lmax))
    return out


@pytest.mark.parametrize("i,B,T,Hq,Hkv,D,W,C,alias,kv_len,Lmax", _append_shapes())
def test_random_fused_append_shape(i, B, T, Hq, Hkv, D, W, C, alias, kv_len, Lmax):
    import torch
    kv = np.asarray(kv_len, np.int32)
    rows = C if C else Lmax
    q = inputs.normal_bf16([1100 + i, T, 0], (B, T, Hq, D) if T > 1 else (B, Hq, D))
    kc = inputs.normal_bf16([1100 + i, T, 1], (B, Hkv, rows, D))  # stale contents everywhere
    vc = None if alias else inputs.normal_bf16([1100 + i, T, 2], (B, Hkv, rows, D))
    kn = inputs.normal_bf16([1100 + i, T, 3], (B, T, Hkv, D) if T > 1 else (B, Hkv, D))
    vn = None if alias else inputs.normal_bf16([1100 + i, T, 4], (B, T, Hkv, D) if T > 1 else (B, Hkv, D))
    kw, vw = kc.copy(), None if vc is None else vc.copy()
    kn4, vn4 = kn.reshape(B, T, Hkv, D), None if vn is None else vn.reshape(B, T, Hkv, D)
    for b in range(B):
        for t in range(T):
            r = (kv[b] - T + t) % C if C else kv[b] - T + t
            kw[b, :, r] = kn4[b, t]
            if vw is not None:
                vw[b, :, r] = vn4[b, t]
    st = Stack([wl.layer_desc(_kind(W), D, Hq, Hkv, _theta(W), W, int(alias), kv_ring=C)])
    kd, vd = to_dev(kc), None if vc is None else to_dev(vc)
    out = st.decode(0, to_dev(q), [kd], [vd], torch.from_numpy(kv).to("cuda:0"), int(kv.max()),
                    k_new=to_dev(kn), v_new=None if vn is None else to_dev(vn))
    torch.cuda.synchronize()
    check(out.cpu().numpy(), oracle.decode(q, kw, vw, kv, W, _theta(W), ring=C),
          "random append %d: B%d T%d Hq%d Hkv%d D%d W%d C%d alias%d" % (i, B, T, Hq, Hkv, D, W, C, alias))
    assert np.array_equal(kd.cpu().view(torch.int16).numpy().view(np.uint16), kw), "key cache after the append"
    if vd is not None:
        assert np.array_equal(vd.cpu().view(torch.int16).numpy().view(np.uint16), vw), "value cache after the append"


def _span_shapes(n=12, seed=20261210):
    """Prefill chunks with random disjoint bidirectional spans."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([256, 512]))
        Hq, Hkv = _heads(rng, [1, 2], [1, 2, 4, 8])
        B = int(rng.integers(1, 3))
        S = int(rng.integers(16, 700))
        P0 = int(rng.choice([0, 0, int(rng.integers(1, 800))]))
        W = 0 if rng.random() < 0.6 else int(rng.integers(1, 900))
        alias = bool(rng.random() < 0.5)
        spans = []
        for b in range(B):
            cuts = np.sort(rng.choice(np.arange(P0, P0 + S), size=min(S, 2 * int(rng.integers(1, 4))), replace=False))
            spans.append([(int(cuts[j]), int(cuts[j + 1])) for j in range(0, len(cuts) - 1, 2)])
        out.append((i, B, S, P0, Hq, Hkv, D, W, alias, spans))
    return out


@pytest.mark.parametrize("i,B,S,P0,Hq,Hkv,D,W,alias,spans", _span_shapes())
def test_random_spans_shape(i, B, S, P0, Hq, Hkv, D, W, alias, spans):
    import torch
    Lmax = P0 + S
    q = inputs.normal_bf16([1200 + i, S, 0], (B, S, Hq, D))
    k = inputs.normal_bf16([1200 + i, S, 1], (B, Hkv, Lmax, D))
    v = None if alias else inputs.normal_bf16([1200 + i, S, 2], (B, Hkv, Lmax, D))
    se = test_gpu_parity._span_end(B, S, P0, spans)
    st = Stack([wl.layer_desc(_kind(W), D, Hq, Hkv, _theta(W), W, int(alias))])
    ws = torch.full((st.prefill_workspace_bytes(0, B, S, P0),), 0xFF, dtype=torch.uint8, device="cuda:0")
    out = st.prefill(0, to_dev(q), [to_dev(k)], [None if v is None else to_dev(v)], workspace=ws, start_pos=P0,
                     span_end=torch.from_numpy(se).to("cuda:0"))
    torch.cuda.synchronize()
    check(out.cpu().numpy(), oracle.prefill(q, k, v, W, _theta(W), start_pos=P0, span_end=se),
          "random spans %d: B%d S%d P0=%d Hq%d Hkv%d D%d W%d alias%d %s" % (i, B, S, P0, Hq, Hkv, D, W, alias, spans))


def _fp8_shapes(n=12, seed=20261211):
    """E4M3 caches with random per-tensor scales: prefill (even i) and decode (odd i)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([256, 512]))
        Hq, Hkv = _heads(rng, [1, 2], [1, 2, 4, 8])
        B = int(rng.integers(1, 4))
        W = 0 if rng.random() < 0.5 else int(rng.integers(1, 1100))
        alias = bool(rng.random() < 0.5)
        ks = float(2.0 ** rng.uniform(-4, 1))
        vs = ks if alias else float(2.0 ** rng.uniform(-4, 1))
        n_len = int(rng.integers(1, 900)) if i % 2 == 0 else int(rng.integers(8, 4000))
        out.append((i, B, n_len, Hq, Hkv, D, W, alias, ks, vs))
    return out


@pytest.mark.parametrize("i,B,n_len,Hq,Hkv,D,W,alias,ks,vs", _fp8_shapes())
def test_random_fp8_cache_shape(i, B, n_len, Hq, Hkv, D, W, alias, ks, vs):
    import torch
    st = Stack([wl.layer_desc(_kind(W), D, Hq, Hkv, _theta(W), W, int(alias), kv_dtype=wl.KV_FP8, k_scale=ks,
                              v_scale=vs)])
    if i % 2 == 0:  # prefill of n_len tokens
        S = n_len
        q = inputs.normal_bf16([1300 + i, S, 0], (B, S, Hq, D))
        k = inputs.normal_e4m3([1300 + i, S, 1], (B, Hkv, S + 3, D), ks)
        v = None if alias else inputs.normal_e4m3([1300 + i, S, 2], (B, Hkv, S + 3, D), vs)
        k[:, :, S:] = inputs.NAN_E4M3
        if v is not None:
            v[:, :, S:] = inputs.NAN_E4M3
        out = st.prefill(0, to_dev(q), [to_dev(k)], [None if v is None else to_dev(v)])
        torch.cuda.synchronize()
        want = oracle.prefill(q, k, v, W, _theta(W), k_scale=ks, v_scale=vs)
    else:  # one-token decode over ragged lengths up to n_len
        kv = np.random.default_rng(1300 + i).integers(1, n_len + 1, size=B).astype(np.int32)
        q = inputs.normal_bf16([1300 + i, n_len, 0], (B, Hq, D))
        k = inputs.poison_beyond(inputs.normal_e4m3([1300 + i, n_len, 1], (B, Hkv, n_len, D), ks), kv)
        v = None if alias else inputs.poison_beyond(inputs.normal_e4m3([1300 + i, n_len, 2], (B, Hkv, n_len, D), vs), kv)
        out = st.decode(0, to_dev(q), [to_dev(k)], [None if v is None else to_dev(v)], torch.from_numpy(kv).to("cuda:0"),
                        int(kv.max()))
        torch.cuda.synchronize()
        want = oracle.decode(q, k, v, kv, W, _theta(W), k_scale=ks, v_scale=vs)
    check(out.cpu().numpy(), want, "random fp8 %d: B%d n%d Hq%d Hkv%d D%d W%d alias%d ks%.3g vs%.3g" % (
        i, B, n_len, Hq, Hkv, D, W, alias, ks, vs))
