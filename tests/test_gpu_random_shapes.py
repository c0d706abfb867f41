"""Parity of the HIP path with the fp64 oracle on seeded random shapes.

The hand-picked cases elsewhere cover each kernel variant at its edges; these
draw batch, sequence length, start position, head counts (group sizes
1-8), head size, window, K=V aliasing, padding of the cache, ragged decode
lengths and tokens per decode step from fixed seeds, so that the work split
(pairs, pieces, 64- or 128-row tiles, both head-size-512 schedules, decode
pieces across ragged streams, column groups) meets combinations nobody
listed.  Each case compares every output element (max |diff| <= 2e-2,
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
