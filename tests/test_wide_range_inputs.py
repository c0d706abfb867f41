"""The wide-range parity inputs (tests/wide_range.py) really take online
softmax's rare paths: checked on the CPU from the oracle's fp64 scores.

The GPU kernels move a row's running maximum only when a block of keys beats
it by more than 8 log2 units (32-key tiles in prefill, 16-key steps in
decode), and the four-wave head-size-256 prefill repeats a pass when a row's
scores rise more than 64 log2 units above its first tile's maximum.  These
tests show that the inputs used by the GPU parity cases cross both bounds.
"""
import numpy as np
import pytest

import wide_range as wr

RESCALE = 8.0
REPEAT = 64.0

PREFILL_CASES = [
    # (B, S, Hq, Hkv, D, W, theta, seed, every, period)
    (1, 1024, 8, 2, 512, 0, 1e6, 0, None, 0),
    (1, 1024, 8, 1, 256, 0, 1e4, 1, None, 0),
    (1, 1024, 8, 1, 256, 512, 1e4, 2, 2, 10),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,W,theta,seed,every,period", PREFILL_CASES)
def test_prefill_inputs_cross_rescale_and_repeat_bounds(orc, B, S, Hq, Hkv, D, W, theta, seed, every, period):
    q, k, v, planted = wr.prefill_case(B, S, Hq, Hkv, D, W, theta, seed, every, period)
    assert len(planted) >= 6
    rows = [(S - 1) * Hq, (S // 2) * Hq + 1, (S - 40) * Hq + Hq - 1]
    jump, rise = wr.prefill_growth(orc, q, k, W, theta, rows)
    assert jump > RESCALE, jump
    assert rise > REPEAT, rise
    # N(0,1) inputs stay far below both bounds
    q0 = wr.inputs.normal_bf16([300 + seed, S, 0], (B, S, Hq, D))
    k0 = wr.inputs.normal_bf16([300 + seed, S, 1], (B, Hkv, S, D))
    j0, r0 = wr.prefill_growth(orc, q0, k0, W, theta, rows)
    assert j0 < RESCALE and r0 < REPEAT


DECODE_CASES = [
    # (B, Hq, Hkv, D, kv_len, Lmax, seed)
    (2, 8, 2, 512, [200, 150], 200, 0),
    (3, 8, 1, 256, [300, 97, 180], 300, 1),
]


@pytest.mark.parametrize("B,Hq,Hkv,D,kv_len,Lmax,seed", DECODE_CASES)
def test_decode_inputs_cross_rescale_bound(orc, B, Hq, Hkv, D, kv_len, Lmax, seed):
    kv = np.array(kv_len, np.int32)
    q, k, v = wr.decode_case(B, Hq, Hkv, D, kv, Lmax, seed)
    theta = 1e6 if D == 512 else 1e4
    assert wr.decode_growth(orc, q, k, kv, 0, theta) > RESCALE


def test_decode_split_covers_every_key_once():
    kv = [200, 150, 1, 4097]
    for Hkv, W in ((1, 0), (2, 0), (2, 100)):
        segs = wr.decode_split(kv, Hkv, W)
        for b, L in enumerate(kv):
            lo = max(0, L - W) if W else 0
            for h in range(Hkv):
                cover = [j for x0, x1 in segs[(b, h)] for j in range(x0, x1)]
                assert cover == list(range(lo, L))
