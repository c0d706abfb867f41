"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module holds no attention arithmetic: it only draws N(0, 1) samples
from numpy's PCG64 generator, rounds them to bfloat16 (round to nearest even)
and hands back the raw uint16 bit patterns.  Both the HIP path (after a copy
to the device) and the fp64 oracle consume exactly these bits.

Seeds follow ``numpy.random.default_rng([workload, layer, tensor])`` with
tensor ids 0 = q, 1 = k, 2 = v, 3 = kv lengths.
"""
from __future__ import annotations

import hashlib
from typing import Sequence

import numpy as np

NAN_BF16 = np.uint16(0x7FC0)
TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_LEN = 0, 1, 2, 3
_CHUNK = 1 << 24


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + np.uint32(0x7FFF) + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = NAN_BF16
    return r


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(seed: Sequence[int], shape) -> np.ndarray:
    """N(0,1) float32 samples rounded to bfloat16, as uint16 bits of ``shape``."""
    rng = np.random.default_rng(list(seed))
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = bf16_bits_from_f32(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


NAN_E4M3 = np.uint8(0x7F)


def normal_e4m3(seed: Sequence[int], shape, scale: float) -> np.ndarray:
    """E4M3 bytes (OCP encoding) of N(0,1) samples divided by ``scale`` (torch's
    round-to-nearest conversion): an 8-bit cache whose elements times
    ``scale`` are about N(0,1)."""
    import torch
    rng = np.random.default_rng(list(seed))
    x = rng.standard_normal(int(np.prod(shape)), dtype=np.float32) / np.float32(scale)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(shape)


def zeros_bf16(shape) -> np.ndarray:
    return np.zeros(shape, np.uint16)


def kv_lengths_uniform(seed: Sequence[int], batch: int, lo: int, hi: int) -> np.ndarray:
    """Per-sequence cache lengths drawn uniformly from [lo, hi] (inclusive)."""
    rng = np.random.default_rng(list(seed))
    return rng.integers(lo, hi, size=batch, endpoint=True).astype(np.int32)


def poison_beyond(cache: np.ndarray, kv_len: np.ndarray) -> np.ndarray:
    """Fill cache rows at or beyond each sequence's length with NaN (bfloat16
    or E4M3, by the array's dtype).

    ``cache`` is [B, H, Lmax, D]; a kernel that reads a row it must not read
    then produces NaN in its output.
    """
    nan = NAN_E4M3 if cache.dtype == np.uint8 else NAN_BF16
    for b, L in enumerate(np.asarray(kv_len)):
        cache[b, :, int(L):, :] = nan
    return cache


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
