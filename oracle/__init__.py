"""Reference oracle (fp64, CPU) for the hybrid sliding/global attention layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``.  The HIP library never imports,
links or calls it, and it shares no code with the HIP library.

The arithmetic lives in ``oracle.c`` (plain C, double precision, OpenMP over
independent rows); this module only compiles it with gcc and marshals numpy
arrays into it.  bfloat16 tensors are passed as their raw uint16 bit patterns.

Source of each definition (the page and section it restates):
  * head sizes 256 / 512, full attention on every fifth layer, RoPE theta
    1e4 / 1e6, 35 layers sharing 15 KV caches: onnxruntime-genai feature
    request "Support for Google Gemma 4 model family", sections
    "Variable Attention Head Dimensions", "KV Cache Sharing",
    "Gemma 4 Model Details";
  * K=V aliasing in sliding layers (V is the raw key projection): the
    Gemma-4 weight loader page (spark_model/weight_loader/gemma4.rs),
    comment in ``supports_tp``; SGLang PR "Support encoder-free unified
    Text/Vision/Audio model", attention_k_eq_v shard duplication;
  * softmax attention with causal / sliding-window masks, RoPE and GQA:
    standard definitions; the readings taken where the pages are silent
    (window counts W keys including self, scale 1/sqrt(D), rotate-half
    pairing, raw keys in the cache) are listed in the design notes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# HSG_ORACLE_LIB lets the mutation test load a deliberately broken copy.
_LIB_OVERRIDE = os.environ.get("HSG_ORACLE_LIB")
_LIB_PATH = _LIB_OVERRIDE or os.path.join(_HERE, "liboracle.so")
_lib = None

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math, OpenMP) into liboracle.so."""
    global _lib
    if _LIB_OVERRIDE:
        return _LIB_PATH
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
        _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.orc_rope_inv_freq.argtypes = [ctypes.c_int32, ctypes.c_double, _f64p]
        lib.orc_rope.argtypes = [_f64p, ctypes.c_int32, ctypes.c_double, ctypes.c_double, _f64p]
        lib.orc_attention_row.argtypes = [_u16p, _u16p, _u16p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int32, ctypes.c_double, ctypes.c_double, _f64p, _f64p]
        lib.orc_attention_row.restype = ctypes.c_int
        lib.orc_scores_row.argtypes = [_u16p, _u16p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_double, ctypes.c_double, _f64p]
        lib.orc_scores_row.restype = ctypes.c_int
        lib.orc_prefill.argtypes = [ctypes.c_int32] * 7 + [ctypes.c_double, ctypes.c_double, _u16p, _u16p, _u16p,
                                                           _i64p, ctypes.c_int64, _f64p, ctypes.c_int32]
        lib.orc_prefill.restype = ctypes.c_int
        lib.orc_decode.argtypes = [ctypes.c_int32] * 6 + [ctypes.c_double, ctypes.c_double, _u16p, _u16p, _u16p,
                                                          _i32p, _i64p, ctypes.c_int64, _f64p, ctypes.c_int32]
        lib.orc_decode.restype = ctypes.c_int
        vp = ctypes.c_void_p
        lib.orc_prefill_ext.argtypes = [ctypes.c_int32] * 7 + [ctypes.c_double, ctypes.c_double, _u16p, vp, vp,
                                                               ctypes.c_int32, ctypes.c_double, ctypes.c_double,
                                                               ctypes.c_int32, _i32p, _i64p, ctypes.c_int64, _f64p,
                                                               ctypes.c_int32]
        lib.orc_prefill_ext.restype = ctypes.c_int
        lib.orc_decode_ext.argtypes = [ctypes.c_int32] * 7 + [ctypes.c_double, ctypes.c_double, _u16p, vp, vp,
                                                              ctypes.c_int32, ctypes.c_double, ctypes.c_double, _i32p,
                                                              ctypes.c_int64, _i64p, ctypes.c_int64, _f64p,
                                                              ctypes.c_int32]
        lib.orc_decode_ext.restype = ctypes.c_int
        lib.orc_fp8_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        lib.orc_fp8_e4m3_to_f64.restype = ctypes.c_double
        lib.orc_fp8_e4m3_quantize.argtypes = [ctypes.c_float, ctypes.c_float]
        lib.orc_fp8_e4m3_quantize.restype = ctypes.c_uint8
        lib.orc_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray], t):
    if a is None:
        return ctypes.cast(None, t)
    return a.ctypes.data_as(t)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bfloat16 tensors are passed as uint16 bit patterns")
    return a


def max_threads() -> int:
    return int(_load().orc_max_threads())


def inv_freq(D: int, theta: float) -> np.ndarray:
    out = np.empty(D // 2, np.float64)
    _load().orc_rope_inv_freq(D, theta, _ptr(out, _f64p))
    return out


def rope(x: np.ndarray, theta: float, pos: float) -> np.ndarray:
    """Rotate-half RoPE of one fp64 D-vector at position ``pos``."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    _load().orc_rope(_ptr(x, _f64p), x.shape[0], theta, float(pos), _ptr(y, _f64p))
    return y


def attention_row(q: np.ndarray, k_slice: np.ndarray, v_slice: Optional[np.ndarray], pos: int, length: int,
                  window: int, theta: float, scale: float = 0.0):
    """One query row over one (batch, kv-head) cache slice.

    Returns ``(weights[length], out[D])``.  ``v_slice=None`` means an aliased
    layer: the value rows are the raw key rows.
    """
    q = _u16(q)
    k_slice = _u16(k_slice)
    v_slice = k_slice if v_slice is None else _u16(v_slice)
    D = q.shape[-1]
    w = np.empty(length, np.float64)
    o = np.empty(D, np.float64)
    rc = _load().orc_attention_row(_ptr(q, _u16p), _ptr(k_slice, _u16p), _ptr(v_slice, _u16p), D, pos, length,
                                   window, theta, scale, _ptr(w, _f64p), _ptr(o, _f64p))
    if rc != 0:
        raise ValueError("oracle: invalid attention row")
    return w, o


def scores_row(q: np.ndarray, k_slice: np.ndarray, pos: int, length: int, window: int, theta: float,
               scale: float = 0.0) -> np.ndarray:
    """Scores (natural units) of one query row over one (batch, kv-head) cache slice.

    Returns ``length`` doubles: scale * <RoPE(q, pos), RoPE(k_j, j)> for the
    keys visible from ``pos``, -inf for the others.
    """
    q = _u16(q)
    k_slice = _u16(k_slice)
    D = q.shape[-1]
    s = np.empty(length, np.float64)
    rc = _load().orc_scores_row(_ptr(q, _u16p), _ptr(k_slice, _u16p), D, pos, length, window, theta, scale,
                                _ptr(s, _f64p))
    if rc != 0:
        raise ValueError("oracle: invalid scores row")
    return s


KV_BF16, KV_FP8 = 0, 1


def fp8_e4m3_value(codes) -> np.ndarray:
    """Exact values of OCP E4M3 bytes (NaN for the two NaN codes)."""
    lib = _load()
    c = np.asarray(codes, np.uint8)
    return np.array([lib.orc_fp8_e4m3_to_f64(int(x)) for x in c.ravel()], np.float64).reshape(c.shape)


def fp8_e4m3_quantize(x, scale: float) -> np.ndarray:
    """E4M3 codes of x / scale (quotient in float32, nearest value, ties to
    even, saturating at +-448): what an 8-bit cache stores for the values x."""
    lib = _load()
    a = np.asarray(x, np.float32)
    return np.array([lib.orc_fp8_e4m3_quantize(float(v), float(scale)) for v in a.ravel()],
                    np.uint8).reshape(a.shape)


def _kv(a: Optional[np.ndarray]):
    """A cache tensor: uint16 (bf16 bits) or uint8 (E4M3 bytes); returns (array, format)."""
    if a is None:
        return None, None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return a, KV_BF16
    if a.dtype == np.uint8:
        return a, KV_FP8
    raise TypeError("cache tensors are uint16 (bfloat16 bits) or uint8 (E4M3 bytes)")


def _vptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def prefill(q: np.ndarray, k: np.ndarray, v: Optional[np.ndarray], window: int, theta: float, scale: float = 0.0,
            rows: Optional[Sequence[int]] = None, nthreads: int = 0, start_pos: int = 0,
            span_end: Optional[np.ndarray] = None, k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Prefill attention; q [B,S,Hq,D] at positions start_pos..start_pos+S-1,
    k/v [B,Hkv,Lmax,D] (bf16 bits, or E4M3 bytes times k_scale / v_scale;
    v None = aliased), span_end None (causal) or int32 [B,S] (last position
    of each query's bidirectional span).

    Returns fp64 [B,S,Hq,D], or [len(rows), D] for flattened rows b*S*Hq+s*Hq+h.
    """
    q = _u16(q)
    k, kf = _kv(k)
    v, vf = _kv(v)
    B, S, Hq, D = q.shape
    _, Hkv, Lmax, Dk = k.shape
    if Dk != D or (v is not None and (v.shape != k.shape or vf != kf)):
        raise ValueError("shape mismatch")
    se = None if span_end is None else np.ascontiguousarray(span_end, dtype=np.int32)
    if se is not None and se.shape != (B, S):
        raise ValueError("span_end must be [B, S]")
    if rows is None:
        out = np.empty((B, S, Hq, D), np.float64)
        r, n = None, -1
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        n = r.shape[0]
        out = np.empty((n, D), np.float64)
    rc = _load().orc_prefill_ext(B, S, Hq, Hkv, D, Lmax, window, theta, scale, _ptr(q, _u16p), _vptr(k), _vptr(v),
                                 kf, k_scale, v_scale, start_pos, _ptr(se, _i32p), _ptr(r, _i64p), n,
                                 _ptr(out, _f64p), nthreads)
    if rc != 0:
        raise ValueError("oracle: invalid prefill arguments")
    return out


def decode(q: np.ndarray, k: np.ndarray, v: Optional[np.ndarray], kv_len: np.ndarray, window: int, theta: float,
           scale: float = 0.0, rows: Optional[Sequence[int]] = None, nthreads: int = 0, ring: int = 0,
           k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Decode attention; q [B,Hq,D] (one token at kv_len-1) or [B,T,Hq,D] (T
    tokens at kv_len-T .. kv_len-1), k/v [B,Hkv,Lmax,D] (bf16 bits or E4M3
    bytes; with ring = Lmax > 0, position j in row j % ring), kv_len [B] (host).
    Returns fp64 shaped like q, or [len(rows), D]."""
    q = _u16(q)
    multi = q.ndim == 4
    if multi:
        B, T, Hq, D = q.shape
    else:
        (B, Hq, D), T = q.shape, 1
    k, kf = _kv(k)
    v, vf = _kv(v)
    _, Hkv, Lmax, Dk = k.shape
    if Dk != D or (v is not None and (v.shape != k.shape or vf != kf)):
        raise ValueError("shape mismatch")
    kl = np.ascontiguousarray(kv_len, dtype=np.int32)
    if rows is None:
        out = np.empty(q.shape, np.float64)
        r, n = None, -1
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        n = r.shape[0]
        out = np.empty((n, D), np.float64)
    rc = _load().orc_decode_ext(B, T, Hq, Hkv, D, Lmax, window, theta, scale, _ptr(q, _u16p), _vptr(k), _vptr(v), kf,
                                k_scale, v_scale, _ptr(kl, _i32p), ring, _ptr(r, _i64p), n, _ptr(out, _f64p),
                                nthreads)
    if rc != 0:
        raise ValueError("oracle: invalid decode arguments")
    return out


def stack_prefill(layers: Sequence[dict], qs: Sequence[np.ndarray], k_caches: Sequence[Optional[np.ndarray]],
                  v_caches: Sequence[Optional[np.ndarray]], rows: Optional[Sequence[int]] = None,
                  nthreads: int = 0) -> list:
    """Prefill over a stack of layers with KV-cache sharing.

    Each layer dict carries ``head_dim, rope_theta, window, kv_alias,
    kv_source_layer``.  A layer with ``kv_source_layer >= 0`` owns no cache
    and reads the source layer's buffers (N layers -> M unique caches, the
    feature request's "KV Cache Sharing" section); an aliased layer reads its
    values from the key buffer.
    """
    outs = []
    for li, d in enumerate(layers):
        src = li if d["kv_source_layer"] < 0 else d["kv_source_layer"]
        k = k_caches[src]
        v = None if d["kv_alias"] else v_caches[src]
        outs.append(prefill(qs[li], k, v, d["window"], d["rope_theta"], d.get("scale", 0.0), rows=rows,
                            nthreads=nthreads))
    return outs
