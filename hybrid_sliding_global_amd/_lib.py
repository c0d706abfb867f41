"""ctypes binding of libgemma4_attn.so (include/gemma4_attn.h).

Argument marshalling only: every step of the attention path runs in the HIP
kernels behind the C ABI.  Torch tensors supply device memory and the
current HIP stream; there is no CPU fallback, and loading fails loudly when
the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgemma4_attn.so")

G4_OK = 0
G4_ERR_INVALID_ARG = -1
G4_ERR_UNSUPPORTED = -2
G4_ERR_BAD_SOURCE = -3
G4_ERR_WORKSPACE = -4
G4_ERR_HIP = -5
G4_SLIDING, G4_FULL = 0, 1

EXPORTED = (
    "gemma4_abi_version",
    "gemma4_status_string",
    "gemma4_last_error",
    "gemma4_validate_layers",
    "gemma4_kv_bytes",
    "gemma4_prefill_workspace_bytes",
    "gemma4_decode_workspace_bytes",
    "gemma4_attn_prefill",
    "gemma4_attn_decode",
    "gemma4_set_profile_events",
)


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("kv_alias", ctypes.c_int32),
        ("kv_source_layer", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("rope_theta", ctypes.c_double),
    ]


class Gemma4Error(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__("%s: %s" % (status_string(status), detail))


_lib = None


def load():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libgemma4_attn.so is not built (run `python -m hybrid_sliding_global_amd.build`)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    i32 = ctypes.c_int32
    lib.gemma4_abi_version.restype = ctypes.c_int
    lib.gemma4_status_string.restype = ctypes.c_char_p
    lib.gemma4_status_string.argtypes = [ctypes.c_int]
    lib.gemma4_last_error.restype = ctypes.c_char_p
    lib.gemma4_validate_layers.argtypes = [P(LayerDesc), i32]
    lib.gemma4_kv_bytes.argtypes = [P(LayerDesc), i32, i32, i32, i32, P(sz), P(sz)]
    lib.gemma4_prefill_workspace_bytes.argtypes = [P(LayerDesc), i32, i32, i32, i32, P(sz)]
    lib.gemma4_decode_workspace_bytes.argtypes = [P(LayerDesc), i32, i32, i32, i32, P(sz)]
    lib.gemma4_attn_prefill.argtypes = [P(LayerDesc), i32, i32, vp, P(vp), P(vp), i32, i32, i32, vp, vp, sz, vp]
    lib.gemma4_attn_decode.argtypes = [P(LayerDesc), i32, i32, vp, P(vp), P(vp), vp, i32, i32, i32, vp, vp, sz, vp]
    lib.gemma4_set_profile_events.argtypes = [vp, vp]
    for name in ("gemma4_set_profile_events", "gemma4_validate_layers", "gemma4_kv_bytes", "gemma4_prefill_workspace_bytes",
                 "gemma4_decode_workspace_bytes", "gemma4_attn_prefill", "gemma4_attn_decode"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().gemma4_status_string(int(status)).decode()


def last_error() -> str:
    return load().gemma4_last_error().decode()


def abi_version() -> int:
    return int(load().gemma4_abi_version())


def _check(rc: int) -> int:
    if rc < 0:
        raise Gemma4Error(rc, last_error())
    return rc


def set_profile_events(before=None, after=None) -> None:
    """Record two torch.cuda.Event objects around the next compute calls' main kernel (None, None: off)."""
    b = None if before is None else int(before.cuda_event)
    a = None if after is None else int(after.cuda_event)
    _check(load().gemma4_set_profile_events(b, a))


def descs(layers: Sequence[dict]):
    """Pack layer dicts (see workloads.layer_desc) into a C array."""
    arr = (LayerDesc * len(layers))()
    for i, d in enumerate(layers):
        arr[i] = LayerDesc(int(d["kind"]), int(d["head_dim"]), int(d["num_q_heads"]), int(d["num_kv_heads"]),
                           int(d["window"]), int(d["kv_alias"]), int(d["kv_source_layer"]), float(d.get("scale", 0.0)),
                           float(d["rope_theta"]))
    return arr


def validate_layers(layers: Sequence[dict]) -> int:
    """Return the status code (0 or negative) without raising."""
    arr = descs(layers)
    return int(load().gemma4_validate_layers(arr, len(layers)))


def kv_bytes(layers, layer: int, batch: int, max_len: int):
    k, v = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().gemma4_kv_bytes(descs(layers), len(layers), layer, batch, max_len, ctypes.byref(k), ctypes.byref(v)))
    return k.value, v.value


def prefill_workspace_bytes(layers, layer: int, batch: int, seq_len: int) -> int:
    n = ctypes.c_size_t()
    _check(load().gemma4_prefill_workspace_bytes(descs(layers), len(layers), layer, batch, seq_len, ctypes.byref(n)))
    return n.value


def decode_workspace_bytes(layers, layer: int, batch: int, max_kv_len: int) -> int:
    n = ctypes.c_size_t()
    _check(load().gemma4_decode_workspace_bytes(descs(layers), len(layers), layer, batch, max_kv_len,
                                                ctypes.byref(n)))
    return n.value


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _ptr_table(ts):
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = _ptr(t)
    return arr


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _check_tensor(t, name, dtype, shape):
    import torch
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


class Stack:
    """A stack of layer descriptors kept as a C array for repeated calls."""

    def __init__(self, layers: Sequence[dict]):
        self.layers = [dict(d) for d in layers]
        self.arr = descs(self.layers)
        _check(load().gemma4_validate_layers(self.arr, len(self.layers)))

    def __len__(self):
        return len(self.layers)

    def source(self, layer: int) -> int:
        s = self.layers[layer]["kv_source_layer"]
        return layer if s < 0 else s

    def prefill_workspace_bytes(self, layer: int, batch: int, seq_len: int) -> int:
        n = ctypes.c_size_t()
        _check(load().gemma4_prefill_workspace_bytes(self.arr, len(self), layer, batch, seq_len, ctypes.byref(n)))
        return n.value

    def decode_workspace_bytes(self, layer: int, batch: int, max_kv_len: int) -> int:
        n = ctypes.c_size_t()
        _check(load().gemma4_decode_workspace_bytes(self.arr, len(self), layer, batch, max_kv_len, ctypes.byref(n)))
        return n.value

    def prefill(self, layer: int, q, k_caches, v_caches, out=None, workspace=None, stream=None):
        """q: bf16 [B,S,Hq,D]; k_caches/v_caches: per-layer lists (None for shared / aliased entries)."""
        import torch
        d = self.layers[layer]
        B, S, Hq, D = q.shape
        src = self.source(layer)
        k = k_caches[src]
        if k is None:
            raise ValueError("k_caches[%d] is None" % src)
        Lmax = k.shape[2]
        _check_tensor(q, "q", torch.bfloat16, (B, S, d["num_q_heads"], d["head_dim"]))
        _check_tensor(k, "k_cache", torch.bfloat16, (B, d["num_kv_heads"], Lmax, d["head_dim"]))
        if not d["kv_alias"]:
            _check_tensor(v_caches[src], "v_cache", torch.bfloat16, tuple(k.shape))
        if out is None:
            out = torch.empty((B, S, Hq, D), dtype=torch.float32, device=q.device)
        _check_tensor(out, "out", torch.float32, (B, S, Hq, D))
        need = self.prefill_workspace_bytes(layer, B, S)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        kt = _ptr_table(list(k_caches))
        vt = _ptr_table(list(v_caches)) if v_caches is not None else None
        _check(load().gemma4_attn_prefill(self.arr, len(self), layer, _ptr(q), kt, vt, B, S, Lmax, _ptr(out),
                                          _ptr(workspace), workspace.numel() * workspace.element_size(),
                                          _stream(stream)))
        return out

    def decode(self, layer: int, q, k_caches, v_caches, kv_len, max_kv_len: int, out=None, workspace=None,
               stream=None):
        """q: bf16 [B,Hq,D]; kv_len: int32 device [B]; max_kv_len: host bound on kv_len."""
        import torch
        d = self.layers[layer]
        B, Hq, D = q.shape
        src = self.source(layer)
        k = k_caches[src]
        if k is None:
            raise ValueError("k_caches[%d] is None" % src)
        Lmax = k.shape[2]
        _check_tensor(q, "q", torch.bfloat16, (B, d["num_q_heads"], d["head_dim"]))
        _check_tensor(k, "k_cache", torch.bfloat16, (B, d["num_kv_heads"], Lmax, d["head_dim"]))
        if not d["kv_alias"]:
            _check_tensor(v_caches[src], "v_cache", torch.bfloat16, tuple(k.shape))
        _check_tensor(kv_len, "kv_len", torch.int32, (B,))
        if out is None:
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
        _check_tensor(out, "out", torch.float32, (B, Hq, D))
        need = self.decode_workspace_bytes(layer, B, max_kv_len)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        kt = _ptr_table(list(k_caches))
        vt = _ptr_table(list(v_caches)) if v_caches is not None else None
        _check(load().gemma4_attn_decode(self.arr, len(self), layer, _ptr(q), kt, vt, _ptr(kv_len), B, Lmax,
                                         int(max_kv_len), _ptr(out), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream)))
        return out
