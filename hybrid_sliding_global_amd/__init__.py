"""MI355X (gfx950) hybrid sliding/global attention: Gemma-4-style prefill and
decode behind a small C ABI (include/gemma4_attn.h), hand-written HIP kernels.

    from hybrid_sliding_global_amd import Stack, workloads
    stack = Stack(workloads.gemma4_stack())
    out = stack.prefill(layer, q, k_caches, v_caches)

The kernels live in libgemma4_attn.so, built in-tree by
``python -m hybrid_sliding_global_amd.build``.  Importing this package does
not load the library; the first call does, and fails if it is missing.
"""
from ._lib import (G4_FULL, G4_SLIDING, Gemma4Error, LayerDesc, Stack, abi_version, decode_workspace_bytes, kv_bytes,
                   last_error, load, prefill_workspace_bytes, status_string, validate_layers)

__all__ = ["Stack", "Gemma4Error", "LayerDesc", "G4_SLIDING", "G4_FULL", "abi_version", "decode_workspace_bytes",
           "kv_bytes", "last_error", "load", "prefill_workspace_bytes", "status_string", "validate_layers"]
