"""Layer descriptors and the synthetic workloads the tests and benchmark use.

Facts from the pages (onnxruntime-genai feature request "Support for Google
Gemma 4 model family", sections "Variable Attention Head Dimensions", "KV
Cache Sharing" and "Gemma 4 Model Details"):
  * sliding layers use head_dim 256, full layers global_head_dim 512;
  * full attention on every fifth layer, indices 4, 9, ..., 34
    (attention_pattern 0 = sliding, 1 = full);
  * RoPE theta 10000 for sliding and 1000000 for full layers;
  * the E2B stack has 35 layers but only 15 unique KV cache pairs
    (num_kv_shared_layers = 20).
K=V aliasing in sliding layers comes from the Gemma-4 weight loader page
(spark_model/weight_loader/gemma4.rs, ``supports_tp``).

Readings where the pages are silent:
  * which layer a shared layer reads: layers 0..14 own their cache; a
    shared layer reads the last owning layer of its own kind (sliding -> 13,
    full -> 14), so head sizes and kv-head counts always match;
  * head counts of the 35-layer stack: sliding Hq=8, Hkv=1; full Hq=8, Hkv=2.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

SLIDING, FULL = 0, 1
HEAD_DIM_SLIDING, HEAD_DIM_FULL = 256, 512
THETA_SLIDING, THETA_FULL = 10000.0, 1000000.0


KV_BF16, KV_FP8 = 0, 1


def layer_desc(kind: int, head_dim: int, num_q_heads: int, num_kv_heads: int, rope_theta: float, window: int,
               kv_alias: int, kv_source_layer: int = -1, scale: float = 0.0, kv_dtype: int = KV_BF16,
               kv_ring: int = 0, k_scale: float = 1.0, v_scale: float = 1.0) -> dict:
    return dict(kind=int(kind), head_dim=int(head_dim), num_q_heads=int(num_q_heads), num_kv_heads=int(num_kv_heads),
                rope_theta=float(rope_theta), window=int(window), kv_alias=int(kv_alias),
                kv_source_layer=int(kv_source_layer), scale=float(scale), kv_dtype=int(kv_dtype),
                kv_ring=int(kv_ring), k_scale=float(k_scale), v_scale=float(v_scale))


def attention_pattern(n_layers: int, period: int = 5) -> List[int]:
    """0 = sliding, 1 = full; full on every ``period``-th layer (index period-1, 2*period-1, ...)."""
    return [1 if (i + 1) % period == 0 else 0 for i in range(n_layers)]


def kv_share_map(pattern: List[int], n_owners: int) -> List[int]:
    """Source layer of each layer (-1 = owns its cache).

    Layers below ``n_owners`` own a cache; every later layer reads the last
    owner of the same kind.
    """
    src = []
    for i, kind in enumerate(pattern):
        if i < n_owners:
            src.append(-1)
        else:
            owners = [j for j in range(n_owners) if pattern[j] == kind]
            if not owners:
                raise ValueError("no owning layer of kind %d" % kind)
            src.append(owners[-1])
    return src


def gemma4_stack(n_layers: int = 35, n_owners: int = 15, window: int = 512, hq_sliding: int = 8,
                 hkv_sliding: int = 1, hq_full: int = 8, hkv_full: int = 2) -> List[dict]:
    pattern = attention_pattern(n_layers)
    src = kv_share_map(pattern, n_owners)
    layers = []
    for i, kind in enumerate(pattern):
        if kind == SLIDING:
            layers.append(layer_desc(SLIDING, HEAD_DIM_SLIDING, hq_sliding, hkv_sliding, THETA_SLIDING, window, 1,
                                     src[i]))
        else:
            layers.append(layer_desc(FULL, HEAD_DIM_FULL, hq_full, hkv_full, THETA_FULL, 0, 0, src[i]))
    return layers


@dataclass
class Workload:
    """One synthetic workload: a list of layers and the call shapes."""
    wid: int
    name: str
    mode: str  # "prefill" or "decode"
    layers: List[dict]
    batch: int
    seq_len: int = 0          # prefill query tokens (= cache rows used)
    max_len: int = 0          # cache capacity Lmax
    kv_len: Optional[int] = None      # decode: fixed length for every sequence
    kv_len_range: Optional[tuple] = None  # decode: uniform [lo, hi] per sequence
    notes: str = ""
    run_layers: List[int] = field(default_factory=list)  # layers evaluated (default: all)


def workloads() -> dict:
    w = {}
    w[1] = Workload(1, "sliding_prefill_s64", "prefill",
                    [layer_desc(SLIDING, 256, 4, 1, THETA_SLIDING, 32, 1)], batch=1, seq_len=64, max_len=64,
                    notes="single sliding layer, K=V aliased, window 32")
    w[2] = Workload(2, "full_prefill_s4096", "prefill",
                    [layer_desc(FULL, 512, 8, 2, THETA_FULL, 0, 0)], batch=1, seq_len=4096, max_len=4096,
                    notes="single full-attention layer, separate K and V")
    w[3] = Workload(3, "decode_b64_l8192", "decode",
                    [layer_desc(SLIDING, 256, 8, 1, THETA_SLIDING, 1024, 1),
                     layer_desc(FULL, 512, 8, 2, THETA_FULL, 0, 0)], batch=64, max_len=8192, kv_len=8192,
                    notes="one new token per sequence; sliding (K=V) plus full layer")
    w[4] = Workload(4, "stack35_prefill_s2048", "prefill", gemma4_stack(), batch=1, seq_len=2048, max_len=2048,
                    notes="35 layers, full at 4,9,...,34, 15 owned caches")
    w[5] = Workload(5, "decode_b4_long", "decode",
                    [layer_desc(SLIDING, 256, 16, 2, THETA_SLIDING, 1024, 1),
                     layer_desc(FULL, 512, 16, 2, THETA_FULL, 0, 0)], batch=4, max_len=131072,
                    kv_len_range=(1024, 131072), notes="per-sequence lengths uniform in [1024, 131072]")
    return w


def prefill_flops(S: int, Hq: int, D: int, window: int) -> int:
    """Algorithmic FLOPs of one prefill layer: 4*D*Hq*sum_i n_i over visible (query, key) pairs."""
    if window <= 0:
        pairs = S * (S + 1) // 2
    else:
        w = min(window, S)
        pairs = w * (w + 1) // 2 + (S - w) * w
    return 4 * D * Hq * pairs


def decode_bytes(kv_lens, Hq: int, Hkv: int, D: int, window: int, alias: bool) -> int:
    """Algorithmic bytes of one decode layer: visible K (+V unless aliased) bf16 rows,
    the bf16 query, the fp32 output and the int32 lengths."""
    total = 0
    for L in kv_lens:
        n = min(int(L), window) if window > 0 else int(L)
        total += n * Hkv * D * 2 * (1 if alias else 2)
    B = len(kv_lens)
    total += B * Hq * D * 2 + B * Hq * D * 4 + B * 4
    return total
