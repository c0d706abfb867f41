"""Inputs whose attention scores span a wide range, and the check that they do.

Online softmax keeps a running maximum per query row and rescales what it
has accumulated when a later block of keys scores higher.  With N(0,1)
inputs those events are rare, so these inputs plant keys whose scores rise
in steps of about STEP log2 units along the sequence:

  * the lowest-frequency rotation pair (dims D/2-1 and D-1, which turn by at
    most a few tenths of a radian over the positions used here) is zeroed in
    every key, and in every query's second half;
  * planted key m (m = 1, 2, ...) is m in dim D/2-1 and zero elsewhere;
  * every query gets the value A in dim D/2-1, with A chosen so that
    scale * log2(e) * A * 1 = STEP.

Planted key m then scores STEP * m (times the cosine of its small relative
angle), while all other scores stay of order one: consecutive planted keys
are STEP apart, so however the bf16 rounding of a score of size S (about
S * 2^-9) moves them, the runner-up's weight stays near 2^-STEP.  (With
N(0,1) noise left on the planted keys two of them can end up a few units
apart, and the rounding noise of scores near 80 units then moves the output
by a few 1e-2 -- the arithmetic, not a defect, but outside the tolerance.)
The threshold checks below read the oracle's fp64 scores, never the GPU's.
"""
import math

import numpy as np

from hybrid_sliding_global_amd import inputs

STEP = 12.0  # log2 units between consecutive planted keys
LOG2E = 1.0 / math.log(2.0)


def _bf16(x: float) -> np.uint16:
    return inputs.bf16_bits_from_f32(np.array([x], np.float32))[0]


def plant(q: np.ndarray, k: np.ndarray, planted, scale: float = 0.0, period: int = 0):
    """Plant rising keys in k ([B, Hkv, Lmax, D] bf16 bits) at the positions
    ``planted`` (the m-th gets amplitude m + 1, or 1 + m % period) and the
    matching query component in q ([..., D]); both modified in place."""
    D = k.shape[-1]
    f = D // 2 - 1
    sc = scale if scale else 1.0 / math.sqrt(D)
    A = STEP / (sc * LOG2E)
    k[..., f] = 0
    k[..., D - 1] = 0
    for m, j in enumerate(planted):
        k[:, :, j, :] = 0
        k[:, :, j, f] = _bf16(float(1 + (m % period if period else m)))
    q[..., f] = _bf16(A)
    q[..., D - 1] = 0
    return q, k


def block_growth(scores_log2: np.ndarray, block: int, start: int = 0):
    """Over blocks of ``block`` keys from ``start`` on (visible keys only):
    the largest jump of a block's maximum above the maximum of all earlier
    blocks, and the rise of the overall maximum above the first visible
    block's maximum."""
    s = scores_log2[start:]
    nb = -(-len(s) // block)
    maxima = []
    for i in range(nb):
        blk = s[i * block:(i + 1) * block]
        vis = blk[np.isfinite(blk)]
        if vis.size:
            maxima.append(vis.max())
    if not maxima:
        return 0.0, 0.0
    jump, run = 0.0, maxima[0]
    for m in maxima[1:]:
        jump = max(jump, m - run)
        run = max(run, m)
    return jump, max(maxima) - maxima[0]


def prefill_growth(orc, q, k, W, theta, rows, block=32):
    """Largest (jump, rise) over the listed prefill rows (flattened
    b*S*Hq + s*Hq + h), from the oracle's scores in log2 units."""
    B, S, Hq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    best_jump = best_rise = 0.0
    for r in rows:
        b, s, h = r // (S * Hq), (r // Hq) % S, r % Hq
        sc = orc.scores_row(q[b, s, h], k[b, h // g], s, S, W, theta) * LOG2E
        j, rise = block_growth(sc, block)
        best_jump, best_rise = max(best_jump, j), max(best_rise, rise)
    return best_jump, best_rise


def decode_split(kv_len, Hkv, W, pieces=512, min_keys=64):
    """The decode key split: the visible keys of all (batch, kv-head) streams
    laid end to end, cut into min(pieces, max(1, T // min_keys)) equal pieces;
    returns per stream the list of (first key, end key) segments."""
    spans = []
    for L in kv_len:
        lo = max(0, int(L) - W) if W > 0 else 0
        spans.append((lo, int(L)))
    T = sum((hi - lo) * Hkv for lo, hi in spans)
    npc = min(pieces, max(1, T // min_keys))
    cuts = [p * T // npc for p in range(npc + 1)]
    segs = {}
    base = 0
    for b, (lo, hi) in enumerate(spans):
        for h in range(Hkv):
            s0, s1 = base, base + (hi - lo)
            out = []
            for p in range(npc):
                x0, x1 = max(s0, cuts[p]), min(s1, cuts[p + 1])
                if x0 < x1:
                    out.append((lo + x0 - s0, lo + x1 - s0))
            segs[(b, h)] = out
            base = s1
    return segs


def decode_growth(orc, q, k, kv_len, W, theta, step=16):
    """Largest jump of a 16-key step's maximum above the earlier steps of the
    same segment, over every decode query (oracle scores, log2 units)."""
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    segs = decode_split(kv_len, Hkv, W)
    best = 0.0
    for b in range(B):
        L = int(kv_len[b])
        for h in range(Hq):
            sc = orc.scores_row(q[b, h], k[b, h // g], L - 1, L, W, theta) * LOG2E
            for x0, x1 in segs[(b, h // g)]:
                best = max(best, block_growth(sc[x0:x1], step)[0])
    return best


def prefill_case(B, S, Hq, Hkv, D, W, theta, seed, every=None, period=0):
    """Seeded prefill inputs (q, k, v; v separate, N(0,1)) with planted keys at
    offset 5 of 32-key tiles: tiles 2, 4, 7, 11, 16, 22, 29, 37, ... (gaps
    growing by one) or, with ``every``, every ``every``-th tile from 1 on;
    amplitudes rise by one per planted key, cycling with ``period`` if given
    (a window then never holds two planted keys of equal amplitude as long
    as it spans fewer than ``period`` of them)."""
    q = inputs.normal_bf16([300 + seed, S, 0], (B, S, Hq, D))
    k = inputs.normal_bf16([300 + seed, S, 1], (B, Hkv, S, D))
    v = inputs.normal_bf16([300 + seed, S, 2], (B, Hkv, S, D))
    if every:
        tiles = list(range(1, -(-S // 32), every))
    else:
        tiles, t, gap = [], 2, 2
        while 32 * t + 5 < S:
            tiles.append(t)
            t, gap = t + gap, gap + 1
    planted = [32 * t + 5 for t in tiles if 32 * t + 5 < S]
    plant(q, k, planted, period=period)
    return q, k, v, planted


def decode_case(B, Hq, Hkv, D, kv_len, Lmax, seed):
    """Seeded decode inputs with a planted key at offset 3 of every 16 positions
    (amplitudes rising along each stream); v separate, N(0,1)."""
    q = inputs.normal_bf16([400 + seed, Lmax, 0], (B, Hq, D))
    k = inputs.normal_bf16([400 + seed, Lmax, 1], (B, Hkv, Lmax, D))
    v = inputs.normal_bf16([400 + seed, Lmax, 2], (B, Hkv, Lmax, D))
    planted = list(range(3, Lmax, 16))
    plant(q, k, planted)
    inputs.poison_beyond(k, kv_len)
    inputs.poison_beyond(v, kv_len)
    return q, k, v
