"""Pins for the fp64 oracle, against facts that do not come from the oracle itself.

Each test fixes the oracle to a closed form, an invariant of the mathematics,
a brute-force index test or an independent library routine (torch's
scaled_dot_product_attention in float64 on the CPU).  They are chosen so that
a plausible slip anywhere in the oracle (a dropped RoPE term, a flipped sign,
the wrong frequency exponent, interleaved instead of rotate-half pairs, an
off-by-one window, a wrong scale, a wrong GQA head map, rotated values, a
wrong decode position, a transposed operand) fails at least one of them.
"""
import math

import numpy as np
import pytest

from hybrid_sliding_global_amd import inputs

RNG = np.random.default_rng(1234)


def bf16(shape, seed):
    return inputs.normal_bf16(seed, shape)


def widen(b):
    return inputs.f32_from_bf16_bits(b).astype(np.float64)


# ---------------------------------------------------------------- RoPE ------

@pytest.mark.parametrize("D,theta", [(256, 1e4), (512, 1e6), (8, 1e4)])
def test_rope_position_zero_is_identity(orc, D, theta):
    x = RNG.standard_normal(D)
    assert np.array_equal(orc.rope(x, theta, 0.0), x)


@pytest.mark.parametrize("D,theta", [(256, 1e4), (512, 1e6)])
@pytest.mark.parametrize("pos", [1, 17, 4095, 131071])
def test_rope_preserves_norm(orc, D, theta, pos):
    x = RNG.standard_normal(D)
    y = orc.rope(x, theta, pos)
    assert abs(np.linalg.norm(y) - np.linalg.norm(x)) <= 1e-12 * np.linalg.norm(x)
    # every (k, k + D/2) pair keeps its own length: rotation acts pairwise
    h = D // 2
    assert np.allclose(x[:h] ** 2 + x[h:] ** 2, y[:h] ** 2 + y[h:] ** 2, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("m,n", [(3, 5), (100, 4000), (65536, 1)])
def test_rope_composition(orc, m, n):
    x = RNG.standard_normal(256)
    a = orc.rope(orc.rope(x, 1e4, n), 1e4, m)
    b = orc.rope(x, 1e4, m + n)
    assert np.allclose(a, b, rtol=0, atol=1e-9 * np.abs(x).max())


@pytest.mark.parametrize("D,theta", [(256, 1e4), (512, 1e6)])
def test_rope_relative_position(orc, D, theta):
    q, k = RNG.standard_normal(D), RNG.standard_normal(D)
    base = orc.rope(q, theta, 40) @ orc.rope(k, theta, 7)
    for t in (1, 1000, 50000):
        shifted = orc.rope(q, theta, 40 + t) @ orc.rope(k, theta, 7 + t)
        assert abs(shifted - base) <= 1e-9 * (np.linalg.norm(q) * np.linalg.norm(k))


def test_rope_closed_form_angles(orc):
    # D=256, theta=1e4: pair 64 has frequency 1e4^(-128/256) = 1e-2, so position 100 turns it by 1 rad.
    D = 256
    e = np.zeros(D); e[64] = 1.0
    y = orc.rope(e, 1e4, 100.0)
    want = np.zeros(D); want[64] = math.cos(1.0); want[64 + 128] = math.sin(1.0)
    assert np.allclose(y, want, atol=1e-12)
    # pair 0 has frequency 1: position 3 turns it by 3 rad; the partner rotates the other way round
    e = np.zeros(D); e[128] = 1.0
    y = orc.rope(e, 1e4, 3.0)
    want = np.zeros(D); want[0] = -math.sin(3.0); want[128] = math.cos(3.0)
    assert np.allclose(y, want, atol=1e-12)
    # D=512, theta=1e6: pair 128 has frequency 1e6^(-1/2) = 1e-3, position 1000 -> 1 rad
    D = 512
    e = np.zeros(D); e[128] = 1.0
    y = orc.rope(e, 1e6, 1000.0)
    want = np.zeros(D); want[128] = math.cos(1.0); want[128 + 256] = math.sin(1.0)
    assert np.allclose(y, want, atol=1e-12)


def test_rope_inverse_frequencies(orc):
    f = orc.inv_freq(512, 1e6)
    assert f[0] == 1.0
    assert abs(f[128] - 1e-3) < 1e-18
    assert np.all(np.diff(f) < 0)
    assert abs(f[-1] - 1e6 ** (-510 / 512)) < 1e-18


@pytest.mark.parametrize("D,theta,pos", [(256, 1e4, 5), (512, 1e6, 77777), (16, 1e4, 12)])
def test_rope_matches_complex_multiplication(orc, D, theta, pos):
    # independent form: z_k = x_k + i x_{k+D/2} multiplied by exp(i * pos * theta^(-2k/D))
    x = RNG.standard_normal(D)
    h = D // 2
    z = x[:h] + 1j * x[h:]
    freq = np.exp(-np.arange(h) * (2.0 / D) * np.log(theta))
    zr = z * np.exp(1j * pos * freq)
    want = np.concatenate([zr.real, zr.imag])
    assert np.allclose(orc.rope(x, theta, pos), want, rtol=0, atol=1e-10)


# ------------------------------------------------------- mask & softmax -----

@pytest.mark.parametrize("W", [0, 1, 2, 3, 5, 12, 20])
def test_window_mask_matches_direct_index_test(orc, W):
    S, D = 12, 8
    q = bf16((S, D), [900, W, 0])
    k = bf16((S, D), [900, W, 1])
    for i in range(S):
        w, _ = orc.attention_row(q[i], k, None, i, S, W, 1e4)
        visible = {j for j in range(S) if j <= i and (W == 0 or i - j < W)}
        assert {j for j in range(S) if w[j] != 0.0} == visible
        assert abs(w.sum() - 1.0) < 1e-12


def test_weights_sum_to_one_long_rows(orc):
    L, D = 700, 256
    q = bf16((D,), [901, 0, 0])
    k = bf16((L, D), [901, 0, 1])
    for W in (0, 64):
        w, _ = orc.attention_row(q, k, None, L - 1, L, W, 1e4)
        assert abs(w.sum() - 1.0) < 1e-12
        assert np.all(w >= 0)


def test_window_one_returns_own_raw_value(orc):
    S, D = 9, 16
    q = bf16((1, S, 2, D), [902, 0, 0])
    k = bf16((1, 1, S, D), [902, 0, 1])
    v = bf16((1, 1, S, D), [902, 0, 2])
    out = orc.prefill(q, k, v, 1, 1e4)
    assert np.array_equal(out[0, :, 0, :], widen(v[0, 0]))
    # aliased: values are the raw (un-rotated) keys
    out = orc.prefill(q, k, None, 1, 1e4)
    assert np.array_equal(out[0, :, 1, :], widen(k[0, 0]))


@pytest.mark.parametrize("W", [0, 4])
def test_row_zero_returns_first_value(orc, W):
    q = bf16((1, 5, 1, 32), [903, W, 0])
    k = bf16((1, 1, 5, 32), [903, W, 1])
    v = bf16((1, 1, 5, 32), [903, W, 2])
    out = orc.prefill(q, k, v, W, 1e6)
    assert np.array_equal(out[0, 0, 0], widen(v[0, 0, 0]))


def test_window_at_least_length_is_causal(orc):
    S = 23
    q = bf16((2, S, 4, 32), [904, 0, 0])
    k = bf16((2, 2, S, 32), [904, 0, 1])
    v = bf16((2, 2, S, 32), [904, 0, 2])
    causal = orc.prefill(q, k, v, 0, 1e4)
    assert np.array_equal(orc.prefill(q, k, v, S, 1e4), causal)
    assert np.array_equal(orc.prefill(q, k, v, 3 * S, 1e4), causal)
    assert not np.array_equal(orc.prefill(q, k, v, S - 1, 1e4), causal)


@pytest.mark.parametrize("D,scale", [(256, 0.0), (512, 0.0), (64, 0.3)])
def test_two_visible_keys_give_a_sigmoid(orc, D, scale):
    # W=2 at position i sees keys i-1 and i.  Key i-1 is zero, so its score is 0;
    # key i sits at the query's own position, so RoPE cancels and its score is
    # scale * <q, k_i> on the raw vectors.
    S = 6
    q = bf16((S, D), [905, D, 0])
    k = bf16((S, D), [905, D, 1])
    k[S - 2] = 0
    eff = scale if scale else 1.0 / math.sqrt(D)
    w, _ = orc.attention_row(q[S - 1], k, None, S - 1, S, 2, 1e4, scale)
    s = eff * float(widen(q[S - 1]) @ widen(k[S - 1]))
    assert abs(w[S - 1] - 1.0 / (1.0 + math.exp(-s))) < 1e-12
    assert abs(w[S - 2] - 1.0 / (1.0 + math.exp(s))) < 1e-12


@pytest.mark.parametrize("W", [0, 4])
def test_zero_keys_average_the_visible_values(orc, W):
    S, D = 10, 32
    q = bf16((1, S, 2, D), [906, W, 0])
    k = np.zeros((1, 1, S, D), np.uint16)
    v = bf16((1, 1, S, D), [906, W, 2])
    out = orc.prefill(q, k, v, W, 1e4)
    vv = widen(v[0, 0])
    for i in range(S):
        lo = 0 if W == 0 else max(0, i - W + 1)
        want = vv[lo:i + 1].mean(axis=0)
        assert np.allclose(out[0, i, 0], want, rtol=0, atol=1e-12)
        assert np.allclose(out[0, i, 1], want, rtol=0, atol=1e-12)


# ------------------------------------------------- GQA, alias, sharing ------

def test_gqa_equals_repeated_kv_heads(orc):
    B, S, Hq, Hkv, D = 2, 19, 8, 2, 32
    q = bf16((B, S, Hq, D), [907, 0, 0])
    k = bf16((B, Hkv, S, D), [907, 0, 1])
    v = bf16((B, Hkv, S, D), [907, 0, 2])
    grouped = orc.prefill(q, k, v, 5, 1e4)
    rep = orc.prefill(q, np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1), 5, 1e4)
    assert np.array_equal(grouped, rep)
    # and head h really reads kv head h // 4, not h % 2
    swapped = orc.prefill(q, np.tile(k, (1, Hq // Hkv, 1, 1)), np.tile(v, (1, Hq // Hkv, 1, 1)), 5, 1e4)
    assert not np.allclose(grouped, swapped)


def test_alias_equals_explicit_duplicate(orc):
    q = bf16((1, 33, 4, 256), [908, 0, 0])
    k = bf16((1, 1, 40, 256), [908, 0, 1])
    assert np.array_equal(orc.prefill(q, k, None, 16, 1e4), orc.prefill(q, k, k.copy(), 16, 1e4))
    qd = bf16((3, 4, 256), [908, 1, 0])
    kv = np.array([40, 17, 1], np.int32)
    kk = bf16((3, 1, 40, 256), [908, 1, 1])
    assert np.array_equal(orc.decode(qd, kk, None, kv, 16, 1e4), orc.decode(qd, kk, kk.copy(), kv, 16, 1e4))


def test_shared_layer_equals_copied_cache(orc):
    from hybrid_sliding_global_amd.workloads import layer_desc
    S = 21
    layers = [layer_desc(0, 32, 4, 1, 1e4, 8, 1), layer_desc(1, 64, 4, 2, 1e6, 0, 0),
              layer_desc(0, 32, 4, 1, 1e4, 8, 1, kv_source_layer=0), layer_desc(1, 64, 4, 2, 1e6, 0, 0, 1)]
    qs = [bf16((1, S, 4, l["head_dim"]), [909, i, 0]) for i, l in enumerate(layers)]
    kc = [bf16((1, 1, S, 32), [909, 0, 1]), bf16((1, 2, S, 64), [909, 1, 1]), None, None]
    vc = [None, bf16((1, 2, S, 64), [909, 1, 2]), None, None]
    outs = orc.stack_prefill(layers, qs, kc, vc)
    assert np.array_equal(outs[2], orc.prefill(qs[2], kc[0].copy(), None, 8, 1e4))
    assert np.array_equal(outs[3], orc.prefill(qs[3], kc[1].copy(), vc[1].copy(), 0, 1e6))


def test_decode_is_last_prefill_row(orc):
    B, Hq, Hkv, D, L = 2, 4, 2, 64, 29
    q = bf16((B, L, Hq, D), [910, 0, 0])
    k = bf16((B, Hkv, L, D), [910, 0, 1])
    v = bf16((B, Hkv, L, D), [910, 0, 2])
    pre = orc.prefill(q, k, v, 7, 1e6)
    dec = orc.decode(np.ascontiguousarray(q[:, L - 1]), k, v, np.full(B, L, np.int32), 7, 1e6)
    assert np.array_equal(dec, pre[:, L - 1])


def test_decode_ignores_rows_beyond_length(orc):
    B, Hq, Hkv, D, Lmax = 2, 2, 1, 32, 16
    q = bf16((B, Hq, D), [911, 0, 0])
    k = bf16((B, Hkv, Lmax, D), [911, 0, 1])
    kv = np.array([9, 16], np.int32)
    a = orc.decode(q, k, None, kv, 0, 1e4)
    k2 = inputs.poison_beyond(k.copy(), kv)
    b = orc.decode(q, k2, None, kv, 0, 1e4)
    assert np.array_equal(a, b) and np.isfinite(b).all()


def test_row_subset_matches_full(orc):
    q = bf16((2, 17, 4, 32), [912, 0, 0])
    k = bf16((2, 2, 17, 32), [912, 0, 1])
    full = orc.prefill(q, k, None, 6, 1e4)
    rows = [0, 5, 17 * 4 + 3, 2 * 17 * 4 - 1]
    sub = orc.prefill(q, k, None, 6, 1e4, rows=rows)
    assert np.array_equal(sub, full.reshape(-1, 32)[rows])


# ------------------------------------------------------------ scores ------

def _rot_complex(x, pos, theta):
    """Rotate-half RoPE in its complex form: z_k = x_k + i x_{k+D/2} times exp(i pos theta^(-2k/D))."""
    D = x.shape[-1]
    h = D // 2
    z = x[..., :h] + 1j * x[..., h:]
    freq = np.exp(-np.arange(h) * (2.0 / D) * np.log(theta))
    zr = z * np.exp(1j * np.asarray(pos, np.float64)[..., None] * freq)
    return np.concatenate([zr.real, zr.imag], axis=-1)


@pytest.mark.parametrize("D,theta,W,p", [(256, 1e4, 0, 39), (512, 1e6, 7, 30), (16, 1e4, 3, 0)])
def test_scores_match_independent_rotation(orc, D, theta, W, p):
    L = 40
    q = bf16((D,), [915, D, 0])
    k = bf16((L, D), [915, D, 1])
    got = orc.scores_row(q, k, p, L, W, theta)
    kr = _rot_complex(widen(k), np.arange(L), theta)
    qr = _rot_complex(widen(q), p, theta)
    want = kr @ qr / math.sqrt(D)
    vis = np.array([j <= p and (W == 0 or p - j < W) for j in range(L)])
    assert np.all(np.isneginf(got[~vis]))
    assert np.max(np.abs(got[vis] - want[vis])) < 1e-10
    # the weights are the softmax of these scores
    w, _ = orc.attention_row(q, k, None, p, L, W, theta)
    e = np.exp(got[vis] - got[vis].max())
    assert np.max(np.abs(w[vis] - e / e.sum())) < 1e-12


# ------------------------------------------------ library cross-check ------

def _sdpa_reference(q, k, v, W, theta, kv_len=None):
    """torch SDPA (float64, CPU) on keys/queries rotated by the complex-number form."""
    import torch
    qf, kf = widen(q), widen(k)
    vf = kf if v is None else widen(v)

    def rot(x, pos):  # x [..., D], pos broadcastable to x[..., 0]
        D = x.shape[-1]
        h = D // 2
        z = x[..., :h] + 1j * x[..., h:]
        freq = np.exp(-np.arange(h) * (2.0 / D) * np.log(theta))
        zr = z * np.exp(1j * pos[..., None] * freq)
        return np.concatenate([zr.real, zr.imag], axis=-1)

    B, Hkv, Lmax, D = kf.shape
    kr = rot(kf, np.arange(Lmax, dtype=np.float64)[None, None, :])
    if q.ndim == 4:  # prefill [B, S, Hq, D]
        S, Hq = q.shape[1], q.shape[2]
        qpos = np.arange(S, dtype=np.float64)
        qr = rot(qf.transpose(0, 2, 1, 3), qpos[None, None, :])  # [B, Hq, S, D]
        lens = np.full(B, S)
    else:  # decode [B, Hq, D]
        Hq = q.shape[1]
        lens = np.asarray(kv_len)
        qpos = (lens - 1).astype(np.float64)
        qr = rot(qf[:, :, None, :], np.broadcast_to(qpos[:, None, None], (B, Hq, 1)))
    g = Hq // Hkv
    K = torch.from_numpy(np.repeat(kr, g, axis=1).copy())
    V = torch.from_numpy(np.repeat(vf, g, axis=1).copy())
    Q = torch.from_numpy(np.ascontiguousarray(qr))
    Sq = Q.shape[2]
    mask = np.zeros((B, 1, Sq, Lmax), bool)
    for b in range(B):
        for i in range(Sq):
            p = i if q.ndim == 4 else lens[b] - 1
            for j in range(Lmax):
                mask[b, 0, i, j] = j <= p and j < lens[b] and (W == 0 or p - j < W)
    out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=torch.from_numpy(mask))
    out = out.numpy()
    return out.transpose(0, 2, 1, 3) if q.ndim == 4 else out[:, :, 0, :]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,W,theta,alias", [
    (2, 37, 4, 2, 16, 0, 1e4, False),
    (1, 70, 8, 1, 256, 24, 1e4, True),
    (1, 45, 4, 2, 512, 0, 1e6, False),
])
def test_prefill_matches_torch_sdpa(orc, B, S, Hq, Hkv, D, W, theta, alias):
    q = bf16((B, S, Hq, D), [913, S, 0])
    k = bf16((B, Hkv, S, D), [913, S, 1])
    v = None if alias else bf16((B, Hkv, S, D), [913, S, 2])
    got = orc.prefill(q, k, v, W, theta)
    want = _sdpa_reference(q, k, v, W, theta)
    assert np.max(np.abs(got - want)) < 1e-10


@pytest.mark.parametrize("W,alias,D", [(0, False, 512), (5, True, 256)])
def test_decode_matches_torch_sdpa(orc, W, alias, D):
    B, Hq, Hkv, Lmax = 3, 8, 2, 33
    q = bf16((B, Hq, D), [914, W, 0])
    k = bf16((B, Hkv, Lmax, D), [914, W, 1])
    v = None if alias else bf16((B, Hkv, Lmax, D), [914, W, 2])
    kv = np.array([33, 1, 12], np.int32)
    got = orc.decode(q, k, v, kv, W, 1e6)
    want = _sdpa_reference(q, k, v, W, 1e6, kv_len=kv)
    assert np.max(np.abs(got - want)) < 1e-10


# ---------------------------------------------------- input generator ------

def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20, np.inf, np.nan], np.float32)
    b = inputs.bf16_bits_from_f32(x)
    assert b.tolist()[:6] == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81, 0x7F80]
    assert b[6] == 0x7FC0
    assert np.array_equal(inputs.f32_from_bf16_bits(b[:4]), np.array([1.0, 1.0, 1.0 + 2 ** -6, -2.5], np.float32))


def test_generator_is_deterministic():
    a = inputs.normal_bf16([1, 0, 0], (3, 5, 7))
    b = inputs.normal_bf16([1, 0, 0], (3, 5, 7))
    c = inputs.normal_bf16([1, 0, 1], (3, 5, 7))
    assert inputs.sha256(a) == inputs.sha256(b) != inputs.sha256(c)
    f = inputs.f32_from_bf16_bits(inputs.normal_bf16([2, 0, 0], (1 << 16,)))
    assert abs(f.mean()) < 0.02 and abs(f.std() - 1.0) < 0.02


# ------------------------------------------- next rows: E4M3 KV elements ---

def test_fp8_e4m3_decoding_matches_torch(orc):
    """Every one of the 256 E4M3 codes against torch's float8_e4m3fn (OCP)."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    got = orc.fp8_e4m3_value(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], want[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0 and got[0xB8] == -1.0


def _fp8_cache(shape, seed):
    """E4M3 codes of N(0,1) samples (torch's round-to-nearest conversion)."""
    import torch
    x = torch.from_numpy(np.random.default_rng(seed).standard_normal(shape).astype(np.float32))
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _bf16_of(values):
    return inputs.bf16_bits_from_f32(values.astype(np.float32))


@pytest.mark.parametrize("alias", [False, True])
def test_fp8_cache_equals_bf16_cache_of_its_values(orc, alias):
    """An E4M3 cache with power-of-two scales holds values bf16 represents
    exactly, so attention over it equals attention over that bf16 cache, bit
    for bit (prefill and decode)."""
    B, S, Hq, Hkv, D = 2, 21, 4, 2, 32
    ks, vs = 0.125, 4.0
    k8 = _fp8_cache((B, Hkv, S, D), [920, 1])
    v8 = None if alias else _fp8_cache((B, Hkv, S, D), [920, 2])
    kb = _bf16_of(orc.fp8_e4m3_value(k8) * ks)
    vb = None if alias else _bf16_of(orc.fp8_e4m3_value(v8) * vs)
    assert np.array_equal(inputs.f32_from_bf16_bits(kb), (orc.fp8_e4m3_value(k8) * ks).astype(np.float32))
    q = bf16((B, S, Hq, D), [920, 0])
    got = orc.prefill(q, k8, v8, 6, 1e4, k_scale=ks, v_scale=vs)
    assert np.array_equal(got, orc.prefill(q, kb, vb, 6, 1e4))
    qd = bf16((B, Hq, D), [920, 3])
    kv = np.array([S, 7], np.int32)
    got = orc.decode(qd, k8, v8, kv, 0, 1e6, k_scale=ks, v_scale=vs)
    assert np.array_equal(got, orc.decode(qd, kb, vb, kv, 0, 1e6))


def test_fp8_decode_matches_torch_sdpa(orc):
    """E4M3 cache dequantised by torch's own float8 conversion, then torch SDPA."""
    import torch
    B, Hq, Hkv, D, Lmax = 2, 4, 2, 64, 30
    ks, vs = 0.75, 1.5
    k8 = _fp8_cache((B, Hkv, Lmax, D), [921, 1])
    v8 = _fp8_cache((B, Hkv, Lmax, D), [921, 2])
    q = bf16((B, Hq, D), [921, 0])
    kv = np.array([30, 11], np.int32)
    got = orc.decode(q, k8, v8, kv, 9, 1e4, k_scale=ks, v_scale=vs)
    deq = lambda a, s: torch.from_numpy(a).view(torch.float8_e4m3fn).to(torch.float64).numpy() * s  # noqa: E731
    want = _sdpa_reference_values(q, deq(k8, ks), deq(v8, vs), 9, 1e4, kv)
    assert np.max(np.abs(got - want)) < 1e-10


def _sdpa_reference_values(q, kf, vf, W, theta, kv_len):
    """torch SDPA (float64) for decode queries [B, Hq, D] over fp64 key/value
    caches [B, Hkv, Lmax, D] (keys rotated here by the complex form)."""
    import torch
    B, Hkv, Lmax, D = kf.shape
    Hq = q.shape[1]
    kr = _rot_complex(kf, np.arange(Lmax)[None, None, :], theta)
    lens = np.asarray(kv_len)
    qr = _rot_complex(widen(q)[:, :, None, :], np.broadcast_to((lens - 1)[:, None, None], (B, Hq, 1)), theta)
    g = Hq // Hkv
    mask = np.zeros((B, 1, 1, Lmax), bool)
    for b in range(B):
        p = lens[b] - 1
        for j in range(Lmax):
            mask[b, 0, 0, j] = j <= p and (W == 0 or p - j < W)
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.ascontiguousarray(qr)), torch.from_numpy(np.repeat(kr, g, axis=1).copy()),
        torch.from_numpy(np.repeat(vf, g, axis=1).copy()), attn_mask=torch.from_numpy(mask))
    return out.numpy()[:, :, 0, :]


# --------------------------------------------- next rows: ring-buffer cache --

@pytest.mark.parametrize("W,C,T", [(8, 8, 1), (8, 11, 1), (5, 9, 3)])
def test_ring_cache_equals_linear_cache(orc, W, C, T):
    """A window-sized cache keeping position j in row j % C gives the decode
    result of the full linear cache, bit for bit; rows holding positions
    older than every window may hold anything."""
    B, Hq, Hkv, D, L = 3, 4, 1, 32, 40
    kl = bf16((B, Hkv, L, D), [922, C, 1])
    vl = bf16((B, Hkv, L, D), [922, C, 2])
    q = bf16((B, T, Hq, D), [922, C, 0]) if T > 1 else bf16((B, Hq, D), [922, C, 0])
    kv = np.array([40, 13, T], np.int32)
    want = orc.decode(q, kl, vl, kv, W, 1e4)
    kr = np.full((B, Hkv, C, D), inputs.NAN_BF16, np.uint16)
    vr = kr.copy()
    for b in range(B):
        lo = max(0, kv[b] - T + 1 - W)
        for j in range(lo, kv[b]):
            kr[b, :, j % C] = kl[b, :, j]
            vr[b, :, j % C] = vl[b, :, j]
    assert np.array_equal(orc.decode(q, kr, vr, kv, W, 1e4, ring=C), want)
    if C > W + T - 1:  # a ring with spare rows: other layers' positions leave the result alone
        assert np.isfinite(want).all()
    with pytest.raises(ValueError):  # a window the ring cannot hold
        orc.decode(q, kr, vr, kv, C + 1, 1e4, ring=C)


# ------------------------------------- next rows: queries against a cache --

@pytest.mark.parametrize("W,alias", [(0, False), (7, True)])
def test_chunked_prefill_equals_full_prefill(orc, W, alias):
    """Prefill of positions P0..P0+S-1 over a cache holding 0..P0+S-1 gives the
    matching rows of the whole prompt's prefill, bit for bit, for any cut."""
    B, S, Hq, Hkv, D = 2, 37, 4, 2, 32
    q = bf16((B, S, Hq, D), [923, W, 0])
    k = bf16((B, Hkv, S + 5, D), [923, W, 1])
    v = None if alias else bf16((B, Hkv, S + 5, D), [923, W, 2])
    full = orc.prefill(q, k, v, W, 1e4)
    for cuts in ([0, 37], [0, 1, 37], [0, 16, 17, 30, 37]):
        for a, b in zip(cuts[:-1], cuts[1:]):
            part = orc.prefill(np.ascontiguousarray(q[:, a:b]), k, v, W, 1e4, start_pos=a)
            assert np.array_equal(part, full[:, a:b])


def test_chunked_prefill_matches_torch_sdpa(orc):
    """Offset positions against torch SDPA on independently rotated vectors."""
    import torch
    B, S, P0, Hq, Hkv, D, W, theta = 1, 9, 14, 4, 2, 64, 10, 1e6
    q = bf16((B, S, Hq, D), [924, 0])
    k = bf16((B, Hkv, P0 + S, D), [924, 1])
    v = bf16((B, Hkv, P0 + S, D), [924, 2])
    got = orc.prefill(q, k, v, W, theta, start_pos=P0)
    L = P0 + S
    kr = _rot_complex(widen(k), np.arange(L)[None, None, :], theta)
    qr = _rot_complex(widen(q).transpose(0, 2, 1, 3), (P0 + np.arange(S))[None, None, :], theta)
    mask = np.array([[j <= P0 + i and P0 + i - j < W for j in range(L)] for i in range(S)])
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.ascontiguousarray(qr)), torch.from_numpy(np.repeat(kr, Hq // Hkv, axis=1).copy()),
        torch.from_numpy(np.repeat(widen(v), Hq // Hkv, axis=1).copy()), attn_mask=torch.from_numpy(mask))
    assert np.max(np.abs(got - out.numpy().transpose(0, 2, 1, 3))) < 1e-10


@pytest.mark.parametrize("W", [0, 6])
def test_multi_token_decode_equals_single_decodes(orc, W):
    """The T queries of a verify step over a frozen cache: query t equals a
    one-token decode with kv_len - T + t + 1 keys, and the prefill chunk at
    kv_len - T, bit for bit."""
    B, T, Hq, Hkv, D, Lmax = 3, 4, 8, 2, 32, 30
    q = bf16((B, T, Hq, D), [925, W, 0])
    k = bf16((B, Hkv, Lmax, D), [925, W, 1])
    v = bf16((B, Hkv, Lmax, D), [925, W, 2])
    kv = np.array([30, 4, 17], np.int32)
    got = orc.decode(q, k, v, kv, W, 1e4)
    for t in range(T):
        one = orc.decode(np.ascontiguousarray(q[:, t]), k, v, kv - T + t + 1, W, 1e4)
        assert np.array_equal(got[:, t], one)
    for b in range(B):
        chunk = orc.prefill(np.ascontiguousarray(q[b:b + 1]), np.ascontiguousarray(k[b:b + 1]),
                            np.ascontiguousarray(v[b:b + 1]), W, 1e4, start_pos=int(kv[b]) - T)
        assert np.array_equal(got[b], chunk[0])


# ---------------------------------------- next rows: bidirectional spans ---

def _span_end(S, spans):
    e = np.arange(S, dtype=np.int32)
    for a, b in spans:  # [a, b] inclusive
        e[a:b + 1] = b
    return e


@pytest.mark.parametrize("W", [0, 5])
def test_bidirectional_spans_match_explicit_mask(orc, W):
    """Queries inside a span see the whole span (earlier and later keys of it)
    plus the usual causal / window keys: against torch SDPA with the mask
    built from the span list by a direct index test."""
    import torch
    B, S, Hq, Hkv, D, theta = 1, 24, 2, 1, 32, 1e4
    spans = [(3, 8), (15, 20)]
    q = bf16((B, S, Hq, D), [926, W, 0])
    k = bf16((B, Hkv, S, D), [926, W, 1])
    v = bf16((B, Hkv, S, D), [926, W, 2])
    se = _span_end(S, spans)[None, :]
    got = orc.prefill(q, k, v, W, theta, span_end=se)
    span_of = {i: n for n, (a, b) in enumerate(spans) for i in range(a, b + 1)}
    mask = np.zeros((S, S), bool)
    for i in range(S):
        for j in range(S):
            same = i in span_of and span_of.get(j) == span_of[i]
            mask[i, j] = (j <= i or same) and (W == 0 or i - j < W)
    kr = _rot_complex(widen(k), np.arange(S)[None, None, :], theta)
    qr = _rot_complex(widen(q).transpose(0, 2, 1, 3), np.arange(S)[None, None, :], theta)
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.ascontiguousarray(qr)), torch.from_numpy(np.repeat(kr, Hq, axis=1).copy()),
        torch.from_numpy(np.repeat(widen(v), Hq, axis=1).copy()), attn_mask=torch.from_numpy(mask))
    assert np.max(np.abs(got - out.numpy().transpose(0, 2, 1, 3))) < 1e-10
    # no spans is the causal prefill, bit for bit
    assert np.array_equal(orc.prefill(q, k, v, W, theta, span_end=np.arange(S, dtype=np.int32)[None, :]),
                          orc.prefill(q, k, v, W, theta))


def test_one_span_over_everything_is_unmasked_attention(orc):
    """A single span covering the whole prompt: every query sees every key
    (closed form: torch SDPA without any mask)."""
    import torch
    S, D = 12, 16
    q = bf16((1, S, 1, D), [927, 0])
    k = bf16((1, 1, S, D), [927, 1])
    got = orc.prefill(q, k, None, 0, 1e4, span_end=np.full((1, S), S - 1, np.int32))
    kr = _rot_complex(widen(k), np.arange(S)[None, None, :], 1e4)
    qr = _rot_complex(widen(q).transpose(0, 2, 1, 3), np.arange(S)[None, None, :], 1e4)
    out = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(np.ascontiguousarray(qr)),
                                                           torch.from_numpy(kr), torch.from_numpy(widen(k)))
    assert np.max(np.abs(got - out.numpy().transpose(0, 2, 1, 3))) < 1e-10


def test_fp8_quantize_matches_torch_and_saturates(orc):
    """x / scale in float32 rounded to E4M3 like torch's float8_e4m3fn
    conversion inside the finite range, saturating to +-448 beyond it."""
    import torch
    rng = np.random.default_rng(928)
    x = np.concatenate([rng.standard_normal(3000).astype(np.float32) * 3,
                        np.arange(-470, 470, 0.25, dtype=np.float32),
                        np.array([2 ** -10, 3 * 2 ** -11, 1.5 * 2 ** -9, 2.5 * 2 ** -9, 0.0, -0.0], np.float32)])
    for scale in (1.0, 0.5, 0.3):
        got = orc.fp8_e4m3_quantize(x, scale)
        q = (x / np.float32(scale)).astype(np.float32)
        inr = np.abs(q) <= 448
        want = torch.from_numpy(q[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(got[inr], want)
        assert np.all(got[~inr & (q > 0)] == 0x7E) and np.all(got[~inr & (q < 0)] == 0xFE)
    # every code decodes to the nearest E4M3 value of the quotient
    vals = orc.fp8_e4m3_value(np.arange(256, dtype=np.uint8))
    fin = vals[np.isfinite(vals)]
    q = (x / np.float32(0.3)).astype(np.float32).astype(np.float64)
    dec = orc.fp8_e4m3_value(orc.fp8_e4m3_quantize(x, 0.3))
    inr = np.abs(q) <= 448
    nearest = np.min(np.abs(fin[None, :] - q[inr, None]), axis=1)
    assert np.allclose(np.abs(dec[inr] - q[inr]), nearest, rtol=0, atol=0)
