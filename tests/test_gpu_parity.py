"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every case feeds the same seeded bf16 inputs to both sides and compares the
outputs element by element: max |diff| <= 2e-2 and mean |diff| <= 2e-3.
Small and medium shapes are compared in full; the full-size workloads are
compared on sampled rows the oracle computes one by one.
"""
import numpy as np
import pytest

import oracle
from hybrid_sliding_global_amd import Stack, inputs
from hybrid_sliding_global_amd import workloads as wl
from gpu_util import check, prefill_rows, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    oracle.build(force=False)
    yield


def _prefill_case(tag, B, S, Hq, Hkv, D, W, alias, Lmax=None, seed=0, rows=None, poison=True, theta=None):
    import torch
    Lmax = Lmax or S
    kind = wl.SLIDING if W > 0 else wl.FULL
    theta = theta or (wl.THETA_SLIDING if kind == wl.SLIDING else wl.THETA_FULL)
    layers = [wl.layer_desc(kind, D, Hq, Hkv, theta, W, int(alias))]
    q = inputs.normal_bf16([100 + seed, S, 0], (B, S, Hq, D))
    k = inputs.normal_bf16([100 + seed, S, 1], (B, Hkv, Lmax, D))
    v = None if alias else inputs.normal_bf16([100 + seed, S, 2], (B, Hkv, Lmax, D))
    if poison and Lmax > S:  # rows past the sequence must never be read
        k[:, :, S:, :] = inputs.NAN_BF16
        if v is not None:
            v[:, :, S:, :] = inputs.NAN_BF16
    st = Stack(layers)
    # Workspace filled with 0xFF bytes (NaN as fp32): any read of a partial
    # result slot that no work-group wrote in this call shows up as NaN.
    ws = torch.full((st.prefill_workspace_bytes(0, B, S),), 0xFF, dtype=torch.uint8, device="cuda:0")
    out = st.prefill(0, to_dev(q), [to_dev(k)], [None if v is None else to_dev(v)], workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = oracle.prefill(q, k, v, W, theta, rows=rows)
    if rows is not None:
        got = got.reshape(-1, D)[rows]
    check(got, want, tag)
    return got


def test_workload1_sliding_prefill_full_compare():
    w = wl.workloads()[1]
    d = w.layers[0]
    q = inputs.normal_bf16([1, 0, inputs.TENSOR_Q], (1, 64, 4, 256))
    k = inputs.normal_bf16([1, 0, inputs.TENSOR_K], (1, 1, 64, 256))
    st = Stack(w.layers)
    import torch
    out = st.prefill(0, to_dev(q), [to_dev(k)], [None])
    torch.cuda.synchronize()
    check(out.cpu().numpy(), oracle.prefill(q, k, None, d["window"], d["rope_theta"]), "workload1")


@pytest.mark.parametrize("B,S,Hq,Hkv,D,W,alias,Lmax", [
    (1, 200, 8, 2, 512, 0, False, 256),    # full layer, ragged S, poisoned rows past S
    (2, 333, 8, 1, 256, 48, True, 333),    # sliding K=V, batch 2, ragged
    (1, 77, 6, 2, 512, 0, False, 77),      # GQA group of 3
    (1, 130, 2, 2, 256, 16, False, 130),   # no GQA sharing, sliding with separate V
    (1, 1, 4, 1, 256, 32, True, 1),        # single token
    (1, 50, 4, 1, 256, 1, True, 64),       # window 1: every row returns its own raw key
    (1, 100, 8, 1, 256, 512, True, 100),   # window wider than the sequence = causal
    (3, 257, 16, 2, 256, 100, True, 300),  # GQA group of 8, three sequences
    (1, 129, 1, 1, 512, 0, False, 129),    # one head, one tile past a 128-row boundary
    (2, 96, 32, 2, 512, 0, False, 96),     # GQA group of 16
    (1, 300, 4, 4, 512, 64, True, 300),    # sliding layer with head size 512 (any kind/size pair works)
    # causal layers long enough that query tiles are cut across work-groups
    (1, 1024, 8, 1, 256, 0, False, 1024),  # single query tiles in up to 4 pieces
    (1, 2048, 4, 1, 256, 0, False, 2048),  # pairs of query tiles in up to 8 pieces
    (1, 640, 8, 2, 512, 0, False, 640),    # head size 512, pairs cut into 11 pieces
    (1, 37, 160, 1, 512, 0, False, 40),    # GQA group of 160: a 128-row tile spans parts of two positions
])
def test_prefill_shapes(B, S, Hq, Hkv, D, W, alias, Lmax):
    _prefill_case("prefill B%d S%d Hq%d Hkv%d D%d W%d alias%d" % (B, S, Hq, Hkv, D, W, alias), B, S, Hq, Hkv, D, W,
                  alias, Lmax)


@pytest.mark.parametrize("split_pv", [0, 1])
@pytest.mark.parametrize("B,S,Hq,Hkv,W,alias,Lmax", [
    (1, 200, 8, 2, 0, False, 256),      # ragged S, poisoned rows past S
    (1, 77, 6, 2, 0, False, 77),        # GQA group of 3
    (1, 1, 4, 1, 0, False, 1),          # single token: one key tile
    (1, 300, 4, 4, 64, True, 300),      # windowed, K=V
    (1, 640, 8, 2, 0, False, 640),      # pairs cut into pieces
    (2, 1100, 8, 2, 0, False, 1100),    # two sequences, long segments
    (1, 37, 160, 1, 0, False, 40),      # GQA group of 160
])
def test_prefill_head512_schedules(monkeypatch, split_pv, B, S, Hq, Hkv, W, alias, Lmax):
    """Head size 512 has two tile schedules (PV in one phase, or split over two); both against the oracle."""
    monkeypatch.setenv("G4_PREFILL_SPLIT_PV", str(split_pv))
    _prefill_case("prefill splitpv%d B%d S%d Hq%d Hkv%d W%d alias%d" % (split_pv, B, S, Hq, Hkv, W, alias), B, S, Hq,
                  Hkv, 512, W, alias, Lmax)


@pytest.mark.parametrize("rows", [64, 128])
@pytest.mark.parametrize("B,S,Hq,Hkv,W,alias,Lmax", [
    (2, 333, 8, 1, 48, True, 333),      # sliding K=V, batch 2, ragged
    (1, 130, 2, 2, 16, False, 130),     # no GQA sharing, separate V
    (1, 1, 4, 1, 32, True, 1),          # single token
    (3, 257, 16, 2, 100, True, 300),    # GQA group of 8, three sequences, poisoned tail
    (1, 200, 8, 2, 0, False, 256),      # causal, ragged, poisoned tail
    (1, 1024, 8, 1, 0, False, 1024),    # causal: 128-row tiles cut into pieces
    (1, 2048, 4, 1, 0, False, 2048),    # causal: pairs of 128-row tiles in up to 8 pieces
    (1, 1000, 8, 1, 512, True, 1000),   # the stack's sliding-layer configuration, shorter
    (1, 45, 96, 1, 16, True, 45),       # GQA group of 96: one position per 64-row tile, less than one per row block
])
def test_prefill_head256_tile_heights(monkeypatch, rows, B, S, Hq, Hkv, W, alias, Lmax):
    """Head size 256 runs 128-row or 64-row query tiles; both against the oracle."""
    monkeypatch.setenv("G4_PREFILL_ROWS", str(rows))
    _prefill_case("prefill rows%d B%d S%d Hq%d Hkv%d W%d alias%d" % (rows, B, S, Hq, Hkv, W, alias), B, S, Hq, Hkv,
                  256, W, alias, Lmax)


def test_prefill_window_one_is_identity_on_raw_keys():
    got = _prefill_case("window1", 1, 40, 4, 1, 256, 1, True)
    k = inputs.normal_bf16([100, 40, 1], (1, 1, 40, 256))
    want = inputs.f32_from_bf16_bits(k[0, 0]).astype(np.float64)
    for h in range(4):
        assert np.max(np.abs(got[0, :, h, :] - want)) <= 2e-2


def test_workload2_full_prefill_sampled_rows():
    w = wl.workloads()[2]
    d = w.layers[0]
    S, Hq, Hkv, D = 4096, 8, 2, 512
    import torch
    q = inputs.normal_bf16([2, 0, inputs.TENSOR_Q], (1, S, Hq, D))
    k = inputs.normal_bf16([2, 0, inputs.TENSOR_K], (1, Hkv, S, D))
    v = inputs.normal_bf16([2, 0, inputs.TENSOR_V], (1, Hkv, S, D))
    out = Stack(w.layers).prefill(0, to_dev(q), [to_dev(k)], [to_dev(v)])
    torch.cuda.synchronize()
    pos = [0, 1, 7, 31, 32, 33, 127, 128, 129, 1000, 2047, 2048, 3000, 4000, 4094, 4095]
    rows = prefill_rows(1, S, Hq, pos)
    got = out.cpu().numpy().reshape(-1, D)[rows]
    check(got, oracle.prefill(q, k, v, 0, d["rope_theta"], rows=rows), "workload2 sampled")


def _stack_inputs(S=2048):
    layers = wl.gemma4_stack()
    qs, kc, vc = [], [], []
    for i, d in enumerate(layers):
        D = d["head_dim"]
        qs.append(inputs.normal_bf16([4, i, inputs.TENSOR_Q], (1, S, d["num_q_heads"], D)))
        if d["kv_source_layer"] < 0:
            kc.append(inputs.normal_bf16([4, i, inputs.TENSOR_K], (1, d["num_kv_heads"], S, D)))
            vc.append(None if d["kv_alias"] else inputs.normal_bf16([4, i, inputs.TENSOR_V],
                                                                    (1, d["num_kv_heads"], S, D)))
        else:
            kc.append(None)
            vc.append(None)
    return layers, qs, kc, vc


def test_workload4_stack_sampled_rows_and_sharing():
    import torch
    S = 2048
    layers, qs, kc, vc = _stack_inputs(S)
    st = Stack(layers)
    kd = [None if k is None else to_dev(k) for k in kc]
    vd = [None if v is None else to_dev(v) for v in vc]
    pos = [0, 5, 255, 256, 511, 512, 513, 1023, 1500, 2047]
    outs = []
    for i, d in enumerate(layers):
        out = st.prefill(i, to_dev(qs[i]), kd, vd)
        torch.cuda.synchronize()
        rows = prefill_rows(1, S, d["num_q_heads"], pos, heads=[0, d["num_q_heads"] - 1])
        got = out.cpu().numpy().reshape(-1, d["head_dim"])[rows]
        src = i if d["kv_source_layer"] < 0 else d["kv_source_layer"]
        want = oracle.prefill(qs[i], kc[src], None if d["kv_alias"] else vc[src], d["window"], d["rope_theta"],
                              rows=rows)
        check(got, want, "stack layer %d (src %d)" % (i, src))
        outs.append(out)
    # a shared layer gives bit-identical results to the same layer owning a copy of the source cache
    for i in (15, 19):
        d = dict(layers[i])
        src = d["kv_source_layer"]
        d["kv_source_layer"] = -1
        own = Stack([d])
        k_copy = kd[src].clone()
        v_copy = None if vd[src] is None else vd[src].clone()
        ref = own.prefill(0, to_dev(qs[i]), [k_copy], [v_copy])
        torch.cuda.synchronize()
        assert torch.equal(ref, outs[i]), "shared layer %d differs from a copied cache" % i


def test_stack_graph_replays_match_eager():
    """The 35-layer stack (S=640) captured in one HIP graph: every replay, with
    eager calls and synchronisations in between, equals the eager outputs bit
    for bit (the prefill kernels are deterministic)."""
    import torch
    S = 640
    layers, qs, kc, vc = _stack_inputs(S)
    st = Stack(layers)
    kd = [None if k is None else to_dev(k) for k in kc]
    vd = [None if v is None else to_dev(v) for v in vc]
    qd = [to_dev(q) for q in qs]
    outs = [torch.empty((1, S, d["num_q_heads"], d["head_dim"]), dtype=torch.float32, device="cuda:0")
            for d in layers]
    wss = [torch.empty(st.prefill_workspace_bytes(i, 1, S), dtype=torch.uint8, device="cuda:0")
           for i in range(len(layers))]

    def one_pass():
        for i in range(len(layers)):
            st.prefill(i, qd[i], kd, vd, out=outs[i], workspace=wss[i])

    one_pass()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one_pass()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_pass()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for i in range(len(layers)):
            assert torch.equal(outs[i], eager[i]), "replay %d, layer %d differs from eager" % (rep, i)
        one_pass()  # eager work between replays
        torch.cuda.synchronize()


def test_alias_equals_explicit_duplicate_values():
    import torch
    S, D = 300, 256
    q = to_dev(inputs.normal_bf16([5, 1, 0], (1, S, 8, D)))
    k = to_dev(inputs.normal_bf16([5, 1, 1], (1, 1, S, D)))
    a = Stack([wl.layer_desc(wl.SLIDING, D, 8, 1, 1e4, 64, 1)]).prefill(0, q, [k], [None])
    b = Stack([wl.layer_desc(wl.SLIDING, D, 8, 1, 1e4, 64, 0)]).prefill(0, q, [k], [k.clone()])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ------------------------------------------------------------------ decode --

def _decode_case(tag, B, Hq, Hkv, D, W, alias, kv_len, Lmax, seed=0, max_kv_len=None, poison=True, theta=None,
                 rows=None):
    import torch
    kind = wl.SLIDING if W > 0 else wl.FULL
    theta = theta or (wl.THETA_SLIDING if kind == wl.SLIDING else wl.THETA_FULL)
    layers = [wl.layer_desc(kind, D, Hq, Hkv, theta, W, int(alias))]
    kv_len = np.asarray(kv_len, np.int32)
    q = inputs.normal_bf16([200 + seed, Lmax, 0], (B, Hq, D))
    k = inputs.normal_bf16([200 + seed, Lmax, 1], (B, Hkv, Lmax, D))
    v = None if alias else inputs.normal_bf16([200 + seed, Lmax, 2], (B, Hkv, Lmax, D))
    if poison:
        inputs.poison_beyond(k, kv_len)
        if v is not None:
            inputs.poison_beyond(v, kv_len)
    st = Stack(layers)
    kl = torch.from_numpy(kv_len).to("cuda:0")
    out = st.decode(0, to_dev(q), [to_dev(k)], [None if v is None else to_dev(v)], kl,
                    int(max_kv_len or kv_len.max()))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = oracle.decode(q, k, v, kv_len, W, theta, rows=rows)
    if rows is not None:
        got = got.reshape(-1, D)[rows]
    check(got, want, tag)
    return got


@pytest.mark.parametrize("B,Hq,Hkv,D,W,alias,kv_len,Lmax", [
    (4, 8, 2, 512, 0, False, [1, 33, 1000, 4096], 4096),    # full layer, ragged lengths, length 1
    (4, 8, 1, 256, 1024, True, [1, 500, 1025, 3000], 3000),  # sliding K=V, window partly / fully used
    (3, 16, 2, 256, 64, True, [64, 65, 2000], 2048),          # GQA group of 8
    (2, 16, 1, 512, 0, False, [777, 12345], 12345),           # GQA group of 16
    (2, 2, 2, 256, 0, False, [31, 32], 40),                   # no sharing, tiny lengths
    (1, 4, 1, 256, 1, True, [100], 100),                      # window 1 -> own raw key
    (2, 4, 2, 512, 300, False, [299, 301], 512),              # sliding, separate values, head size 512
    # 300 short sequences: the batch scan runs over two blocks of 256 entries,
    # and one piece of the key split covers many whole streams
    (300, 4, 1, 256, 48, True, [1 + (37 * i) % 97 for i in range(300)], 97),
    (300, 8, 2, 512, 0, False, [1 + (53 * i) % 60 for i in range(300)], 64),
])
def test_decode_shapes(B, Hq, Hkv, D, W, alias, kv_len, Lmax):
    _decode_case("decode B%d Hq%d Hkv%d D%d W%d alias%d L%s" % (B, Hq, Hkv, D, W, alias, kv_len), B, Hq, Hkv, D, W,
                 alias, kv_len, Lmax)


def test_decode_split_invariance():
    """The result does not depend on how the keys are cut into pieces (only
    fp32 rounding): the pieces are equal shares of all streams' keys, so a
    longer second sequence moves every piece boundary of the first."""
    kw = dict(B=2, Hq=8, Hkv=2, D=512, W=0, alias=False, Lmax=65536)
    a = _decode_case("split: companion 3000 keys", kv_len=[5000, 3000], **kw)
    b = _decode_case("split: companion 60000 keys", kv_len=[5000, 60000], **kw)
    assert np.max(np.abs(a[0] - b[0])) < 1e-3


@pytest.mark.parametrize("split_pv", [0, 1])
def test_prefill_head512_repeatable(monkeypatch, split_pv):
    """Tiles cut into pieces are merged by whichever piece arrives last, in
    ascending piece order: two calls agree bit for bit under both schedules."""
    monkeypatch.setenv("G4_PREFILL_SPLIT_PV", str(split_pv))
    kw = (1, 640, 8, 2, 512, 0, False, 640)
    a = _prefill_case("repeat 1 splitpv%d" % split_pv, *kw)
    b = _prefill_case("repeat 2 splitpv%d" % split_pv, *kw)
    assert np.array_equal(a, b)


def test_decode_repeatable():
    """Decode has no atomics and merges partials in a fixed order: two calls on
    the same inputs agree bit for bit."""
    kw = dict(B=3, Hq=8, Hkv=2, D=512, W=0, alias=False, kv_len=[2000, 37, 4096], Lmax=4096)
    a = _decode_case("repeat 1", **kw)
    b = _decode_case("repeat 2", **kw)
    assert np.array_equal(a, b)


def test_workload3_decode():
    w = wl.workloads()[3]
    import torch
    B, L = 64, 8192
    kv = np.full(B, L, np.int32)
    kl = torch.from_numpy(kv).to("cuda:0")
    for li, d in enumerate(w.layers):
        D, Hq, Hkv = d["head_dim"], d["num_q_heads"], d["num_kv_heads"]
        q = inputs.normal_bf16([3, li, inputs.TENSOR_Q], (B, Hq, D))
        k = inputs.normal_bf16([3, li, inputs.TENSOR_K], (B, Hkv, L, D))
        v = None if d["kv_alias"] else inputs.normal_bf16([3, li, inputs.TENSOR_V], (B, Hkv, L, D))
        out = Stack([d]).decode(0, to_dev(q), [to_dev(k)], [None if v is None else to_dev(v)], kl, L)
        torch.cuda.synchronize()
        want = oracle.decode(q, k, v, kv, d["window"], d["rope_theta"])
        check(out.cpu().numpy(), want, "workload3 layer %d" % li)
        del k, v


def test_workload5_long_context_decode():
    w = wl.workloads()[5]
    import torch
    B, Lmax = 4, 131072
    kv = inputs.kv_lengths_uniform([5, 0, inputs.TENSOR_LEN], B, 1024, Lmax)
    kl = torch.from_numpy(kv).to("cuda:0")
    for li, d in enumerate(w.layers):
        D, Hq, Hkv = d["head_dim"], d["num_q_heads"], d["num_kv_heads"]
        q = inputs.normal_bf16([5, li, inputs.TENSOR_Q], (B, Hq, D))
        k = inputs.normal_bf16([5, li, inputs.TENSOR_K], (B, Hkv, Lmax, D))
        inputs.poison_beyond(k, kv)
        v = None
        if not d["kv_alias"]:
            v = inputs.normal_bf16([5, li, inputs.TENSOR_V], (B, Hkv, Lmax, D))
            inputs.poison_beyond(v, kv)
        out = Stack([d]).decode(0, to_dev(q), [to_dev(k)], [None if v is None else to_dev(v)], kl, Lmax)
        torch.cuda.synchronize()
        want = oracle.decode(q, k, v, kv, d["window"], d["rope_theta"])
        check(out.cpu().numpy(), want, "workload5 layer %d L=%s" % (li, kv.tolist()))
        del k, v
