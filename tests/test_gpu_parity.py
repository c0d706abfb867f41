"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every case feeds the same seeded bf16 inputs to both sides and compares the
outputs element by element: max |diff| <= 2e-2, mean |diff| <= 2e-3 and
relative RMS error <= 1e-2.  Every case is compared in full except the
long-context decode ones, whose oracle rows are sampled.
"""
import numpy as np
import pytest

import oracle
from hybrid_sliding_global_amd import Stack, inputs
from hybrid_sliding_global_amd import workloads as wl
from gpu_util import check, to_dev
import wide_range as wr

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


@pytest.mark.parametrize("rows,producer", [(64, 1), (64, 0), (128, 1)])
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
def test_prefill_head256_tile_heights(monkeypatch, rows, producer, B, S, Hq, Hkv, W, alias, Lmax):
    """Head size 256 runs 128-row or 64-row query tiles, the 64-row ones with
    or without producer waves for the tile copies; all against the oracle."""
    monkeypatch.setenv("G4_PREFILL_ROWS", str(rows))
    monkeypatch.setenv("G4_PREFILL_PRODUCER", str(producer))
    _prefill_case("prefill rows%d producer%d B%d S%d Hq%d Hkv%d W%d alias%d" % (rows, producer, B, S, Hq, Hkv, W, alias),
                  B, S, Hq, Hkv, 256, W, alias, Lmax)


def test_prefill_window_one_is_identity_on_raw_keys():
    got = _prefill_case("window1", 1, 40, 4, 1, 256, 1, True)
    k = inputs.normal_bf16([100, 40, 1], (1, 1, 40, 256))
    want = inputs.f32_from_bf16_bits(k[0, 0]).astype(np.float64)
    for h in range(4):
        assert np.max(np.abs(got[0, :, h, :] - want)) <= 2e-2


def test_workload2_full_prefill_every_row():
    w = wl.workloads()[2]
    d = w.layers[0]
    S, Hq, Hkv, D = 4096, 8, 2, 512
    import torch
    q = inputs.normal_bf16([2, 0, inputs.TENSOR_Q], (1, S, Hq, D))
    k = inputs.normal_bf16([2, 0, inputs.TENSOR_K], (1, Hkv, S, D))
    v = inputs.normal_bf16([2, 0, inputs.TENSOR_V], (1, Hkv, S, D))
    out = Stack(w.layers).prefill(0, to_dev(q), [to_dev(k)], [to_dev(v)])
    torch.cuda.synchronize()
    check(out.cpu().numpy(), oracle.prefill(q, k, v, 0, d["rope_theta"]), "workload2 full")


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


def test_workload4_stack_every_row_and_sharing():
    import torch
    S = 2048
    layers, qs, kc, vc = _stack_inputs(S)
    st = Stack(layers)
    kd = [None if k is None else to_dev(k) for k in kc]
    vd = [None if v is None else to_dev(v) for v in vc]
    outs = []
    for i, d in enumerate(layers):
        out = st.prefill(i, to_dev(qs[i]), kd, vd)
        torch.cuda.synchronize()
        src = i if d["kv_source_layer"] < 0 else d["kv_source_layer"]
        want = oracle.prefill(qs[i], kc[src], None if d["kv_alias"] else vc[src], d["window"], d["rope_theta"])
        check(out.cpu().numpy(), want, "stack layer %d (src %d)" % (i, src))
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


@pytest.mark.parametrize("S,rows", [(640, None), (1000, "128")])
def test_shared_layers_reuse_source_images(monkeypatch, S, rows):
    """A layer sharing another's cache (same kind, so the same rotation) may
    reuse the key/value operand images its source left in the workspace
    (g4_prefill_opts.images_ready): the key pass is skipped and the output is
    bit-identical to a call that builds them, and matches the oracle.  S=1000
    with 128-row tiles cuts tiles into pieces, so the reused workspace's split
    counters are reset without the key pass."""
    import torch
    if rows:
        monkeypatch.setenv("G4_PREFILL_ROWS", rows)
    layers, qs, kc, vc = _stack_inputs(S)
    st = Stack(layers)
    kd = [None if k is None else to_dev(k) for k in kc]
    vd = [None if v is None else to_dev(v) for v in vc]
    # one workspace per layer kind: the last owner of each kind leaves its
    # images there, and every shared layer of that kind reads the same cache
    kinds = sorted({d["kind"] for d in layers})
    ws = {kd_: torch.full((max(st.prefill_workspace_bytes(i, 1, S) for i, d in enumerate(layers) if d["kind"] == kd_),),
                          0xFF, dtype=torch.uint8, device="cuda:0") for kd_ in kinds}
    checked = 0
    for i, d in enumerate(layers):
        shared = d["kv_source_layer"] >= 0
        out = st.prefill(i, to_dev(qs[i]), kd, vd, workspace=ws[d["kind"]], images_ready=shared)
        torch.cuda.synchronize()
        if not shared:
            continue
        ref = st.prefill(i, to_dev(qs[i]), kd, vd)  # fresh workspace: builds the images
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "layer %d: reused images differ" % i
        if checked < 2 or i in (19, 34):
            src = d["kv_source_layer"]
            want = oracle.prefill(qs[i], kc[src], None if d["kv_alias"] else vc[src], d["window"], d["rope_theta"])
            check(out.cpu().numpy(), want, "reused images layer %d (src %d) S%d" % (i, src, S))
            checked += 1


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


@pytest.mark.parametrize("S,rows", [(1000, "128"), (1000, None)])
def test_stack_graph_replays_with_image_reuse(monkeypatch, S, rows):
    """The launch configuration of the stack benchmark, captured in one HIP
    graph: every shared layer runs in its source layer's workspace and skips
    the key pass (images_ready), so nothing zeroes the split tiles' counters
    inside the graph -- each launch must leave them zero itself.  S=1000 cuts
    tiles into pieces in the head-size-512 kernel (and, with 128-row tiles,
    in the head-size-256 one); every replay, with eager passes in between,
    equals the eager outputs bit for bit."""
    import torch
    if rows:
        monkeypatch.setenv("G4_PREFILL_ROWS", rows)
    layers, qs, kc, vc = _stack_inputs(S)
    st = Stack(layers)
    kd = [None if k is None else to_dev(k) for k in kc]
    vd = [None if v is None else to_dev(v) for v in vc]
    qd = [to_dev(q) for q in qs]
    outs = [torch.empty((1, S, d["num_q_heads"], d["head_dim"]), dtype=torch.float32, device="cuda:0")
            for d in layers]
    src = [i if d["kv_source_layer"] < 0 else d["kv_source_layer"] for i, d in enumerate(layers)]
    need = {}
    for i in range(len(layers)):
        need[src[i]] = max(need.get(src[i], 0), st.prefill_workspace_bytes(i, 1, S))
    wss = {o: torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda:0") for o, n in need.items()}

    def one_pass():
        for i in range(len(layers)):
            st.prefill(i, qd[i], kd, vd, out=outs[i], workspace=wss[src[i]], images_ready=src[i] != i)

    one_pass()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for i in (0, 4, 19, 34):  # owners and sharers of both kinds against the oracle
        d = layers[i]
        want = oracle.prefill(qs[i], kc[src[i]], None if d["kv_alias"] else vc[src[i]], d["window"], d["rope_theta"])
        check(eager[i].cpu().numpy(), want, "graph stack layer %d (src %d) S%d rows %s" % (i, src[i], S, rows))
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
    (3, 8, 2, 512, 0, True, [1, 700, 4096], 4096),            # head size 512 with K=V (full kind)
    (2, 16, 1, 512, 1024, True, [5000, 1030], 5000),          # head size 512 with K=V, windowed, GQA group 16
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


@pytest.mark.parametrize("pieces", [1, 3, 37, 512])
@pytest.mark.parametrize("D,W,alias", [(512, 0, False), (256, 1024, True)])
def test_decode_piece_counts(monkeypatch, pieces, D, W, alias):
    """The decode split at the extremes of its piece count (G4_DECODE_PIECES):
    one work-group for every stream's keys, a few pieces each covering
    several streams, and the default 512; every count matches the oracle."""
    monkeypatch.setenv("G4_DECODE_PIECES", str(pieces))
    _decode_case("decode pieces %d D%d W%d" % (pieces, D, W), B=5, Hq=8, Hkv=2, D=D, W=W, alias=alias,
                 kv_len=[1, 700, 5000, 33, 2049], Lmax=5000)


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


# ------------------------------------------------------- wide score range --
# Planted keys whose scores rise 12 log2 units apart (tests/wide_range.py):
# the running maximum of online softmax then moves many times per row, the
# four-wave head-size-256 prefill repeats its pass (rise above 64 log2
# units), and split tiles merge pieces whose maxima differ by tens of units.
# Each case first shows on the CPU, from the oracle's scores, that it
# crosses those bounds.

import test_wide_range_inputs as wri  # noqa: E402


def _wide_prefill(case, tag):
    import torch
    B, S, Hq, Hkv, D, W, theta, seed, every, period = case
    q, k, v, planted = wr.prefill_case(B, S, Hq, Hkv, D, W, theta, seed, every, period)
    jump, rise = wr.prefill_growth(oracle, q, k, W, theta, [(S - 1) * Hq, (S // 2) * Hq + 1, (S - 40) * Hq + Hq - 1])
    assert jump > wri.RESCALE and rise > wri.REPEAT, (jump, rise)
    kind = wl.SLIDING if W > 0 else wl.FULL
    st = Stack([wl.layer_desc(kind, D, Hq, Hkv, theta, W, 0)])
    ws = torch.full((st.prefill_workspace_bytes(0, B, S),), 0xFF, dtype=torch.uint8, device="cuda:0")
    out = st.prefill(0, to_dev(q), [to_dev(k)], [to_dev(v)], workspace=ws)
    torch.cuda.synchronize()
    check(out.cpu().numpy(), oracle.prefill(q, k, v, W, theta), tag)


@pytest.mark.parametrize("split_pv", [0, 1])
def test_wide_range_prefill_head512(monkeypatch, split_pv):
    monkeypatch.setenv("G4_PREFILL_SPLIT_PV", str(split_pv))
    _wide_prefill(wri.PREFILL_CASES[0], "wide prefill D512 splitpv%d" % split_pv)


@pytest.mark.parametrize("case", [1, 2])
@pytest.mark.parametrize("rows,producer", [(64, 1), (64, 0), (128, 1)])
def test_wide_range_prefill_head256(monkeypatch, rows, producer, case):
    """(64-row tiles run with and without their producer waves: the repeated
    pass must replay the same barrier sequence in both roles.)"""
    monkeypatch.setenv("G4_PREFILL_ROWS", str(rows))
    monkeypatch.setenv("G4_PREFILL_PRODUCER", str(producer))
    _wide_prefill(wri.PREFILL_CASES[case], "wide prefill D256 case%d rows%d producer%d" % (case, rows, producer))


@pytest.mark.parametrize("case", wri.DECODE_CASES)
def test_wide_range_decode(case):
    import torch
    B, Hq, Hkv, D, kv_len, Lmax, seed = case
    kv = np.array(kv_len, np.int32)
    q, k, v = wr.decode_case(B, Hq, Hkv, D, kv, Lmax, seed)
    theta = wl.THETA_FULL if D == 512 else wl.THETA_SLIDING
    assert wr.decode_growth(oracle, q, k, kv, 0, theta) > wri.RESCALE
    st = Stack([wl.layer_desc(wl.FULL, D, Hq, Hkv, theta, 0, 0)])
    out = st.decode(0, to_dev(q), [to_dev(k)], [to_dev(v)], torch.from_numpy(kv).to("cuda:0"), Lmax)
    torch.cuda.synchronize()
    check(out.cpu().numpy(), oracle.decode(q, k, v, kv, 0, theta), "wide decode D%d" % D)


def test_decode_long_pieces():
    """16 sequences of about 131k keys, two kv heads: each of the 512 work-groups
    takes about 8192 keys (512 steps of 16), so the query rotation runs its
    per-step recurrence far beyond the lengths of the other cases.  The cache
    repeats one seeded block of 4099 rows (so the rows of a piece are not
    aligned with the repetition); sampled rows are compared with the oracle."""
    import torch
    B, Hq, Hkv, D, L = 16, 8, 2, 256, 131072
    kv = np.array([L - 7 * b for b in range(B)], np.int32)
    block = inputs.normal_bf16([500, 0, 1], (4099, D))
    k = np.resize(block, (B, Hkv, L, D))
    inputs.poison_beyond(k, kv)
    q = inputs.normal_bf16([500, 0, 0], (B, Hq, D))
    st = Stack([wl.layer_desc(wl.FULL, D, Hq, Hkv, wl.THETA_FULL, 0, 1)])
    out = st.decode(0, to_dev(q), [to_dev(k)], [None], torch.from_numpy(kv).to("cuda:0"), L)
    torch.cuda.synchronize()
    rows = np.array([0 * Hq + 0, 5 * Hq + 3, 9 * Hq + 4, 15 * Hq + 7], np.int64)
    got = out.cpu().numpy().reshape(-1, D)[rows]
    check(got, oracle.decode(q, k, None, kv, 0, wl.THETA_FULL, rows=rows), "decode long pieces")


# ------------------------------------- queries against an existing cache --
# A chunk of a prompt at start position P0 (keys 0 .. P0+S-1 already in the
# cache) and T > 1 decode tokens per sequence (the verify step of
# speculative decoding over a frozen cache).

@pytest.mark.parametrize("B,S,P0,Hq,Hkv,D,W,alias,override", [
    (1, 300, 1000, 8, 2, 512, 0, False, ("G4_PREFILL_SPLIT_PV", "0")),
    (1, 300, 1000, 8, 2, 512, 0, False, ("G4_PREFILL_SPLIT_PV", "1")),
    (1, 128, 3968, 8, 2, 512, 0, False, None),      # the last 128 queries of the 4096-token layer
    (2, 200, 1500, 8, 1, 256, 512, True, ("G4_PREFILL_ROWS", "64")),
    (2, 200, 1500, 8, 1, 256, 512, True, ("G4_PREFILL_ROWS", "128")),
    (1, 1, 37, 4, 1, 256, 0, False, None),           # one query: a decode step through the prefill path
    (1, 77, 5, 6, 2, 512, 64, True, None),           # short history, windowed, GQA group of 3
    (1, 640, 640, 8, 1, 256, 0, False, ("G4_PREFILL_ROWS", "128")),  # tiles cut into pieces
])
def test_chunked_prefill(monkeypatch, B, S, P0, Hq, Hkv, D, W, alias, override):
    import torch
    if override:
        monkeypatch.setenv(*override)
    Lmax = P0 + S + 7
    kind = wl.SLIDING if W > 0 else wl.FULL
    theta = wl.THETA_SLIDING if kind == wl.SLIDING else wl.THETA_FULL
    q = inputs.normal_bf16([700, P0, 0], (B, S, Hq, D))
    k = inputs.normal_bf16([700, P0, 1], (B, Hkv, Lmax, D))
    v = None if alias else inputs.normal_bf16([700, P0, 2], (B, Hkv, Lmax, D))
    k[:, :, P0 + S:] = inputs.NAN_BF16  # rows past the chunk must never be read
    if v is not None:
        v[:, :, P0 + S:] = inputs.NAN_BF16
    st = Stack([wl.layer_desc(kind, D, Hq, Hkv, theta, W, int(alias))])
    ws = torch.full((st.prefill_workspace_bytes(0, B, S, P0),), 0xFF, dtype=torch.uint8, device="cuda:0")
    out = st.prefill(0, to_dev(q), [to_dev(k)], [None if v is None else to_dev(v)], workspace=ws, start_pos=P0)
    torch.cuda.synchronize()
    check(out.cpu().numpy(), oracle.prefill(q, k, v, W, theta, start_pos=P0),
          "chunk B%d S%d P0=%d D%d W%d %s" % (B, S, P0, D, W, override))


@pytest.mark.parametrize("B,T,Hq,Hkv,D,W,alias,kv_len,Lmax", [
    (3, 2, 8, 2, 512, 0, False, [2, 700, 4096], 4096),      # T*g = 8
    (3, 4, 8, 2, 512, 0, False, [4, 33, 3000], 3000),       # T*g = 16: one full column group
    (2, 7, 8, 2, 512, 0, False, [5000, 7], 5000),           # T*g = 28: two column groups
    (4, 2, 8, 1, 256, 1024, True, [2, 500, 1025, 3000], 3000),  # sliding K=V, windows of both tokens
    (3, 3, 16, 2, 256, 64, True, [64, 65, 2000], 2048),     # T*g = 24, window smaller than the span of tokens
    (2, 5, 4, 4, 256, 0, False, [31, 40], 40),              # no GQA sharing
    (2, 3, 32, 1, 512, 0, False, [900, 3], 900),            # 32 query heads per kv head: six column groups
])
def test_multi_token_decode(B, T, Hq, Hkv, D, W, alias, kv_len, Lmax):
    import torch
    kind = wl.SLIDING if W > 0 else wl.FULL
    theta = wl.THETA_SLIDING if kind == wl.SLIDING else wl.THETA_FULL
    kv = np.asarray(kv_len, np.int32)
    q = inputs.normal_bf16([710, T, 0], (B, T, Hq, D))
    k = inputs.poison_beyond(inputs.normal_bf16([710, T, 1], (B, Hkv, Lmax, D)), kv)
    v = None if alias else inputs.poison_beyond(inputs.normal_bf16([710, T, 2], (B, Hkv, Lmax, D)), kv)
    st = Stack([wl.layer_desc(kind, D, Hq, Hkv, theta, W, int(alias))])
    ws = torch.full((st.decode_workspace_bytes(0, B, Lmax, T),), 0xFF, dtype=torch.uint8, device="cuda:0")
    out = st.decode(0, to_dev(q), [to_dev(k)], [None if v is None else to_dev(v)], torch.from_numpy(kv).to("cuda:0"),
                    Lmax, workspace=ws)
    torch.cuda.synchronize()
    check(out.cpu().numpy(), oracle.decode(q, k, v, kv, W, theta),
          "decode T%d B%d Hq%d Hkv%d D%d W%d L%s" % (T, B, Hq, Hkv, D, W, kv_len))


# -------------------------------- window-sized ring caches, fused append --
# A sliding layer's cache of C >= W rows per (batch, kv head) keeps position
# j in row j mod C; the decode call can also write the current tokens' keys
# and values itself (into the ring or a linear cache) and attend to them.

def _ring_from_linear(lin, kv, C, poison_old=0):
    """Ring of C rows holding positions max(0, L-C) .. L-1 of each sequence;
    rows of the ``poison_old`` oldest positions it holds are set to NaN."""
    B, H, _, D = lin.shape
    ring = np.full((B, H, C, D), inputs.NAN_BF16, np.uint16)
    for b, L in enumerate(kv):
        lo = max(0, int(L) - C)
        for j in range(lo, int(L)):
            ring[b, :, j % C] = lin[b, :, j]
        for j in range(lo, min(int(L), lo + poison_old)):
            ring[b, :, j % C] = inputs.NAN_BF16
    return ring


@pytest.mark.parametrize("B,T,Hq,Hkv,D,W,C,alias,kv_len", [
    (4, 1, 8, 1, 256, 1024, 1024, True, [5000, 1024, 1, 3000]),   # the batched sliding layer's shape, ring = window
    (3, 1, 16, 2, 256, 1024, 1100, True, [1100, 70000, 2047]),    # spare rows hold older positions (poisoned)
    (2, 3, 8, 2, 512, 300, 302, False, [303, 9999]),               # three tokens: ring = window + 2
])
def test_ring_cache_decode(B, T, Hq, Hkv, D, W, C, alias, kv_len):
    import torch
    kv = np.asarray(kv_len, np.int32)
    Lmax = int(kv.max())
    q = inputs.normal_bf16([720, C, 0], (B, T, Hq, D) if T > 1 else (B, Hq, D))
    k = inputs.normal_bf16([720, C, 1], (B, Hkv, Lmax, D))
    v = None if alias else inputs.normal_bf16([720, C, 2], (B, Hkv, Lmax, D))
    spare = C - (W + T - 1)
    kr = _ring_from_linear(k, kv, C, spare)
    vr = None if alias else _ring_from_linear(v, kv, C, spare)
    st = Stack([wl.layer_desc(wl.SLIDING, D, Hq, Hkv, wl.THETA_SLIDING, W, int(alias), kv_ring=C)])
    out = st.decode(0, to_dev(q), [to_dev(kr)], [None if vr is None else to_dev(vr)],
                    torch.from_numpy(kv).to("cuda:0"), Lmax)
    torch.cuda.synchronize()
    want = oracle.decode(q, kr, vr, kv, W, wl.THETA_SLIDING, ring=C)
    assert np.array_equal(want, oracle.decode(q, k, v, kv, W, wl.THETA_SLIDING))
    check(out.cpu().numpy(), want, "ring decode C%d T%d D%d" % (C, T, D))


@pytest.mark.parametrize("B,T,Hq,Hkv,D,W,C,alias,kv_len,Lmax", [
    (3, 1, 8, 2, 512, 0, 0, False, [1, 700, 4096], 4096),       # linear full layer, one token
    (3, 2, 8, 1, 256, 1024, 0, True, [2, 1500, 800], 1500),      # linear sliding K=V, two tokens
    (4, 1, 8, 1, 256, 1024, 1024, True, [5000, 1024, 1, 3000], 0),  # ring = window
    (2, 3, 8, 2, 512, 300, 310, False, [303, 9999], 0),           # ring, three tokens, separate values
])
def test_decode_with_fused_append(B, T, Hq, Hkv, D, W, C, alias, kv_len, Lmax):
    """The call writes the T tokens' keys/values into the cache and attends to
    them: its output equals the oracle's on the cache with those rows
    written, and afterwards the device cache holds exactly that cache."""
    import torch
    kind = wl.SLIDING if W > 0 else wl.FULL
    theta = wl.THETA_SLIDING if kind == wl.SLIDING else wl.THETA_FULL
    kv = np.asarray(kv_len, np.int32)
    rows = C if C else Lmax
    q = inputs.normal_bf16([730, T, 0], (B, T, Hq, D) if T > 1 else (B, Hq, D))
    kc = inputs.normal_bf16([730, T, 1], (B, Hkv, rows, D))  # stale contents everywhere
    vc = None if alias else inputs.normal_bf16([730, T, 2], (B, Hkv, rows, D))
    kn = inputs.normal_bf16([730, T, 3], (B, T, Hkv, D) if T > 1 else (B, Hkv, D))
    vn = None if alias else inputs.normal_bf16([730, T, 4], (B, T, Hkv, D) if T > 1 else (B, Hkv, D))
    # the host copy with the new rows written where the call must write them
    kw, vw = kc.copy(), None if vc is None else vc.copy()
    kn4 = kn.reshape(B, T, Hkv, D)
    vn4 = None if vn is None else vn.reshape(B, T, Hkv, D)
    for b in range(B):
        for t in range(T):
            r = (kv[b] - T + t) % C if C else kv[b] - T + t
            kw[b, :, r] = kn4[b, t]
            if vw is not None:
                vw[b, :, r] = vn4[b, t]
    st = Stack([wl.layer_desc(kind, D, Hq, Hkv, theta, W, int(alias), kv_ring=C)])
    kd, vd = to_dev(kc), None if vc is None else to_dev(vc)
    out = st.decode(0, to_dev(q), [kd], [vd], torch.from_numpy(kv).to("cuda:0"), int(kv.max()),
                    k_new=to_dev(kn), v_new=None if vn is None else to_dev(vn))
    torch.cuda.synchronize()
    want = oracle.decode(q, kw, vw, kv, W, theta, ring=C)
    check(out.cpu().numpy(), want, "append C%d T%d D%d" % (C, T, D))
    assert np.array_equal(kd.cpu().view(torch.int16).numpy().view(np.uint16), kw), "key cache after the append"
    if vd is not None:
        assert np.array_equal(vd.cpu().view(torch.int16).numpy().view(np.uint16), vw), "value cache after the append"


# ------------------------------------------------- bidirectional spans --
# Queries inside a span (image tokens) also see the span's later keys.

def _span_end(B, S, P0, spans_per_batch):
    """int32 [B, S]: for query s (position P0 + s) the last position of its
    span, or its own position; spans are inclusive (first, last) positions."""
    e = np.tile(np.arange(P0, P0 + S, dtype=np.int32), (B, 1))
    for b, spans in enumerate(spans_per_batch):
        for a, z in spans:
            e[b, a - P0:z - P0 + 1] = z
    return e


@pytest.mark.parametrize("B,S,P0,Hq,Hkv,D,W,alias,spans,override", [
    (2, 600, 0, 8, 2, 512, 0, False, [[(50, 305), (400, 420)], [(0, 31), (100, 100), (570, 599)]], None),
    (1, 300, 0, 8, 2, 512, 0, False, [[(10, 290)]], ("G4_PREFILL_SPLIT_PV", "0")),  # short segments, spans
    (2, 700, 0, 8, 1, 256, 0, True, [[(64, 319)], [(5, 6), (200, 455)]], ("G4_PREFILL_ROWS", "64")),
    (2, 700, 0, 8, 1, 256, 0, True, [[(64, 319)], [(5, 6), (200, 455)]], ("G4_PREFILL_ROWS", "128")),
    (2, 700, 0, 8, 1, 256, 0, True, [[(64, 319)], [(5, 6), (200, 455)]],
     [("G4_PREFILL_ROWS", "64"), ("G4_PREFILL_PRODUCER", "0")]),  # 64-row tiles, copies from the compute waves
    (1, 500, 0, 8, 1, 256, 64, True, [[(100, 300)]], None),          # a span longer than the window
    (1, 256, 900, 8, 2, 512, 0, False, [[(950, 1100)]], None),        # a chunk at a start position
    (1, 1024, 0, 8, 1, 256, 0, False, [[(300, 900)]], ("G4_PREFILL_ROWS", "128")),  # tiles cut into pieces
])
def test_bidirectional_spans(monkeypatch, B, S, P0, Hq, Hkv, D, W, alias, spans, override):
    import torch
    for name, value in ([override] if override and isinstance(override[0], str) else override or []):
        monkeypatch.setenv(name, value)
    Lmax = P0 + S
    kind = wl.SLIDING if W > 0 else wl.FULL
    theta = wl.THETA_SLIDING if kind == wl.SLIDING else wl.THETA_FULL
    q = inputs.normal_bf16([740, S, 0], (B, S, Hq, D))
    k = inputs.normal_bf16([740, S, 1], (B, Hkv, Lmax, D))
    v = None if alias else inputs.normal_bf16([740, S, 2], (B, Hkv, Lmax, D))
    se = _span_end(B, S, P0, spans)
    st = Stack([wl.layer_desc(kind, D, Hq, Hkv, theta, W, int(alias))])
    ws = torch.full((st.prefill_workspace_bytes(0, B, S, P0),), 0xFF, dtype=torch.uint8, device="cuda:0")
    out = st.prefill(0, to_dev(q), [to_dev(k)], [None if v is None else to_dev(v)], workspace=ws, start_pos=P0,
                     span_end=torch.from_numpy(se).to("cuda:0"))
    torch.cuda.synchronize()
    want = oracle.prefill(q, k, v, W, theta, start_pos=P0, span_end=se)
    assert not np.array_equal(want, oracle.prefill(q, k, v, W, theta, start_pos=P0))  # the spans matter
    check(out.cpu().numpy(), want, "spans B%d S%d P0=%d D%d W%d %s" % (B, S, P0, D, W, override))


# ----------------------------------------------------- 8-bit KV caches --
# A layer's cache may hold E4M3 bytes with one scale per tensor: element =
# code * k_scale (keys) or code * v_scale (values; k_scale when aliased).

@pytest.mark.parametrize("B,S,Hq,Hkv,D,W,alias,ks,vs,override", [
    (1, 640, 8, 2, 512, 0, False, 0.3, 1.7, ("G4_PREFILL_SPLIT_PV", "0")),
    (1, 640, 8, 2, 512, 0, False, 0.3, 1.7, ("G4_PREFILL_SPLIT_PV", "1")),
    (2, 333, 8, 1, 256, 48, True, 0.125, 1.0, ("G4_PREFILL_ROWS", "64")),
    (2, 333, 8, 1, 256, 48, True, 0.125, 1.0, ("G4_PREFILL_ROWS", "128")),
    (1, 1000, 8, 1, 256, 512, False, 0.07, 0.4, None),
])
def test_fp8_cache_prefill(monkeypatch, B, S, Hq, Hkv, D, W, alias, ks, vs, override):
    import torch
    if override:
        monkeypatch.setenv(*override)
    kind = wl.SLIDING if W > 0 else wl.FULL
    theta = wl.THETA_SLIDING if kind == wl.SLIDING else wl.THETA_FULL
    q = inputs.normal_bf16([750, S, 0], (B, S, Hq, D))
    k = inputs.normal_e4m3([750, S, 1], (B, Hkv, S + 3, D), ks)
    v = None if alias else inputs.normal_e4m3([750, S, 2], (B, Hkv, S + 3, D), vs)
    k[:, :, S:] = inputs.NAN_E4M3
    if v is not None:
        v[:, :, S:] = inputs.NAN_E4M3
    st = Stack([wl.layer_desc(kind, D, Hq, Hkv, theta, W, int(alias), kv_dtype=wl.KV_FP8, k_scale=ks, v_scale=vs)])
    out = st.prefill(0, to_dev(q), [to_dev(k)], [None if v is None else to_dev(v)])
    torch.cuda.synchronize()
    check(out.cpu().numpy(), oracle.prefill(q, k, v, W, theta, k_scale=ks, v_scale=vs),
          "fp8 prefill D%d W%d alias%d %s" % (D, W, alias, override))


@pytest.mark.parametrize("B,T,Hq,Hkv,D,W,alias,ring,kv_len,ks,vs", [
    (4, 1, 8, 2, 512, 0, False, 0, [1, 33, 1000, 4096], 0.3, 1.7),     # three 16-row stages beside the value tile
    (3, 1, 8, 2, 512, 0, True, 0, [700, 2, 3000], 0.5, 0.5),
    (4, 1, 8, 1, 256, 1024, True, 0, [1, 500, 1025, 3000], 0.125, 0.125),
    (3, 1, 16, 2, 256, 0, False, 0, [64, 65, 2000], 0.2, 3.0),
    (2, 3, 8, 2, 512, 0, False, 0, [5000, 3], 0.3, 1.7),               # multi-token
    (3, 1, 8, 1, 256, 1024, True, 1024, [5000, 1024, 17], 0.25, 0.25),  # ring
])
def test_fp8_cache_decode(B, T, Hq, Hkv, D, W, alias, ring, kv_len, ks, vs):
    import torch
    kind = wl.SLIDING if W > 0 else wl.FULL
    theta = wl.THETA_SLIDING if kind == wl.SLIDING else wl.THETA_FULL
    kv = np.asarray(kv_len, np.int32)
    rows = ring if ring else int(kv.max())
    q = inputs.normal_bf16([760, T, 0], (B, T, Hq, D) if T > 1 else (B, Hq, D))
    k = inputs.normal_e4m3([760, T, 1], (B, Hkv, rows, D), ks)
    v = None if alias else inputs.normal_e4m3([760, T, 2], (B, Hkv, rows, D), vs)
    if not ring:
        inputs.poison_beyond(k, kv)
        if v is not None:
            inputs.poison_beyond(v, kv)
    st = Stack([wl.layer_desc(kind, D, Hq, Hkv, theta, W, int(alias), kv_dtype=wl.KV_FP8, kv_ring=ring,
                              k_scale=ks, v_scale=vs)])
    out = st.decode(0, to_dev(q), [to_dev(k)], [None if v is None else to_dev(v)], torch.from_numpy(kv).to("cuda:0"),
                    int(kv.max()))
    torch.cuda.synchronize()
    check(out.cpu().numpy(), oracle.decode(q, k, v, kv, W, theta, ring=ring, k_scale=ks, v_scale=vs),
          "fp8 decode T%d D%d W%d alias%d ring%d" % (T, D, W, alias, ring))


@pytest.mark.parametrize("B,T,Hq,Hkv,D,W,alias,ring,kv_len,ks,vs", [
    (3, 1, 8, 2, 512, 0, False, 0, [1, 700, 2048], 0.3, 1.7),
    (4, 1, 8, 1, 256, 1024, True, 1024, [5000, 1024, 1, 3000], 0.03, 0.03),  # ring
    (2, 2, 8, 2, 512, 300, False, 301, [303, 9999], 0.25, 2.0),
])
def test_fp8_cache_decode_with_append(B, T, Hq, Hkv, D, W, alias, ring, kv_len, ks, vs):
    """New keys / values are stored as E4M3 codes of x / scale (the oracle's
    quantiser) and attended to as such; the cache bytes are checked too."""
    import torch
    kind = wl.SLIDING if W > 0 else wl.FULL
    theta = wl.THETA_SLIDING if kind == wl.SLIDING else wl.THETA_FULL
    kv = np.asarray(kv_len, np.int32)
    rows = ring if ring else int(kv.max())
    q = inputs.normal_bf16([770, T, 0], (B, T, Hq, D) if T > 1 else (B, Hq, D))
    kc = inputs.normal_e4m3([770, T, 1], (B, Hkv, rows, D), ks)
    vc = None if alias else inputs.normal_e4m3([770, T, 2], (B, Hkv, rows, D), vs)
    nshape = (B, T, Hkv, D) if T > 1 else (B, Hkv, D)
    kn = inputs.normal_bf16([770, T, 3], nshape)
    vn = None if alias else inputs.normal_bf16([770, T, 4], nshape)
    kw, vw = kc.copy(), None if vc is None else vc.copy()
    kn4, vn4 = kn.reshape(B, T, Hkv, D), None if vn is None else vn.reshape(B, T, Hkv, D)
    # two elements of every new key far beyond the E4M3 range at this scale: stored saturated at +-448
    kn4[..., 0] = inputs.bf16_bits_from_f32(np.array([1000.0], np.float32))[0]
    kn4[..., 1] = inputs.bf16_bits_from_f32(np.array([-1000.0], np.float32))[0]
    for b in range(B):
        for t in range(T):
            r = (kv[b] - T + t) % ring if ring else kv[b] - T + t
            kw[b, :, r] = oracle.fp8_e4m3_quantize(inputs.f32_from_bf16_bits(kn4[b, t]), ks)
            if vw is not None:
                vw[b, :, r] = oracle.fp8_e4m3_quantize(inputs.f32_from_bf16_bits(vn4[b, t]), vs)
    st = Stack([wl.layer_desc(kind, D, Hq, Hkv, theta, W, int(alias), kv_dtype=wl.KV_FP8, kv_ring=ring,
                              k_scale=ks, v_scale=vs)])
    kd, vd = to_dev(kc), None if vc is None else to_dev(vc)
    out = st.decode(0, to_dev(q), [kd], [vd], torch.from_numpy(kv).to("cuda:0"), int(kv.max()),
                    k_new=to_dev(kn), v_new=None if vn is None else to_dev(vn))
    torch.cuda.synchronize()
    assert np.array_equal(kd.cpu().numpy(), kw), "E4M3 key cache after the append"
    if vd is not None:
        assert np.array_equal(vd.cpu().numpy(), vw), "E4M3 value cache after the append"
    check(out.cpu().numpy(), oracle.decode(q, kw, vw, kv, W, theta, ring=ring, k_scale=ks, v_scale=vs),
          "fp8 append T%d D%d ring%d" % (T, D, ring))
