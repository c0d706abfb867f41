"""The Python binding's marshalling, on the CPU: temporaries a call creates
(the output when none is given, the workspace) are allocated for the stream
the kernels are launched on, and that stream is the one passed to the C ABI."""
import contextlib
import ctypes

import pytest

from hybrid_sliding_global_amd import _lib as L


class _FakeStream:
    def __init__(self, handle):
        self.cuda_stream = handle


class _FakeTensor:
    def __init__(self, shape, dtype, stream=None):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.stream = stream
        self.device = "cuda:0"

    def data_ptr(self):
        return 0x1000

    def dim(self):
        return len(self.shape)

    def numel(self):
        n = 1
        for x in self.shape:
            n *= x
        return n

    def element_size(self):
        return 1


class _FakeLib:
    """Stands in for libgemma4_attn.so: sizes queries answer 1 KiB, compute
    calls record the stream handle they receive."""

    def __init__(self):
        self.streams = []

    def gemma4_validate_layers(self, arr, n):
        return 0

    def gemma4_prefill_workspace_bytes(self, arr, n, layer, b, s, out):
        ctypes.cast(out, ctypes.POINTER(ctypes.c_size_t))[0] = 1024
        return 0

    gemma4_decode_workspace_bytes = gemma4_prefill_workspace_bytes

    def gemma4_attn_prefill(self, *args):
        self.streams.append(args[-1])
        return 0

    def gemma4_attn_decode(self, *args):
        self.streams.append(args[-1])
        return 0


@pytest.fixture
def fake(monkeypatch):
    import torch
    current = {"s": _FakeStream(1)}  # the "current" stream
    allocs = []

    @contextlib.contextmanager
    def stream_ctx(s):
        prev = current["s"]
        current["s"] = s
        try:
            yield
        finally:
            current["s"] = prev

    def empty(shape, dtype=None, device=None):
        t = _FakeTensor(shape, dtype, current["s"])
        allocs.append(t)
        return t

    lib = _FakeLib()
    monkeypatch.setattr(torch.cuda, "stream", stream_ctx)
    monkeypatch.setattr(torch.cuda, "current_stream", lambda: current["s"])
    monkeypatch.setattr(torch, "empty", empty)
    monkeypatch.setattr(L, "_check_tensor", lambda *a, **k: None)
    monkeypatch.setattr(L, "load", lambda: lib)
    return lib, allocs, current


@pytest.mark.parametrize("call", ["prefill", "decode"])
@pytest.mark.parametrize("explicit", [False, True])
def test_temporaries_follow_the_launch_stream(fake, call, explicit):
    import torch
    from hybrid_sliding_global_amd import workloads as wl
    lib, allocs, current = fake
    st = L.Stack([wl.layer_desc(wl.FULL, 512, 8, 2, 1e6, 0, 0)])
    side = _FakeStream(7)
    k = _FakeTensor((1, 2, 64, 512), torch.bfloat16)
    if call == "prefill":
        q = _FakeTensor((1, 64, 8, 512), torch.bfloat16)
        st.prefill(0, q, [k], [k], stream=side if explicit else None)
    else:
        q = _FakeTensor((1, 8, 512), torch.bfloat16)
        kv = _FakeTensor((1,), torch.int32)
        st.decode(0, q, [k], [k], kv, 64, stream=side if explicit else None)
    launch = side if explicit else current["s"]
    assert lib.streams == [launch.cuda_stream]
    assert len(allocs) == 2  # the output and the workspace
    assert all(t.stream is launch for t in allocs)


def test_images_ready_needs_the_workspace_that_holds_them(fake):
    """Reusing a source layer's operand images only makes sense with the
    workspace they were written to: the binding refuses to allocate one."""
    import torch
    from hybrid_sliding_global_amd import workloads as wl
    lib, allocs, current = fake
    st = L.Stack([wl.layer_desc(wl.FULL, 512, 8, 2, 1e6, 0, 0)])
    k = _FakeTensor((1, 2, 64, 512), torch.bfloat16)
    q = _FakeTensor((1, 64, 8, 512), torch.bfloat16)
    with pytest.raises(ValueError):
        st.prefill(0, q, [k], [k], images_ready=True)
    assert lib.streams == []
