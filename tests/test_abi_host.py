"""Host-side checks of the C ABI (include/gemma4_attn.h) -- no GPU needed.

The library must load, export every function the header declares, and reject
bad descriptors / arguments with the documented status codes before it
touches the HIP runtime.
"""
import ctypes
import os
import re

import pytest

from hybrid_sliding_global_amd import _lib as L
from hybrid_sliding_global_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemma4_attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        import hybrid_sliding_global_amd.build as b
        b.build()
    return L.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemma4_\w+)\s*\(", text)))


def test_header_symbols_exported(lib):
    names = header_functions()
    assert names, "no functions parsed from the header"
    assert set(names) == set(L.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


CITE_TAGS = ("[FR]", "[HF]", "[LD]", "[SG]")
UNCITED_OK = ("no passage of the pages defines", "Library plumbing", "is cited at")


def _decl_comments():
    """(declaration, the comment block right above it) for every function the header declares."""
    text = open(HEADER).read()
    out = []
    for m in re.finditer(r"/\*((?:(?!\*/).)*)\*/\s*\n((?:[^;/])*?\b(gemma4_\w+)\s*\([^;]*;)", text, flags=re.S):
        out.append((m.group(3), re.sub(r"\s*\n\s*\*\s*", " ", m.group(1))))
    return out


def test_every_header_declaration_cites_its_passage():
    decls = dict(_decl_comments())
    assert set(decls) == set(header_functions())
    for name, comment in decls.items():
        assert any(t in comment for t in CITE_TAGS + UNCITED_OK), "%s has no citation" % name
    # every descriptor field names the passage that defines it
    text = open(HEADER).read()
    block = text[text.index("Per-layer descriptor."):text.index("typedef struct")]
    for field in ("kind", "head_dim", "num_q_heads", "num_kv_heads", "window", "kv_alias", "kv_source_layer",
                  "scale", "rope_theta"):
        m = re.search(r"\n \*   %s\s+(.*?)(?=\n \*   \w+\s{2,}|\n \*/)" % field, block, flags=re.S)
        assert m, field
        assert any(t in m.group(1) for t in CITE_TAGS), "field %s has no citation" % field


def test_abi_version_and_status_strings(lib):
    assert L.abi_version() == 3
    for code, name in [(0, "G4_OK"), (-1, "G4_ERR_INVALID_ARG"), (-2, "G4_ERR_UNSUPPORTED"),
                       (-3, "G4_ERR_BAD_SOURCE"), (-4, "G4_ERR_WORKSPACE"), (-5, "G4_ERR_HIP")]:
        assert L.status_string(code) == name


def _c_layout(struct, fields):
    """sizeof and offsetof of a header struct, from a C program compiled against include/gemma4_attn.h."""
    import shutil
    import subprocess
    import tempfile
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    prog = "#include <stdio.h>\n#include <stddef.h>\n#include \"gemma4_attn.h\"\nint main(void){printf(\"%%zu\", sizeof(%s));" % struct
    prog += "".join('printf(" %%zu", offsetof(%s, %s));' % (struct, f) for f in fields) + "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "l.c"), os.path.join(d, "l")
        open(src, "w").write(prog)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), src, "-o", exe], check=True)
        return [int(x) for x in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]


@pytest.mark.parametrize("struct,cls", [("g4_layer_desc", "LayerDesc"), ("g4_prefill_opts", "PrefillOpts"),
                                        ("g4_decode_opts", "DecodeOpts")])
def test_struct_layouts_match_header(lib, struct, cls):
    c = getattr(L, cls)
    fields = [f[0] for f in c._fields_]
    got = _c_layout(struct, fields)
    assert got == [ctypes.sizeof(c)] + [getattr(c, f).offset for f in fields]


def test_gemma4_stack_validates(lib):
    assert L.validate_layers(wl.gemma4_stack()) == 0


def _one(**kw):
    d = wl.layer_desc(wl.SLIDING, 256, 8, 1, 1e4, 512, 1)
    d.update(kw)
    return d


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=128), L.G4_ERR_UNSUPPORTED),
    (dict(head_dim=384), L.G4_ERR_UNSUPPORTED),
    (dict(num_q_heads=6, num_kv_heads=4), L.G4_ERR_UNSUPPORTED),
    (dict(num_kv_heads=0), L.G4_ERR_INVALID_ARG),
    (dict(window=0), L.G4_ERR_INVALID_ARG),
    (dict(window=-3), L.G4_ERR_INVALID_ARG),
    (dict(kind=wl.FULL, head_dim=512, window=512), L.G4_ERR_INVALID_ARG),
    (dict(kind=7), L.G4_ERR_UNSUPPORTED),
    (dict(rope_theta=0.0), L.G4_ERR_INVALID_ARG),
    (dict(rope_theta=float("nan")), L.G4_ERR_INVALID_ARG),
    (dict(scale=-1.0), L.G4_ERR_INVALID_ARG),
    (dict(kv_alias=2), L.G4_ERR_INVALID_ARG),
])
def test_bad_descriptor_rejected(lib, kw, code):
    assert L.validate_layers([_one(**kw)]) == code
    assert L.last_error() != ""


def test_bad_sources_rejected(lib):
    full = wl.layer_desc(wl.FULL, 512, 8, 2, 1e6, 0, 0)
    sl = _one()
    # source must be earlier
    assert L.validate_layers([_one(kv_source_layer=0)]) == L.G4_ERR_BAD_SOURCE
    assert L.validate_layers([sl, _one(kv_source_layer=1)]) == L.G4_ERR_BAD_SOURCE
    assert L.validate_layers([sl, _one(kv_source_layer=5)]) == L.G4_ERR_BAD_SOURCE
    # source must own its cache
    assert L.validate_layers([sl, _one(kv_source_layer=0), _one(kv_source_layer=1)]) == L.G4_ERR_BAD_SOURCE
    # head dim / kv heads / alias must match
    assert L.validate_layers([full, _one(kv_source_layer=0)]) == L.G4_ERR_BAD_SOURCE
    assert L.validate_layers([sl, _one(num_q_heads=4, num_kv_heads=2, kv_source_layer=0)]) == L.G4_ERR_BAD_SOURCE
    assert L.validate_layers([sl, _one(kv_alias=0, kv_source_layer=0)]) == L.G4_ERR_BAD_SOURCE
    # matching source accepted (query heads may differ)
    assert L.validate_layers([sl, _one(num_q_heads=4, kv_source_layer=0)]) == 0


def test_kv_bytes_and_sharing(lib):
    stack = wl.gemma4_stack()
    total_k = total_v = 0
    for i in range(len(stack)):
        k, v = L.kv_bytes(stack, i, 1, 2048)
        total_k += k
        total_v += v
        if stack[i]["kv_source_layer"] >= 0:
            assert k == v == 0
    # 12 aliased sliding owners (one 1 MiB buffer each) + 3 full owners (K and V, 4 MiB each)
    assert total_k + total_v == 12 * 2048 * 256 * 2 + 3 * 2 * (2 * 2048 * 512 * 2) == 37748736


def _ws_parts(B, S, Hq, Hkv, D, rows):
    """Lower bounds of the prefill workspace: both operand images (rotated
    keys and values, 32-key tiles, bf16) and one arrival counter per query
    tile of ``rows`` rows, each part rounded up to 256 bytes; and the size of
    one partial-result slot (a 32 x D fp32 block per row group plus the
    running maximum and sum of every lane)."""
    rnd = lambda x: -(-x // 256) * 256  # noqa: E731
    img = rnd(B * Hkv * (-(-S // 32)) * 32 * D * 2)
    nqt = -(-(S * (Hq // Hkv)) // rows)
    base = rnd(2 * img + B * Hkv * nqt * 4)
    waves = 8 if D == 512 else 4
    return base, 32 * D * 16 + waves * 64 * 2 * 4


def _split_slots(B, S, Hq, Hkv, D, W):
    """Number of partial-result slots the workspace holds beyond images and
    counters, for whichever query-tile height the library picked (None if no
    height explains the size)."""
    stack = [wl.layer_desc(wl.SLIDING if W else wl.FULL, D, Hq, Hkv, 1e4, W, 0)]
    ws = L.prefill_workspace_bytes(stack, 0, B, S)
    for rows in ((128, 64) if D == 256 else (128,)):
        base, slot = _ws_parts(B, S, Hq, Hkv, D, rows)
        if ws >= base and (ws - base) % slot == 0:
            return (ws - base) // slot
    return None


def test_workspace_sizes(lib):
    """Properties of the prefill workspace size: it holds the operand images
    and counters, plus whole partial-result slots only when query tiles are
    cut into pieces (two slots per work-group, each work-group covering up to
    two query tiles)."""
    # one key tile: nothing can be split, so there are no slots
    for D, W in ((512, 0), (256, 0), (256, 16)):
        for S in (1, 17, 32):
            assert _split_slots(1, S, 8, 2, D, W) == 0
    # the 4096-token full layer is cut into pieces: slots present
    n = _split_slots(1, 4096, 8, 2, 512, 0)
    assert n is not None and n > 0 and n % 2 == 0
    # windowed 2048-token sliding layer (128 query tiles of 128 rows): whole tiles per work-group
    assert _split_slots(1, 2048, 8, 1, 256, 512) == 0
    # every shape is explained by images + counters + whole slots
    for (B, S, Hq, Hkv, D, W) in ((2, 333, 8, 1, 256, 48), (1, 1024, 8, 1, 256, 0), (1, 640, 8, 2, 512, 0),
                                  (3, 257, 16, 2, 256, 100), (1, 2048, 8, 2, 512, 0)):
        assert _split_slots(B, S, Hq, Hkv, D, W) is not None, (B, S, Hq, Hkv, D, W)
    stack = wl.gemma4_stack()
    assert L.prefill_workspace_bytes(stack, 0, 1, 2048) >= 2 * 1 * 1 * 2048 * 256 * 2
    w = L.decode_workspace_bytes(stack, 4, 64, 8192)
    # one fp32 partial (head_dim values and a log-sum-exp) per query head for
    # every stream plus every piece of the split: (B*Hkv + 512) * g * (D + 1) * 4
    assert w == (64 * 2 + 512) * 4 * (512 + 1) * 4
    # T query tokens: T*g columns per (batch, kv head), in groups of 16
    st = L.Stack(stack)
    assert st.decode_workspace_bytes(4, 64, 8192, 3) == (64 * 2 + 512) * 12 * (512 + 1) * 4
    assert st.decode_workspace_bytes(4, 64, 8192, 5) == (64 * 2 * 2 + 512) * 16 * (512 + 1) * 4
    # a chunk at start position P0 images keys 0 .. P0 + S - 1
    assert st.prefill_workspace_bytes(0, 1, 64, 1000) >= 2 * (1064 + 31) // 32 * 32 * 256 * 2
    with pytest.raises(L.Gemma4Error):
        L.prefill_workspace_bytes(stack, 4, 0, 2048)


def test_compute_calls_reject_bad_arguments_without_gpu(lib):
    """Argument errors are reported before anything is enqueued (no HIP call)."""
    stack = wl.gemma4_stack()
    arr = L.descs(stack)
    n = len(stack)
    null_tab = (ctypes.c_void_p * n)()
    fake = ctypes.c_void_p(0x1000)
    # NULL q / out
    assert lib.gemma4_attn_prefill(arr, n, 0, None, null_tab, null_tab, 1, 16, 16, None, fake, 1 << 20, None) \
        == L.G4_ERR_INVALID_ARG
    # seq_len > max_len
    assert lib.gemma4_attn_prefill(arr, n, 0, fake, null_tab, null_tab, 1, 32, 16, fake, fake, 1 << 20, None) \
        == L.G4_ERR_INVALID_ARG
    # missing cache pointer of the source layer (layer 20 reads layer 13)
    assert lib.gemma4_attn_prefill(arr, n, 20, fake, null_tab, null_tab, 1, 16, 16, fake, fake, 1 << 20, None) \
        == L.G4_ERR_INVALID_ARG
    assert "k_cache[13]" in L.last_error()
    # workspace too small
    tab = (ctypes.c_void_p * n)(*([0x2000] * n))
    assert lib.gemma4_attn_prefill(arr, n, 4, fake, tab, tab, 1, 2048, 2048, fake, fake, 16, None) \
        == L.G4_ERR_WORKSPACE
    assert lib.gemma4_attn_prefill(arr, n, 4, fake, tab, tab, 1, 2048, 2048, fake, None, 1 << 30, None) \
        == L.G4_ERR_WORKSPACE
    # non-aliased layer without a value buffer
    assert lib.gemma4_attn_prefill(arr, n, 4, fake, tab, None, 1, 16, 16, fake, fake, 1 << 20, None) \
        == L.G4_ERR_INVALID_ARG
    # decode: max_kv_len > max_len, NULL kv_len, too many query heads per kv head
    assert lib.gemma4_attn_decode(arr, n, 4, fake, tab, tab, fake, 4, 100, 200, fake, fake, 1 << 20, None) \
        == L.G4_ERR_INVALID_ARG
    assert lib.gemma4_attn_decode(arr, n, 4, fake, tab, tab, None, 4, 100, 100, fake, fake, 1 << 20, None) \
        == L.G4_ERR_INVALID_ARG
    # 32 query heads per kv head: two groups of 16 MFMA columns, accepted (here stopped by the workspace)
    wide = L.descs([wl.layer_desc(wl.FULL, 512, 32, 1, 1e6, 0, 0)])
    assert lib.gemma4_attn_decode(wide, 1, 0, fake, tab, tab, fake, 4, 100, 100, fake, fake, 8, None) \
        == L.G4_ERR_WORKSPACE
    # ext calls: start_pos + seq_len beyond the cache, n_tokens above max_kv_len, reserved options set
    po = L.PrefillOpts(start_pos=10)
    assert lib.gemma4_attn_prefill_ext(arr, n, 4, fake, tab, tab, 1, 16, 20, ctypes.byref(po), fake, fake, 1 << 20,
                                       None) == L.G4_ERR_INVALID_ARG
    po = L.PrefillOpts(start_pos=-1)
    assert lib.gemma4_attn_prefill_ext(arr, n, 4, fake, tab, tab, 1, 16, 20, ctypes.byref(po), fake, fake, 1 << 20,
                                       None) == L.G4_ERR_INVALID_ARG
    do = L.DecodeOpts(5, None, None)
    assert lib.gemma4_attn_decode_ext(arr, n, 4, fake, tab, tab, fake, 4, 100, 4, ctypes.byref(do), fake, fake,
                                      1 << 30, None) == L.G4_ERR_INVALID_ARG
    do = L.DecodeOpts(0, None, None)
    assert lib.gemma4_attn_decode_ext(arr, n, 4, fake, tab, tab, fake, 4, 100, 100, ctypes.byref(do), fake, fake,
                                      1 << 30, None) == L.G4_ERR_INVALID_ARG
    assert lib.gemma4_attn_decode(arr, n, 4, fake, tab, tab, fake, 64, 8192, 8192, fake, fake, 8, None) \
        == L.G4_ERR_WORKSPACE
    # layer index out of range
    assert lib.gemma4_attn_prefill(arr, n, n, fake, tab, tab, 1, 16, 16, fake, fake, 1 << 20, None) \
        == L.G4_ERR_INVALID_ARG


def test_noalloc_decode_rejects_oversize_calls_without_gpu(lib):
    """The scratch-size check of the no-allocation decode runs before anything
    touches the GPU."""
    d = L.descs([wl.layer_desc(wl.FULL, 512, 16, 1, 1e6, 0, 0)])
    fake = ctypes.c_void_p(0x1000)
    tab = (ctypes.c_void_p * 1)(0x2000)
    need = L.decode_workspace_bytes([wl.layer_desc(wl.FULL, 512, 16, 1, 1e6, 0, 0)], 0, 600, 64)
    assert need > L.STATIC_SCRATCH_BYTES
    assert lib.gemma4_attn_decode_noalloc(d, 1, 0, fake, tab, tab, fake, 600, 64, 64, fake, None) \
        == L.G4_ERR_WORKSPACE
    assert "static scratch" in L.last_error()
