"""Host-side layer planning against the structural facts the pages print
(tests/golden/gemma4_e2b_layer_facts.txt cites the page and sections)."""
import os

from hybrid_sliding_global_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gemma4_e2b_layer_facts.txt")


def facts():
    out = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        out[key] = vals
    return out


def test_attention_pattern_matches_pages():
    f = facts()
    n = int(f["num_hidden_layers"][0])
    pat = wl.attention_pattern(n)
    assert [i for i, k in enumerate(pat) if k == wl.FULL] == [int(x) for x in f["full_attention_layers"]]
    assert pat[:10] == [int(x) for x in f["attention_pattern_prefix"]]


def test_stack_descriptors_match_pages():
    f = facts()
    stack = wl.gemma4_stack()
    assert len(stack) == int(f["num_hidden_layers"][0])
    for d in stack:
        if d["kind"] == wl.SLIDING:
            assert d["head_dim"] == int(f["head_dim"][0])
            assert d["rope_theta"] == float(f["rope_theta_sliding"][0])
            assert d["kv_alias"] == 1 and d["window"] > 0
        else:
            assert d["head_dim"] == int(f["global_head_dim"][0])
            assert d["rope_theta"] == float(f["rope_theta_full"][0])
            assert d["kv_alias"] == 0 and d["window"] == 0
    owners = [i for i, d in enumerate(stack) if d["kv_source_layer"] < 0]
    shared = [i for i, d in enumerate(stack) if d["kv_source_layer"] >= 0]
    assert len(owners) == int(f["unique_kv_caches"][0])
    assert len(shared) == int(f["num_kv_shared_layers"][0])


def test_shared_layers_read_an_owner_of_their_own_kind():
    stack = wl.gemma4_stack()
    for i, d in enumerate(stack):
        s = d["kv_source_layer"]
        if s < 0:
            continue
        src = stack[s]
        assert s < i and src["kv_source_layer"] < 0
        assert (src["kind"], src["head_dim"], src["num_kv_heads"], src["kv_alias"]) == \
            (d["kind"], d["head_dim"], d["num_kv_heads"], d["kv_alias"])


def test_algorithmic_work_of_the_workloads():
    assert wl.prefill_flops(64, 4, 256, 32) == 6356992
    assert wl.prefill_flops(4096, 8, 512, 0) == 137472507904
    total = sum(wl.prefill_flops(2048, d["num_q_heads"], d["head_dim"], d["window"]) for d in wl.gemma4_stack())
    assert total == 451147726848
    assert wl.decode_bytes([8192] * 64, 8, 2, 512, 0, False) == 2149056768
    assert wl.decode_bytes([8192] * 64, 8, 1, 256, 1024, True) == 34341120
