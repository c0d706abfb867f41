"""Plant one plausible mistake at a time in a scratch copy of the oracle (CPU
only) and check that the oracle pins reject every one of them."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = {
    # name: (anchor, replacement, occurrence to replace; None = every one)
    "rope_sin_sign": ("y[k] = x0 * c - x1 * s;", "y[k] = x0 * c + x1 * s;", None),
    "rope_dropped_term": ("y[k + half] = x1 * c + x0 * s;", "y[k + half] = x1 * c;", None),
    "rope_exponent": ("out[k] = pow(theta, -2.0", "out[k] = pow(theta, -1.0", None),
    "rope_interleaved_pairs": ("double x0 = x[k], x1 = x[k + half];",
                               "double x0 = x[2 * k % D], x1 = x[(2 * k + 1) % D];", None),
    "key_position": ("orc_rope_freq(tmp, D, f, (double)j, krot + (size_t)j * D);\n    }\n    free(tmp);",
                     "orc_rope_freq(tmp, D, f, (double)(j + 1), krot + (size_t)j * D);\n    }\n    free(tmp);",
                     None),
    "window_off_by_one": ("if (W > 0 && p - j >= W) return 0;", "if (W > 0 && p - j > W) return 0;", None),
    "causal_off_by_one": ("if (j < 0 || j > e || j >= L) return 0;", "if (j < 0 || j > e + 1 || j >= L) return 0;",
                          None),
    "scale": ("scale = 1.0 / sqrt((double)D);", "scale = 1.0 / (double)D;", None),
    "gqa_prefill_map": ("if (rb != b || h / g != kvh) continue;", "if (rb != b || h % Hkv != kvh) continue;", 0),
    "gqa_decode_map": ("if (rb != b || h / g != kvh) continue;", "if (rb != b || h % Hkv != kvh) continue;", 1),
    "decode_position": ("qpos[nq] = L - T + t;", "qpos[nq] = L - T + t + 1;", None),
    "value_row_index": ("orc_row(vr, j, D, v);", "orc_row(vr, j / 2, D, v);", None),
    "values_from_rotated_keys": ("for (int32_t d = 0; d < D; ++d) out[d] += w * v[d];",
                                 "for (int32_t d = 0; d < D; ++d) out[d] += w * krot[(size_t)j * D + d];", None),
    "fp8_exponent_bias": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);", None),
    "fp8_subnormal_scale": ("v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);", None),
    "fp8_alias_value_scale": ("const double vs = v ? v_scale : k_scale;", "const double vs = v_scale;", None),
    "ring_row": ("const int64_t r = c->ring > 0 ? j % c->ring : j;",
                 "const int64_t r = c->ring > 0 ? (j + 1) % c->ring : j;", None),
    "chunk_query_position": ("qpos[nq] = start_pos + s;", "qpos[nq] = s;", None),
    "span_ignored": ("if (j < 0 || j > e || j >= L) return 0;", "if (j < 0 || j > p || j >= L) return 0;", None),
    "verify_all_at_last_position": ("qpos[nq] = L - T + t;", "qpos[nq] = L - 1;", None),
    "fp8_quantize_ties_to_odd": ("if (dc < db || (dc == db && (c & 1) == 0)) best = c;",
                                 "if (dc < db || (dc == db && (c & 1) == 1)) best = c;", None),
    "softmax_no_max_shift": ("s[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);",
                             "s[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m) + 1e-3;", None),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_reject_planted_mistake(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    old, new, which = MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    n = src.count(old)
    assert n >= 1, "mutation anchor missing: " + old
    if which is None:
        out = src.replace(old, new)
    else:
        assert which < n
        parts = src.split(old)
        out = "".join(p + (new if i == which else old) for i, p in enumerate(parts[:-1])) + parts[-1]
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(out)
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", str(lib), str(mutated), "-lm"],
                   check=True)
    env = dict(os.environ, HSG_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "planted mistake %s survived every pin" % name
    assert "failed" in r.stdout
