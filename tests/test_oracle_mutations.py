"""Plant one plausible mistake at a time in a scratch copy of the oracle (CPU
only) and check that the oracle pins reject every one of them."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = {
    "rope_sin_sign": ("y[k] = x0 * c - x1 * s;", "y[k] = x0 * c + x1 * s;"),
    "rope_dropped_term": ("y[k + half] = x1 * c + x0 * s;", "y[k + half] = x1 * c;"),
    "rope_exponent": ("double a = pos * pow(theta, -2.0", "double a = pos * pow(theta, -1.0"),
    "rope_interleaved_pairs": ("double x0 = x[k], x1 = x[k + half];", "double x0 = x[2 * k % D], x1 = x[(2 * k + 1) % D];"),
    "window_off_by_one": ("if (W > 0 && p - j >= W) return 0;", "if (W > 0 && p - j > W) return 0;"),
    "causal_off_by_one": ("if (j < 0 || j > p || j >= L) return 0;", "if (j < 0 || j > p + 1 || j >= L) return 0;"),
    "scale": ("scale = 1.0 / sqrt((double)D);", "scale = 1.0 / (double)D;"),
    "gqa_prefill_map": ("int64_t kvh = h / g;", "int64_t kvh = h % Hkv;"),
    "gqa_decode_map": ("int64_t b = r / Hq, h = r % Hq, kvh = h / g;", "int64_t b = r / Hq, h = r % Hq, kvh = h % Hkv;"),
    "decode_position": ("D, L - 1, L, W, theta", "D, L, L, W, theta"),
    "values_from_keys": ("const uint16_t* v = vbase + (size_t)j * (size_t)D;",
                         "const uint16_t* v = kbase + (size_t)j * (size_t)D;"),
    "softmax_no_max_shift": ("s[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);",
                             "s[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m) + 1e-3;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_reject_planted_mistake(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    old, new = MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert src.count(old) >= 1, "mutation anchor missing: " + old
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", str(lib), str(mutated), "-lm"],
                   check=True)
    env = dict(os.environ, HSG_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "planted mistake %s survived every pin" % name
    assert "failed" in r.stdout
