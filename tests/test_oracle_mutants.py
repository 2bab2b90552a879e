"""The pins must bite: plant one plausible mistake at a time in a copy of the
oracle (on the CPU), build it, and check that the pin suite fails on it."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "diagonal-excluded": ("&ks, pos + 1, Hkv", "&ks, pos, Hkv"),
    "top-left-alignment": ("(int64_t)k_lens[s] - q_lens[s] + i", "i"),
    "gqa-modulo-heads": ("Hkv, h / g, d", "Hkv, h % Hkv, d"),
    "dropped-last-dim": ("        for (int32_t e = 0; e < d; ++e)\n            dot +=",
                         "        for (int32_t e = 0; e < d - 1; ++e)\n            dot +="),
    "softmax-sign": ("exp(x[j] - m)", "exp(m - x[j])"),
    "scale-dropped": ("x[j] = scale * dot;", "x[j] = dot;"),
    "no-normalise": ("        o[e] /= den;", "        o[e] /= 1.0;"),
    "slot-offset-index": ("return (int64_t)table[lb] * bs + p % bs;",
                          "return (int64_t)table[lb] * bs + p / bs;"),
    "slot-block-unscaled": ("return (int64_t)table[lb] * bs + p % bs;",
                            "return (int64_t)table[lb] + p % bs;"),
    "store-half-row": ("(size_t)row_bytes);", "(size_t)row_bytes / 2);"),
    "store-skips-slot-zero": ("if (s < 0)\n            continue;", "if (s <= 0)\n            continue;"),
    "rope-sign": ("v[ia] = a * c - b * sn;", "v[ia] = a * c + b * sn;"),
    "rope-exponent": ("pow(base, -2.0 * j / rot_dim)", "pow(base, -1.0 * j / rot_dim)"),
    "rope-cos-sin-swapped": ("const double c = cos(theta), sn = sin(theta);",
                             "const double c = sin(theta), sn = cos(theta);"),
    "rope-position-offset": ("(double)pos[t] * pow", "(double)(pos[t] + 1) * pow"),
    "rope-half-pairing": ("style == 0 ? j + half : 2 * j + 1", "style == 0 ? half - 1 - j + half : 2 * j + 1"),
    "rope-interleaved-pairing": ("style == 0 ? j : 2 * j;", "style == 0 ? j : j;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, name
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           str(mutated), "-o", str(lib), "-lm"])
    env = dict(os.environ, PKV_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
