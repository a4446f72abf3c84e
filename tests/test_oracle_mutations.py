"""The pins catch plausible mistakes in the oracle (CPU only).

Each case plants one mistake in a copy of oracle/attn_oracle.c (a dropped
scale, an off-by-one causal mask, a missing normalisation, a wrong sign or a
transposed index), builds the copy with the oracle's own compiler flags, and
runs tests/test_oracle_pins.py against it in a subprocess: at least one pin
must fail.  The unmodified copy must pass all of them, which shows that the
harness itself runs the pins.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attn_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, text in the source, replacement): each text occurs exactly once
MUTATIONS = [
    ("causal mask excludes the diagonal", "if (ks->causal && j > i) return 0;", "if (ks->causal && j >= i) return 0;"),
    ("scale dropped from S (naive forward)",
     "S[i * N + j] = allowed(&ks, i, j) ? scale * dot(Q + i * d, K + j * d, d) : -INFINITY;",
     "S[i * N + j] = allowed(&ks, i, j) ? dot(Q + i * d, K + j * d, d) : -INFINITY;"),
    ("softmax not normalised",
     "P[i * N + j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m) / l;",
     "P[i * N + j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);"),
    ("max added instead of subtracted",
     "for (long j = 0; j < N; ++j) P[i * N + j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m) / l;",
     "for (long j = 0; j < N; ++j) P[i * N + j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] + m) / l;"),
    ("LSE without the logarithm", "        LSE[i] = m + log(l);\n    }\n\n    /* O = P V */",
     "        LSE[i] = m + l;\n    }\n\n    /* O = P V */"),
    ("D_i summed without P", "            acc += P[i * N + j] * dp;", "            acc += dp;"),
    ("dS with the wrong sign of D", "dS[i * N + j] = P[i * N + j] * (dS[i * N + j] - D[i]);",
     "dS[i * N + j] = P[i * N + j] * (dS[i * N + j] + D[i]);"),
    ("dQ built from Q instead of K", "for (long k = 0; k < d; ++k) g[k] += s * K[j * d + k];",
     "for (long k = 0; k < d; ++k) g[k] += s * Q[j * d + k];"),
    ("dQ without the scale", "            for (long k = 0; k < d; ++k) g[k] += s * K[j * d + k];\n        }\n"
     "        for (long k = 0; k < d; ++k) g[k] *= scale;",
     "            for (long k = 0; k < d; ++k) g[k] += s * K[j * d + k];\n        }\n"),
    ("dV from the key's own dO row (P not transposed)",
     "            double s = dS[i * N + j], p = P[i * N + j];\n            for (long k = 0; k < d; ++k) {\n"
     "                gk[k] += s * Q[i * d + k];\n                gv[k] += p * dO[i * d + k];",
     "            double s = dS[i * N + j], p = P[i * N + j];\n            for (long k = 0; k < d; ++k) {\n"
     "                gk[k] += s * Q[i * d + k];\n                gv[k] += p * dO[j * d + k];"),
    ("online rescale factor inverted", "exp(m[r] - mnew);", "exp(mnew - m[r]);"),
    ("online forward without the final division", "l[r] > 0.0 ? acc[r * d + k] / l[r] : 0.0;",
     "l[r] > 0.0 ? acc[r * d + k] : 0.0;"),
    ("block mask indexed transposed", "ks->bmask[(i / ks->block) * ks->nblk + j / ks->block]",
     "ks->bmask[(j / ks->block) * ks->nblk + i / ks->block]"),
    ("block mask ignored", "return !ks->bmask || ks->bmask[", "return 1 || ks->bmask["),
    ("online forward: empty rows divided by zero", "l[r] > 0.0 ? acc[r * d + k] / l[r] : 0.0;",
     "acc[r * d + k] / l[r];"),
    ("rows: D_i left out of dS", "double D = dot(g, o, d);", "double D = 0.0;"),
    ("cols: P normalised by the key's statistic", "K + j * d, d) - LSE[i]);", "K + j * d, d) - LSE[j]);"),
]


def _build(tmp_path, text, name):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    lib = tmp_path / f"{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(lib), str(src), "-lm"],
                   check=True, capture_output=True)
    return str(lib)


def _run_pins(lib):
    env = dict(os.environ, ATTN_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout[-2000:]


def test_unmodified_copy_passes_the_pins(tmp_path):
    with open(SRC) as f:
        text = f.read()
    rc, out = _run_pins(_build(tmp_path, text, "control"))
    assert rc == 0, out


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(tmp_path, name, old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation text must occur once: {name}"
    rc, out = _run_pins(_build(tmp_path, text.replace(old, new), "mutant"))
    assert rc != 0, f"no pin caught the mutation '{name}':\n{out}"
