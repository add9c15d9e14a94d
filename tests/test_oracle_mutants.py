"""Plant plausible mistakes in copies of the oracle's C source and check that
the pins reject every one of them (CPU only; the real oracle is untouched)."""
import json
import os
import subprocess
import sys

import pytest

import pins
from oracle import oracle as O

SRC = os.path.join(os.path.dirname(O.__file__), "oracle.c")

# (name, original text, mistaken text): each a one-token slip
MUTANTS = [
    ("beam keys dropped", "const int N = L + T;", "const int N = L;"),
    ("context keys dropped", "const int N = L + T;", "const int N = T + 0 * L;"),
    ("wrong GQA head map", "const int g = h / (J->Hq / J->Hkv);", "const int g = h % J->Hkv;"),
    ("scale missing", "z[j] = J->scale * dot;", "z[j] = dot;"),
    ("scale squared", "z[j] = J->scale * dot;", "z[j] = J->scale * J->scale * dot;"),
    ("lse without max", "*lse = M + log(Z);", "*lse = log(Z);"),
    ("lse base 2", "*lse = M + log(Z);", "*lse = M + log2(Z);"),
    ("no normalisation", "out[d] /= Z;", "out[d] /= 1.0;"),
    ("max not subtracted", "double p = exp(z[j] - M);", "double p = exp(z[j]);"),
    ("sign of max", "double p = exp(z[j] - M);", "double p = exp(M - z[j]);"),
    ("beam V read from beam K", "v = kv_row(J->beam_v,", "v = kv_row(J->beam_k,"),
    ("ctx V read from ctx K", "v = kv_row(J->ctx_v,", "v = kv_row(J->ctx_k,"),
    ("path step off by one", "+ (j - L)], g);\n        double dot",
     "+ (j - L + 1) % J->T_cap], g);\n        double dot"),
    ("context off by one", "if (j < L)\n            k =", "if (j <= L)\n            k ="),
    ("request 0 for every row", "return buf + (((int64_t)b * cap + t) * Hkv + g) * D;",
     "return buf + (((int64_t)0 * b * cap + t) * Hkv + g) * D;"),
    ("transposed KV layout", "return buf + (((int64_t)b * cap + t) * Hkv + g) * D;",
     "return buf + (((int64_t)b * Hkv + g) * cap + t) * D;"),
    ("query head g instead of h", "const uint16_t *qv = J->q + ((int64_t)r * J->Hq + h) * D;",
     "const uint16_t *qv = J->q + ((int64_t)r * J->Hq + g) * D;"),
    ("path row of wrong beam", "J->beam_path[(int64_t)r * J->T_cap + (j - L)], g);\n        double",
     "J->beam_path[(int64_t)(r ^ 1) * J->T_cap + (j - L)], g);\n        double"),
    ("max over first key only", "if (z[j] > M)\n            M = z[j];",
     "if (j == 0)\n            M = z[j];"),
]


RUNNER = """
import json, sys
sys.path[:0] = {paths!r}
import pins
from oracle import oracle as O
print(json.dumps(pins.battery(O.from_library({so!r}))))
"""


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


def test_real_oracle_passes_battery():
    assert pins.battery(O.decode_attn) == []


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_rejected(workdir, name, orig, bad):
    src = open(SRC).read()
    assert orig in src, f"mutation anchor not found: {orig!r}"
    mutated = src.replace(orig, bad, 1)
    tag = "".join(ch if ch.isalnum() else "_" for ch in name)
    c_path = os.path.join(workdir, f"{tag}.c")
    so_path = os.path.join(workdir, f"{tag}.so")
    with open(c_path, "w") as f:
        f.write(mutated)
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", c_path, "-o",
                           so_path, "-lpthread", "-lm"])
    # a separate process: a mutant may also read out of bounds and crash
    paths = [os.path.dirname(os.path.abspath(__file__)),
             os.path.dirname(os.path.dirname(os.path.abspath(__file__)))]
    res = subprocess.run([sys.executable, "-c", RUNNER.format(paths=paths, so=so_path)],
                         capture_output=True, text=True, timeout=300)
    if res.returncode != 0:
        assert res.returncode < 0 or "Error" in res.stderr, res.stderr[-2000:]
        return  # crashed: rejected, though not by a pin
    failed = json.loads(res.stdout.strip().splitlines()[-1])
    assert failed, f"no pin rejects the mutant '{name}'"
