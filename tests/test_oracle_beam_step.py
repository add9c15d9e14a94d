"""Pins of the beam-step oracle (BeamKV append + BeamPath update), and planted
mistakes in copies of its C source that the pins must reject (CPU only)."""
import json
import os
import subprocess
import sys

import pytest

import pins_step
from oracle import oracle as O

SRC = os.path.join(os.path.dirname(O.__file__), "oracle.c")


def test_p1_chain_walk():
    pins_step.pin_p1_chain_walk(O.beam_step)


def test_p2_append():
    pins_step.pin_p2_append(O.beam_step)


def test_p3_composition_with_attention():
    pins_step.pin_p3_composition(O.beam_step)


def test_p4_special_cases():
    pins_step.pin_p4_special(O.beam_step)


# (name, original text, mistaken text): each a one-token slip in oracle_beam_step
MUTANTS = [
    ("parent ignored", "path_old[(int64_t)(row_offset_old[b] + p) * T_cap + t]",
     "path_old[(int64_t)(row_offset_old[b] + k) * T_cap + t]"),
    ("request base missing", "path_old[(int64_t)(row_offset_old[b] + p) * T_cap + t]",
     "path_old[(int64_t)(p) * T_cap + t]"),
    ("slot stride of the step width", "const int64_t slot = (int64_t)s * W_cap + k;",
     "const int64_t slot = (int64_t)s * w_new + k;"),
    ("path copy one short", "for (int t = 0; t < s; ++t)\n",
     "for (int t = 0; t + 1 < s; ++t)\n"),
    ("length not advanced", "beam_len_new[b] = w_new > 0 ? s + 1 : s;",
     "beam_len_new[b] = s;"),
    ("V taken from new K", "= new_v[(int64_t)r * row_elems + e];",
     "= new_k[(int64_t)r * row_elems + e];"),
    ("own slot of the next step", "path_new[(int64_t)r * T_cap + s] = (int32_t)slot;",
     "path_new[(int64_t)r * T_cap + s] = (int32_t)(slot + W_cap);"),
    ("parent bound off by one", "(s > 0 && (p < 0 || p >= w_old))",
     "(s > 0 && (p < 0 || p > w_old))"),
]

RUNNER = """
import json, sys
sys.path[:0] = {paths!r}
import pins_step
from oracle import oracle as O
print(json.dumps(pins_step.battery(O.beam_step_from_library({so!r}))))
"""


def test_real_oracle_passes_battery():
    assert pins_step.battery(O.beam_step) == []


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_rejected(tmp_path, name, orig, bad):
    src = open(SRC).read()
    assert orig in src, f"mutation anchor not found: {orig!r}"
    start = src.index("int oracle_beam_step(")
    mutated = src[:start] + src[start:].replace(orig, bad, 1)
    assert mutated != src
    c_path = os.path.join(tmp_path, "m.c")
    so_path = os.path.join(tmp_path, "m.so")
    with open(c_path, "w") as f:
        f.write(mutated)
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", c_path, "-o",
                           so_path, "-lpthread", "-lm"])
    paths = [os.path.dirname(os.path.abspath(__file__)),
             os.path.dirname(os.path.dirname(os.path.abspath(__file__)))]
    res = subprocess.run([sys.executable, "-c", RUNNER.format(paths=paths, so=so_path)],
                         capture_output=True, text=True, timeout=300)
    if res.returncode != 0:
        assert res.returncode < 0 or "Error" in res.stderr, res.stderr[-2000:]
        return  # crashed: rejected, though not by a pin
    failed = json.loads(res.stdout.strip().splitlines()[-1])
    assert failed, f"no pin rejects the mutant '{name}'"
