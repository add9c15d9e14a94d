"""Write tests/golden/oracle_golden.json.

Records (a) SHA-256 digests of the five seeded workloads' input buffers and
(b) fp64 oracle outputs for workload 1 (all rows) and three rows of workload
2.  Only the seeded generator and ``oracle/`` are called.  The stored oracle
values are a regression guard for the oracle itself; the oracle is pinned to
independent facts by tests/pins.py.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import oracle as O                     # noqa: E402
from shared_prefix_beam_amd import inputs as I     # noqa: E402


def main():
    res = {"input_sha256": {}, "oracle": {}}
    for cfg in range(1, 6):
        inp = I.generate(I.WORKLOADS[cfg])
        res["input_sha256"][str(cfg)] = inp.digest()
        if cfg in (1, 2):
            rows = list(range(inp.R)) if cfg == 1 else [0, 517, 1023]
            out, lse = O.decode_attn_inputs(inp, rows=rows)
            res["oracle"][str(cfg)] = {"rows": rows, "out": out.tolist(), "lse": lse.tolist()}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_golden.json")
    with open(path, "w") as f:
        json.dump(res, f)
    print("wrote", path)


if __name__ == "__main__":
    main()
