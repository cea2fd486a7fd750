"""Write tests/golden/oracle_tiny_digest.json from the CPU oracle alone.

Digests of the oracle's outputs on the tiny workload (cos/sin tables,
rotate-half, GEGLU) and of its full 65536-entry bf16 GELU table, so that any
later change of the oracle's arithmetic shows up as a failing test and has to
be justified.  Calls only oracle/ and the seeded inputs of workloads.py.

    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads  # noqa: E402

OUT = os.path.join(HERE, "oracle_tiny_digest.json")


def digests():
    o = oracle.get()
    w = workloads.WORKLOADS[0]
    r, g = w["rope"], w["geglu"]
    cos, sin = o.rope_cossin(workloads.workload_freqs(0))
    x = workloads.normal_bf16((r["B"], r["S"], r["H"], r["D"]), workloads.seed_for(0, "x"))
    rope = o.rope_rotate_half(x, cos, sin)
    gate = workloads.normal_bf16((g["rows"], g["hidden"]), workloads.seed_for(0, "gate"),
                                 g["gate_sigma"])
    up = workloads.normal_bf16((g["rows"], g["hidden"]), workloads.seed_for(0, "up"))
    geglu = o.gelu_and_mul(np.concatenate([gate, up], axis=1))
    table = o.gelu_table()

    def h(a):
        return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()

    return {
        "cos": h(cos), "sin": h(sin), "rope": h(rope), "geglu": h(geglu),
        "gelu_table": h(table),
        "samples": {
            "cos[255,1]": int(cos[255, 1]), "sin[255,1]": int(sin[255, 1]),
            "rope[0,100,2,5]": int(rope[0, 100, 2, 5]), "geglu[7,9]": int(geglu[7, 9]),
        },
    }


if __name__ == "__main__":
    with open(OUT, "w") as f:
        json.dump(digests(), f, indent=1, sort_keys=True)
        f.write("\n")
    print(OUT)
