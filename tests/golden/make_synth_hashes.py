"""Writes tests/golden/synth_hashes.json: SHA-256 prefixes of seed-0 generator
outputs, so a change in the seeded workload recipe is noticed. Calls only the
``synth`` input generators."""

import hashlib
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from synth import gen  # noqa: E402


def _h(*arrays):
    m = hashlib.sha256()
    for a in arrays:
        m.update(np.ascontiguousarray(a).tobytes())
    return m.hexdigest()[:16]


def main():
    a = gen.w4a16_problem(16, 1024, 1024, seed=0)
    w8 = gen.w4a8_problem(16, 512, 256, seed=0)
    w2 = gen.w2w4_problem(4, 1024, 512, seed=0)
    out = {
        "w4a16_m16_k1024_n1024": _h(a["A"], a["codes"], a["scales"]),
        "w4a8_m16_k512_n256": _h(w8["A"], w8["a_scale"], w8["codes"], w8["group_scales"],
                                 w8["chan_scales"]),
        "w2w4_m4_k1024_n512": _h(w2["A"], w2["codes"], w2["scales"], w2["bitmap"]),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "synth_hashes.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
