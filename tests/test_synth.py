"""Pins for the seeded input generators (synth/): determinism, canonical packing,
value ranges and the mixed 2/4-bit group selection."""

import hashlib
import json
import os

import numpy as np

from synth import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "synth_hashes.json")


def _h(*arrays):
    m = hashlib.sha256()
    for a in arrays:
        m.update(np.ascontiguousarray(a).tobytes())
    return m.hexdigest()[:16]


def test_pack_nibbles_hand():
    codes = np.arange(16, dtype=np.uint8).reshape(16, 1)
    out = gen.pack_nibbles_u32(codes)
    assert out[:, 0].tolist() == [0x76543210, 0xFEDCBA98]


def test_determinism_and_ranges():
    a = gen.w4a16_problem(16, 1024, 1024, seed=0)
    b = gen.w4a16_problem(16, 1024, 1024, seed=0)
    c = gen.w4a16_problem(16, 1024, 1024, seed=1)
    assert _h(a["A"], a["codes"], a["scales"]) == _h(b["A"], b["codes"], b["scales"])
    assert _h(a["codes"]) != _h(c["codes"])
    assert a["A"].dtype == np.float16 and a["scales"].dtype == np.float16
    s = a["scales"].astype(np.float64)
    assert s.min() >= 0.0049 and s.max() <= 0.0201
    # weights do not depend on M
    d = gen.w4a16_problem(1, 1024, 1024, seed=0)
    assert _h(d["codes"], d["scales"]) == _h(a["codes"], a["scales"])
    w8 = gen.w4a8_problem(16, 1024, 1024, seed=0)
    assert w8["A"].min() >= -127 and w8["A"].max() <= 127
    assert w8["group_scales"].min() >= 1 and w8["group_scales"].max() <= 16


def test_select_4bit_groups_count_and_ties():
    K, N = 4096, 4096
    p = gen.w2w4_problem(1, K, N, seed=0)
    G = (K // 128) * N
    assert int(p["mask"].sum()) == round(0.1 * G) == 13107
    # all selected groups have range >= every unselected group's range
    lat = gen.rng_for(0, 3, 1, K, N).standard_normal(size=(K, N), dtype=np.float32)
    blk = lat.reshape(K // 128, 128, N)
    r = blk.max(axis=1) - blk.min(axis=1)
    assert r[p["mask"]].min() >= r[~p["mask"]].max()
    # 2-bit groups hold codes 0..3
    wide = np.repeat(p["mask"], 128, axis=0)
    assert p["codes"][~wide].max() <= 3 and p["codes"][wide].max() <= 15
    # tie-break toward the lower linear index
    flat = np.zeros((2, 128, 3), dtype=np.float32)
    flat[:, 0, :] = 1.0                                    # every group has range 1
    m = gen.select_4bit_groups(flat.reshape(256, 3), frac=2 / 6)
    assert m.ravel().tolist() == [True, True, False, False, False, False]


def test_golden_hashes():
    with open(GOLDEN) as f:
        want = json.load(f)
    a = gen.w4a16_problem(16, 1024, 1024, seed=0)
    w8 = gen.w4a8_problem(16, 512, 256, seed=0)
    w2 = gen.w2w4_problem(4, 1024, 512, seed=0)
    got = {
        "w4a16_m16_k1024_n1024": _h(a["A"], a["codes"], a["scales"]),
        "w4a8_m16_k512_n256": _h(w8["A"], w8["a_scale"], w8["codes"], w8["group_scales"],
                                 w8["chan_scales"]),
        "w2w4_m4_k1024_n512": _h(w2["A"], w2["codes"], w2["scales"], w2["bitmap"]),
    }
    assert got == want
