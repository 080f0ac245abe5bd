"""The planner decides whether every workgroup of a launch is resident at once
from a table of the waves per SIMD that each streaming-kernel instance's
register use allows, and skips instances that spill. This test compiles the
kernel sources for gfx950 with the compiler's resource-usage report and checks
the table in api.cpp against it, so a kernel change that moves a register
count fails here instead of silently skewing the plans. Needs hipcc and
c++filt; no GPU."""

import concurrent.futures
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_weight_quantized_qgemm_amd", "csrc")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
SOURCES = ["w4a16.hip", "w4a8.hip", "w2w4.hip", "w4g.hip", "sp24.hip", "bitplane_lo.hip", "bitplane_hi.hip"]
SHAPES = [(1, 1), (1, 2), (2, 1), (2, 2)]


def _report(src):
    cmd = [HIPCC, "--offload-arch=gfx950", "--cuda-device-only", "-c", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(CSRC, src), "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: +(Function Name|Occupancy \[waves/SIMD\]|ScratchSize \[bytes/lane\]): (\S+)", line)
        if not m:
            continue
        if m.group(1) == "Function Name":
            cur = m.group(2)
            out[cur] = {}
        else:
            out[cur][m.group(1).split()[0]] = int(m.group(2))
    return out


def _demangle(names):
    r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True, check=True)
    return r.stdout.splitlines()


def _table():
    src = open(os.path.join(CSRC, "api.cpp")).read()
    rows = {k: v for k, v in re.findall(r'kOcc(\w+) = "(\w{12})"', src)}
    bp = re.search(r"kOccBP\[8\] = \{([^}]*)\}", src).group(1)
    for b, v in enumerate(re.findall(r'"(\w{12})"', bp), start=1):
        rows[f"BP{b}"] = v
    return rows


def test_occupancy_table_matches_compiler():
    if not os.path.exists(HIPCC) or not shutil.which("c++filt"):
        pytest.skip("hipcc or c++filt not available")
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        reports = list(ex.map(_report, SOURCES))
    kernels = {}
    for rep in reports:
        for mangled, demangled in zip(rep, _demangle(list(rep))):
            m = re.search(r"skinny_gemm_kp(\d)<qg::fmt::(\w+(?:<[^>]*>)?), (\d), (\d)>", demangled)
            if m:
                kp, pol, mb, nb = int(m.group(1)), m.group(2), int(m.group(3)), int(m.group(4))
                kernels.setdefault(pol, {})[(mb, nb, kp)] = rep[mangled]
    policies = {"W4A16": ["PolicyW4A16"], "W4A8": ["PolicyW4A8"], "W2W4": ["PolicyW2W4"], "SP24": ["PolicySP24"],
                "W4GH": [p for p in kernels if p.startswith("PolicyW4G<false,") and p.endswith("true>")],
                "W4GLH": [p for p in kernels if p.startswith("PolicyW4G<false,") and p.endswith("false>")],
                "W4GB": [p for p in kernels if p.startswith("PolicyW4G<true,") and p.endswith("true>")],
                "W4GLB": [p for p in kernels if p.startswith("PolicyW4G<true,") and p.endswith("false>")]}
    policies.update({f"BP{b}": [f"PolicyBP<{b}>"] for b in range(1, 9)})
    assert all(len(policies[r]) == 2 for r in ("W4GH", "W4GLH", "W4GB", "W4GLB"))
    table = _table()
    assert set(table) == set(policies)
    for row, pols in policies.items():
        want = ""
        for mb, nb in SHAPES:
            use = ["PolicyW4A16M32"] if (row == "W4A16" and (mb, nb) == (2, 2)) else pols
            for kp in (1, 2, 4):
                rs = [kernels[p][(mb, nb, kp)] for p in use]
                occ = min(r["Occupancy"] for r in rs)
                spills = any(r["ScratchSize"] > 0 for r in rs)
                want += chr(ord("a") + occ - 1) if spills else str(occ)
        assert table[row] == want, (row, table[row], want)


@pytest.mark.parametrize("row", ["W4A16", "W4A8", "W2W4", "W4G", "W4G-bf16", "SP24"] + [f"BP{b}" for b in range(1, 9)])
def test_automatic_plans_avoid_spilling_kernels(row):
    import bit_weight_quantized_qgemm_amd as qg
    fmt = {"W4A16": qg.FMT_W4A16, "W4A8": qg.FMT_W4A8, "W2W4": qg.FMT_W2W4, "W4G": qg.FMT_W4G, "W4G-bf16": qg.FMT_W4G,
           "SP24": qg.FMT_W4A16_SP24}.get(row, qg.FMT_BITPLANE)
    act = qg.DT_BF16 if row == "W4G-bf16" else qg.DT_F16
    bits = int(row[2:]) if row.startswith("BP") else 4
    for K, N in [(1024, 1024), (4096, 11008), (11008, 4096), (8192, 28672), (28672, 8192)]:
        if fmt == qg.FMT_W4A8 and K > 16384:
            continue
        for M in (1, 8, 16, 17, 32, 64, 100, 128):
            p = qg.plan(fmt, M, K, N, bits=bits, act_dtype=act)
            if p["kernel"] == 2:
                continue
            if row.startswith("W4G"):
                h = "B" if act == qg.DT_BF16 else "H"
                occ = _table()[("W4GL" if p["kernel"] == 3 else "W4G") + h]
            else:
                occ = _table()[row]
            kp = p["wpt"] // 4
            ch = occ[SHAPES.index((p["mb"], p["nb"])) * 3 + (0 if kp == 1 else 1 if kp == 2 else 2)]
            assert ch.isdigit(), (row, K, N, M, p)
