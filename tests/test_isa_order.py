"""The streaming and wide kernels count their outstanding vector-memory
operations to know when a group's activations (direct-to-LDS loads) have
landed; the count assumes a fixed issue order in each loop iteration
(streaming kernel: the weights of a later group, the wait, the barrier, the
activation loads; wide kernel: the wait, the barrier, the activation loads,
the weights), so after each loop barrier the first vector-memory load a wave
issues is an activation load. This test compiles kernels to gfx950 assembly and checks that
after every barrier (a compiler that issued weight loads first made the count
wait too little and the kernel read activation slots still being filled).
Needs hipcc; no GPU."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_weight_quantized_qgemm_amd", "csrc")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


@pytest.mark.parametrize("src", ["w4a16.hip", "wide.hip", "bitplane_lo.hip"])
def test_activation_loads_issue_before_weight_loads(src, tmp_path):
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path / "k.s"
    cmd = [HIPCC if os.path.exists(HIPCC) else "hipcc", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    s = out.read_text()
    checked = 0
    for m in re.finditer(r"^(_ZN2qg\w+):", s, re.M):
        end = s.index("s_endpgm", m.end())
        body = [l.strip() for l in s[m.end():end].split("\n") if l.strip() and not l.strip().startswith(";")]
        for b, line in enumerate(body):
            if not line.startswith("s_barrier"):
                continue
            rest = body[b + 1:]
            stop = next((k for k, x in enumerate(rest) if x.startswith("s_barrier")), len(rest))
            window = rest[:stop]
            loads = [x for x in window if x.startswith("buffer_load")]
            if not any(x.endswith(" lds") or " lds " in x for x in loads):
                continue   # no activation loads after this barrier
            checked += 1
            assert loads[0].endswith(" lds") or " lds " in loads[0], (m.group(1), b, loads[:3])
    assert checked > 0
