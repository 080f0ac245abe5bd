"""Host sanitizer tier: the CPU tests of the C ABI (argument validation, the
planner, blob-layout sizes; tests/test_abi_cpu.py) run again in a child process
against a build of the library whose host code carries AddressSanitizer and
UndefinedBehaviorSanitizer (bit_weight_quantized_qgemm_amd/build_sanitized.py).
Any sanitizer report aborts the child and fails this test. No GPU is used.
"""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_cpu_tests_pass_under_host_asan_and_ubsan():
    from bit_weight_quantized_qgemm_amd import build_sanitized as bs

    lib = bs.build()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the library is not instrumented"
    env = dict(os.environ)
    env.update({
        "QGEMM_LIB": lib,
        "LD_PRELOAD": bs.asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    code = ("import sys, pytest, bit_weight_quantized_qgemm_amd as qg; "
            f"assert qg.lib_path() == {lib!r}; "
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', 'tests/test_abi_cpu.py']))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
