"""The C ABI's host validation and the CPU oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; no GPU is touched): the check program
in tests/sanitize drives every entry point through its rejection paths and the
workspace-size arithmetic over many argument sets, and runs the oracle's
attention and LMSD functions on small inputs with every mask form."""

import os
import shutil
import subprocess
import sys

import pytest

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "sanitize"))


@pytest.mark.timeout(600)
def test_abi_and_oracle_under_asan_ubsan():
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc is not available")
    import build_check

    exe = build_check.build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"stdout:\n{r.stdout}\nstderr:\n{r.stderr[-4000:]}"
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
