"""include/hstu.h is a C header: a C99 program (tests/c_consumer/consumer.c) built
with gcc -std=c99 -pedantic -Werror against it alone, linked to libhstu.so, drives
the host-side paths of the ABI (version, status strings, workspace sizes against
the sizes the header states, rejections and their messages, the release build's
hstu_debug_take).  No GPU is used."""

import os
import shutil
import subprocess

import pytest

from generative_recommender_attention_amd import hstu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = "/opt/rocm"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c99_program_uses_the_abi(tmp_path):
    lib = hstu.library_path(debug=False)
    if not os.path.exists(lib):
        pytest.skip("libhstu.so is not built")
    exe = tmp_path / "consumer"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include"),
           os.path.join(HERE, "c_consumer", "consumer.c"), "-o", str(exe),
           "-L", os.path.dirname(lib), "-l:libhstu.so", "-Wl,-rpath," + os.path.dirname(lib),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
