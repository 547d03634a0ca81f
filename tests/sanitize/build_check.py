"""Build tests/sanitize/abi_check with AddressSanitizer and UndefinedBehaviorSanitizer
on the host code: the library's sources (hipcc; the sanitizers go to the host pass
only, each -fsanitize= right after -Xarch_host, the device code is built as usual),
the oracle's C sources (ROCm's clang, no OpenMP) and the check program, linked into
one executable with clang's sanitizer runtimes.  Rebuilt when a source is newer."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from generative_recommender_attention_amd import build as libbuild  # noqa: E402

OUT_DIR = os.path.join(ROOT, "_build", "sanitize")
EXE = os.path.join(OUT_DIR, "abi_check")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["address", "undefined"]
HOST_SAN = [f for s in SAN for f in ("-Xarch_host", f"-fsanitize={s}")] + [
    "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def _sources():
    lib = [os.path.join(libbuild.CSRC, s) for s in libbuild.SOURCES]
    oracle = [os.path.join(ROOT, "oracle", f) for f in ("hstu_oracle.c", "lmsd_oracle.c")]
    return lib, oracle, os.path.join(HERE, "abi_check.cpp")


def _stale(target, deps):
    if not os.path.exists(target):
        return True
    t = os.path.getmtime(target)
    return any(os.path.getmtime(d) > t for d in deps)


def build() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    lib, oracle, check = _sources()
    headers = [os.path.join(libbuild.CSRC, f) for f in os.listdir(libbuild.CSRC) if f.endswith(".h")]
    headers.append(os.path.join(libbuild.INCLUDE, "hstu.h"))
    if not _stale(EXE, lib + oracle + headers + [check, __file__]):
        return EXE
    hipcc = libbuild.hipcc()
    objs, procs = [], []
    base = ["-std=c++17", "-O1", "-g", f"--offload-arch={libbuild.ARCH}", "-I", libbuild.INCLUDE, "-I", libbuild.CSRC,
            *libbuild.DEVICE_FLAGS, *HOST_SAN]
    for src in lib + [check]:
        obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
        procs.append(subprocess.Popen([hipcc, *base, "-c", src, "-o", obj], stderr=subprocess.PIPE, text=True))
        objs.append(obj)
    for src in oracle:
        obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
        procs.append(subprocess.Popen([CLANG, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                                       "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-c", src, "-o",
                                       obj], stderr=subprocess.PIPE, text=True))
        objs.append(obj)
    for p in procs:
        err = p.communicate()[1]
        if p.returncode:
            raise RuntimeError(f"sanitizer build failed:\n{err}")
    link = [hipcc, f"--offload-arch={libbuild.ARCH}", "-fsanitize=address", "-fsanitize=undefined",
            "-fno-gpu-sanitize", "-o", EXE + ".tmp", *objs]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"sanitizer link failed:\n{r.stderr}")
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())
