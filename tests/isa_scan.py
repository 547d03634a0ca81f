"""Scan gfx950 assembly of the HIP kernels for hazards the compiler cannot see.

The tile loads are inline assembly (global_load_lds_dwordx4 with an SGPR base
and M0 as the LDS destination), so LLVM's hazard recognizer does not know
which registers they read.  The hardware needs, before a vector memory
instruction, 5 wait states after a VALU instruction wrote an SGPR it reads, and
1 wait state after M0 was written.  Missing them makes the load use a stale
base address.  The scanner walks back from every such load through the
straight-line code before it and counts wait states (one per instruction,
N + 1 for ``s_nop N``).
"""

from __future__ import annotations

import os
import re
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "generative_recommender_attention_amd")

_SGPR_RANGE = re.compile(r"\bs\[(\d+):(\d+)\]")
_SGPR_ONE = re.compile(r"\bs(\d+)\b")


def sgprs(text: str) -> set:
    out = set()
    for a, b in _SGPR_RANGE.findall(text):
        out.update(range(int(a), int(b) + 1))
    text = _SGPR_RANGE.sub("", text)
    out.update(int(x) for x in _SGPR_ONE.findall(text))
    return out


def instructions(asm: str):
    """(mnemonic, operand text) for each instruction line; labels and directives split blocks."""
    for line in asm.splitlines():
        line = line.split(";")[0].strip()
        if not line:
            continue
        if line.endswith(":") or line.startswith("."):
            yield ("<label>", "")
            continue
        parts = line.split(None, 1)
        yield (parts[0], parts[1] if len(parts) > 1 else "")


def valu_sgpr_dests(mn: str, ops: str) -> set:
    """SGPRs a VALU instruction writes (scalar destination or carry-out)."""
    if not mn.startswith("v_"):
        return set()
    fields = [f.strip() for f in ops.split(",")]
    dst = set()
    if fields and (fields[0].startswith("s") or fields[0] == "vcc"):
        dst |= sgprs(fields[0])
    if len(fields) > 1 and re.match(r"^s\[\d+:\d+\]$", fields[1]):  # v_add_co_u32 v, s[..], ... / v_mad_u64_u32
        dst |= sgprs(fields[1])
    return dst


def find_hazards(asm: str):
    """Return a list of (index, text) of LDS DMA loads with too few wait states before them."""
    insts = list(instructions(asm))
    bad = []
    for i, (mn, ops) in enumerate(insts):
        if not mn.startswith("global_load_lds") and not (mn.startswith("buffer_load") and "lds" in ops):
            continue
        reads = sgprs(ops)
        waits, j = 0, i - 1
        while j >= 0 and waits < 5:
            pmn, pops = insts[j]
            if pmn == "<label>":
                # a branch target: the code before it in the file need not run first,
                # so require the padding to sit inside the straight-line run
                bad.append((i, f"{mn} {ops}: label {5 - waits} wait states before it"))
                break
            if valu_sgpr_dests(pmn, pops) & reads:
                bad.append((i, f"{mn} {ops}: {pmn} {pops} only {waits} wait states earlier"))
                break
            if waits < 1 and re.search(r"\bm0\b", pops.split(",")[0] if pops else "") and pmn.startswith("s_"):
                bad.append((i, f"{mn} {ops}: M0 written by {pmn} with no wait state"))
                break
            m = re.match(r"s_nop", pmn)
            waits += (int(pops, 0) + 1) if m and pops else 1
            j -= 1
    return bad


def device_asm(source: str, extra_flags=()) -> str:
    """gfx950 assembly of one source file, compiled as the library build compiles it."""
    import sys

    sys.path.insert(0, ROOT)
    from generative_recommender_attention_amd import build

    cmd = [build.hipcc(), *build.compile_flags(), *build.FILE_FLAGS.get(source, []), *extra_flags,
           "--cuda-device-only", "-S", "-o", "-", os.path.join(build.CSRC, source)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(r.stderr)
    return r.stdout
