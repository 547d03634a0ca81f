#!/usr/bin/env python3
"""Benchmark: HSTU attention forward + backward on one MI355X.

One step = the whole path over one batch of synthetic input, launched through
the C ABI on the current stream: hstu_fwd, then the backward as hstu_bwd runs it
-- hstu_bwd_dkdv_ds (dK, dV, and dS stored in a workspace allocated before the
timed region) then hstu_bwd_dq_ds, or with --recompute-dq hstu_bwd_dq then
hstu_bwd_dkdv.  Default
workload: B=32 sequences with Zipf(1.2) lengths clipped to [16, 4096]
(T = 23460), H=4, D=128, causal, bf16, plus an upstream gradient.

Metric: useful TFLOP/s = useful flops / time, counting only visible (query,
key) pairs P: forward 4*D*H*P, backward 10*D*H*P (five matmul-equivalents,
including the score recompute the backward needs).  Inputs are resident in HBM
before the timed region starts.

Prints one JSON line.  `--gpus N` with N > 1 is refused: this build measures a
single GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0
CLOCK_WGS = 2048  # one-wave workgroups per clock sample: about 8 per CU, so most CUs appear in both
DEFAULT_WORKLOAD = "zipf_b32_h4_d128_causal_fwdbwd"
# Algorithmic flops per visible (query, key) pair and head, per unit of D:
# forward: S (2) + A.V (2); dq kernel: S (2) + dO.V^T (2) + dS.K (2);
# dk/dv kernel: S (2) + dO.V^T (2) + A^T.dO (2) + dS^T.Q (2) (also when it stores
# dS); dq from stored dS: dS.K (2).
FLOPS_PER_PAIR_D = {"fwd": 4, "bwd_dq": 6, "bwd_dkdv": 8, "bwd_dkdv_ds": 8, "bwd_dq_ds": 2, "bwd_fused": 10}
USEFUL_PER_PAIR_D = {"fwd": 4, "bwd": 10}
KERNEL_SYMBOL = {"fwd": "fwd_kernel", "bwd_dq": "bwd_dq_kernel", "bwd_dkdv": "bwd_dkdv_kernel",
                 "bwd_dkdv_ds": "bwd_dkdv_kernel", "bwd_dq_ds": "bwd_dq_ds_kernel", "bwd_fused": "bwd_dkdv_kernel"}


def dq_ds_bytes(wl, pairs: int) -> int:
    """Algorithmic HBM bytes of one dq-from-stored-dS launch: the bf16 dS of every
    visible pair and head, K read once and dQ written once."""
    h, d = wl.num_heads, wl.head_dim
    return 2 * h * pairs + 2 * h * d * (wl.total_k + wl.total_q)


def visible_pairs(lengths_q, lengths_k, window) -> int:
    """Count of (query, key) pairs a token window (left, right) keeps: key j is
    visible to query i iff i - left <= j <= i + right, -1 = unbounded side (so
    (-1, 0) is top-left causal and (-1, -1) full attention)."""
    left, right = window
    total = 0
    for lq, lk in zip(np.asarray(lengths_q, dtype=np.int64), np.asarray(lengths_k, dtype=np.int64)):
        i = np.arange(lq, dtype=np.int64)
        lo = np.zeros_like(i) if left < 0 else np.maximum(0, i - left)
        hi = np.full_like(i, lk) if right < 0 else np.minimum(lk, i + right + 1)
        total += int(np.maximum(0, hi - lo).sum())
    return total


def func_visible_pairs(func, lengths_q, lengths_k) -> int:
    """Count of (query, key) pairs an interval-list mask keeps: packed row r sees the
    local keys [0, F0) u [F1, F2) u ... (F_n = func[n, r]) inside [0, L_k)."""
    total, r0 = 0, 0
    for lq, lk in zip(np.asarray(lengths_q, dtype=np.int64), np.asarray(lengths_k, dtype=np.int64)):
        j = np.arange(lk, dtype=np.int64)[None, :]
        for c0 in range(0, int(lq), 1024):
            f = func[:, r0 + c0:r0 + min(int(lq), c0 + 1024)].astype(np.int64)
            seen = j < f[0][:, None]
            for n in range(1, f.shape[0] - 1, 2):
                seen |= (f[n][:, None] <= j) & (j < f[n + 1][:, None])
            total += int(seen.sum())
        r0 += int(lq)
    return total


def workload_pairs(wl) -> int:
    if wl.func is not None:
        return func_visible_pairs(wl.func, wl.lengths_q, wl.lengths_k)
    return visible_pairs(wl.lengths_q, wl.lengths_k, wl.window_size)


def _code_only(text: str) -> str:
    """C/C++/HIP source with comments removed and whitespace collapsed, so that a
    comment edit does not count as a kernel change."""
    import re

    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_digest() -> str:
    """Digest of the kernel sources (code only) and of the build script that sets
    their compile flags."""
    pkg = os.path.join(ROOT, "generative_recommender_attention_amd")
    csrc = os.path.join(pkg, "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8", errors="replace") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    with open(os.path.join(pkg, "build.py"), "rb") as f:
        h.update(b"build.py\0" + f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed PMC summary, if it matches these
    sources and this workload."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != kernel_source_digest() or t.get("workload") != workload:
        return None
    k = t.get("kernels", {}).get(kernel)
    if not k:
        return None
    return int(k["hbm_bytes_per_launch"])


PROFILE_COMMANDS = {
    "kt": ("rocprofv3 --kernel-trace --stats -T --output-format csv -d {d}/kt -o run -- python3 bench.py "
           "--no-cpu-baseline --no-reference-gemm --workload {w} --clock-out {d}/kt/clock.json --json-out {d}/kt/bench.json"),
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/fetch -o run -- python3 bench.py --steps 5 --warmup 1 --no-cpu-baseline --no-reference-gemm --workload {w}",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/write -o run -- python3 bench.py --steps 5 --warmup 1 --no-cpu-baseline --no-reference-gemm --workload {w}",
    "cfetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/cfetch -o run -- python3 bench.py --calibrate-copy-mib 256",
    "cwrite": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/cwrite -o run -- python3 bench.py --calibrate-copy-mib 256",
    "mfma": ("rocprofv3 --pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_VALU SQ_INSTS_LDS "
             "SQ_WAVE_CYCLES SQ_ACTIVE_INST_VALU SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE --output-format csv "
             "-d {d}/mfma -o run -- python3 bench.py --steps 5 --warmup 1 --no-cpu-baseline --no-reference-gemm --workload {w}"),
}
MFMA_FLOPS = 2 * 32 * 32 * 16  # one v_mfma_f32_32x32x16_bf16 (the only MFMA the attention kernels issue)
ALG_TENSORS = {"fwd_kernel": 4, "bwd_dq_kernel": 5, "bwd_dkdv_kernel": 6}  # (T, H, D) bf16 tensors read + written
PROFILED_KERNELS = ["fwd_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel", "bwd_dq_ds_kernel"]


def alg_bytes(kernel: str, wl, pairs: int, stored: bool) -> int:
    """Algorithmic HBM bytes of one launch: each (T, H, D) bf16 tensor the kernel
    reads or writes once, plus the bf16 dS of every visible pair and head that the
    dk/dv kernel stores (stored route) or the dq kernel reads back."""
    tensor = wl.total_q * wl.num_heads * wl.head_dim * 2
    if kernel == "bwd_dq_ds_kernel":
        return dq_ds_bytes(wl, pairs)
    return ALG_TENSORS[kernel] * tensor + (2 * wl.num_heads * pairs if stored and kernel == "bwd_dkdv_kernel" else 0)


def summarize_profiles(prof_dir: str, workload: str) -> None:
    """Turn the rocprofv3 outputs of PROFILE_COMMANDS (run from the repository root,
    prof_dir relative to it) into the kernel-trace summary and, when the PMC passes
    are there too, profiles/traffic.json and the HBM-traffic summary."""
    import csv
    import glob

    def rows(sub, pattern):
        out = []
        for path in glob.glob(os.path.join(prof_dir, sub, "**", pattern), recursive=True):
            with open(path) as f:
                out.extend(csv.DictReader(f))
        if not out:
            raise SystemExit(f"no {pattern} under {os.path.join(prof_dir, sub)}")
        return out

    def counter_kib(sub, counter, match):
        vals = {}
        for r in rows(sub, "*counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            name = next((m for m in match if m in r["Kernel_Name"]), None)
            if name and ("<128," in r["Kernel_Name"] or "copyBuffer" in name):
                vals.setdefault(name, []).append(float(r["Counter_Value"]))
        return {k: float(np.mean(v)) for k, v in vals.items()}

    kernels = list(PROFILED_KERNELS)
    copy = ["copyBuffer"]
    from generative_recommender_attention_amd.workloads import lmsd_named_workload, named_workload

    if workload.startswith("lmsd_"):
        lw = lmsd_named_workload(workload)
        title = "HSTU LMSD fwd + bwd"
        what = (f"Workload: N={lw.n} rows, D={lw.d}, {lw.segments} output segments (SiLU(u), x, LN(x) SiLU(u)), "
                "bf16, seeded synthetic inputs; one bench step = hstu_lmsd_fwd + hstu_lmsd_bwd (row kernel, "
                "column sums).")
        kernels = ["lmsd_fwd_kernel", "lmsd_bwd_kernel", "lmsd_colsum_kernel"]
    else:
        wl = named_workload(workload)
        title = "HSTU attention fwd + bwd"
        stored = True
        what = (f"Workload: B={wl.batch} packed sequences (T={wl.total_q}), H={wl.num_heads}, D={wl.head_dim}, "
                f"mask {wl.mask_name}, bf16, seeded synthetic inputs; one bench step = hstu_fwd + " +
                ("hstu_bwd_dkdv_ds (bwd_dkdv_kernel storing dS) + hstu_bwd_dq_ds." if stored else
                 "hstu_bwd_dq + hstu_bwd_dkdv."))
    # a run of the fused backward (bench.py --fused-bwd) gets its own summary file
    suffix, kt_cmd = "", PROFILE_COMMANDS["kt"].format(d=prof_dir, w=workload)
    bpath0 = os.path.join(prof_dir, "kt", "bench.json")
    if os.path.exists(bpath0):
        with open(bpath0) as f:
            backward = (json.loads(f.readline()).get("config") or {}).get("backward") or ""
        if backward.startswith("fused"):
            suffix, kt_cmd = "_fused", kt_cmd + " --fused-bwd"
            title = "HSTU attention fwd + fused bwd"
            what = what.split("one bench step")[0] + ("one bench step = hstu_fwd + hstu_bwd_fused (fill_zero_kernel, "
                                                      "bwd_dkdv_kernel with the fp32-atomic dQ phase, "
                                                      "dq_convert_kernel).")
            kernels = kernels + ["fill_zero_kernel", "dq_convert_kernel"]
    stats = rows("kt", "*kernel_stats.csv")
    clock_note = []
    cpath = os.path.join(prof_dir, "kt", "clock.json")
    if os.path.exists(cpath):
        with open(cpath) as f:
            clk = json.load(f)
        clock_note = [f"Shader clock over the timed steps of the same run: {clk['shader_mhz']} MHz (mean over XCDs; "
                      f"per XCD {clk['per_xcd_mhz']}), from s_memtime / s_memrealtime samples taken just before "
                      "and after them.", ""]
    out = [f"# rocprofv3 kernel trace: {title}, workload {workload}", "", what, "",
           "Command (GPU box, from the repository root):",
           "    " + kt_cmd, ""] + clock_note + [
           f"{'kernel':26s}{'calls':>8s}{'avg ns':>11s}{'min ns':>11s}{'max ns':>11s}{'share':>8s}"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"]
        short = next((k for k in kernels if k in name), name.split("(")[0][-26:])
        out.append(f"{short:26s}{int(r['Calls']):8d}{float(r['AverageNs']):11.0f}{float(r['MinNs']):11.0f}"
                   f"{float(r['MaxNs']):11.0f}{float(r['Percentage']):7.1f}%")
    bpath = os.path.join(prof_dir, "kt", "bench.json")
    if os.path.exists(bpath):
        with open(bpath) as f:
            line = json.loads(f.readline())
        out += ["", f"The same run's bench line (HIP events on the launch stream, mean over {line['steps']} timed steps "
                    f"after {line['warmup']} warmup steps; the trace above also counts the warmup launches):",
                f"  value {line['value']} {line['unit']} ({line.get('frac_of_peak')} of the 2500 TFLOP/s peak), "
                f"{line['ms_per_step']} ms per step"]
        for kname, d in line.get("kernels", {}).items():
            extra = f", {d['alg_gbs']} GB/s of algorithmic bytes" if "alg_gbs" in d else ""
            out.append(f"  {kname:12s} {d['ms'] * 1e3:8.1f} us  {d['alg_tflops']:7.1f} TFLOP/s "
                       f"({d['frac_of_peak']:.1%} of peak){extra}")
        rl = line.get("roofline")
        if rl:
            tr = next((float(r["AverageNs"]) for r in stats if rl["kernel"] in r["Name"]), None)
            out.append(f"  roofline: {rl['kernel']} {rl['achieved']} TFLOP/s = frac {rl['frac']} from the events; "
                       + (f"{rl['alg_flops_per_launch']} flops / {tr / 1e3:.1f} us (trace average) = "
                          f"{rl['alg_flops_per_launch'] / (tr * 1e-9) / 1e12:.1f} TFLOP/s = frac "
                          f"{rl['alg_flops_per_launch'] / (tr * 1e-9) / 1e12 / PEAK_BF16_TFLOPS:.4f} from the trace"
                          if tr else "(kernel not in the trace)"))
    with open(os.path.join(ROOT, "profiles", f"hstu_kernels_{workload}{suffix}_kernel_trace.txt"), "w") as f:
        f.write("\n".join(out) + "\n")
    if suffix:
        print(f"wrote the kernel-trace summary for {workload}{suffix}")
        return
    if os.path.isdir(os.path.join(prof_dir, "mfma")) and not workload.startswith("lmsd_"):
        avg_ns = {k: float(r["AverageNs"]) for r in stats for k in kernels if k in r["Name"]}
        ctr = {}
        for r in rows("mfma", "*counter_collection.csv"):
            name = next((k for k in kernels if k in r["Kernel_Name"]), None)
            if name and "<128," in r["Kernel_Name"]:
                ctr.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        mean = {k: {c: float(np.mean(v)) for c, v in d.items()} for k, d in ctr.items()}
        m = [f"# rocprofv3 MFMA / VALU / LDS counters per dispatch, workload {workload}", "",
             "Command (GPU box, repository root; one pass, 8 SQ counters and GRBM_GUI_ACTIVE):",
             "    " + PROFILE_COMMANDS["mfma"].format(d=prof_dir, w=workload), "",
             "Executed MFMA flops = SQ_INSTS_MFMA x 32768 (every MFMA the kernels issue is "
             "v_mfma_f32_32x32x16_bf16); utilisation against the dense bf16 peak (2500 TFLOP/s) uses",
             "the kernel's average duration from the kernel trace of the same workload.", "",
             "MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (4 SQ_BUSY_CU_CYCLES), the fraction of the cycles in which a",
             "CU was busy that a SIMD's matrix core was busy (the MFMA counter sums the 4 SIMDs of a CU).", "",
             f"{'kernel':18s}{'MFMA insts':>12s}{'exec TFLOP':>11s}{'avg us':>9s}{'exec TF/s':>10s}{'of peak':>9s}"
             f"{'MFMA busy':>11s}{'VALU/MFMA':>10s}{'LDS/MFMA':>9s}{'bank confl/LDS':>15s}"]
        for k in kernels:
            if k not in mean or k not in avg_ns:
                continue
            c = mean[k]
            flops = c["SQ_INSTS_MFMA"] * MFMA_FLOPS
            tfs = flops / (avg_ns[k] * 1e-9) / 1e12
            m.append(f"{k:18s}{c['SQ_INSTS_MFMA']:12.4g}{flops / 1e12:11.3f}{avg_ns[k] / 1e3:9.1f}{tfs:10.1f}"
                     f"{tfs / PEAK_BF16_TFLOPS:9.1%}{c['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * c['SQ_BUSY_CU_CYCLES']):11.1%}"
                     f"{c['SQ_INSTS_VALU'] / c['SQ_INSTS_MFMA']:10.2f}{c['SQ_INSTS_LDS'] / c['SQ_INSTS_MFMA']:9.2f}"
                     f"{c['SQ_LDS_BANK_CONFLICT'] / max(c['SQ_INSTS_LDS'], 1):15.3f}")
        m += ["", "Raw means per dispatch:"]
        for k in kernels:
            if k in mean:
                m.append(f"  {k}: " + ", ".join(f"{c}={v:.4g}" for c, v in sorted(mean[k].items())))
        with open(os.path.join(ROOT, "profiles", f"hstu_kernels_{workload}_mfma_counters.txt"), "w") as f:
            f.write("\n".join(m) + "\n")
        print(f"wrote the MFMA counter summary for {workload}")
    if not os.path.isdir(os.path.join(prof_dir, "fetch")):
        print(f"wrote the kernel-trace summary for {workload} (no PMC passes under {prof_dir})")
        return
    fetch, write = counter_kib("fetch", "FETCH_SIZE", kernels), counter_kib("write", "WRITE_SIZE", kernels)
    cfetch, cwrite = counter_kib("cfetch", "FETCH_SIZE", copy), counter_kib("cwrite", "WRITE_SIZE", copy)
    copy_kib = 256 * 1024.0
    ff, wf = copy_kib / cfetch["copyBuffer"], copy_kib / cwrite["copyBuffer"]
    tensor_bytes = wl.total_q * wl.num_heads * wl.head_dim * 2
    pairs = workload_pairs(wl)
    traffic = {"source_digest": kernel_source_digest(), "workload": workload, "fetch_factor": ff, "write_factor": wf,
               "kernels": {}}
    lines = [f"# HBM traffic per dispatch (rocprofv3 PMC), workload {workload}", "",
             "Commands (GPU box, repository root; one counter per pass):"]
    lines += ["    " + PROFILE_COMMANDS[k].format(d=prof_dir, w=workload) for k in ("fetch", "write", "cfetch", "cwrite")]
    lines += ["", f"copy of {copy_kib:.0f} KiB (the HIP runtime's __amd_rocclr_copyBuffer): FETCH_SIZE reads "
                  f"{cfetch['copyBuffer']:.1f} KiB -> fetch factor {ff:.4f}",
              f"{'':48s}WRITE_SIZE reads {cwrite['copyBuffer']:.1f} KiB -> write factor {wf:.4f}", "",
              f"{'kernel':18s}{'FETCH KiB':>12s}{'WRITE KiB':>12s}{'HBM MB (scaled)':>18s}{'algorithmic MB':>16s}{'ratio':>8s}"]
    for k in kernels:
        if k not in fetch or k not in write:
            continue
        hbm = (fetch[k] * ff + write[k] * wf) * 1024.0
        alg = alg_bytes(k, wl, pairs, stored)
        traffic["kernels"][k] = {"fetch_kib": fetch[k], "write_kib": write[k], "hbm_bytes_per_launch": int(hbm),
                                 "algorithmic_bytes_per_launch": alg}
        lines.append(f"{k:18s}{fetch[k]:12.1f}{write[k]:12.1f}{hbm / 1e6:18.1f}{alg / 1e6:16.1f}{hbm / alg:8.2f}")
    lines += ["", "Algorithmic bytes: fwd reads q, k, v and writes o (4 tensors); dq kernel reads q, do, k, v and",
              "writes dq (5); dk/dv kernel reads q, do, k, v and writes dk, dv (6), and on the stored-dS route",
              "also writes 2 bytes of dS per visible pair and head; the dq-from-dS kernel reads that dS and k and",
              f"writes dq; each tensor T*H*D*2 = {tensor_bytes} bytes, {pairs} visible pairs per head."]
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    with open(os.path.join(ROOT, "profiles", f"hstu_kernels_{workload}_hbm_traffic.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    print(f"wrote profiles/traffic.json and the summaries for {workload}")


def cpu_baseline(wl, max_pairs: int):
    """Time the fp64 oracle (fwd + bwd) on whole sequences of the workload whose
    visible pairs add up to at most ``max_pairs`` (shortest first)."""
    import oracle

    oracle.build(force=False)
    order = np.argsort(wl.lengths_q, kind="stable")
    chosen, pairs = [], 0
    for b in order:
        if wl.func is not None:
            r0 = int(wl.cu_seqlens_q[b])
            p = func_visible_pairs(wl.func[:, r0:r0 + int(wl.lengths_q[b])], [wl.lengths_q[b]], [wl.lengths_k[b]])
        else:
            p = visible_pairs([wl.lengths_q[b]], [wl.lengths_k[b]], wl.window_size)
        if max_pairs and pairs + p > max_pairs and chosen:
            continue
        chosen.append(int(b))
        pairs += p
    cu_q, cu_k = wl.cu_seqlens_q, wl.cu_seqlens_k
    rows_q = np.concatenate([np.arange(cu_q[b], cu_q[b + 1]) for b in chosen])
    rows_k = np.concatenate([np.arange(cu_k[b], cu_k[b + 1]) for b in chosen])
    t0 = time.perf_counter()
    oracle.fwd_workload(wl, rows_q)
    if wl.do is not None:
        oracle.bwd_workload(wl, rows_q, rows_k)
    dt = time.perf_counter() - t0
    per_pair = USEFUL_PER_PAIR_D["fwd"] + (USEFUL_PER_PAIR_D["bwd"] if wl.do is not None else 0)
    flops = per_pair * wl.head_dim * wl.num_heads * pairs
    lens = sorted(int(wl.lengths_q[b]) for b in chosen)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"fp64 oracle fwd+bwd on {len(chosen)} of {wl.batch} sequences (lengths {lens[0]}..{lens[-1]}, "
                   f"{pairs} visible pairs x {wl.num_heads} heads = {pairs / workload_pairs(wl):.1%} "
                   f"of the workload's pairs), {dt:.1f} s"),
        "seconds": dt,
        "cpu": cpu_model(),
    }


ORACLE_CONFIGS = [  # (workload, runs): the five configurations; the long ones once
    ("tiny_b2_h1_d16_causal", 3), ("uniform_b8_h2_d64_full", 3), ("zipf_b32_h4_d128_causal", 3),
    ("long_b4_h8_d128_causal", 1), ("zipf_b32_h4_d128_causal_fwdbwd", 1)]


def time_oracle_configs() -> int:
    """Wall time of the fp64 oracle on every configuration, whole workloads, on this
    host's threads; written to profiles/oracle_cpu_baseline.txt."""
    import oracle
    from generative_recommender_attention_amd.workloads import named_workload

    oracle.build(force=False)
    lines = ["# fp64 CPU oracle on the five workload configurations (whole workloads)", "",
             f"Host: {cpu_model()}, {os.cpu_count()} logical CPUs visible, oracle threads "
             f"(OMP_NUM_THREADS) {oracle.num_threads()}.",
             "Command (from the repository root): python3 bench.py --oracle-configs", "",
             "The oracle is the plain fp64 definition (libm exp, no blocking), OpenMP over output rows; "
             "useful flops count visible pairs only (fwd 4 D H P, bwd 10 D H P).", "",
             f"{'workload':34s}{'runs':>5s}{'median s':>10s}{'useful GFLOP':>14s}{'GFLOP/s':>10s}"]
    out = {}
    for name, runs in ORACLE_CONFIGS:
        wl = named_workload(name)
        times = []
        for _ in range(runs):
            t0 = time.perf_counter()
            oracle.fwd_workload(wl)
            if wl.do is not None:
                oracle.bwd_workload(wl)
            times.append(time.perf_counter() - t0)
        t = float(np.median(times))
        per_pair = USEFUL_PER_PAIR_D["fwd"] + (USEFUL_PER_PAIR_D["bwd"] if wl.do is not None else 0)
        flops = per_pair * wl.head_dim * wl.num_heads * workload_pairs(wl)
        out[name] = {"runs": runs, "median_s": t, "useful_gflop": flops / 1e9, "gflops": flops / t / 1e9}
        lines.append(f"{name:34s}{runs:5d}{t:10.3f}{flops / 1e9:14.3f}{flops / t / 1e9:10.2f}")
        print(f"[oracle] {name}: {t:.3f} s ({runs} runs)", file=sys.stderr, flush=True)
    with open(os.path.join(ROOT, "profiles", "oracle_cpu_baseline.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({"oracle_configs": out, "cpu": cpu_model(), "threads": oracle.num_threads()}))
    return 0


def cpu_model() -> str:
    """The host CPU's model name with its family / model / stepping numbers (from the
    first processor of /proc/cpuinfo; a virtual machine may report a short name), else
    the machine type."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break  # the first processor's block ends here
                key, _, val = line.partition(":")
                fields[key.strip()] = val.strip()
    except OSError:
        pass
    name = fields.get("model name")
    if not name:
        return platform.processor() or platform.machine()
    ids = ", ".join(f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields)
    return f"{name} ({ids})" if ids else name


def board_power(fn, seconds: float, device_index: int = 0) -> dict:
    """Run fn() back to back for about `seconds` while another thread polls
    `amd-smi metric -p -c` (socket power and the GFX clock the firmware reports);
    returns the median of the samples taken after the first second (the readings
    lag the load by up to ~1 s).  Measurement only."""
    import subprocess
    import threading

    import torch

    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            t = time.perf_counter()
            try:
                r = subprocess.run(["amd-smi", "metric", "-p", "-c", "-g", str(device_index), "--json"],
                                   capture_output=True, text=True, timeout=20)
                d = json.loads(r.stdout)
                g = d[0] if isinstance(d, list) else d.get("gpu_data", [d])[0]
                pw = g["power"]["socket_power"]["value"]
                clk = g["clock"]["gfx_0"]["clk"]["value"]
                samples.append((t, float(pw), float(clk)))
            except Exception:  # tool missing or output changed: no sample
                if stop.wait(0.5):
                    break

    fn()
    torch.cuda.synchronize()
    th = threading.Thread(target=poll, daemon=True)
    t0 = time.perf_counter()
    th.start()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn()
        n += 20
        torch.cuda.synchronize()
    t1 = time.perf_counter()
    stop.set()
    th.join(timeout=30)
    use = [(p, c) for t, p, c in samples if t0 + 1.0 <= t <= t1]
    if not use:
        return {"samples": 0, "launches": n, "seconds": round(t1 - t0, 2)}
    return {"socket_w": float(np.median([p for p, _ in use])), "gfx_mhz": float(np.median([c for _, c in use])),
            "samples": len(use), "launches": n, "seconds": round(t1 - t0, 2)}


def reference_gemm(dev, stream, n: int = 8192, reps: int = 10, power_seconds: float = 0.0) -> dict:
    """What a plain dense bf16 GEMM reaches on this board, timed in the same process
    after the attention steps: torch.mm (the ROCm BLAS library's kernel) on two
    n x n N(0,1) bf16 matrices, with the shader clock over its timed launches.  A
    context figure for the roofline (the chip runs near its board power limit under
    matrix-core load, far below the 2.4 GHz the published peak assumes); it is not
    part of the attention path."""
    import torch

    from generative_recommender_attention_amd import hstu

    g = torch.Generator(device=dev).manual_seed(0)
    a = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.mm(a, b, out=c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    clk0 = hstu.clock_sample(CLOCK_WGS, dev, stream)
    e0.record(stream)
    for _ in range(reps):
        torch.mm(a, b, out=c)
    e1.record(stream)
    clk1 = hstu.clock_sample(CLOCK_WGS, dev, stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    mhz = clock_summary(clk0.cpu().numpy(), clk1.cpu().numpy())["shader_mhz"]
    print(f"[bench] reference GEMM: torch.mm bf16 {n}^3 {ms:.3f} ms = {tf:.1f} TFLOP/s at {mhz} MHz",
          file=sys.stderr, flush=True)
    out = {"what": f"torch.mm bf16 {n}x{n}x{n}, N(0,1) operands (ROCm BLAS library kernel), "
                   "same process, after the timed steps; not part of the attention path",
           "ms": round(ms, 4), "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
           "shader_mhz": mhz}
    if power_seconds > 0:
        out["board_power"] = board_power(lambda: torch.mm(a, b, out=c), power_seconds, dev.index or 0)
    return out


def clock_summary(before, after) -> dict:
    """Average shader clock between two clock_sample launches (rows of (real time at
    100 MHz, shader cycles, XCC id, HW_ID)).  The cycle counter is per compute unit
    (its readings on different CUs of one XCD differ by arbitrary offsets), so
    readings are paired by CU -- the XCC id and the CU, SH and SE fields of HW_ID
    (bits 8-15) -- and each CU seen in both launches gives d(cycles) / d(real time)
    x 100 MHz; an XCD's clock is the median over its CUs, the chip's the mean over
    XCDs.  counter_spread_cycles is the largest spread of one CU's readings inside
    one launch (its workgroups start within microseconds of each other)."""
    b, a = np.asarray(before, dtype=np.int64), np.asarray(after, dtype=np.int64)

    def by_cu(s):
        out, spread = {}, 0
        for row in s:
            key = (int(row[2]), (int(row[3]) >> 8) & 0xFF)
            out.setdefault(key, []).append((int(row[0]), int(row[1])))
        for v in out.values():
            cy = [c for _, c in v]
            spread = max(spread, max(cy) - min(cy))
        return {k: min(v) for k, v in out.items()}, spread

    sb, spb = by_cu(b)
    sa, spa = by_cu(a)
    per_xcd = {}
    for key in sorted(set(sb) & set(sa)):
        drt = sa[key][0] - sb[key][0]
        if drt > 0:
            per_xcd.setdefault(key[0], []).append((sa[key][1] - sb[key][1]) / drt * 100.0)
    med = {x: float(np.median(v)) for x, v in per_xcd.items()}
    vals = list(med.values())
    region_us = float(np.median(a[:, 0]) - np.median(b[:, 0])) / 100.0
    return {"shader_mhz": round(float(np.mean(vals)), 1) if vals else None,
            "per_xcd_mhz": {str(k): round(v, 1) for k, v in sorted(med.items())},
            "cus_paired": int(sum(len(v) for v in per_xcd.values())),
            "region_us_by_realtime": round(region_us, 1), "counter_spread_cycles": int(max(spb, spa)),
            "method": "s_memtime / s_memrealtime deltas per CU between samples taken just before and after "
                      "the timed steps on the same stream; median per XCD, mean over XCDs"}


def lmsd_bytes(n: int, d: int, segs: int) -> dict:
    """Algorithmic HBM bytes of one LMSD forward and backward (bf16 matrices, fp32
    statistics; weight and bias read once): fwd reads x, u, writes y (S segments),
    mean, rstd; bwd reads dy, x, u, mean, rstd, writes dx, du (the workspace of
    column partials is not algorithmic)."""
    fwd = 2 * n * d * 2 + segs * n * d * 2 + 8 * n + 4 * d
    bwd = segs * n * d * 2 + 2 * n * d * 2 + 8 * n + 2 * n * d * 2 + 8 * d
    return {"fwd": fwd, "bwd": bwd}


def run_lmsd(args, name: str) -> int:
    """One step = hstu_lmsd_fwd + hstu_lmsd_bwd on an LMSD workload; HBM-bound, so the
    line reports effective bandwidth (algorithmic bytes / time) against 8 TB/s."""
    import torch

    from generative_recommender_attention_amd import hstu
    from generative_recommender_attention_amd.workloads import lmsd_named_workload

    dev = torch.device("cuda:0")
    wl = lmsd_named_workload(name)
    print(f"[bench] LMSD workload {name}: N={wl.n} D={wl.d} segments={wl.segments}", file=sys.stderr, flush=True)

    def td(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    x, u, w, b, dy = td(wl.x), td(wl.u), td(wl.weight), td(wl.bias), td(wl.dy)
    flags = dict(apply_u_silu=wl.silu_u, concat_u=wl.concat_u, concat_x=wl.concat_x)
    y = torch.empty((wl.n, wl.segments * wl.d), dtype=torch.bfloat16, device=dev)
    mean = torch.empty(wl.n, dtype=torch.float32, device=dev)
    rstd = torch.empty_like(mean)
    dx, du = torch.empty_like(x), torch.empty_like(u)
    dw, db = torch.empty_like(w), torch.empty_like(b)
    ws = torch.empty(hstu.lmsd_bwd_workspace_size(x, u, eps=wl.eps, **flags), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        hstu.lmsd_fwd(x, u, w, b, eps=wl.eps, y=y, mean=mean, rstd=rstd, stream=stream, **flags)
        if ev is not None:
            ev[1].record(stream)
        hstu.lmsd_bwd(dy, x, u, w, b, mean, rstd, eps=wl.eps, dx=dx, du=du, dweight=dw, dbias=db, workspace=ws,
                      stream=stream, **flags)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    nbytes = lmsd_bytes(wl.n, wl.d, wl.segments)
    ms_per_step = elapsed * 1e3 / args.steps
    value = (nbytes["fwd"] + nbytes["bwd"]) / (ms_per_step * 1e-3) / 1e9
    dominant = "bwd" if bwd_ms >= fwd_ms else "fwd"
    dom_ms = bwd_ms if dominant == "bwd" else fwd_ms
    achieved = nbytes[dominant] / (dom_ms * 1e-3) / 1e9
    result = {
        "metric": "HSTU LMSD fwd+bwd effective HBM bandwidth (algorithmic bytes / time)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "rows": wl.n, "hidden": wl.d, "segments": wl.segments,
                   "apply_u_silu": wl.silu_u, "concat_u": wl.concat_u, "concat_x": wl.concat_x,
                   "parallelism": "single GPU"},
        "kernels": {"fwd": {"ms": round(fwd_ms, 5), "GB_s": round(nbytes["fwd"] / (fwd_ms * 1e-3) / 1e9, 1)},
                    "bwd": {"ms": round(bwd_ms, 5), "GB_s": round(nbytes["bwd"] / (bwd_ms * 1e-3) / 1e9, 1)}},
        "roofline": {"bound": "hbm", "kernel": f"lmsd_{dominant}", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": None, "alg_bytes_per_launch": nbytes[dominant], "avg_launch_ms": round(dom_ms, 5)},
    }
    if not args.no_cpu_baseline:
        import oracle

        oracle.build(force=False)
        rows = wl.n  # the whole workload: the oracle takes well under a second
        t0 = time.perf_counter()
        yy, mm, rr = oracle.lmsd_fwd(wl.x[:rows], wl.u[:rows], wl.weight, wl.bias, wl.eps, wl.silu_u, wl.concat_u,
                                     wl.concat_x)
        oracle.lmsd_bwd(wl.dy[:rows], wl.x[:rows], wl.u[:rows], wl.weight, wl.bias, mm, rr, wl.silu_u, wl.concat_u,
                        wl.concat_x)
        dt = time.perf_counter() - t0
        sub = lmsd_bytes(rows, wl.d, wl.segments)
        result["cpu_baseline"] = {"value": round((sub["fwd"] + sub["bwd"]) / dt / 1e9, 3), "unit": "GB/s",
                                  "cores": oracle.num_threads(), "kind": "oracle",
                                  "sample": f"fp64 oracle fwd+bwd on all {rows} rows, {dt:.2f} s"}
    print(json.dumps(result))
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-reference-gemm", action="store_true",
                    help="skip the plain bf16 GEMM timed after the steps as a context figure")
    ap.add_argument("--recompute-dq", action="store_true",
                    help="time the backward route without stored dS (hstu_bwd_dq + hstu_bwd_dkdv)")
    ap.add_argument("--fused-bwd", action="store_true",
                    help="time the fused single-pass backward with fp32-atomic dQ (hstu_bwd_fused: clear, "
                         "pass, convert, timed together)")
    ap.add_argument("--cpu-max-pairs", type=int, default=0,
                    help="bound on the oracle sample in visible pairs per head (0: the whole workload, "
                         "about 15 s on 16 host threads for the default workload)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="only write profiles/ from the rocprofv3 outputs under DIR (see PROFILE_COMMANDS)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (PMC byte-counter calibration)")
    ap.add_argument("--power-seconds", type=float, default=0.0,
                    help="after the timed steps, loop the step (then the reference GEMM) this many seconds each "
                         "while polling board power and clock with amd-smi; adds a 'board_power' object")
    ap.add_argument("--clock-out", metavar="PATH", help="also write the shader-clock reading to PATH (JSON)")
    ap.add_argument("--json-out", metavar="PATH", help="also write the JSON line to PATH")
    ap.add_argument("--oracle-configs", action="store_true",
                    help="only time the CPU oracle on every workload configuration (median of 3 runs for the "
                         "small ones, one run for the long ones) and write profiles/oracle_cpu_baseline.txt")
    args = ap.parse_args(argv)

    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.workload)
        return 0
    if args.oracle_configs:
        return time_oracle_configs()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU; --gpus must be 1 "
                                   "(every (sequence, head) pair is independent; see the sharding design notes)"}))
        return 2

    import torch

    from generative_recommender_attention_amd import hstu
    from generative_recommender_attention_amd.workloads import named_workload

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 1
    dev = torch.device("cuda:0")
    if args.workload.startswith("lmsd_"):
        return run_lmsd(args, args.workload)

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20)
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                          "launches": 5}))
        return 0

    lib = hstu.library()
    del lib
    wl = named_workload(args.workload)
    print(f"[bench] workload {wl.name}: B={wl.batch} T={wl.total_q} H={wl.num_heads} D={wl.head_dim} "
          f"mask={wl.mask_name}", file=sys.stderr, flush=True)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    q, k, v = to_dev(wl.q), to_dev(wl.k), to_dev(wl.v)
    has_bwd = wl.do is not None
    do = to_dev(wl.do) if has_bwd else None
    cu_q = torch.from_numpy(wl.cu_seqlens_q).to(dev)
    cu_k = torch.from_numpy(wl.cu_seqlens_k).to(dev)
    o = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    kw = dict(max_seqlen_q=wl.max_seqlen_q, max_seqlen_k=wl.max_seqlen_k, alpha=float(wl.alpha),
              scaling_seqlen=wl.scaling_seqlen, causal=wl.causal, window_size=wl.window,
              func=torch.from_numpy(wl.func).to(dev) if wl.func is not None else None)
    stream = torch.cuda.current_stream(dev)
    ws_bytes = hstu.hstu_bwd_workspace_size(do, q, k, v, cu_q, cu_k, **kw) if has_bwd else 0
    fused = has_bwd and args.fused_bwd
    stored = has_bwd and ws_bytes > 0 and not args.recompute_dq and not fused
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if stored else None
    if stored:
        print(f"[bench] backward through stored dS: workspace {ws_bytes / 2**20:.0f} MiB", file=sys.stderr, flush=True)
    kernels = ["fwd"] + ((["bwd_fused"] if fused else ["bwd_dkdv_ds", "bwd_dq_ds"] if stored else ["bwd_dq", "bwd_dkdv"])
                         if has_bwd else [])
    fws = (torch.empty(wl.total_q * wl.num_heads * wl.head_dim * 4 + 256, dtype=torch.uint8, device=dev)
           if fused else None)

    def step(events=None):
        if events is not None:
            events[0].record(stream)
        hstu.hstu_fwd(q, k, v, cu_q, cu_k, out=o, stream=stream, **kw)
        if events is not None:
            events[1].record(stream)
        if fused:
            hstu.hstu_bwd_fused(do, q, k, v, cu_q, cu_k, dq=dq, dk=dk, dv=dv, workspace=fws, stream=stream, **kw)
            if events is not None:
                events[2].record(stream)
        elif stored:
            hstu.hstu_bwd_dkdv_ds(do, q, k, v, cu_q, cu_k, ds=ws, dk=dk, dv=dv, stream=stream, **kw)
            if events is not None:
                events[2].record(stream)
            hstu.hstu_bwd_dq_ds(q, k, cu_q, cu_k, ds=ws, dq=dq, stream=stream, **kw)
            if events is not None:
                events[3].record(stream)
        elif has_bwd:
            hstu.hstu_bwd_dq(do, q, k, v, cu_q, cu_k, dq=dq, stream=stream, **kw)
            if events is not None:
                events[2].record(stream)
            hstu.hstu_bwd_dkdv(do, q, k, v, cu_q, cu_k, dk=dk, dv=dv, stream=stream, **kw)
            if events is not None:
                events[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()  # barrier: one rank
    clk0 = hstu.clock_sample(CLOCK_WGS, dev, stream)
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    clk1 = hstu.clock_sample(CLOCK_WGS, dev, stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    clock = clock_summary(clk0.cpu().numpy(), clk1.cpu().numpy())
    print(f"[bench] timed {args.steps} steps in {elapsed:.3f} s; shader clock {clock['shader_mhz']} MHz "
          f"(per XCD {clock['per_xcd_mhz']}, {clock['cus_paired']} CUs paired, counter spread "
          f"{clock['counter_spread_cycles']} cycles, "
          f"region {clock['region_us_by_realtime']} us by the real-time counter)", file=sys.stderr, flush=True)
    if args.clock_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.clock_out)), exist_ok=True)
        with open(args.clock_out, "w") as f:
            json.dump(dict(clock, samples_before=clk0.cpu().tolist(), samples_after=clk1.cpu().tolist()), f)

    per_kernel_ms = {}
    for i, name in enumerate(kernels):
        per_kernel_ms[name] = float(np.mean([e[i].elapsed_time(e[i + 1]) for e in ev]))
    ms_per_step = elapsed * 1e3 / args.steps

    pairs = workload_pairs(wl)
    unit_pd = wl.head_dim * wl.num_heads * pairs
    useful = USEFUL_PER_PAIR_D["fwd"] * unit_pd + (USEFUL_PER_PAIR_D["bwd"] * unit_pd if has_bwd else 0)
    value = useful / (ms_per_step * 1e-3) / 1e12

    dominant = max(per_kernel_ms, key=per_kernel_ms.get)
    alg_flops = FLOPS_PER_PAIR_D[dominant] * unit_pd
    achieved = alg_flops / (per_kernel_ms[dominant] * 1e-3) / 1e12
    # the PMC counters behind profiles/traffic.json were taken on the default (stored-dS) route; the dk/dv
    # kernel of the other routes runs in another mode, so they report no traffic
    traffic = load_traffic(KERNEL_SYMBOL[dominant], wl.name) if stored or dominant == "fwd" else None

    detail = {}
    for name in kernels:
        f = FLOPS_PER_PAIR_D[name] * unit_pd
        tf = f / (per_kernel_ms[name] * 1e-3) / 1e12
        detail[name] = {"ms": round(per_kernel_ms[name], 5), "alg_tflops": round(tf, 2),
                        "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        if name == "bwd_dq_ds":  # a stream of stored dS: its HBM rate is the telling figure
            gbs = dq_ds_bytes(wl, pairs) / (per_kernel_ms[name] * 1e-3) / 1e9
            detail[name].update({"alg_bytes": dq_ds_bytes(wl, pairs), "alg_gbs": round(gbs, 1),
                                 "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)})
    fwd_useful_tf = USEFUL_PER_PAIR_D["fwd"] * unit_pd / (per_kernel_ms["fwd"] * 1e-3) / 1e12
    result = {
        "metric": "HSTU attn fwd/bwd useful TFLOP/s @H=4,D=128 causal jagged; % of BF16 MFMA peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "total_tokens": wl.total_q,
                   "heads": wl.num_heads, "head_dim": wl.head_dim, "mask": wl.mask_name,
                   "max_seqlen": wl.max_seqlen_q, "visible_pairs_per_head": pairs,
                   "useful_flops_per_step": useful, "parallelism": "single GPU",
                   "backward": "fused (fp32 atomic dQ)" if fused else "stored dS" if stored else
                               "recompute" if has_bwd else None,
                   "workspace_bytes": ws_bytes if stored else 0},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_useful_tflops": round(fwd_useful_tf, 2),
        "fwd_frac_of_peak": round(fwd_useful_tf / PEAK_BF16_TFLOPS, 4),
        "kernels": detail,
        "roofline": {"bound": "mfma", "kernel": KERNEL_SYMBOL[dominant], "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "alg_flops_per_launch": alg_flops,
                     "avg_launch_ms": round(per_kernel_ms[dominant], 5)},
    }
    if args.power_seconds > 0:
        print(f"[bench] board power over {args.power_seconds} s of back-to-back steps", file=sys.stderr, flush=True)
        result["board_power"] = board_power(step, args.power_seconds, dev.index or 0)
        print(f"[bench] board power: {result['board_power']}", file=sys.stderr, flush=True)
    if not args.no_reference_gemm:
        try:  # a context figure only: a failure of the library GEMM must not cost the bench line
            ref = reference_gemm(dev, stream, power_seconds=args.power_seconds)
            ref["attention_step_frac"] = round(value / ref["tflops"], 4)
            ref["fwd_frac"] = round(fwd_useful_tf / ref["tflops"], 4)
            ref["dominant_kernel_frac"] = round(achieved / ref["tflops"], 4)
        except Exception as e:  # noqa: BLE001
            ref = {"error": f"{type(e).__name__}: {e}"}
        result["reference_gemm"] = ref
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_max_pairs)
    props = torch.cuda.get_device_properties(dev)
    result["device"] = {"name": props.name, "compute_units": props.multi_processor_count,
                        "gcn_arch": getattr(props, "gcnArchName", ""), "shader_clock": clock,
                        "peak_basis": "2500 TFLOP/s = 256 CUs x 2.4 GHz x 4096 bf16 flop/clk/CU (published); "
                                      "at the measured clock the same CUs peak at "
                                      f"{256 * 4096 * (clock['shader_mhz'] or 0) / 1e6:.0f} TFLOP/s"}
    print(json.dumps(result))
    if args.json_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.json_out)), exist_ok=True)
        with open(args.json_out, "w") as f:
            f.write(json.dumps(result) + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
