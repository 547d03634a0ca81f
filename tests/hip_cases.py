"""Helpers for the GPU tests: move a seeded workload to the device, run the HIP
path through the binding, compare with the fp64 oracle.

Tolerances:
* the bar, for X in {O, dQ, dK, dV}:  max|X_gpu - X_ref| <= 1e-2 max|X_ref| + 1e-3;
* a supplementary per-sequence check, because the absolute 1e-3 term alone would
  accept all-zero output for the many short sequences of the Zipf workload:
  max_b|X_gpu - X_ref| <= 2e-2 max_b|X_ref| + 1e-6 for every sequence b.  The GPU
  rounds the SiLU scores (or dS) to bf16 before the second product and its
  outputs to bf16 (relative 2^-9 each), so a correct kernel sits near 4e-3 of
  each sequence's maximum; 2e-2 leaves headroom while any dropped tile, wrong
  row or wrong sign lands far above it.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

from generative_recommender_attention_amd import hstu
from generative_recommender_attention_amd.workloads import Workload

REL_BAR, ABS_BAR = 1e-2, 1e-3
REL_SEQ, ABS_SEQ = 2e-2, 1e-6


def say(msg: str) -> None:
    """Name the case before each GPU step, flushed, so a fault can be located."""
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def to_dev(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


class DeviceWorkload:
    def __init__(self, wl: Workload, device="cuda"):
        self.wl = wl
        self.q, self.k, self.v = to_dev(wl.q, device), to_dev(wl.k, device), to_dev(wl.v, device)
        self.do = to_dev(wl.do, device) if wl.do is not None else None
        self.cu_q = torch.from_numpy(wl.cu_seqlens_q).to(device)
        self.cu_k = torch.from_numpy(wl.cu_seqlens_k).to(device)
        self.func = torch.from_numpy(wl.func).to(device) if wl.func is not None else None

    def kw(self):
        wl = self.wl
        return dict(max_seqlen_q=wl.max_seqlen_q, max_seqlen_k=wl.max_seqlen_k, alpha=float(wl.alpha),
                    scaling_seqlen=wl.scaling_seqlen, causal=wl.causal, window_size=wl.window, func=self.func)

    def fwd(self, **over):
        kw = self.kw()
        kw.update(over)
        return hstu.hstu_fwd(self.q, self.k, self.v, self.cu_q, self.cu_k, **kw)

    def workspace(self, fill=0xFF, **over):
        """A dS workspace for hstu_bwd, or None when the mask has none; filled with
        bf16 NaN by default, so that a read of an entry no kernel wrote shows."""
        kw = self.kw()
        kw.update(over)
        kw.pop("store_ds", None)
        need = hstu.hstu_bwd_workspace_size(self.do, self.q, self.k, self.v, self.cu_q, self.cu_k, **kw)
        return torch.full((need,), fill, dtype=torch.uint8, device=self.q.device) if need else None

    def bwd(self, **over):
        """hstu_bwd; on the stored-dS path (the default where the mask allows it)
        with a NaN-filled workspace unless one is given."""
        kw = self.kw()
        kw.update(over)
        if kw.get("store_ds", True) and "workspace" not in kw:
            kw["workspace"] = self.workspace(**over)
        return hstu.hstu_bwd(self.do, self.q, self.k, self.v, self.cu_q, self.cu_k, **kw)


def check_close(name, got, ref, cu, rows=None):
    """Assert the bar and the per-sequence check; return (err/max, worst per-seq ratio)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    diff = np.abs(got - ref)
    refmax = float(np.abs(ref).max()) if ref.size else 0.0
    err = float(diff.max()) if diff.size else 0.0
    assert err <= REL_BAR * refmax + ABS_BAR, f"{name}: max err {err:.3e} > bar (max|ref| {refmax:.3e})"
    worst = 0.0
    rows = np.arange(ref.shape[0]) if rows is None else np.asarray(rows)
    for b in range(len(cu) - 1):
        sel = (rows >= cu[b]) & (rows < cu[b + 1])
        if not np.any(sel):
            continue
        e_b = float(diff[sel].max())
        m_b = float(np.abs(ref[sel]).max())
        assert e_b <= REL_SEQ * m_b + ABS_SEQ, \
            f"{name}: sequence {b}: err {e_b:.3e} vs max|ref| {m_b:.3e}"
        if m_b > 0:
            worst = max(worst, e_b / m_b)
    return (err / refmax if refmax > 0 else 0.0), worst


def sample_rows(cu: np.ndarray, per_seq: int = 48, seed: int = 0) -> np.ndarray:
    """Rows to compare at full size: all rows of short sequences; for long ones the
    first and last rows, rows around every 64/128 tile edge in a stride, and random rows."""
    rng = np.random.default_rng(seed)
    out = []
    for b in range(len(cu) - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        n = hi - lo
        if n <= per_seq:
            out.extend(range(lo, hi))
            continue
        pick = {0, 1, n - 1, n - 2}
        for edge in range(64, n, 64 * max(1, n // (64 * 8))):
            pick.update({edge - 1, edge})
        pick.update(rng.integers(0, n, size=per_seq // 2).tolist())
        out.extend(lo + i for i in sorted(p for p in pick if 0 <= p < n))
    return np.array(sorted(set(out)), dtype=np.int64)
