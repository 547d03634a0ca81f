"""Seeded synthetic inputs for HSTU attention over packed (THD) sequences.

This module only draws numbers: sequence lengths, cumulative offsets and the
bf16 bit patterns of q, k, v and the upstream gradient.  It holds none of the
attention arithmetic, so the CPU oracle and the HIP path can both take their
inputs from here without sharing any of the computation they are compared on.

Layout (HSTU Attention page, "Tensor layout" table): q/k/v/do are
``(T, H, D)`` packed token-major tensors; ``cu_seqlens`` is an int32 array of
``B + 1`` cumulative lengths starting at zero.

Recipe for every workload: ``numpy.random.default_rng(seed)`` (PCG64); the
lengths are drawn first (unless fixed), then q, k, v, each as
``standard_normal((T, H, D), float32) * scale`` rounded to bf16 with
round-to-nearest-even, then (for the backward workload) the upstream gradient
``standard_normal((T, H, D), float32)`` rounded the same way.  Key lengths equal
query lengths; the score scale is the fp32 value of ``1/sqrt(D)``; the
normaliser ``scaling_seqlen`` is the longest query length.  The mask is causal
or full (``causal``) unless a token window ``(left, right)`` is given (HSTU
Attention page, "Mask support": ``window_size``, -1 = unbounded side), or an
arbitrary mask: the page's ``func_tensor``, held here as an int32 ``(N, T_q)``
array whose column r lists the endpoints of packed query row r (visible keys
``[0, F0) u [F1, F2) u ...`` in local key indices).
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Workload",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "make_workload",
    "named_workload",
    "func_target_mask",
    "func_random_mask",
    "LmsdWorkload",
    "make_lmsd_workload",
    "lmsd_named_workload",
    "LMSD_WORKLOAD_NAMES",
    "WORKLOAD_NAMES",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    Inputs are finite normals, so NaN/Inf handling is not needed; it is
    rejected rather than silently mangled.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("f32_to_bf16_bits: non-finite input")
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    """One synthetic HSTU attention problem (host copies only)."""

    name: str
    seed: int
    lengths_q: np.ndarray          # (B,) int32
    lengths_k: np.ndarray          # (B,) int32
    cu_seqlens_q: np.ndarray       # (B+1,) int32
    cu_seqlens_k: np.ndarray       # (B+1,) int32
    num_heads: int
    head_dim: int
    causal: bool
    alpha: np.float32              # score scale as the fp32 value both sides use
    scaling_seqlen: int            # L_scale
    q: np.ndarray                  # (T_q, H, D) uint16 bf16 bits
    k: np.ndarray                  # (T_k, H, D) uint16
    v: np.ndarray                  # (T_k, H, D) uint16
    do: Optional[np.ndarray] = None  # (T_q, H, D) uint16, backward only
    window: Optional[Tuple[int, int]] = None  # (left, right); None: causal / full per `causal`
    func: Optional[np.ndarray] = None         # (N, T_q) int32 interval endpoints; overrides the rest

    @property
    def window_size(self) -> Tuple[int, int]:
        """The mask as a (left, right) token window, -1 = unbounded."""
        if self.window is not None:
            return self.window
        return (-1, 0) if self.causal else (-1, -1)

    @property
    def mask_spec(self):
        """The mask as the oracle takes it: the func array, else the window pair."""
        return self.func if self.func is not None else self.window_size

    @property
    def mask_name(self) -> str:
        if self.func is not None:
            return f"func(N={self.func.shape[0]})"
        left, right = self.window_size
        if (left, right) == (-1, -1):
            return "none"
        if (left, right) == (-1, 0):
            return "causal"
        return f"window({left},{right})"

    @property
    def batch(self) -> int:
        return int(self.lengths_q.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def total_k(self) -> int:
        return int(self.cu_seqlens_k[-1])

    @property
    def max_seqlen_q(self) -> int:
        return int(self.lengths_q.max()) if self.batch else 0

    @property
    def max_seqlen_k(self) -> int:
        return int(self.lengths_k.max()) if self.batch else 0


def _cumulative(lengths: np.ndarray) -> np.ndarray:
    cu = np.zeros(lengths.shape[0] + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    if cu[-1] > np.iinfo(np.int32).max:
        raise ValueError("total token count does not fit int32")
    return cu.astype(np.int32)


def _normal_bf16(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x = x * np.float32(scale)
    return f32_to_bf16_bits(x)


def make_workload(
    name: str,
    seed: int,
    lengths_q: Sequence[int],
    num_heads: int,
    head_dim: int,
    causal: bool,
    scale: float = 1.0,
    lengths_k: Optional[Sequence[int]] = None,
    with_do: bool = False,
    alpha: Optional[float] = None,
    scaling_seqlen: Optional[int] = None,
    rng: Optional[np.random.Generator] = None,
    window: Optional[Tuple[int, int]] = None,
    func: Optional[np.ndarray] = None,
) -> Workload:
    """Build a workload from explicit lengths.

    ``rng`` continues an existing stream (used when the lengths were drawn from
    it first); otherwise a fresh ``default_rng(seed)`` is used.
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    lq = np.asarray(lengths_q, dtype=np.int64)
    lk = lq.copy() if lengths_k is None else np.asarray(lengths_k, dtype=np.int64)
    if lq.shape != lk.shape or lq.ndim != 1:
        raise ValueError("lengths_q/lengths_k must be 1-D of equal length")
    if np.any(lq < 0) or np.any(lk < 0):
        raise ValueError("negative sequence length")
    if window is not None:
        window = (int(window[0]), int(window[1]))
        if min(window) < -1:
            raise ValueError("window bounds must be >= -1")
    cu_q = _cumulative(lq)
    cu_k = _cumulative(lk)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    H, D = int(num_heads), int(head_dim)
    q = _normal_bf16(rng, (tq, H, D), scale)
    k = _normal_bf16(rng, (tk, H, D), scale)
    v = _normal_bf16(rng, (tk, H, D), scale)
    do = _normal_bf16(rng, (tq, H, D), 1.0) if with_do else None
    a = np.float32(1.0 / np.sqrt(D)) if alpha is None else np.float32(alpha)
    if scaling_seqlen is None:
        ls = max(int(lq.max()) if lq.size else 0, 1)
    else:
        ls = int(scaling_seqlen)
    return Workload(
        name=name,
        seed=seed,
        lengths_q=lq.astype(np.int32),
        lengths_k=lk.astype(np.int32),
        cu_seqlens_q=cu_q,
        cu_seqlens_k=cu_k,
        num_heads=H,
        head_dim=D,
        causal=bool(causal),
        alpha=a,
        scaling_seqlen=int(ls),
        q=q,
        k=k,
        v=v,
        do=do,
        window=window,
        func=None if func is None else _check_func(func, tq),
    )


def _check_func(func: np.ndarray, total_q: int) -> np.ndarray:
    f = np.ascontiguousarray(func, dtype=np.int32)
    if f.ndim != 2 or f.shape[0] % 2 != 1 or f.shape[1] != total_q:
        raise ValueError("func must be (N, T_q) int32 with N odd")
    return f


def func_target_mask(lengths: Sequence[int], max_candidates: int = 256) -> np.ndarray:
    """Arbitrary-mask endpoints (N = 3) for a history + candidates layout: in a
    sequence of length L the last c = min(max_candidates, max(1, L // 8)) tokens are
    candidates.  History row i sees keys [0, i + 1) (causal); candidate row i sees
    the whole history [0, L - c) and itself [i, i + 1), no other candidate."""
    lengths = np.asarray(lengths, dtype=np.int64)
    total = int(lengths.sum())
    f = np.zeros((3, total), dtype=np.int32)
    r = 0
    for L in lengths.tolist():
        c = min(max_candidates, max(1, L // 8)) if L else 0
        h = L - c
        i = np.arange(L)
        hist = i < h
        f[0, r:r + L] = np.where(hist, i + 1, h)
        f[1, r:r + L] = np.where(hist, 0, i)
        f[2, r:r + L] = np.where(hist, 0, i + 1)
        r += L
    return f


def func_random_mask(rng: np.random.Generator, lengths_q: Sequence[int], lengths_k: Sequence[int],
                     n: int) -> np.ndarray:
    """Random endpoints, n (odd) per query row, drawn uniformly from
    [-3, L_k + 3] of the row's sequence: intervals overlap, come in any order,
    may be empty or reversed, and reach past both ends of the sequence."""
    if n % 2 != 1:
        raise ValueError("n must be odd")
    cols = []
    for lq, lk in zip(np.asarray(lengths_q).tolist(), np.asarray(lengths_k).tolist()):
        cols.append(rng.integers(-3, lk + 3, size=(n, lq), endpoint=True))
    f = np.concatenate(cols, axis=1) if cols else np.zeros((n, 0))
    return f.astype(np.int32)


# The seven synthetic workloads the measurement is defined on.  Names say what
# they are: batch, length law, heads, head dim and mask.
WORKLOAD_NAMES = (
    "tiny_b2_h1_d16_causal",          # B=2, lengths [5, 11]
    "uniform_b8_h2_d64_full",         # B=8, lengths U[64, 512]
    "zipf_b32_h4_d128_causal",        # B=32, Zipf(1.2) clipped to [16, 4096]
    "long_b4_h8_d128_causal",         # B=4, lengths U[8192, 16384]
    "zipf_b32_h4_d128_causal_fwdbwd",  # the Zipf workload plus an upstream gradient
    "long_b4_h8_d128_window1024",      # the long workload, sliding window (1024, 0), with gradient
    "zipf_b32_h4_d128_target_fwdbwd",  # the Zipf workload, history + candidates func mask, with gradient
)


def named_workload(name: str) -> Workload:
    """Return one of the seven synthetic workloads, fully deterministic."""
    if name == "tiny_b2_h1_d16_causal":
        return make_workload(name, 0, [5, 11], 1, 16, True, 1.0)
    if name == "uniform_b8_h2_d64_full":
        rng = np.random.default_rng(1)
        lens = rng.integers(64, 512, size=8, endpoint=True)
        return make_workload(name, 1, lens, 2, 64, False, 1.0, rng=rng)
    if name in ("zipf_b32_h4_d128_causal", "zipf_b32_h4_d128_causal_fwdbwd"):
        rng = np.random.default_rng(2)
        lens = np.clip(rng.zipf(1.2, size=32), 16, 4096)
        return make_workload(name, 2, lens, 4, 128, True, 0.5, rng=rng,
                             with_do=name.endswith("fwdbwd"))
    if name == "zipf_b32_h4_d128_target_fwdbwd":
        rng = np.random.default_rng(2)
        lens = np.clip(rng.zipf(1.2, size=32), 16, 4096)
        return make_workload(name, 2, lens, 4, 128, False, 0.5, rng=rng, with_do=True,
                             func=func_target_mask(lens))
    if name == "long_b4_h8_d128_causal":
        rng = np.random.default_rng(3)
        lens = rng.integers(8192, 16384, size=4, endpoint=True)
        return make_workload(name, 3, lens, 8, 128, True, 0.5, rng=rng)
    if name == "long_b4_h8_d128_window1024":
        rng = np.random.default_rng(3)
        lens = rng.integers(8192, 16384, size=4, endpoint=True)
        return make_workload(name, 3, lens, 8, 128, False, 0.5, rng=rng, with_do=True, window=(1024, 0))
    raise KeyError(f"unknown workload {name!r}; known: {WORKLOAD_NAMES}")


# ---------------------------------------------------------------------------
# HSTU LMSD (LayerNorm, affine, times SiLU(u)) inputs
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class LmsdWorkload:
    """One synthetic LMSD problem: N rows of D values (host copies, bf16 bits)."""

    name: str
    seed: int
    x: np.ndarray        # (N, D) uint16
    u: np.ndarray        # (N, D) uint16
    weight: np.ndarray   # (D,) uint16
    bias: np.ndarray     # (D,) uint16
    dy: Optional[np.ndarray]  # (N, S D) uint16, backward only
    eps: float
    silu_u: bool
    concat_u: bool
    concat_x: bool

    @property
    def n(self) -> int:
        return int(self.x.shape[0])

    @property
    def d(self) -> int:
        return int(self.x.shape[1])

    @property
    def segments(self) -> int:
        return 1 + int(self.concat_u) + int(self.concat_x)


def make_lmsd_workload(name: str, seed: int, n: int, d: int, silu_u: bool = True, concat_u: bool = True,
                       concat_x: bool = True, eps: float = 1e-6, with_dy: bool = True) -> LmsdWorkload:
    """Recipe: ``default_rng(seed)``; x, u ~ N(0, 1); weight ~ 1 + 0.1 N(0, 1);
    bias ~ 0.1 N(0, 1); then dy ~ N(0, 1) over the (N, S D) output; all float32
    draws rounded to bf16 (nearest, ties to even), in that order."""
    rng = np.random.default_rng(seed)
    x = _normal_bf16(rng, (n, d), 1.0)
    u = _normal_bf16(rng, (n, d), 1.0)
    w = f32_to_bf16_bits(1.0 + 0.1 * rng.standard_normal(d, dtype=np.float32))
    b = f32_to_bf16_bits(0.1 * rng.standard_normal(d, dtype=np.float32))
    s = 1 + int(concat_u) + int(concat_x)
    dy = _normal_bf16(rng, (n, s * d), 1.0) if with_dy else None
    return LmsdWorkload(name, seed, x, u, w, b, dy, float(eps), bool(silu_u), bool(concat_u), bool(concat_x))


# The LMSD workloads: the HSTU layer's normalisation of the attention output, one
# row per token of the Zipf workload (T = 23460) and D = H x d = 4 x 128 = 512,
# with both auxiliary segments (the page's first example's flags); and the
# page's own example shape (N = 257, D = 128).
LMSD_WORKLOAD_NAMES = ("lmsd_n23460_d512", "lmsd_n257_d128")


def lmsd_named_workload(name: str) -> LmsdWorkload:
    if name == "lmsd_n23460_d512":
        return make_lmsd_workload(name, 7, 23460, 512)
    if name == "lmsd_n257_d128":
        return make_lmsd_workload(name, 8, 257, 128)
    raise KeyError(f"unknown LMSD workload {name!r}; known: {LMSD_WORKLOAD_NAMES}")
