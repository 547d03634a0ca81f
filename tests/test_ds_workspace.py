"""The stored-dS workspace size (hstu_bwd_workspace_size) against the blocks the
backward kernels address, on the host only.

The library sizes the workspace from T_q, T_k, B, max_seqlen_q/k alone (it never
reads cu_seqlens on the host), so the size must bound the packed layout for every
length mix those sizes allow: sequence b keeps ceil(L_q/32) row blocks, each with
min(R + 1, ceil(L_k/32)) key groups under the causal mask (row block R) and all
ceil(L_k/32) otherwise; the heads follow one another.  Random mixes, including
ones that reach the bound, must all fit."""

import ctypes
import os

import numpy as np
import pytest

from generative_recommender_attention_amd import hstu


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hstu.library_path()):
        pytest.skip("libhstu.so is not built")
    return hstu.library()


def needed_blocks(lq, lk, causal):
    n = 0
    for a, b in zip(lq, lk):
        nR, nG = -(-a // 32), -(-b // 32)
        n += sum(min(R + 1, nG) for R in range(nR)) if causal else nR * nG
    return n


def ws_blocks(lib, lq, lk, causal, H=3):
    a = hstu.HstuArgs()
    a.batch, a.total_q, a.total_k, a.num_heads, a.head_dim = len(lq), sum(lq), sum(lk), H, 64
    a.max_seqlen_q, a.max_seqlen_k, a.alpha, a.scaling_seqlen = max(lq), max(lk), 0.1, 0
    a.mask = hstu.HSTU_MASK_CAUSAL if causal else hstu.HSTU_MASK_NONE
    n = ctypes.c_size_t(0)
    assert lib.hstu_bwd_workspace_size(ctypes.byref(a), ctypes.byref(n)) == hstu.HSTU_OK
    assert n.value % (2048 * H) == 0
    return n.value // (2048 * H)


@pytest.mark.parametrize("causal", [True, False])
def test_workspace_covers_every_length_mix(lib, causal):
    rng = np.random.default_rng(11 if causal else 12)
    tight = 0
    for _ in range(3000):
        B = int(rng.integers(1, 40))
        lmax = int(rng.choice([31, 32, 33, 100, 500, 4096]))
        lq = rng.integers(0, lmax + 1, size=B).tolist()
        lk = list(lq) if rng.random() < 0.5 else rng.integers(0, lmax + 1, size=B).tolist()
        if rng.random() < 0.3:  # push mass to the longest length, where the bound is reached
            lq = [lmax if rng.random() < 0.7 else x for x in lq]
            lk = list(lq)
        lk = [max(a, b) for a, b in zip(lq, lk)] if max(lk) < max(lq) else lk
        if max(lq) == 0 or max(lk) == 0:
            continue
        need, have = needed_blocks(lq, lk, causal), ws_blocks(lib, lq, lk, causal)
        assert need <= have, (lq, lk, need, have)
        tight += need == have
    assert tight > 0  # the bound is reached by some mixes, not just an overestimate


def test_compact_sizes_of_the_named_workloads(lib):
    """Zipf (B=32, T=23460, max 4096, H=4) and the long workload (B=4, T=43527, max
    14840, H=8), causal: the triangle bound against the per-row-block-slot layout
    it replaced (every row block slot holding all 4 ceil(max/128) key groups)."""
    for B, T, L, H, mb in ((32, 23460, 4096, 4, 402), (4, 43527, 14840, 8, 5096)):
        a = hstu.HstuArgs()
        a.batch, a.total_q, a.total_k, a.num_heads, a.head_dim = B, T, T, H, 128
        a.max_seqlen_q, a.max_seqlen_k, a.alpha, a.scaling_seqlen, a.mask = L, L, 0.1, 0, hstu.HSTU_MASK_CAUSAL
        n = ctypes.c_size_t(0)
        assert lib.hstu_bwd_workspace_size(ctypes.byref(a), ctypes.byref(n)) == hstu.HSTU_OK
        old = H * ((T + 31 * B) // 32) * 4 * (-(-L // 128)) * 2048
        assert round(n.value / 1e6) == mb and n.value < 0.51 * old, (n.value, old)
