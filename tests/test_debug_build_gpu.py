"""The debug build (libhstu_debug.so, -DHSTU_DEBUG) on the GPU: its kernels test the
global indices they form and record failed tests (hstu_debug_take).

* On valid inputs across the masks, head dims and entry points, no test may fail,
  and every output must equal the release build's bit for bit (the tests only
  observe; the fused backward's dQ, whose summation order is not fixed, is compared
  against the bar instead).
* A test does fire: the arguments claim fewer query rows than the cumulative
  lengths give, while the tensors are views of larger allocations that hold every
  row the kernels touch -- the report comes from the bounds test alone, with no
  access outside any buffer.
"""

import numpy as np
import pytest
import torch

from generative_recommender_attention_amd import hstu
from generative_recommender_attention_amd.workloads import func_random_mask, make_lmsd_workload, make_workload

from hip_cases import DeviceWorkload, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu_and_debug_build():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    hstu.library(debug=False)
    hstu.library(debug=True)
    prev = hstu.select_library(False)
    yield
    hstu.select_library(prev)


def _cases():
    lens = [200, 64, 129, 7, 0, 300]
    rng = np.random.default_rng(401)
    f3 = func_random_mask(rng, lens, lens, 3)
    f5 = func_random_mask(rng, lens, lens, 5)
    return [
        ("causal_d128", make_workload("dbg0", 400, lens, 3, 128, True, 0.5, with_do=True)),
        ("full_d64", make_workload("dbg1", 401, lens, 2, 64, False, 0.5, with_do=True)),
        ("window_d32", make_workload("dbg2", 402, lens, 2, 32, False, 0.5, with_do=True, window=(50, 3))),
        ("func3_d16", make_workload("dbg3", 403, lens, 2, 16, False, 0.5, with_do=True, func=f3)),
        ("func5_d128", make_workload("dbg4", 404, lens, 1, 128, False, 0.5, with_do=True, func=f5)),
        ("b70_causal_d64", make_workload("dbg5", 405, [int(x) for x in rng.integers(0, 90, 70)], 2, 64, True, 0.5,
                                         with_do=True)),
    ]


CASES = _cases()


def _run(dw):
    """O; dQ, dK, dV through both backward routes; the fused backward."""
    kw = dw.kw()
    out = {"o": dw.fwd()}
    for name, store in (("stored", True), ("recompute", False)):
        out[name] = dw.bwd(store_ds=store)
    out["fused"] = hstu.hstu_bwd_fused(dw.do, dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name,wl", CASES, ids=[c[0] for c in CASES])
def test_debug_build_records_nothing_and_matches_release(name, wl):
    dw = DeviceWorkload(wl)
    hstu.select_library(False)  # the fixture restores the session's choice
    say(f"release build: {name}")
    ref = _run(dw)
    prev = hstu.select_library(True)
    try:
        hstu.debug_take()  # clear anything an earlier call left
        say(f"debug build: {name}")
        got = _run(dw)
        sites = hstu.debug_take()
    finally:
        hstu.select_library(prev)
    assert sites == 0, {b: n for b, n in hstu.DEBUG_SITES.items() if sites >> b & 1}
    assert torch.equal(got["o"], ref["o"])
    for route in ("stored", "recompute"):
        for i, t in enumerate("qkv"):
            assert torch.equal(got[route][i], ref[route][i]), f"{route} d{t}"
    assert torch.equal(got["fused"][1], ref["fused"][1]) and torch.equal(got["fused"][2], ref["fused"][2])
    a, b = got["fused"][0].float(), ref["fused"][0].float()
    assert (a - b).abs().max() <= 1e-2 * b.abs().max() + 1e-3  # fp32 atomics in arrival order


def test_debug_build_lmsd_records_nothing_and_matches_release():
    wl = make_lmsd_workload("dbglmsd", 406, 700, 256)
    x, u, w, b, dy = (to_dev(t) for t in (wl.x, wl.u, wl.weight, wl.bias, wl.dy))
    res = {}
    prev = hstu.select_library(False)
    try:
        for debug in (False, True):
            hstu.select_library(debug)
            say(f"LMSD fwd + bwd + bwd_noalloc, {'debug' if debug else 'release'} build")
            y, mean, rstd = hstu.lmsd_fwd(x, u, w, b)
            g = hstu.lmsd_bwd(dy, x, u, w, b, mean, rstd)
            dx, du, dwt, db = (torch.empty_like(t) for t in g)
            hstu.lmsd_bwd_noalloc(dy, x, u, w, b, mean, rstd, dx, du, dwt, db)
            torch.cuda.synchronize()
            res[debug] = (y, mean, rstd, *g, dx, du, dwt, db)
            if debug:
                sites = hstu.debug_take()
    finally:
        hstu.select_library(prev)
    assert sites == 0, {k: n for k, n in hstu.DEBUG_SITES.items() if sites >> k & 1}
    for i, (a, r) in enumerate(zip(res[True], res[False])):
        assert torch.equal(a, r), i


def test_debug_build_reports_rows_past_the_claimed_total():
    """cu_seqlens reaches T = 400 query rows while the arguments say 392 (q and o
    are the first 392 rows of 400-row tensors): the forward reads and writes rows
    392..399 of those allocations, and the debug build reports the sequence-bounds
    site.  k and v are whole; every access stays inside the buffers."""
    lens = [150, 250]
    wl = make_workload("dbglie", 407, lens, 2, 64, True, 0.5)
    dw = DeviceWorkload(wl)
    T = int(wl.total_q)
    o_full = torch.zeros_like(dw.q)
    q_view, o_view = dw.q[: T - 8], o_full[: T - 8]
    kw = dw.kw()
    prev = hstu.select_library(True)
    try:
        hstu.debug_take()
        say("debug build: forward with total_q below cu_seqlens_q[B] (views of larger buffers)")
        hstu.hstu_fwd(q_view, dw.k, dw.v, dw.cu_q, dw.cu_k, out=o_view, **kw)
        sites = hstu.debug_take()
    finally:
        hstu.select_library(prev)
    assert sites & 1, sites  # bit 0: a sequence's tokens outside [0, total)
