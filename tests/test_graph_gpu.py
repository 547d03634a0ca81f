"""The entry points under HIP graph capture (the header's claim: calls keep no
state, never synchronise and never allocate, so they can be captured).

Each graph is replayed several times with eager work and synchronisation in
between, and every replay is compared bit for bit with the eager result (the
library records no memset nodes; the check would catch one that goes stale
after the first replay)."""

import numpy as np
import pytest
import torch

from generative_recommender_attention_amd import hstu
from generative_recommender_attention_amd.workloads import func_random_mask, make_lmsd_workload, make_workload

from hip_cases import DeviceWorkload, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    hstu.library()


@pytest.mark.parametrize("mask", ["causal", "window", "func"])
def test_attention_fwd_bwd_graph_replays(mask):
    lens = [200, 64, 129, 7]
    if mask == "func":
        i = np.concatenate([np.arange(n) for n in lens])
        func = np.stack([i // 2 + 1, i, i + 3]).astype(np.int32)  # [0, i/2 + 1) u [i, i + 3)
        wl = make_workload("g", 160, lens, 2, 128, False, with_do=True, func=func)
    elif mask == "window":
        wl = make_workload("g", 161, lens, 2, 128, False, with_do=True, window=(50, 3))
    else:
        wl = make_workload("g", 162, lens, 2, 128, True, with_do=True)
    dw = DeviceWorkload(wl)
    kw = dw.kw()
    o = torch.empty_like(dw.q)
    dq, dk, dv = torch.empty_like(dw.q), torch.empty_like(dw.k), torch.empty_like(dw.v)
    ws = dw.workspace()  # stored dS under the causal mask; None (recompute) under the others
    say(f"graph capture: attention fwd + bwd, mask {mask}")
    o_ref = dw.fwd()
    g_ref = dw.bwd()
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            hstu.hstu_fwd(dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, out=o, **kw)
            hstu.hstu_bwd(dw.do, dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for t in (o, dq, dk, dv):
            t.fill_(float("nan"))  # eager work between replays; the replay must overwrite it all
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {rep}: O"
        for name, got, ref in (("dQ", dq, g_ref[0]), ("dK", dk, g_ref[1]), ("dV", dv, g_ref[2])):
            assert torch.equal(got, ref), f"replay {rep}: {name}"


def test_func_changed_in_place_is_seen_on_replay():
    """The arbitrary mask's endpoints are read by the kernels at run time (HSTU page,
    "Mask support": an in-place change of func_tensor is visible, also under graph
    replay): the graph is captured once on one set of endpoints, the endpoint tensor
    is overwritten in place before each replay, and every replay must equal, bit for
    bit, an eager run on the endpoints it saw."""
    lens = [200, 64, 129, 7]
    rng = np.random.default_rng(164)
    i = np.concatenate([np.arange(n) for n in lens])
    ends = [np.stack([i + 1, i, i]).astype(np.int32),                   # causal
            np.stack([i // 2 + 1, i, i + 3]).astype(np.int32),          # [0, i/2 + 1) u [i, i + 3)
            np.stack([np.zeros_like(i), np.maximum(i - 20, 0), i + 1]).astype(np.int32),  # window (20, 0)
            func_random_mask(rng, lens, lens, 3)]
    wl = make_workload("gf", 165, lens, 2, 128, False, with_do=True, func=ends[0])
    dw = DeviceWorkload(wl)
    kw = dw.kw()
    func = kw["func"]  # the device tensor the graph reads
    o = torch.empty_like(dw.q)
    dq, dk, dv = torch.empty_like(dw.q), torch.empty_like(dw.k), torch.empty_like(dw.v)
    say("graph capture: attention fwd + bwd under the arbitrary mask, endpoints changed in place")
    hstu.hstu_fwd(dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, out=o, **kw)  # warm up outside capture
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            hstu.hstu_fwd(dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, out=o, **kw)
            hstu.hstu_bwd(dw.do, dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, dq=dq, dk=dk, dv=dv, **kw)
    torch.cuda.current_stream().wait_stream(s)
    for rep, e in enumerate(ends[1:] + ends[:1]):
        func.copy_(torch.from_numpy(e))  # in place: same storage the graph captured
        ref_kw = dict(kw, func=torch.from_numpy(e.copy()).cuda())
        o_ref = hstu.hstu_fwd(dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, **ref_kw)
        g_ref = hstu.hstu_bwd(dw.do, dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, **ref_kw)
        for t in (o, dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {rep}: O"
        for name, got, ref in (("dQ", dq, g_ref[0]), ("dK", dk, g_ref[1]), ("dV", dv, g_ref[2])):
            assert torch.equal(got, ref), f"replay {rep}: {name}"


def test_lmsd_graph_replays():
    wl = make_lmsd_workload("glmsd", 163, 700, 256)
    x, u, w, b, dy = (to_dev(t) for t in (wl.x, wl.u, wl.weight, wl.bias, wl.dy))
    say("graph capture: LMSD fwd + bwd")
    y_ref, m_ref, r_ref = hstu.lmsd_fwd(x, u, w, b)
    g_ref = hstu.lmsd_bwd(dy, x, u, w, b, m_ref, r_ref)
    torch.cuda.synchronize()
    y, mean, rstd = torch.empty_like(y_ref), torch.empty_like(m_ref), torch.empty_like(r_ref)
    dx, du, dwt, db = torch.empty_like(x), torch.empty_like(u), torch.empty_like(w), torch.empty_like(b)
    ws = torch.empty(hstu.lmsd_bwd_workspace_size(x, u), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            hstu.lmsd_fwd(x, u, w, b, y=y, mean=mean, rstd=rstd)
            hstu.lmsd_bwd(dy, x, u, w, b, mean, rstd, dx=dx, du=du, dweight=dwt, dbias=db, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for t in (y, dx, du, dwt, db, mean, rstd):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(mean, m_ref) and torch.equal(rstd, r_ref), f"replay {rep}: fwd"
        for name, got, ref in zip(("dx", "du", "dweight", "dbias"), (dx, du, dwt, db), g_ref):
            assert torch.equal(got, ref), f"replay {rep}: {name}"
