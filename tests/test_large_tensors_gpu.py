"""Tensors past 2^31 elements and 4 GiB: T = 2^21 tokens in 8192 causal sequences
of 256, H = 16, D = 128, so every (T, H, D) tensor holds 2^32 bf16 elements (8 GiB)
and the kernels form element offsets up to 2^32 and byte offsets up to 8 GiB
(32-bit offset arithmetic anywhere would show here).  The forward and the
stored-dS backward run on the whole tensors, then the fused backward (its fp32 dQ
accumulator holds 16 GiB; its dK and dV must equal the stored route's bit for bit
over the whole tensors) and a forward under a token window (64, 0) -- ~120 GiB of
device memory in all.  Sequences at the start, middle and end of the buffers are
compared with the fp64 oracle, each as its own problem, to the bar of
tests/hip_cases.py.

Inputs are drawn on the device by torch's seeded generator (bf16 normals times 0.5,
an exact scaling); the oracle reads the same bits, copied back per sequence."""

import math

import numpy as np
import pytest
import torch

from generative_recommender_attention_amd import hstu

from hip_cases import check_close, say, to_f64

pytestmark = pytest.mark.gpu

T, B, L, H, D = 1 << 21, 8192, 256, 16, 128
NEED_BYTES = 140 << 30  # inputs, outputs, workspaces and headroom
SAMPLED = [0, 1, B // 2, B - 2, B - 1]


def test_tensors_past_4gib_fwd_bwd(oracle_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    free, _ = torch.cuda.mem_get_info()
    if free < NEED_BYTES:
        pytest.skip(f"needs {NEED_BYTES >> 30} GiB of free device memory, {free >> 30} GiB free")
    gen = torch.Generator(device="cuda").manual_seed(500)

    def draw():
        t = torch.randn((T, H, D), generator=gen, device="cuda", dtype=torch.bfloat16)
        return t.mul_(0.5)

    say(f"large tensors: T={T} B={B} L={L} H={H} D={D}, {T * H * D} elements per tensor")
    q, k, v, do = draw(), draw(), draw(), draw()
    cu = torch.arange(0, T + 1, L, dtype=torch.int32, device="cuda")
    alpha = float(np.float32(1.0 / math.sqrt(D)))
    kw = dict(max_seqlen_q=L, max_seqlen_k=L, alpha=alpha, scaling_seqlen=L, causal=True)
    assert q.numel() == 1 << 32 and q.numel() * q.element_size() == 8 << 30
    say("large tensors: hstu_fwd")
    o = hstu.hstu_fwd(q, k, v, cu, cu, **kw)
    say("large tensors: hstu_bwd (stored dS)")
    ws_bytes = hstu.hstu_bwd_workspace_size(do, q, k, v, cu, cu, **kw)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    dq, dk, dv = hstu.hstu_bwd(do, q, k, v, cu, cu, workspace=ws, **kw)
    torch.cuda.synchronize()
    del ws
    say("large tensors: hstu_bwd_fused")
    fdq, fdk, fdv = hstu.hstu_bwd_fused(do, q, k, v, cu, cu, **kw)
    torch.cuda.synchronize()
    assert torch.equal(fdk, dk) and torch.equal(fdv, dv)  # the same pass computes them
    del fdk, fdv
    say("large tensors: hstu_fwd under the window (64, 0)")
    ow = hstu.hstu_fwd(q, k, v, cu, cu, **dict(kw, causal=False), window_size=(64, 0))
    torch.cuda.synchronize()

    cu1 = np.array([0, L], dtype=np.int32)
    bits = lambda t, r0: t[r0:r0 + L].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    for b in SAMPLED:
        r0 = b * L
        say(f"large tensors: sequence {b} (rows {r0}..{r0 + L - 1}) against the oracle")
        qs, ks, vs, dos = bits(q, r0), bits(k, r0), bits(v, r0), bits(do, r0)
        ro = oracle_lib.fwd(cu1, cu1, qs, ks, vs, alpha, L, (-1, 0))
        rq = oracle_lib.bwd_dq(cu1, cu1, dos, qs, ks, vs, alpha, L, (-1, 0))
        rk, rv = oracle_lib.bwd_dkdv(cu1, cu1, dos, qs, ks, vs, alpha, L, (-1, 0))
        rw = oracle_lib.fwd(cu1, cu1, qs, ks, vs, alpha, L, (64, 0))
        for name, got, ref in (("O", o, ro), ("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv),
                               ("fused dQ", fdq, rq), ("window O", ow, rw)):
            check_close(f"{name} of sequence {b}", to_f64(got[r0:r0 + L]), ref, cu1)
