"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Every problem is compared element by element on whole tensors, except the
backward of the long 4 x 8k-15k causal workload, whose oracle would take
minutes: there the rows compared are sampled (every row of short sequences,
first/last rows, rows on both sides of tile edges, random rows).
"""

import numpy as np
import pytest
import torch

import oracle
from generative_recommender_attention_amd import hstu
from generative_recommender_attention_amd.workloads import func_random_mask, make_workload, named_workload

from hip_cases import DeviceWorkload, check_close, sample_rows, say, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    hstu.library()  # no fallback: a missing library fails here


def run_fwd_check(wl, rows=None, tag=""):
    dw = DeviceWorkload(wl)
    say(f"hstu_fwd {wl.name}{tag}: B={wl.batch} T={wl.total_q} H={wl.num_heads} D={wl.head_dim} mask={wl.mask_name}")
    o = dw.fwd()
    torch.cuda.synchronize()
    got = to_f64(o)
    ref = oracle.fwd_workload(wl, rows)
    if rows is not None:
        got = got[rows]
    return check_close("O", got, ref, wl.cu_seqlens_q, rows)


def run_bwd_check(wl, rows_q=None, rows_k=None, tag=""):
    """Both backward routes against one oracle evaluation: dQ from stored dS and dQ
    from recomputed scores."""
    dw = DeviceWorkload(wl)
    routes = [True, False]
    rq, rk, rv = oracle.bwd_workload(wl, rows_q, rows_k)
    res = []
    for store in routes:
        say(f"hstu_bwd {wl.name}{tag} ({'stored dS' if store else 'recompute'}): B={wl.batch} Tq={wl.total_q} "
            f"Tk={wl.total_k} H={wl.num_heads} D={wl.head_dim} mask={wl.mask_name}")
        dq, dk, dv = dw.bwd(store_ds=store)
        torch.cuda.synchronize()
        gq, gk, gv = to_f64(dq), to_f64(dk), to_f64(dv)
        if rows_q is not None:
            gq = gq[rows_q]
        if rows_k is not None:
            gk, gv = gk[rows_k], gv[rows_k]
        res.append((check_close("dQ", gq, rq, wl.cu_seqlens_q, rows_q),
                    check_close("dK", gk, rk, wl.cu_seqlens_k, rows_k),
                    check_close("dV", gv, rv, wl.cu_seqlens_k, rows_k)))
    return res[0]


# ---------------------------------------------------------------- the workloads
def test_tiny_workload_fwd(oracle_lib):
    run_fwd_check(named_workload("tiny_b2_h1_d16_causal"))


def test_uniform_workload_fwd(oracle_lib):
    run_fwd_check(named_workload("uniform_b8_h2_d64_full"))


def test_zipf_workloads_full(oracle_lib):
    """The Zipf forward workload and the Zipf forward + backward workload, every row:
    both draw q, k, v from seed 2 in the same order (the backward one draws dO after
    them), so one forward comparison covers both; the backward goes through both
    routes against one oracle evaluation."""
    fwd_wl = named_workload("zipf_b32_h4_d128_causal")
    wl = named_workload("zipf_b32_h4_d128_causal_fwdbwd")
    for name in ("q", "k", "v", "cu_seqlens_q", "cu_seqlens_k"):
        assert np.array_equal(getattr(fwd_wl, name), getattr(wl, name)), name
    rel, worst = run_fwd_check(wl)
    print(f"zipf fwd: err/max {rel:.2e}, worst per-sequence {worst:.2e}")
    res = run_bwd_check(wl)
    print("zipf bwd (err/max, worst per-seq):", res)


def test_long_workload_fwd_full(oracle_lib):
    wl = named_workload("long_b4_h8_d128_causal")
    rel, worst = run_fwd_check(wl)
    print(f"long fwd: err/max {rel:.2e}, worst per-sequence {worst:.2e}")


def test_long_workload_fwd_bwd_sampled(oracle_lib):
    # the longest walks (up to 256 tiles of 64) through both backward routes, at full
    # size; the oracle's backward over all 43527 rows and 8 heads would take minutes,
    # so the rows compared are sampled (every tile edge in a stride, first and last
    # rows, random rows), dK and dV on the same row set
    rng = np.random.default_rng(3)  # the long causal workload's lengths and inputs, plus dO
    lens = rng.integers(8192, 16384, size=4, endpoint=True)
    wl = make_workload("long_b4_h8_d128_causal_fwdbwd", 3, lens, 8, 128, True, 0.5, rng=rng, with_do=True)
    rows = sample_rows(wl.cu_seqlens_q, per_seq=48, seed=6)
    res = run_bwd_check(wl, rows, rows, " (sampled rows)")
    print("long bwd (err/max, worst per-seq):", res)


# ------------------------------------------------------------------ large scores
def large_score_workload(tag, seed, D, q_k_scale=1.0, alpha=None):
    """Scores far outside the N(0, 1) range of the named workloads: q and k scaled by
    a power of two (exact in bf16) or a large alpha.  With |s| in the hundreds,
    2^y in the kernels' sigmoid overflows to infinity for large negative s (the
    reciprocal then gives 0), sig(s) rounds to exactly 0 or 1 on both sides, and
    SiLU(s) and SiLU'(s) approach their asymptotes s, 0 and 1, 0."""
    wl = make_workload(f"big{tag}", seed, [300, 129, 64, 17, 1], 2, D, True, 1.0, with_do=True, alpha=alpha)
    if q_k_scale != 1.0:
        from generative_recommender_attention_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits

        wl.q = f32_to_bf16_bits(bf16_bits_to_f32(wl.q) * np.float32(q_k_scale))
        wl.k = f32_to_bf16_bits(bf16_bits_to_f32(wl.k) * np.float32(q_k_scale))
    return wl


LARGE_SCORE_CASES = [
    # (tag, seed, D, q and k scale, alpha, least max|s| the case must reach)
    ("qk8_d64", 200, 64, 8.0, None, 150.0),      # 2^(c x) overflows to +inf (alpha x < -88.7)
    ("qk8_d128", 201, 128, 8.0, None, 150.0),
    ("qk2_d128", 202, 128, 2.0, None, 15.0),     # sig(s) rounds to 1 in fp32 (s > 16.6)
    ("alpha4_d128", 203, 128, 1.0, 4.0, 100.0),
]


@pytest.mark.parametrize("case", LARGE_SCORE_CASES, ids=[c[0] for c in LARGE_SCORE_CASES])
def test_large_scores_fwd_bwd(oracle_lib, case):
    tag, seed, D, scale, alpha, least = case
    wl = large_score_workload(tag, seed, D, scale, alpha)
    q, k = oracle.widen(wl.q), oracle.widen(wl.k)
    smax = float(wl.alpha) * max(float(np.abs(q[:300, h] @ k[:300, h].T).max()) for h in range(wl.num_heads))
    say(f"large scores {tag}: max |s| over the first sequence {smax:.0f}")
    assert smax > least  # the case reaches the saturated range it is meant to cover
    run_fwd_check(wl, tag=f" ({tag})")
    run_bwd_check(wl, tag=f" ({tag})")


# ------------------------------------------------------------ shapes and edges
EDGE_LENGTHS = [0, 1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 200]

RANDOM_CASES = [
    # (seed, lengths_q, lengths_k or None, H, D, causal)
    (100, EDGE_LENGTHS, None, 2, 16, True),
    (101, EDGE_LENGTHS, None, 2, 32, False),
    (102, EDGE_LENGTHS, None, 1, 64, True),
    (103, EDGE_LENGTHS, None, 2, 128, True),
    (104, EDGE_LENGTHS, None, 2, 128, False),
    (105, [300, 5, 0, 257], [310, 9, 4, 257], 2, 64, True),     # L_k > L_q, top-left causal
    (106, [130, 40, 7], [131, 38, 3], 3, 32, False),            # L_k < L_q in two sequences, full
    (107, [3] * 40 + [250], None, 1, 128, True),                # many tiny sequences
]


@pytest.mark.parametrize("case", RANDOM_CASES, ids=[f"seed{c[0]}_d{c[4]}_{'causal' if c[5] else 'full'}"
                                                    for c in RANDOM_CASES])
def test_random_shapes_fwd_bwd(oracle_lib, case):
    seed, lq, lk, H, D, causal = case
    wl = make_workload(f"edge{seed}", seed, lq, H, D, causal, 1.0, lengths_k=lk, with_do=True)
    run_fwd_check(wl)
    run_bwd_check(wl)


@pytest.mark.parametrize("mask", ["causal", "full", "window", "func"])
def test_more_than_64_sequences(oracle_lib, mask):
    """B > 64: the live-block numbering sums the sequences' block counts over
    several 64-sequence chunks; zero-length sequences sit in every chunk."""
    rng = np.random.default_rng(170)
    lens = rng.integers(0, 300, size=150)
    lens[::17] = 0
    lens[5] = 700
    if mask == "func":
        f = func_random_mask(np.random.default_rng(171), lens, lens, 3)
        wl = make_workload("b150f", 172, lens, 2, 64, False, 1.0, with_do=True, func=f)
    elif mask == "window":
        wl = make_workload("b150w", 173, lens, 2, 64, False, 1.0, with_do=True, window=(40, 7))
    else:
        wl = make_workload("b150", 174, lens, 2, 64, mask == "causal", 1.0, with_do=True)
    run_fwd_check(wl)
    run_bwd_check(wl)


def test_explicit_scaling_seqlen_and_alpha(oracle_lib):
    wl = make_workload("ls", 110, [90, 33], 2, 64, True, 1.0, with_do=True, alpha=0.3, scaling_seqlen=7)
    run_fwd_check(wl)
    run_bwd_check(wl)


def test_single_long_sequence_full_mask(oracle_lib):
    wl = make_workload("single", 111, [777], 1, 128, False, 0.5, with_do=True)
    run_fwd_check(wl)
    run_bwd_check(wl)


# ------------------------------------------------------------------ token windows
WINDOW_CASES = [
    # (seed, lengths_q, lengths_k or None, H, D, (left, right))
    (130, EDGE_LENGTHS, None, 2, 128, (64, 0)),
    (131, EDGE_LENGTHS, None, 2, 64, (0, 0)),                    # diagonal only
    (132, EDGE_LENGTHS, None, 1, 32, (100, 37)),                 # bounds off the tile grid
    (133, EDGE_LENGTHS, None, 2, 16, (-1, 65)),                  # right bound only
    (134, EDGE_LENGTHS, None, 2, 128, (129, -1)),                # left bound only
    (135, [300, 5, 0, 257], [310, 9, 4, 257], 2, 64, (31, 3)),   # L_k > L_q
    (136, [130, 40, 7], [131, 38, 3], 3, 128, (5, 70)),          # L_k < L_q
    (137, [700, 1000], None, 2, 128, (256, 128)),                # interior tiles with no per-element test
    (138, [3] * 40 + [250], None, 1, 128, (1, 1)),               # many tiny sequences
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=[f"seed{c[0]}_d{c[4]}_w{c[5][0]}_{c[5][1]}"
                                                    for c in WINDOW_CASES])
def test_window_fwd_bwd(oracle_lib, case):
    seed, lq, lk, H, D, window = case
    wl = make_workload(f"win{seed}", seed, lq, H, D, False, 1.0, lengths_k=lk, with_do=True, window=window)
    run_fwd_check(wl)
    run_bwd_check(wl)


def test_long_window_workload_full(oracle_lib):
    wl = named_workload("long_b4_h8_d128_window1024")
    rel, worst = run_fwd_check(wl)
    print(f"long window fwd: err/max {rel:.2e}, worst per-sequence {worst:.2e}")
    res = run_bwd_check(wl)
    print("long window bwd (err/max, worst per-seq):", res)


def test_windows_naming_full_and_causal_are_those_masks_bitwise():
    """(-1, 0) and (-1, -1) run the causal and full kernels; a window whose bounds
    reach past every sequence runs the window kernel and must agree bit for bit
    with full attention (same tiles, same order, only the masking path differs)."""
    wl = make_workload("wnames", 139, [200, 64, 129], 2, 64, True, with_do=True)
    dw = DeviceWorkload(wl)
    say("window (-1, 0) vs causal, (-1, -1) and (500, 500) vs full")
    oc, gc = dw.fwd(causal=True), dw.bwd(causal=True)
    ow, gw = dw.fwd(window_size=(-1, 0)), dw.bwd(window_size=(-1, 0))
    of, gf = dw.fwd(causal=False), dw.bwd(causal=False)
    on, gn = dw.fwd(window_size=(-1, -1)), dw.bwd(window_size=(-1, -1))
    ob, gb = dw.fwd(window_size=(500, 500)), dw.bwd(window_size=(500, 500))
    gfr, gbr = dw.bwd(causal=False, store_ds=False), dw.bwd(window_size=(500, 500), store_ds=False)
    torch.cuda.synchronize()
    assert torch.equal(oc, ow) and all(torch.equal(a, b) for a, b in zip(gc, gw))
    assert torch.equal(of, on) and all(torch.equal(a, b) for a, b in zip(gf, gn))
    # the wide window stores dS relative to each row block, the full mask by key group: same values
    assert torch.equal(of, ob) and all(torch.equal(a, b) for a, b in zip(gf, gb))
    assert all(torch.equal(a, b) for a, b in zip(gfr, gbr))


def test_window_invalid_bounds_raise():
    wl = make_workload("wbad", 140, [10], 1, 16, True)
    dw = DeviceWorkload(wl)
    with pytest.raises(hstu.HstuError):
        dw.fwd(window_size=(-2, 0))
    with pytest.raises(hstu.HstuError):
        hstu.hstu_bwd(dw.q, dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, 10, 10, window_size=(3, -7))


# ------------------------------------------------------------------ arbitrary interval masks
FUNC_CASES = [
    # (seed, lengths_q, lengths_k or None, H, D, endpoints per row)
    (150, EDGE_LENGTHS, None, 2, 128, 3),
    (151, EDGE_LENGTHS, None, 2, 64, 1),
    (152, EDGE_LENGTHS, None, 1, 32, 5),
    (153, EDGE_LENGTHS, None, 2, 16, 3),
    (154, [300, 5, 0, 257], [310, 9, 4, 257], 2, 128, 5),     # L_k > L_q
    (155, [130, 40, 7], [131, 38, 3], 3, 64, 3),              # L_k < L_q
    (156, [700, 1000], None, 2, 128, 1),                      # long rows, one interval [0, F0)
]


@pytest.mark.parametrize("case", FUNC_CASES, ids=[f"seed{c[0]}_d{c[4]}_n{c[5]}" for c in FUNC_CASES])
def test_func_mask_fwd_bwd(oracle_lib, case):
    seed, lq, lk, H, D, n = case
    lk = lq if lk is None else lk
    f = func_random_mask(np.random.default_rng(seed), lq, lk, n)
    wl = make_workload(f"func{seed}", seed, lq, H, D, False, 1.0, lengths_k=lk, with_do=True, func=f)
    run_fwd_check(wl)
    run_bwd_check(wl)


def test_func_target_workload_full(oracle_lib):
    wl = named_workload("zipf_b32_h4_d128_target_fwdbwd")
    rel, worst = run_fwd_check(wl)
    print(f"target fwd: err/max {rel:.2e}, worst per-sequence {worst:.2e}")
    res = run_bwd_check(wl)
    print("target bwd (err/max, worst per-seq):", res)


def test_func_spelling_causal_and_window_is_bitwise_those_masks():
    """Endpoints that spell causal (F0 = i + 1) or a window walk the same tiles in the
    same order as those kernels, so the results agree bit for bit."""
    lens = [200, 64, 129, 1]
    wl = make_workload("fspell", 157, lens, 2, 128, True, with_do=True)
    dw = DeviceWorkload(wl)
    i = np.concatenate([np.arange(n) for n in lens])
    causal_f = torch.from_numpy((i + 1)[None, :].astype(np.int32)).cuda()
    left, right = 70, 0
    win_f = torch.from_numpy(np.stack([np.zeros_like(i), i - left, i + right + 1]).astype(np.int32)).cuda()
    say("func spelling causal / window (70, 0) vs those kernels, both backward routes")
    for store in (False, True):
        # stored dS: the row blocks' key-group ranges from the endpoints are the causal and
        # window kernels' ranges, so dQ reads the same blocks in the same order
        oc, gc = dw.fwd(causal=True), dw.bwd(causal=True, store_ds=store)
        of, gf = dw.fwd(func=causal_f), dw.bwd(func=causal_f, store_ds=store)
        ow, gw = dw.fwd(window_size=(left, right)), dw.bwd(window_size=(left, right), store_ds=store)
        ofw, gfw = dw.fwd(func=win_f), dw.bwd(func=win_f, store_ds=store)
        torch.cuda.synchronize()
        assert torch.equal(oc, of) and all(torch.equal(a, b) for a, b in zip(gc, gf)), store
        assert torch.equal(ow, ofw) and all(torch.equal(a, b) for a, b in zip(gw, gfw)), store


def test_func_invalid_arguments_raise():
    wl = make_workload("fbad", 158, [10], 1, 16, True)
    dw = DeviceWorkload(wl)
    even = torch.zeros(2, 10, dtype=torch.int32, device="cuda")
    short = torch.zeros(3, 9, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        dw.fwd(func=even)
    with pytest.raises(ValueError):
        dw.fwd(func=short)
    with pytest.raises(ValueError):
        dw.fwd(func=torch.zeros(1, 10, dtype=torch.int32, device="cuda"), window_size=(1, 1))


# ------------------------------------------------------------------ limits and degenerate cases
def test_alpha_zero_gives_exact_zeros():
    """alpha = 0: every score is 0 and SiLU(0) = 0, so O, dV, dQ and dK are exactly 0."""
    wl = make_workload("a0", 180, [70, 150, 1], 2, 64, True, with_do=True)
    dw = DeviceWorkload(wl)
    say("alpha = 0")
    o = dw.fwd(alpha=0.0)
    dq, dk, dv = dw.bwd(alpha=0.0)
    torch.cuda.synchronize()
    for name, t in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert torch.all(t == 0), name


def test_largest_token_stride(oracle_lib):
    """A key tensor with the largest token stride the library accepts (2^24 elements):
    the 64-row tile copies address it with 32-bit byte offsets up to 2 (63 * 2^24 + 120)."""
    wl = make_workload("maxstride", 181, [100, 30], 1, 16, True, 1.0, with_do=True)
    dw = DeviceWorkload(wl)
    stride = 1 << 24
    say(f"largest token stride: k viewed with token stride {stride} ({wl.total_k * stride * 2 / 2**30:.1f} GiB)")
    big = torch.zeros(wl.total_k * stride, dtype=torch.bfloat16, device="cuda")
    k_view = big.as_strided((wl.total_k, 1, 16), (stride, 16, 1))
    k_view.copy_(dw.k)
    kw = dw.kw()
    o = hstu.hstu_fwd(dw.q, k_view, dw.v, dw.cu_q, dw.cu_k, **kw)
    dq, dk, dv = hstu.hstu_bwd(dw.do, dw.q, k_view, dw.v, dw.cu_q, dw.cu_k, **kw)
    torch.cuda.synchronize()
    del big
    check_close("O", to_f64(o), oracle.fwd_workload(wl), wl.cu_seqlens_q)
    rq, rk, rv = oracle.bwd_workload(wl)
    check_close("dQ", to_f64(dq), rq, wl.cu_seqlens_q)
    check_close("dK", to_f64(dk), rk, wl.cu_seqlens_k)
    check_close("dV", to_f64(dv), rv, wl.cu_seqlens_k)


# ------------------------------------------------------------------ stored dS
@pytest.mark.parametrize("D,causal", [(16, True), (64, False), (128, True)])
def test_stored_ds_entry_points(oracle_lib, D, causal):
    """hstu_bwd_dkdv_ds then hstu_bwd_dq_ds: dK and dV bit-identical to
    hstu_bwd_dkdv's, dQ bit-identical to hstu_bwd's stored route; the workspace
    starts as NaN, and a second, smaller problem reuses it as the first left it."""
    big = make_workload(f"dsbig{D}", 190 + D, [300, 129, 64, 0, 33], 2, D, causal, with_do=True)
    small = make_workload(f"dssmall{D}", 191 + D, [65, 1, 200], 2, D, causal, with_do=True)
    ws = DeviceWorkload(big).workspace()
    for wl in (big, small):
        dw = DeviceWorkload(wl)
        kw = dw.kw()
        kw.pop("func")
        say(f"stored dS entry points {wl.name}: lengths {list(wl.lengths_q)} D={D} mask={wl.mask_name}")
        dk, dv = hstu.hstu_bwd_dkdv_ds(dw.do, dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, ds=ws, **kw)
        dq = hstu.hstu_bwd_dq_ds(dw.q, dw.k, dw.cu_q, dw.cu_k, ds=ws, **kw)
        dk_r, dv_r = hstu.hstu_bwd_dkdv(dw.do, dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, **kw)
        g = dw.bwd()
        torch.cuda.synchronize()
        assert torch.equal(dk, dk_r) and torch.equal(dv, dv_r)
        assert torch.equal(dq, g[0]) and torch.equal(dk, g[1]) and torch.equal(dv, g[2])
        rq, rk, rv = oracle.bwd_workload(wl)
        check_close("dQ", to_f64(dq), rq, wl.cu_seqlens_q)


def test_stored_ds_needs_the_workspace_it_asks_for():
    wl = make_workload("dsws", 195, [100, 40], 1, 32, True, with_do=True)
    dw = DeviceWorkload(wl)
    kw = dw.kw()
    kw.pop("func")
    ws = dw.workspace()
    with pytest.raises(hstu.HstuError):
        hstu.hstu_bwd(dw.do, dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, workspace=ws[:-256], **kw)
    with pytest.raises(hstu.HstuError):
        hstu.hstu_bwd_dq_ds(dw.q, dw.k, dw.cu_q, dw.cu_k, ds=ws[:2048], **kw)
    # a window asks for its own (relative) layout: the causal-sized workspace is not that
    wsw = dw.workspace(window_size=(8, 0))
    assert wsw.numel() < ws.numel()


# ------------------------------------------------------------------ invariants
def test_zero_queries_give_exact_zeros():
    wl = make_workload("zq", 120, [70, 150], 2, 128, True, with_do=True)
    dw = DeviceWorkload(wl)
    dw.q.zero_()
    say("hstu_fwd/bwd zero queries")
    o = dw.fwd()
    dq, dk, dv = dw.bwd()
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(dk == 0) and torch.all(dv == 0)
    assert torch.any(dq != 0)


def test_alpha_folds_into_queries_bitwise():
    wl = make_workload("alpha2", 121, [100, 31, 260], 2, 64, True, with_do=True)
    dw = DeviceWorkload(wl)
    say("hstu_fwd/bwd alpha=2 vs doubled q")
    o1 = dw.fwd(alpha=2.0)
    g1 = dw.bwd(alpha=2.0)
    q2 = dw.q * 2  # exact in bf16
    o2 = hstu.hstu_fwd(q2, dw.k, dw.v, dw.cu_q, dw.cu_k, wl.max_seqlen_q, wl.max_seqlen_k, alpha=1.0,
                       scaling_seqlen=wl.scaling_seqlen, causal=True)
    g2 = hstu.hstu_bwd(dw.do, q2, dw.k, dw.v, dw.cu_q, dw.cu_k, wl.max_seqlen_q, wl.max_seqlen_k, alpha=1.0,
                       scaling_seqlen=wl.scaling_seqlen, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(g1[0], g2[0] * 2)   # dQ(alpha=2, Q) = 2 dQ(alpha=1, 2Q)
    assert torch.equal(g1[1], g2[1]) and torch.equal(g1[2], g2[2])


def test_outputs_written_exactly_on_real_rows():
    """Canary: outputs start as NaN; every real row is overwritten, the guard rows past T are not."""
    wl = make_workload("canary", 122, [5, 0, 129, 64], 2, 32, True, with_do=True)
    dw = DeviceWorkload(wl)
    T, H, D, guard = wl.total_q, wl.num_heads, wl.head_dim, 40
    nan = torch.full((T + guard, H, D), float("nan"), device="cuda", dtype=torch.bfloat16)
    o_buf, dq_buf, dk_buf, dv_buf = (nan.clone() for _ in range(4))
    kw = dw.kw()
    say("canary fwd/bwd")
    hstu.hstu_fwd(dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, out=o_buf[:T], **kw)
    hstu.hstu_bwd(dw.do, dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, dq=dq_buf[:T], dk=dk_buf[:T], dv=dv_buf[:T], **kw)
    torch.cuda.synchronize()
    for name, buf in (("o", o_buf), ("dq", dq_buf), ("dk", dk_buf), ("dv", dv_buf)):
        assert not torch.any(torch.isnan(buf[:T])), name
        assert torch.all(torch.isnan(buf[T:])), name


def test_strided_views():
    """dk/dv split from one packed KV gradient buffer, head-major q, padded-token v."""
    wl = make_workload("views", 123, [80, 200, 33], 2, 64, True, with_do=True)
    dw = DeviceWorkload(wl)
    T, H, D = wl.total_q, wl.num_heads, wl.head_dim
    kw = dw.kw()
    say("strided views")
    o_ref = dw.fwd()
    dq_ref, dk_ref, dv_ref = dw.bwd()
    q_hm = dw.q.permute(1, 0, 2).contiguous().permute(1, 0, 2)         # (T, H, D) view of (H, T, D)
    v_pad = torch.zeros(T, H, D + 64, device="cuda", dtype=torch.bfloat16)
    v_pad[:, :, :D] = dw.v
    v_view = v_pad[:, :, :D]                                              # token stride H*(D+64)
    kv_grad = torch.empty(T, 2, H, D, device="cuda", dtype=torch.bfloat16)
    o = hstu.hstu_fwd(q_hm, dw.k, v_view, dw.cu_q, dw.cu_k, **kw)
    dq, dk, dv = hstu.hstu_bwd(dw.do, q_hm, dw.k, v_view, dw.cu_q, dw.cu_k, dk=kv_grad[:, 0], dv=kv_grad[:, 1], **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    assert torch.equal(dq, dq_ref) and torch.equal(kv_grad[:, 0], dk_ref) and torch.equal(kv_grad[:, 1], dv_ref)


def test_repeat_runs_are_bitwise_identical():
    wl = named_workload("zipf_b32_h4_d128_causal_fwdbwd")
    dw = DeviceWorkload(wl)
    say("determinism: zipf fwd+bwd twice")
    o1, g1 = dw.fwd(), dw.bwd()
    o2, g2 = dw.fwd(), dw.bwd()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_permuting_sequences_permutes_outputs_bitwise():
    wl = make_workload("perm", 124, [130, 7, 300, 64], 2, 128, True, with_do=True)
    perm = [2, 0, 3, 1]
    cu = wl.cu_seqlens_q
    rows = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in perm])
    wl_p = make_workload("perm_p", 124, [int(wl.lengths_q[b]) for b in perm], 2, 128, True, with_do=True)
    wl_p.q, wl_p.k, wl_p.v, wl_p.do = wl.q[rows], wl.k[rows], wl.v[rows], wl.do[rows]
    wl_p.scaling_seqlen = wl.scaling_seqlen
    a, b = DeviceWorkload(wl), DeviceWorkload(wl_p)
    say("permutation")
    oa, ga = a.fwd(), a.bwd()
    ob, gb = b.fwd(), b.bwd()
    torch.cuda.synchronize()
    idx = torch.from_numpy(rows).cuda()
    assert torch.equal(ob, oa[idx])
    for x, y in zip(gb, ga):
        assert torch.equal(x, y[idx])


def test_runs_on_caller_stream(oracle_lib):
    wl = make_workload("stream", 125, [100, 60], 2, 64, False, with_do=True)
    dw = DeviceWorkload(wl)
    s = torch.cuda.Stream()
    say("non-default stream")
    with torch.cuda.stream(s):
        o = dw.fwd()
    s.synchronize()
    check_close("O", to_f64(o), oracle.fwd_workload(wl), wl.cu_seqlens_q)


def test_bwd_on_side_stream_allocates_there(oracle_lib):
    """hstu_bwd on a side stream with no workspace given: the binding allocates the dS
    workspace and the outputs while that stream is current, so a block freed at
    return is not handed to the current stream's next allocation while the side
    stream's kernels still use it.  The current stream allocates and NaN-fills
    blocks of the workspace's size right after the call, without waiting."""
    wl = make_workload("sidestream", 127, [1500, 900, 64], 4, 128, True, 0.5, with_do=True)
    dw = DeviceWorkload(wl)
    kw = dw.kw()
    need = hstu.hstu_bwd_workspace_size(dw.do, dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, **kw)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    say("hstu_bwd on a side stream, workspace allocated by the binding")
    dq, dk, dv = hstu.hstu_bwd(dw.do, dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, stream=s, **kw)
    junk = [torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda") for _ in range(4)]
    s.synchronize()
    torch.cuda.synchronize()
    del junk
    rq, rk, rv = oracle.bwd_workload(wl)
    check_close("dQ", to_f64(dq), rq, wl.cu_seqlens_q)
    check_close("dK", to_f64(dk), rk, wl.cu_seqlens_k)
    check_close("dV", to_f64(dv), rv, wl.cu_seqlens_k)


def test_unsupported_raise():
    wl = make_workload("unsup", 126, [10], 1, 16, True)
    dw = DeviceWorkload(wl)
    q48 = torch.zeros(10, 1, 48, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(NotImplementedError):
        hstu.hstu_fwd(q48, q48, q48, dw.cu_q, dw.cu_k, 10, 10)
    with pytest.raises(hstu.HstuError):
        hstu.hstu_fwd(dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, 11, 10)  # max_seqlen_q > max_seqlen_k


# ------------------------------------------------------------------ fused backward (fp32 atomic dQ)
FUSED_CASES = [
    # (name, seed, lengths_q, lengths_k or None, H, D, mask)
    ("edge_d16_causal", 300, EDGE_LENGTHS, None, 2, 16, True),
    ("edge_d32_full", 301, EDGE_LENGTHS, None, 2, 32, False),
    ("edge_d64_causal", 302, EDGE_LENGTHS, None, 1, 64, True),
    ("edge_d128_causal", 303, EDGE_LENGTHS, None, 2, 128, True),
    ("lq_ne_lk_full", 304, [130, 40, 7], [131, 38, 3], 3, 64, False),
    ("window", 305, [700, 1000, 33], None, 2, 128, (256, 128)),
    ("func", 306, [300, 5, 0, 257], [310, 9, 4, 257], 2, 128, "func"),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fused_backward(oracle_lib, case):
    """hstu_bwd_fused: dK and dV bit-identical to hstu_bwd_dkdv's (the same pass), dQ
    (fp32 atomics, any summation order) within the bar of the oracle's."""
    name, seed, lq, lk, H, D, mask = case
    kw = {}
    if mask == "func":
        kw["func"] = func_random_mask(np.random.default_rng(seed), lq, lk, 3)
        causal = False
    elif isinstance(mask, tuple):
        kw["window"], causal = mask, False
    else:
        causal = mask
    wl = make_workload(f"fused_{name}", seed, lq, H, D, causal, 1.0, lengths_k=lk, with_do=True, **kw)
    dw = DeviceWorkload(wl)
    dkw = dw.kw()
    ws = torch.full((wl.total_q * H * D * 4 + 256,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN-filled
    say(f"hstu_bwd_fused {name}: lengths {list(wl.lengths_q)} H={H} D={D} mask={wl.mask_name}")
    dq, dk, dv = hstu.hstu_bwd_fused(dw.do, dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, workspace=ws, **dkw)
    dk_r, dv_r = hstu.hstu_bwd_dkdv(dw.do, dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, **dkw)
    torch.cuda.synchronize()
    assert torch.equal(dk, dk_r) and torch.equal(dv, dv_r)
    rq, rk, rv = oracle.bwd_workload(wl)
    check_close("dQ", to_f64(dq), rq, wl.cu_seqlens_q)
    check_close("dK", to_f64(dk), rk, wl.cu_seqlens_k)


def test_fused_backward_zipf_workload_full(oracle_lib):
    wl = named_workload("zipf_b32_h4_d128_causal_fwdbwd")
    dw = DeviceWorkload(wl)
    say("hstu_bwd_fused on the Zipf workload (every row)")
    dq, dk, dv = hstu.hstu_bwd_fused(dw.do, dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, **dw.kw())
    torch.cuda.synchronize()
    rq, rk, rv = oracle.bwd_workload(wl)
    print("fused zipf dQ (err/max, worst per-seq):", check_close("dQ", to_f64(dq), rq, wl.cu_seqlens_q))
    check_close("dK", to_f64(dk), rk, wl.cu_seqlens_k)
    check_close("dV", to_f64(dv), rv, wl.cu_seqlens_k)


# ------------------------------------------------------------------ long walks, odd head counts
SPLIT_CASES = [
    # (seed, lengths, H, D, causal): blocks walking 33 to 64 key tiles next to short and
    # empty sequences; odd H so that neighbouring work items differ in head and row block
    (310, [4100, 100, 2049, 0, 33], 1, 128, True),
    (311, [2500, 3000], 3, 64, False),
    (312, [2113, 17, 4000], 2, 32, True),
    (313, [2200, 900], 1, 16, False),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[f"seed{c[0]}_h{c[2]}_d{c[3]}_{'causal' if c[4] else 'full'}"
                                                   for c in SPLIT_CASES])
def test_split_walks_fwd(oracle_lib, case):
    seed, lens, H, D, causal = case
    wl = make_workload(f"split{seed}", seed, lens, H, D, causal, 0.5)
    run_fwd_check(wl)
    dw = DeviceWorkload(wl)
    o1, o2 = dw.fwd(), dw.fwd()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)  # each output row is summed in one fixed order


# ------------------------------------------------------------------ dQ from stored dS: long walks
DQ_LONG_CASES = [
    # (seed, lengths, H, D, causal): 256-row blocks walking 33 to 110 key tiles of stored
    # dS beside short and empty sequences, odd and even head counts
    (320, [4100, 100, 2049, 0, 3000], 3, 128, True),
    (321, [2500, 2113], 2, 64, False),
    (322, [7000], 8, 32, True),
    (323, [2200, 17, 2600], 5, 16, True),
]


@pytest.mark.parametrize("case", DQ_LONG_CASES, ids=[f"seed{c[0]}_h{c[2]}_d{c[3]}_{'causal' if c[4] else 'full'}"
                                                     for c in DQ_LONG_CASES])
def test_dq_ds_long_walks(oracle_lib, case):
    seed, lens, H, D, causal = case
    wl = make_workload(f"dqlong{seed}", seed, lens, H, D, causal, 0.5, with_do=True)
    run_bwd_check(wl)
    dw = DeviceWorkload(wl)
    kw = dw.kw()
    ws = dw.workspace()
    hstu.hstu_bwd_dkdv_ds(dw.do, dw.q, dw.k, dw.v, dw.cu_q, dw.cu_k, ds=ws, **kw)
    dq1 = hstu.hstu_bwd_dq_ds(dw.q, dw.k, dw.cu_q, dw.cu_k, ds=ws, **kw)
    dq2 = hstu.hstu_bwd_dq_ds(dw.q, dw.k, dw.cu_q, dw.cu_k, ds=ws, **kw)  # again, on the same dS
    dq3 = dw.bwd()[0]  # a whole backward on a fresh workspace
    torch.cuda.synchronize()
    assert torch.equal(dq1, dq2) and torch.equal(dq1, dq3)


# ------------------------------------------------------------------ closed forms at full size
def test_closed_forms_on_the_zipf_workload(oracle_lib):
    """Properties the method fixes at any size (HSTU page, "Overview" equations), on the
    Zipf forward + backward workload's shapes: with Q = 0 every score is 0 and
    SiLU(0) = 0, so O, dK and dV are exactly 0 on both backward routes, while dQ =
    alpha SiLU'(0) / L_s sum_j (dO_i . v_j) k_j (SiLU'(0) = 1/2) meets the bar against
    the oracle; with V = 1 every column of O is the same masked SiLU row sum, so all
    columns of O are bit-identical."""
    wl = named_workload("zipf_b32_h4_d128_causal_fwdbwd")
    dw = DeviceWorkload(wl)
    v1 = torch.ones_like(dw.v)
    say("closed forms: Zipf workload with V = 1")
    o1 = hstu.hstu_fwd(dw.q, dw.k, v1, dw.cu_q, dw.cu_k, **dw.kw())
    torch.cuda.synchronize()
    assert torch.equal(o1, o1[:, :, :1].expand_as(o1))
    dw.q.zero_()
    say("closed forms: Zipf workload with Q = 0")
    o = dw.fwd()
    assert torch.all(o == 0)
    zero_q = np.zeros_like(wl.q)
    rq = oracle_lib.bwd_dq(wl.cu_seqlens_q, wl.cu_seqlens_k, wl.do, zero_q, wl.k, wl.v, float(wl.alpha),
                           wl.scaling_seqlen, wl.mask_spec)
    for store in (True, False):
        dq, dk, dv = dw.bwd(store_ds=store)
        torch.cuda.synchronize()
        assert torch.all(dk == 0) and torch.all(dv == 0), store
        check_close(f"dQ with Q = 0 ({'stored dS' if store else 'recompute'})", to_f64(dq), rq, wl.cu_seqlens_q)
