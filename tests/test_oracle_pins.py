"""Pins for the fp64 oracle: checks against things other than the oracle itself.

None of these tests touches a GPU.  Each pin is chosen so that a plausible slip
in the oracle (a dropped term of SiLU or SiLU', a wrong sign, an offset taken
from the wrong cumulative array, a transposed operand, a wrong mask alignment,
a missing 1/L_scale) fails at least one of them:

* a dense brute force over the whole packed batch (global indices, explicit
  block-diagonal mask, library matmul and library SiLU) for the forward;
* PyTorch autograd of that dense forward, in fp64, for the backward;
* central finite differences of <dO, O(Q, K, V)> through the oracle's own
  forward, for the backward;
* closed forms and invariants of the definition on the HSTU Attention page
  ("Overview" equations): Q = 0 gives O = 0; V = 1 gives every output column
  equal to the masked SiLU row sum over L_scale; the first causal row; linearity
  in V; alpha folded into Q; permutation and locality across sequences;
  <dV, V> = <dO, O> and <dQ, Q> = <dK, K>;
* for the token window of the page's "Mask support" table: the dense brute
  force with the band built by library ``tril``/``triu`` diagonals, the
  special windows the table names ((-1, 0) is causal, (-1, -1) full), bounds
  past the sequence acting as unbounded, the diagonal-only window (0, 0) in
  closed form, and the count of visible keys per row against an independent
  closed form (equal keys make every score of a row equal).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from generative_recommender_attention_amd.workloads import make_workload, named_workload


# ----------------------------------------------------------------------------
# independent brute force: dense (T_q x T_k) formulation with a global mask
# ----------------------------------------------------------------------------
def dense_mask(cu_q, cu_k, causal):
    """Block-diagonal mask over global token indices, built by brute force."""
    if not isinstance(causal, bool):
        return dense_band_mask(cu_q, cu_k, *causal)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    m = np.zeros((tq, tk))
    for b in range(len(cu_q) - 1):
        for r in range(cu_q[b], cu_q[b + 1]):
            for c in range(cu_k[b], cu_k[b + 1]):
                i, j = r - cu_q[b], c - cu_k[b]
                if (not causal) or j <= i:  # top-left causal: key j visible to query i iff j <= i
                    m[r, c] = 1.0
    return m


def dense_band_mask(cu_q, cu_k, left, right):
    """Block-diagonal mask of a token window: each sequence's block is the band
    of diagonals -left .. +right of an all-ones (L_q x L_k) block (numpy ``tril``
    keeps diagonals <= right, ``triu`` those >= -left; -1 drops that cut)."""
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    m = np.zeros((tq, tk))
    for b in range(len(cu_q) - 1):
        blk = np.ones((cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]))
        if right >= 0:
            blk = np.tril(blk, right)
        if left >= 0:
            blk = np.triu(blk, -left)
        m[cu_q[b]:cu_q[b + 1], cu_k[b]:cu_k[b + 1]] = blk
    return m


def dense_forward_torch(cu_q, cu_k, q, k, v, alpha, ls, causal):
    """O = ((M * silu(alpha Q K^T)) / ls) V per head, fp64 torch tensors in/out.
    ``causal`` is a bool (causal / full) or a (left, right) window."""
    m = torch.from_numpy(dense_mask(cu_q, cu_k, causal))
    outs = []
    for h in range(q.shape[1]):
        s = alpha * (q[:, h, :] @ k[:, h, :].T)
        a = m * torch.nn.functional.silu(s) / ls
        outs.append(a @ v[:, h, :])
    return torch.stack(outs, dim=1)


def random_problem(seed, lq, lk, H, D, causal, scale=1.0):
    """``causal`` is a bool or a (left, right) window."""
    if isinstance(causal, bool):
        return make_workload("pin", seed, lq, H, D, causal, scale, lengths_k=lk, with_do=True)
    return make_workload("pin", seed, lq, H, D, False, scale, lengths_k=lk, with_do=True, window=causal)


def f64(bits):
    return oracle.widen(bits)


TINY_CASES = [
    # (seed, lengths_q, lengths_k, H, D, causal)
    (10, [5, 11], None, 1, 16, True),
    (11, [3, 0, 7], None, 2, 8, True),
    (12, [4, 9, 1], None, 2, 4, False),
    (13, [6, 2], [9, 5], 1, 8, True),     # L_k > L_q (top-left causal)
    (14, [7, 3], [4, 3], 2, 4, False),    # L_k < L_q, full mask
    (15, [12], None, 3, 16, True),
    (16, [0, 0, 5], [0, 3, 5], 1, 4, True),
    # token windows (left, right)
    (17, [9, 14], None, 2, 8, (3, 0)),
    (18, [11, 6], None, 1, 8, (2, 4)),
    (19, [7, 12], [10, 5], 2, 4, (0, 2)),   # L_k != L_q both ways
    (20, [13], None, 1, 8, (0, 0)),
    (41, [10, 4], None, 2, 4, (-1, 3)),     # right bound only
    (42, [8, 0, 15], None, 1, 8, (5, -1)),  # left bound only
]


@pytest.mark.parametrize("case", TINY_CASES, ids=[f"seed{c[0]}" for c in TINY_CASES])
def test_forward_matches_dense_brute_force(oracle_lib, case):
    seed, lq, lk, H, D, causal = case
    wl = random_problem(seed, lq, lk, H, D, causal)
    q, k, v = (torch.from_numpy(f64(x)) for x in (wl.q, wl.k, wl.v))
    want = dense_forward_torch(wl.cu_seqlens_q, wl.cu_seqlens_k, q, k, v,
                               float(wl.alpha), wl.scaling_seqlen, causal).numpy()
    got = oracle.fwd_workload(wl)
    assert got.shape == want.shape
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("case", TINY_CASES, ids=[f"seed{c[0]}" for c in TINY_CASES])
def test_backward_matches_autograd_of_dense_forward(oracle_lib, case):
    seed, lq, lk, H, D, causal = case
    wl = random_problem(seed, lq, lk, H, D, causal)
    q, k, v = (torch.from_numpy(f64(x)).requires_grad_(True) for x in (wl.q, wl.k, wl.v))
    do = torch.from_numpy(f64(wl.do))
    o = dense_forward_torch(wl.cu_seqlens_q, wl.cu_seqlens_k, q, k, v,
                            float(wl.alpha), wl.scaling_seqlen, causal)
    (o * do).sum().backward()
    dq, dk, dv = oracle.bwd_workload(wl)
    np.testing.assert_allclose(dq, q.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dk, k.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dv, v.grad.numpy(), rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False, (1, 1)], ids=["causal", "full", "window11"])
def test_backward_matches_finite_differences(oracle_lib, causal):
    """Central differences of f = <dO, O(Q,K,V)> through the oracle's forward."""
    lq, lk, H, D = [4, 3], [4, 3], 2, 4
    wl = random_problem(5, lq, lk, H, D, causal)
    q, k, v, do = (f64(x) for x in (wl.q, wl.k, wl.v, wl.do))
    # make the scores large enough that SiLU is far from linear
    q = q * 3.0
    alpha, ls = 0.7, 5.0
    cu_q, cu_k = wl.cu_seqlens_q, wl.cu_seqlens_k

    def f(qq, kk, vv):
        return float(np.sum(do * oracle.fwd(cu_q, cu_k, qq, kk, vv, alpha, ls, causal)))

    dq = oracle.bwd_dq(cu_q, cu_k, do, q, k, v, alpha, ls, causal)
    dk, dv = oracle.bwd_dkdv(cu_q, cu_k, do, q, k, v, alpha, ls, causal)
    eps = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[idx] = (f(*args_p) - f(*args_m)) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=f"d{name}")


def test_silu_derivative_closed_form_matches_finite_difference(oracle_lib):
    """The SiLU' closed form the oracle's backward uses, against differences of
    the library SiLU, through a one-pair problem: with q = [s], k = [1], v = [1],
    alpha = 1, L_scale = 1 and dO = 1, dQ equals SiLU'(s) exactly by the chain rule."""
    for s in (-30.0, -4.5, -1.0, -0.1, 0.0, 0.3, 2.0, 9.0):
        cu = np.array([0, 1], dtype=np.int32)
        q = np.array([[[s]]]); k = np.array([[[1.0]]]); v = np.array([[[1.0]]]); do = np.array([[[1.0]]])
        got = oracle.bwd_dq(cu, cu, do, q, k, v, 1.0, 1.0, True)[0, 0, 0]
        h = 1e-6
        t = torch.tensor([s - h, s + h], dtype=torch.float64)
        y = torch.nn.functional.silu(t)
        num = float((y[1] - y[0]) / (2 * h))
        assert abs(got - num) <= 1e-8 * max(1.0, abs(num)), (s, got, num)


# ----------------------------------------------------------------------------
# closed forms and invariants
# ----------------------------------------------------------------------------
def test_zero_queries_give_zero_output_and_zero_dk_dv(oracle_lib):
    wl = random_problem(21, [7, 4, 9], None, 2, 8, True)
    q = np.zeros_like(f64(wl.q))
    k, v, do = f64(wl.k), f64(wl.v), f64(wl.do)
    a, ls = float(wl.alpha), wl.scaling_seqlen
    o = oracle.fwd(wl.cu_seqlens_q, wl.cu_seqlens_k, q, k, v, a, ls, True)
    assert np.all(o == 0.0)
    dk, dv = oracle.bwd_dkdv(wl.cu_seqlens_q, wl.cu_seqlens_k, do, q, k, v, a, ls, True)
    assert np.all(dk == 0.0) and np.all(dv == 0.0)
    # with s = 0 everywhere, SiLU'(0) = 1/2, so dQ_i = alpha * (1/2) / L * sum_{j<=i} (dO_i . v_j) k_j
    dq = oracle.bwd_dq(wl.cu_seqlens_q, wl.cu_seqlens_k, do, q, k, v, a, ls, True)
    cu = wl.cu_seqlens_q
    for b in range(3):
        for h in range(2):
            for i in range(cu[b + 1] - cu[b]):
                r = cu[b] + i
                want = np.zeros(8)
                for j in range(i + 1):
                    want += a * 0.5 / ls * float(do[r, h] @ v[cu[b] + j, h]) * k[cu[b] + j, h]
                np.testing.assert_allclose(dq[r, h], want, rtol=1e-12, atol=1e-15)


def test_unit_values_give_masked_silu_row_sums(oracle_lib):
    wl = random_problem(22, [6, 10], None, 2, 16, True)
    q, k = f64(wl.q), f64(wl.k)
    v = np.ones_like(f64(wl.v))
    a, ls = float(wl.alpha), wl.scaling_seqlen
    o = oracle.fwd(wl.cu_seqlens_q, wl.cu_seqlens_k, q, k, v, a, ls, True)
    cu = wl.cu_seqlens_q
    for b in range(2):
        for h in range(2):
            for i in range(cu[b + 1] - cu[b]):
                r = cu[b] + i
                row = 0.0
                for j in range(i + 1):
                    s = a * math.fsum(q[r, h] * k[cu[b] + j, h])
                    row += s / (1.0 + math.exp(-s))
                np.testing.assert_allclose(o[r, h], np.full(16, row / ls), rtol=1e-12)


def test_first_causal_row_is_single_term(oracle_lib):
    wl = random_problem(23, [5, 8], None, 3, 16, True, scale=2.0)
    q, k, v = f64(wl.q), f64(wl.k), f64(wl.v)
    a, ls = float(wl.alpha), wl.scaling_seqlen
    o = oracle.fwd(wl.cu_seqlens_q, wl.cu_seqlens_k, q, k, v, a, ls, True)
    for b in range(2):
        r = wl.cu_seqlens_q[b]
        for h in range(3):
            s = a * math.fsum(q[r, h] * k[r, h])
            want = s / (1.0 + math.exp(-s)) * v[r, h] / ls
            np.testing.assert_allclose(o[r, h], want, rtol=1e-13)


def test_causal_last_row_equals_full_last_row(oracle_lib):
    wl = random_problem(24, [9, 13], None, 2, 8, True)
    args = (wl.cu_seqlens_q, wl.cu_seqlens_k, wl.q, wl.k, wl.v, float(wl.alpha), wl.scaling_seqlen)
    last = wl.cu_seqlens_q[1:] - 1
    oc = oracle.fwd(*args, True, rows=last)
    of = oracle.fwd(*args, False, rows=last)
    np.testing.assert_array_equal(oc, of)


def test_linear_in_values(oracle_lib):
    wl = random_problem(25, [8, 5], None, 2, 8, False)
    wl2 = random_problem(26, [8, 5], None, 2, 8, False)
    q, k, v1, v2 = f64(wl.q), f64(wl.k), f64(wl.v), f64(wl2.v)
    a, ls = float(wl.alpha), wl.scaling_seqlen
    run = lambda vv: oracle.fwd(wl.cu_seqlens_q, wl.cu_seqlens_k, q, k, vv, a, ls, False)
    np.testing.assert_allclose(run(v1 + 2.0 * v2), run(v1) + 2.0 * run(v2), rtol=1e-12, atol=1e-14)


def test_alpha_folds_into_queries_exactly(oracle_lib):
    wl = random_problem(27, [7, 6], None, 2, 16, True)
    q, k, v = f64(wl.q), f64(wl.k), f64(wl.v)
    cu = wl.cu_seqlens_q
    o_alpha = oracle.fwd(cu, cu, q, k, v, 2.0, 7, True)
    o_scaled = oracle.fwd(cu, cu, 2.0 * q, k, v, 1.0, 7, True)
    np.testing.assert_array_equal(o_alpha, o_scaled)


def test_output_times_scaling_seqlen_is_independent_of_it(oracle_lib):
    wl = random_problem(28, [7, 6], None, 1, 8, True)
    cu = wl.cu_seqlens_q
    o3 = oracle.fwd(cu, cu, wl.q, wl.k, wl.v, float(wl.alpha), 3, True)
    o11 = oracle.fwd(cu, cu, wl.q, wl.k, wl.v, float(wl.alpha), 11, True)
    np.testing.assert_allclose(o3 * 3.0, o11 * 11.0, rtol=1e-14)


def test_permuting_sequences_permutes_outputs(oracle_lib):
    wl = random_problem(29, [4, 9, 6], None, 2, 8, True)
    cu = wl.cu_seqlens_q
    perm = [2, 0, 1]
    rows = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in perm])
    lens = np.array([cu[b + 1] - cu[b] for b in perm])
    cu_p = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v, do = (f64(x)[rows] for x in (wl.q, wl.k, wl.v, wl.do))
    a, ls = float(wl.alpha), wl.scaling_seqlen
    o = oracle.fwd(cu, cu, wl.q, wl.k, wl.v, a, ls, True)
    o_p = oracle.fwd(cu_p, cu_p, q, k, v, a, ls, True)
    np.testing.assert_array_equal(o_p, o[rows])
    dq, dk, dv = oracle.bwd_workload(wl)
    dq_p = oracle.bwd_dq(cu_p, cu_p, do, q, k, v, a, ls, True)
    dk_p, dv_p = oracle.bwd_dkdv(cu_p, cu_p, do, q, k, v, a, ls, True)
    np.testing.assert_array_equal(dq_p, dq[rows])
    np.testing.assert_array_equal(dk_p, dk[rows])
    np.testing.assert_array_equal(dv_p, dv[rows])


def test_changing_one_sequence_leaves_others_unchanged(oracle_lib):
    wl = random_problem(30, [5, 7, 4], None, 1, 8, True)
    cu = wl.cu_seqlens_q
    q, k, v = f64(wl.q), f64(wl.k), f64(wl.v)
    a, ls = float(wl.alpha), wl.scaling_seqlen
    o = oracle.fwd(cu, cu, q, k, v, a, ls, True)
    k2, v2 = k.copy(), v.copy()
    k2[cu[1]:cu[2]] += 1.5
    v2[cu[1]:cu[2]] -= 0.75
    o2 = oracle.fwd(cu, cu, q, k2, v2, a, ls, True)
    keep = np.r_[cu[0]:cu[1], cu[2]:cu[3]]
    np.testing.assert_array_equal(o2[keep], o[keep])
    assert not np.allclose(o2[cu[1]:cu[2]], o[cu[1]:cu[2]])


@pytest.mark.parametrize("causal", [True, False])
def test_backward_inner_product_identities(oracle_lib, causal):
    """<dV, V> = <dO, O> and <dQ, Q> = <dK, K> per (sequence, head)."""
    wl = random_problem(31, [9, 14, 3], None, 2, 16, causal, scale=1.5)
    o = oracle.fwd_workload(wl)
    dq, dk, dv = oracle.bwd_workload(wl)
    q, k, v, do = (f64(x) for x in (wl.q, wl.k, wl.v, wl.do))
    cu = wl.cu_seqlens_q
    for b in range(3):
        sl = slice(cu[b], cu[b + 1])
        for h in range(2):
            lhs, rhs = np.sum(dv[sl, h] * v[sl, h]), np.sum(do[sl, h] * o[sl, h])
            assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(rhs))
            lhs, rhs = np.sum(dq[sl, h] * q[sl, h]), np.sum(dk[sl, h] * k[sl, h])
            assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(rhs))


def test_empty_rows_are_zero(oracle_lib):
    """L_k = 0 gives zero output rows; keys no query sees get zero dK, dV."""
    wl = random_problem(32, [3, 4], [0, 6], 1, 8, True)
    o = oracle.fwd_workload(wl)
    assert np.all(o[:3] == 0.0)
    dq, dk, dv = oracle.bwd_workload(wl)
    assert np.all(dq[:3] == 0.0)
    # second sequence: L_q = 4, L_k = 6, top-left causal -> keys 4 and 5 are seen by no query
    assert np.all(dk[4:6] == 0.0) and np.all(dv[4:6] == 0.0)
    assert np.any(dk[:4] != 0.0)


def test_row_subsets_match_full_evaluation(oracle_lib):
    wl = random_problem(33, [13, 2, 8], None, 2, 16, True)
    full = oracle.fwd_workload(wl)
    rows = np.array([22, 0, 14, 5, 13])
    np.testing.assert_array_equal(oracle.fwd_workload(wl, rows), full[rows])
    dq, dk, dv = oracle.bwd_workload(wl)
    sq, sk, sv = oracle.bwd_workload(wl, rows_q=rows, rows_k=rows[::-1])
    np.testing.assert_array_equal(sq, dq[rows])
    np.testing.assert_array_equal(sk, dk[rows[::-1]])
    np.testing.assert_array_equal(sv, dv[rows[::-1]])


def test_out_of_range_row_is_rejected(oracle_lib):
    wl = random_problem(34, [3], None, 1, 4, True)
    with pytest.raises(ValueError):
        oracle.fwd_workload(wl, rows=np.array([3]))


def test_tiny_workload_matches_dense_brute_force(oracle_lib):
    """The B=2, lengths [5, 11], H=1, D=16 causal workload end to end."""
    wl = named_workload("tiny_b2_h1_d16_causal")
    q, k, v = (torch.from_numpy(f64(x)) for x in (wl.q, wl.k, wl.v))
    want = dense_forward_torch(wl.cu_seqlens_q, wl.cu_seqlens_k, q, k, v,
                               float(wl.alpha), wl.scaling_seqlen, True).numpy()
    np.testing.assert_allclose(oracle.fwd_workload(wl), want, rtol=1e-12, atol=1e-15)


def test_oracle_matches_its_committed_fixtures(oracle_lib):
    """Regression against values the oracle wrote earlier (tests/golden/make_golden.py)."""
    import json
    import os

    here = os.path.join(os.path.dirname(__file__), "golden")
    with open(os.path.join(here, "tiny_b2_h1_d16_causal_fwd.json")) as f:
        g = json.load(f)
    wl = named_workload("tiny_b2_h1_d16_causal")
    np.testing.assert_allclose(oracle.fwd_workload(wl).ravel(), g["o"], rtol=1e-14, atol=0)
    with open(os.path.join(here, "tiny_bwd_b3_h2_d16_causal.json")) as f:
        g = json.load(f)
    wl = make_workload("tiny_bwd_b3_h2_d16_causal", 40, [6, 0, 9], 2, 16, True, with_do=True)
    dq, dk, dv = oracle.bwd_workload(wl)
    for name, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        np.testing.assert_allclose(x.ravel(), g[name], rtol=1e-14, atol=0)


# ----------------------------------------------------------------------------
# token windows ("Mask support" table)
# ----------------------------------------------------------------------------
def _fwd_bwd(wl, mask):
    args = (wl.cu_seqlens_q, wl.cu_seqlens_k)
    a, ls = float(wl.alpha), wl.scaling_seqlen
    o = oracle.fwd(*args, wl.q, wl.k, wl.v, a, ls, mask)
    dq = oracle.bwd_dq(*args, wl.do, wl.q, wl.k, wl.v, a, ls, mask)
    dk, dv = oracle.bwd_dkdv(*args, wl.do, wl.q, wl.k, wl.v, a, ls, mask)
    return o, dq, dk, dv


def test_named_windows_are_causal_and_full(oracle_lib):
    """(-1, 0) is causal and (-1, -1) is full attention, bit for bit."""
    wl = random_problem(43, [9, 1, 17], [12, 1, 17], 2, 8, True)
    for window, flag in (((-1, 0), True), ((-1, -1), False)):
        for x, y in zip(_fwd_bwd(wl, window), _fwd_bwd(wl, flag)):
            np.testing.assert_array_equal(x, y)


def test_bounds_past_the_sequence_are_unbounded(oracle_lib):
    """A left bound >= L_q - 1 cuts nothing, nor does a right bound >= L_k - 1."""
    wl = random_problem(44, [9, 6], [7, 10], 1, 8, True)
    full = _fwd_bwd(wl, (-1, -1))
    for window in ((8, 9), (8, -1), (-1, 9), (100, 100)):
        for x, y in zip(_fwd_bwd(wl, window), full):
            np.testing.assert_array_equal(x, y)
    causal = _fwd_bwd(wl, (-1, 0))
    for x, y in zip(_fwd_bwd(wl, (8, 0)), causal):
        np.testing.assert_array_equal(x, y)


def test_diagonal_window_closed_form(oracle_lib):
    """Window (0, 0): query i sees key i only, so O_i = SiLU(alpha q_i.k_i) v_i / L_scale,
    dV_i = SiLU(s_ii) dO_i / L, dQ_i = alpha SiLU'(s_ii) (dO_i.v_i) k_i / L and
    dK_i = alpha SiLU'(s_ii) (dO_i.v_i) q_i / L; rows i >= L_k see nothing."""
    wl = random_problem(45, [6, 9], [6, 7], 2, 8, (0, 0), scale=1.5)
    q, k, v, do = (f64(x) for x in (wl.q, wl.k, wl.v, wl.do))
    a, ls = float(wl.alpha), wl.scaling_seqlen
    o, dq, dk, dv = _fwd_bwd(wl, (0, 0))
    for b in range(2):
        lq, lk = int(wl.lengths_q[b]), int(wl.lengths_k[b])
        for i in range(lq):
            r, c = wl.cu_seqlens_q[b] + i, wl.cu_seqlens_k[b] + i
            for h in range(2):
                if i >= lk:
                    assert np.all(o[r, h] == 0.0) and np.all(dq[r, h] == 0.0)
                    continue
                s = a * math.fsum(q[r, h] * k[c, h])
                sig = 1.0 / (1.0 + math.exp(-s))
                dsilu = sig * (1.0 + s * (1.0 - sig))
                da = math.fsum(do[r, h] * v[c, h])
                np.testing.assert_allclose(o[r, h], s * sig * v[c, h] / ls, rtol=1e-12, atol=1e-15)
                np.testing.assert_allclose(dv[c, h], s * sig * do[r, h] / ls, rtol=1e-12, atol=1e-15)
                np.testing.assert_allclose(dq[r, h], a * dsilu * da * k[c, h] / ls, rtol=1e-11, atol=1e-15)
                np.testing.assert_allclose(dk[c, h], a * dsilu * da * q[r, h] / ls, rtol=1e-11, atol=1e-15)
        for j in range(lq, lk):  # keys no query reaches
            c = wl.cu_seqlens_k[b] + j
            assert np.all(dk[c] == 0.0) and np.all(dv[c] == 0.0)


@pytest.mark.parametrize("window", [(0, 0), (1, 0), (3, 0), (0, 1), (2, 5), (-1, 2), (4, -1), (6, 6)])
def test_visible_key_count_per_row(oracle_lib, window):
    """With every key of a sequence equal and V = 1, every score of query row i is
    the same value s_i, so O_i = n_i SiLU(s_i) / L_scale in every column, where
    n_i = #{j in [0, L_k) : i - left <= j <= i + right} is counted here from the
    interval's clamped ends, not by testing keys one by one."""
    left, right = window
    lq, lk = [11, 5, 8], [9, 7, 8]
    wl = random_problem(46, lq, lk, 1, 8, window)
    q, k = f64(wl.q), f64(wl.k)
    cu_q, cu_k = wl.cu_seqlens_q, wl.cu_seqlens_k
    for b in range(3):
        k[cu_k[b]:cu_k[b + 1]] = k[cu_k[b]]
    v = np.ones_like(f64(wl.v))
    a, ls = float(wl.alpha), wl.scaling_seqlen
    o = oracle.fwd(cu_q, cu_k, q, k, v, a, ls, window)
    for b in range(3):
        for i in range(lq[b]):
            lo = 0 if left < 0 else max(0, i - left)
            hi = lk[b] - 1 if right < 0 else min(lk[b] - 1, i + right)
            n = max(0, hi - lo + 1)
            r = cu_q[b] + i
            s = a * math.fsum(q[r, 0] * k[cu_k[b], 0])
            want = n * s / (1.0 + math.exp(-s)) / ls
            np.testing.assert_allclose(o[r, 0], np.full(8, want), rtol=1e-12, atol=1e-15)


def test_band_splits_into_its_two_sides(oracle_lib):
    """Keys [i - l, i + r] are the disjoint union of [i - l, i] and [i + 1, i + r], and
    the masked sum is linear in the key set: O(l, r) = O(l, 0) + O(-1, r) - O(-1, 0)."""
    wl = random_problem(47, [15, 9], [12, 14], 2, 8, True)
    args = (wl.cu_seqlens_q, wl.cu_seqlens_k, wl.q, wl.k, wl.v, float(wl.alpha), wl.scaling_seqlen)
    for l, r in ((2, 3), (0, 5), (4, 1)):
        lhs = oracle.fwd(*args, (l, r))
        rhs = oracle.fwd(*args, (l, 0)) + oracle.fwd(*args, (-1, r)) - oracle.fwd(*args, (-1, 0))
        np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-13)


def test_window_bounds_below_minus_one_are_rejected(oracle_lib):
    wl = random_problem(48, [3], None, 1, 4, True)
    with pytest.raises(ValueError):
        oracle.fwd(wl.cu_seqlens_q, wl.cu_seqlens_k, wl.q, wl.k, wl.v, 1.0, 3, (-2, 0))


# ----------------------------------------------------------------------------
# arbitrary interval mask ("Mask support": func_tensor)
# ----------------------------------------------------------------------------
from generative_recommender_attention_amd.workloads import func_random_mask, func_target_mask  # noqa: E402


def func_of_window(wl, left, right):
    """Endpoints (N = 3) that spell a token window: [0, 0) u [i - left, i + right + 1)."""
    cols = []
    for b in range(wl.batch):
        i = np.arange(int(wl.lengths_q[b]))
        lk = int(wl.lengths_k[b])
        lo = np.zeros_like(i) if left < 0 else i - left
        hi = np.full_like(i, lk + 5) if right < 0 else i + right + 1
        cols.append(np.stack([np.zeros_like(i), lo, hi]))
    return np.concatenate(cols, axis=1).astype(np.int32)


def func_run(wl, f):
    args = (wl.cu_seqlens_q, wl.cu_seqlens_k)
    a, ls = float(wl.alpha), wl.scaling_seqlen
    o = oracle.fwd(*args, wl.q, wl.k, wl.v, a, ls, f)
    dq = oracle.bwd_dq(*args, wl.do, wl.q, wl.k, wl.v, a, ls, f)
    dk, dv = oracle.bwd_dkdv(*args, wl.do, wl.q, wl.k, wl.v, a, ls, f)
    return o, dq, dk, dv


def test_func_spelling_causal_full_and_windows_matches_them(oracle_lib):
    """Endpoints that spell causal (F0 = i + 1), full (F0 = L_k) and windows give those
    masks bit for bit; column r is the packed row, the endpoints local key indices."""
    wl = random_problem(60, [7, 12, 0, 5], [9, 12, 2, 4], 2, 8, True)
    i_local = np.concatenate([np.arange(n) for n in wl.lengths_q])
    lk_row = np.repeat(wl.lengths_k, wl.lengths_q)
    causal = (i_local + 1)[None, :].astype(np.int32)
    full = lk_row[None, :].astype(np.int32)
    for f, m in ((causal, (-1, 0)), (full, (-1, -1))):
        for x, y in zip(func_run(wl, f), _fwd_bwd(wl, m)):
            np.testing.assert_array_equal(x, y)
    for window in ((2, 0), (1, 3), (-1, 2), (4, -1), (0, 0)):
        for x, y in zip(func_run(wl, func_of_window(wl, *window)), _fwd_bwd(wl, window)):
            np.testing.assert_array_equal(x, y)


def test_func_union_is_order_free_and_idempotent(oracle_lib):
    """Swapping interval pairs, repeating one, adding a reversed (empty) one, or splitting
    one into two overlapping pieces leaves every output unchanged."""
    rng = np.random.default_rng(61)
    wl = random_problem(61, [9, 14], [11, 14], 2, 8, True)
    f = func_random_mask(rng, wl.lengths_q, wl.lengths_k, 5)
    base = func_run(wl, f)
    swapped = f[[0, 3, 4, 1, 2]]
    repeated = np.concatenate([f, f[1:3]])
    rev = np.concatenate([f, np.stack([f[2] + 3, f[2] - 2])]).astype(np.int32)   # start above end: empty
    mid = ((f[1].astype(np.int64) + f[2]) // 2).astype(np.int32)
    ok = f[1] < f[2]  # split proper intervals into two overlapping pieces, keep the others whole
    first_end = np.where(ok, mid + 1, f[2])
    second = np.where(ok, np.maximum(mid - 1, f[1]), 0), np.where(ok, f[2], 0)
    split = np.concatenate([f[[0]], np.stack([f[1], first_end, second[0], second[1]]), f[3:]]).astype(np.int32)
    for g in (swapped, repeated, rev, split):
        for x, y in zip(func_run(wl, g), base):
            np.testing.assert_array_equal(x, y)


def test_func_disjoint_intervals_add(oracle_lib):
    """With disjoint key sets A and B, O(A u B) = O(A) + O(B) (the masked sum is linear
    in the key set), and likewise every gradient."""
    wl = random_problem(62, [10, 13], None, 2, 8, True)
    rng = np.random.default_rng(62)
    cut = np.concatenate([rng.integers(0, n + 1, size=n) for n in wl.lengths_k]).astype(np.int32)
    zero = np.zeros_like(cut)
    a = np.stack([cut])                                    # [0, cut)
    b = np.stack([zero, cut, cut + 20])                    # [cut, past the end)
    ab = np.stack([cut, cut, cut + 20])
    for x, y, z in zip(func_run(wl, ab), func_run(wl, a), func_run(wl, b)):
        np.testing.assert_allclose(x, y + z, rtol=1e-12, atol=1e-14)


def union_length(f_col, lk):
    """|[0, F0) u [F1, F2) u ...| inside [0, lk), by sorting and merging the intervals."""
    iv = [(0, int(f_col[0]))] + [(int(f_col[n]), int(f_col[n + 1])) for n in range(1, len(f_col) - 1, 2)]
    iv = sorted((max(0, a), min(lk, b)) for a, b in iv if min(lk, b) > max(0, a))
    total, end = 0, 0
    for a, b in iv:
        if b <= end:
            continue
        total += b - max(a, end)
        end = b
    return total


@pytest.mark.parametrize("n", [1, 3, 7])
def test_func_visible_key_count_per_row(oracle_lib, n):
    """Equal keys and V = 1: O_i = |visible keys of row i| SiLU(s_i) / L_scale, the count
    from a sort-and-merge of the row's intervals."""
    rng = np.random.default_rng(63 + n)
    lq, lk = [11, 6, 9], [9, 12, 9]
    wl = random_problem(63 + n, lq, lk, 1, 8, True)
    f = func_random_mask(rng, lq, lk, n)
    q, k = f64(wl.q), f64(wl.k)
    for b in range(3):
        k[wl.cu_seqlens_k[b]:wl.cu_seqlens_k[b + 1]] = k[wl.cu_seqlens_k[b]]
    v = np.ones_like(f64(wl.v))
    a, ls = float(wl.alpha), wl.scaling_seqlen
    o = oracle.fwd(wl.cu_seqlens_q, wl.cu_seqlens_k, q, k, v, a, ls, f)
    for b in range(3):
        for i in range(lq[b]):
            r = wl.cu_seqlens_q[b] + i
            cnt = union_length(f[:, r], lk[b])
            s = a * math.fsum(q[r, 0] * k[wl.cu_seqlens_k[b], 0])
            want = cnt * s / (1.0 + math.exp(-s)) / ls
            np.testing.assert_allclose(o[r, 0], np.full(8, want), rtol=1e-12, atol=1e-15)


def test_func_matches_dense_brute_force_and_autograd(oracle_lib):
    """Random endpoints: the dense forward with the mask built by per-key membership
    over global indices, and its fp64 autograd for the backward."""
    rng = np.random.default_rng(70)
    lq, lk = [6, 0, 11, 4], [8, 3, 11, 2]
    wl = random_problem(70, lq, lk, 2, 8, True)
    f = func_random_mask(rng, lq, lk, 5)
    m = np.zeros((wl.total_q, wl.total_k))
    for b in range(4):
        for i in range(lq[b]):
            r = wl.cu_seqlens_q[b] + i
            keys = set(range(0, min(lk[b], max(0, f[0, r]))))
            for p in range(1, 5, 2):
                keys |= set(range(max(0, f[p, r]), min(lk[b], f[p + 1, r])))
            for j in keys:
                m[r, wl.cu_seqlens_k[b] + j] = 1.0
    q, k, v = (torch.from_numpy(f64(x)).requires_grad_(True) for x in (wl.q, wl.k, wl.v))
    mt = torch.from_numpy(m)
    a, ls = float(wl.alpha), wl.scaling_seqlen
    o = torch.stack([(mt * torch.nn.functional.silu(a * (q[:, h] @ k[:, h].T)) / ls) @ v[:, h]
                     for h in range(2)], dim=1)
    do = torch.from_numpy(f64(wl.do))
    (o * do).sum().backward()
    got = func_run(wl, f)
    np.testing.assert_allclose(got[0], o.detach().numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(got[1], q.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(got[2], k.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(got[3], v.grad.numpy(), rtol=1e-11, atol=1e-13)


def test_target_mask_layout():
    """History rows causal; candidate rows see the history and themselves only."""
    f = func_target_mask([10, 40, 1])
    # sequence 0: L = 10, one candidate (row 9); sequence 1: L = 40, 5 candidates; sequence 2: L = 1, row 0 a candidate
    assert f[:, 0].tolist() == [1, 0, 0] and f[:, 8].tolist() == [9, 0, 0] and f[:, 9].tolist() == [9, 9, 10]
    assert f[:, 10 + 34].tolist() == [35, 0, 0] and f[:, 10 + 35].tolist() == [35, 35, 36]
    assert f[:, 50].tolist() == [0, 0, 1]
