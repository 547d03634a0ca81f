"""The parity checker itself, on the CPU: it must accept outputs that are off by
bf16-level rounding and reject the plausible wrong outputs that the plain bar
alone would let through on the Zipf workload (B=32, H=4, D=128, causal), where
most sequences are short and their outputs sit below the bar's absolute term.

The reference is the fp64 oracle on sampled rows of that workload (every row of
the short sequences, edges and random rows of the long ones)."""

import numpy as np
import pytest

from generative_recommender_attention_amd.workloads import named_workload
from hip_cases import check_close, sample_rows


@pytest.fixture(scope="module")
def zipf_ref(oracle_lib):
    wl = named_workload("zipf_b32_h4_d128_causal")
    rows = sample_rows(wl.cu_seqlens_q, per_seq=24)
    ref = oracle_lib.fwd_workload(wl, rows)
    return wl, rows, ref


def _fails(got, ref, cu, rows):
    with pytest.raises(AssertionError):
        check_close("o", got, ref, cu, rows)


def test_accepts_bf16_level_error(zipf_ref):
    wl, rows, ref = zipf_ref
    rng = np.random.default_rng(0)
    # relative noise of 4e-3 per element, about what two bf16 roundings leave
    got = ref * (1.0 + 4e-3 * rng.uniform(-1, 1, size=ref.shape))
    err, worst = check_close("o", got, ref, wl.cu_seqlens_q, rows)
    assert err < 5e-3 and worst < 5e-3


def test_rejects_all_zero_output(zipf_ref):
    wl, rows, ref = zipf_ref
    _fails(np.zeros_like(ref), ref, wl.cu_seqlens_q, rows)


def test_rejects_one_short_sequence_zeroed(zipf_ref):
    wl, rows, ref = zipf_ref
    cu = wl.cu_seqlens_q
    lengths = np.diff(cu)
    b = int(np.argmin(lengths))  # a 16-token sequence, far below the bar's absolute term
    sel = (rows >= cu[b]) & (rows < cu[b + 1])
    assert np.abs(ref[sel]).max() < 1e-3  # the plain bar alone would accept zeros here
    got = ref.copy()
    got[sel] = 0.0
    _fails(got, ref, cu, rows)


def test_rejects_sign_flip_of_one_sequence(zipf_ref):
    wl, rows, ref = zipf_ref
    cu = wl.cu_seqlens_q
    b = int(np.argsort(np.diff(cu))[len(cu) // 2])
    sel = (rows >= cu[b]) & (rows < cu[b + 1])
    got = ref.copy()
    got[sel] = -got[sel]
    _fails(got, ref, cu, rows)


def test_rejects_rows_shifted_by_one(zipf_ref):
    wl, rows, ref = zipf_ref
    got = np.roll(ref, 1, axis=0)  # an off-by-one row index
    _fails(got, ref, wl.cu_seqlens_q, rows)


def test_rejects_non_finite(zipf_ref):
    wl, rows, ref = zipf_ref
    got = ref.copy()
    got[0, 0, 0] = np.nan
    _fails(got, ref, wl.cu_seqlens_q, rows)
