"""Host logic of the benchmark: the visible-pair count its flop figures rest on,
and the refusal of more than one GPU.  No GPU is touched."""

import json

import numpy as np
import pytest

import bench


def brute_pairs(lq, lk, left, right):
    n = 0
    for i in range(lq):
        for j in range(lk):
            if (left < 0 or j >= i - left) and (right < 0 or j <= i + right):
                n += 1
    return n


@pytest.mark.parametrize("window", [(-1, -1), (-1, 0), (0, 0), (3, 0), (2, 5), (-1, 4), (7, -1), (40, 40)])
def test_visible_pairs_matches_brute_force(window):
    lens_q, lens_k = [0, 1, 9, 17, 30], [4, 1, 12, 17, 25]
    want = sum(brute_pairs(a, b, *window) for a, b in zip(lens_q, lens_k))
    assert bench.visible_pairs(lens_q, lens_k, window) == want


def test_causal_pairs_closed_form():
    n = np.array([1, 64, 4096])
    assert bench.visible_pairs(n, n, (-1, 0)) == int((n * (n + 1) // 2).sum())


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    out = json.loads(capsys.readouterr().out.strip())
    assert "one GPU" in out["error"]


def test_func_pairs_match_window_and_random_brute_force():
    from generative_recommender_attention_amd.workloads import func_random_mask

    lens_q, lens_k = [5, 0, 13, 9], [7, 2, 13, 4]
    i = np.concatenate([np.arange(n) for n in lens_q])
    f = np.stack([np.zeros_like(i), i - 2, i + 4]).astype(np.int32)  # window (2, 3)
    assert bench.func_visible_pairs(f, lens_q, lens_k) == bench.visible_pairs(lens_q, lens_k, (2, 3))
    f = func_random_mask(np.random.default_rng(3), lens_q, lens_k, 5)
    want, r0 = 0, 0
    for lq, lk in zip(lens_q, lens_k):
        for r in range(r0, r0 + lq):
            keys = set(range(0, min(lk, max(0, f[0, r]))))
            for n in (1, 3):
                keys |= set(range(max(0, f[n, r]), min(lk, f[n + 1, r])))
            want += len(keys)
        r0 += lq
    assert bench.func_visible_pairs(f, lens_q, lens_k) == want


def test_source_digest_ignores_comments():
    code = "int f(int x) { // add one\n  return x + 1; /* done */ }\n"
    assert bench._code_only(code) == bench._code_only("int f(int x) {\n return x + 1; }")
    assert bench._code_only(code) != bench._code_only("int f(int x) { return x + 2; }")


def test_clock_summary_pairs_readings_by_cu():
    """Two launches 1 ms apart (100 MHz real-time ticks); every CU's cycle counter has
    its own offset; the CUs of XCD 0 advance 1.8e6 cycles, those of XCD 1 2.0e6, and
    one CU of XCD 1 appears only in the first launch."""
    before, after = [], []
    for w in range(16):
        x, cu = w % 2, w // 2
        hwid = cu << 8
        off = 10_000_000 * (w + 1)  # per-CU counter offset
        before.append([1000 + w, off, x, hwid])
        if w != 15:
            after.append([101_000 + w, off + (1_800_000 if x == 0 else 2_000_000), x, hwid])
    before.append([1003, 10_000_000 + 50, 0, 0])  # a second workgroup on CU 0 of XCD 0
    c = bench.clock_summary(np.array(before), np.array(after))
    assert c["per_xcd_mhz"] == {"0": 1800.0, "1": 2000.0}
    assert c["shader_mhz"] == 1900.0
    assert c["cus_paired"] == 15
    assert c["region_us_by_realtime"] == 1000.0
    assert c["counter_spread_cycles"] == 50


def test_cpu_model_is_named():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()
