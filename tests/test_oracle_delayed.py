"""Pins of the oracle's delayed tensorwise scaling (amax history), the case the
weight-caching issue contrasts with block scaling (TransformerEngine issue
2852, question 3).  Each check ties the function to something outside itself:
hand-derived OCP codes, a reduction to current scaling, the closed form of
the history roll, the special cases of the scale rule, and the caching
consequence itself.
"""
import numpy as np

import oracle

BF16 = {1.0: 0x3F80, -2.0: 0xC000, 0.5: 0x3F00, 0.0: 0x0000, 3.0: 0x4040}


def _x(vals):
    return np.array([[BF16[v] for v in vals]], np.uint16)


def test_worked_example_e4m3():
    # history [4, 0]: scale = 448 / 4 = 112.  1 * 112 = 1.75 * 2^6 -> exponent
    # field 6 + 7 = 13, mantissa .75 -> 0 1101 110 = 0x6E; -224 = 1.75 * 2^7 ->
    # 1 1110 110 = 0xF6; 56 = 1.75 * 2^5 -> 0 1100 110 = 0x66; 0 -> 0x00.
    r = oracle.quant_delayed(_x([1.0, -2.0, 0.5, 0.0]), "e4m3", [4.0, 0.0])
    assert list(r["q_row"][0]) == [0x6E, 0xF6, 0x66, 0x00]
    assert r["scale"] == np.float32(112.0) and r["scale_inv"] == np.float32(1.0 / 112.0)
    # this call's amax (2) goes in front, the oldest entry drops out
    assert list(r["history"]) == [2.0, 4.0]
    assert r["amax"] == np.float32(2.0)


def test_worked_example_e5m2():
    # history [4]: scale = 57344 / 4 = 14336 = 1.75 * 2^13.  E5M2 bias 15:
    # 14336 -> 0 11100 11 = 0x73; -28672 -> 1 11101 11 = 0xF7; 7168 -> 0x6F.
    r = oracle.quant_delayed(_x([1.0, -2.0, 0.5]), "e5m2", [4.0])
    assert list(r["q_row"][0]) == [0x73, 0xF7, 0x6F]
    assert list(r["history"]) == [2.0]


def test_history_max_equal_to_amax_is_current_scaling():
    rng = np.random.default_rng(3)
    x = oracle.bf16_rne(rng.standard_normal((256, 384)).astype(np.float32))
    a = float(oracle.amax_bf16(x))
    for fmt in ("e4m3", "e5m2"):
        ref = oracle.quant_tensor(x, fmt)
        d = oracle.quant_delayed(x, fmt, [0.5 * a, a, 0.25 * a])
        assert np.array_equal(d["q_row"], ref["q_row"]) and np.array_equal(d["q_col"], ref["q_col"])
        assert d["scale"] == ref["scale"] and d["scale_inv"] == ref["scale_inv"]


def test_history_roll_closed_form():
    # after k calls on tensors whose amaxes are 1, 2, ..., k (here x = [[k]]
    # encoded in bf16), a length-H history holds k, k-1, ..., down to k-H+1
    # (zeros where fewer calls were made)
    H = 3
    h = np.zeros(H, np.float32)
    for k in range(1, 6):
        x = np.array([[oracle.bf16_rne(np.array([k], np.float32))[0]]], np.uint16)
        h = oracle.quant_delayed(x, "e4m3", h)["history"]
        expect = [float(max(k - i, 0)) for i in range(H)]
        assert list(h) == expect, (k, list(h))


def test_special_histories():
    x = _x([1.0, 3.0])
    # all zeros (no earlier call): scale 1
    assert oracle.quant_delayed(x, "e4m3", [0.0, 0.0])["scale"] == np.float32(1.0)
    # a NaN anywhere in the history: scale 1 (the NaN / Inf rule of current scaling)
    r = oracle.quant_delayed(x, "e4m3", [0.5, np.nan])
    assert r["scale"] == np.float32(1.0)
    # +Inf: scale 1; a tiny amax: the scale saturates at FLT_MAX
    assert oracle.quant_delayed(x, "e4m3", [np.inf])["scale"] == np.float32(1.0)
    r = oracle.quant_delayed(x, "e4m3", [np.float32(1e-38)])
    assert r["scale"] == np.finfo(np.float32).max


def _weights(cycles, rng, K=128, M=128):
    # one weight per accumulation cycle (an optimizer step between cycles),
    # with clearly different amaxes
    return [oracle.bf16_rne((rng.standard_normal((M, K)) * (0.02 * (c + 1))).astype(np.float32))
            for c in range(cycles)]


def test_caching_changes_results_under_delayed_scaling_only():
    """Three accumulation cycles of four microbatches.  Uncached: W is
    quantized every microbatch; cached: only on the first microbatch of a
    cycle (is_first_microbatch True, then False), the others reuse its bytes.
    Under current scaling both use identical bytes in every microbatch.
    Under delayed scaling the uncached run's second microbatch already sees
    this cycle's own amax in W's history, while the cache still holds bytes
    scaled by the previous cycle's history: the runs differ."""
    rng = np.random.default_rng(7)
    W = _weights(3, rng)
    H = 4
    h_unc = np.zeros(H, np.float32)
    h_cac = np.zeros(H, np.float32)
    differ_delayed = 0
    for c, w in enumerate(W):
        cached_codes = None
        for mb in range(4):
            cur = oracle.quant_tensor(w, "e4m3")["q_row"]
            unc = oracle.quant_delayed(w, "e4m3", h_unc)
            h_unc = unc["history"]
            if mb == 0:
                cac = oracle.quant_delayed(w, "e4m3", h_cac)
                h_cac = cac["history"]
                cached_codes = cac["q_row"]
                cached_cur = cur
            # current scaling: the cache is exactly what requantizing gives
            assert np.array_equal(cached_cur, cur)
            if not np.array_equal(unc["q_row"], cached_codes):
                differ_delayed += 1
    # every cycle after the first scale change differs on microbatches 1..3
    assert differ_delayed >= 3
