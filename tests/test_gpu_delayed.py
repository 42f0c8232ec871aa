"""Delayed tensorwise scaling (amax history) on the GPU against the oracle,
through the C ABI: every code, scale and history entry bit-exact over
sequences of calls; and the weight-caching consequence the oracle pins
(cached differs from requantizing under delayed scaling) reproduced byte for
byte."""
import numpy as np
import pytest
import torch

import oracle
from _util import to_np_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    import fp8_mixed_precision_amax_amd as m
    m.lib()
    return m


def _bf16(shape, sigma, seed):
    rng = np.random.default_rng(seed)
    return oracle.bf16_rne((rng.standard_normal(shape) * sigma).astype(np.float32))


def _u32(t):
    return t.detach().cpu().numpy().view(np.uint32)


def _check(got, ref, hist_dev, hist_ref, name):
    assert np.array_equal(to_np_u8(got.q_row), ref["q_row"]), name + ": row codes"
    assert np.array_equal(to_np_u8(got.q_col), ref["q_col"]), name + ": col codes"
    assert _u32(got.scale)[0] == np.float32(ref["scale"]).view(np.uint32), name + ": scale"
    assert _u32(got.scale_inv)[0] == np.float32(ref["scale_inv"]).view(np.uint32), name + ": scale_inv"
    assert _u32(got.amax)[0] == np.float32(ref["amax"]).view(np.uint32), name + ": amax"
    assert np.array_equal(_u32(hist_dev), hist_ref.view(np.uint32)), name + ": history"


# rows, cols, history length, format
CASES = [(256, 384, 1, "e4m3"), (640, 512, 16, "e5m2"), (1024, 2048, 1024, "e4m3"), (128, 128, 7, "e5m2")]


@pytest.mark.parametrize("R,C,H,fmt", CASES)
def test_delayed_sequence_matches_oracle(fp8, R, C, H, fmt):
    dev = torch.device("cuda")
    F = fp8.E4M3 if fmt == "e4m3" else fp8.E5M2
    hist_ref = np.zeros(H, np.float32)
    hist_dev = torch.zeros(H, dtype=torch.float32, device=dev)
    # five calls on tensors of growing and shrinking spread: the history fills
    # and (H < 5) rolls over
    for k, sigma in enumerate([1.0, 4.0, 0.25, 2.0, 1.0]):
        x = _bf16((R, C), sigma, 100 * k + R)
        ref = oracle.quant_delayed(x, fmt, hist_ref)
        hist_ref = ref["history"]
        got = fp8.quantize_delayed(torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16), F, hist_dev)
        torch.cuda.synchronize()
        _check(got, ref, hist_dev, hist_ref, "call %d" % k)


def test_delayed_special_histories(fp8):
    dev = torch.device("cuda")
    x = _bf16((256, 256), 1.0, 9)
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    for h in ([0.0, 0.0], [0.5, np.nan], [np.inf, 1.0], [np.float32(1e-38)], [3.0, 7.5, 0.0, 2.0]):
        href = np.array(h, np.float32)
        ref = oracle.quant_delayed(x, "e4m3", href)
        hd = torch.from_numpy(href.copy()).to(dev)
        got = fp8.quantize_delayed(xd, fp8.E4M3, hd)
        torch.cuda.synchronize()
        _check(got, ref, hd, ref["history"], "history %s" % (h,))


def test_delayed_nan_input_patched(fp8):
    dev = torch.device("cuda")
    x = _bf16((256, 256), 1.0, 10)
    x[7, 9] = 0x7FC0          # NaN
    x[200, 3] = 0xFF80        # -Inf
    ref = oracle.quant_delayed(x, "e5m2", np.array([2.0], np.float32))
    hd = torch.tensor([2.0], device=dev)
    got = fp8.quantize_delayed(torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16), fp8.E5M2, hd)
    torch.cuda.synchronize()
    _check(got, ref, hd, ref["history"], "NaN input")


def test_weight_cache_under_delayed_scaling(fp8):
    """Three accumulation cycles of four microbatches, as the oracle pin:
    uncached requantizes W every microbatch, cached only on the first.  The
    GPU bytes equal the oracle's in both runs, and the runs differ."""
    dev = torch.device("cuda")
    H = 4
    rng = np.random.default_rng(7)
    W = [oracle.bf16_rne((rng.standard_normal((256, 512)) * (0.02 * (c + 1))).astype(np.float32)) for c in range(3)]
    h_unc_ref, h_cac_ref = np.zeros(H, np.float32), np.zeros(H, np.float32)
    h_unc, h_cac = torch.zeros(H, device=dev), torch.zeros(H, device=dev)
    differ = 0
    for w in W:
        wd = torch.from_numpy(w.view(np.int16)).to(dev).view(torch.bfloat16)
        for mb in range(4):
            ref_u = oracle.quant_delayed(w, "e4m3", h_unc_ref)
            h_unc_ref = ref_u["history"]
            got_u = fp8.quantize_delayed(wd, fp8.E4M3, h_unc)
            if mb == 0:
                ref_c = oracle.quant_delayed(w, "e4m3", h_cac_ref)
                h_cac_ref = ref_c["history"]
                got_c = fp8.quantize_delayed(wd, fp8.E4M3, h_cac)
            torch.cuda.synchronize()
            _check(got_u, ref_u, h_unc, h_unc_ref, "uncached")
            _check(got_c, ref_c, h_cac, h_cac_ref, "cached")
            if not torch.equal(got_u.q_row, got_c.q_row):
                differ += 1
    assert differ >= 3
