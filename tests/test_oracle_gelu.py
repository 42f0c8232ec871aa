"""Pins of the oracle's GELU and GELU' (the activation between the two
linears of the MLP block, exact erf form) and of the dGELU gradient.

The oracle evaluates GELU(x) = x Phi(x) and GELU'(x) = Phi(x) + x phi(x) in
fp64 with the C library's erfc and exp and rounds once to fp32.  These tests
tie it to things outside itself:
  - a 45-digit evaluation (mpmath) of both functions at every bf16 input with
    2^-40 <= |x| < 16: the oracle's fp32 must be the correctly rounded value,
    and each exact value must keep a stated distance from the nearest fp32
    rounding boundary, so that any fp64 evaluation accurate to a few units
    in the last place (the GPU's own, with another math library) rounds the
    same way;
  - the closed forms outside that range (|x| < 2^-40: GELU = x/2, GELU' = 1/2;
    |x| >= 16: GELU = x or -0, GELU' = 1 or -0) on every bf16 input there;
  - special values (signed zeros, infinities, NaN) and the canonical NaN;
  - the standard normal table values Phi(1), Phi(2), phi(1);
  - PyTorch's float32 exact GELU and its backward (another implementation),
    within a few fp32 units;
  - the dGELU composition bf16(fl32(dy * fl32(GELU'(x)))) against numpy's
    IEEE fp32 multiply.
"""
import mpmath
import numpy as np
import pytest
import torch

import oracle

ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)
MAG = ALL & 0x7FFF
F32 = (ALL.astype(np.uint32) << 16).view(np.float32)
TABLE = (MAG >= (87 << 7)) & (MAG < (131 << 7))      # 2^-40 <= |x| < 16
TINY = MAG < (87 << 7)
BIG = (MAG >= (131 << 7)) & (MAG < 0x7F80)           # 16 <= |x| < Inf
NEG = (ALL >> 15).astype(bool)


def _bits(f32):
    return np.asarray(f32, np.float32).view(np.uint32)


def _round_f32(v):
    """Correctly rounded fp32 of the mpmath value v (v != 0), and the distance
    of v from the nearest rounding boundary in units of the fp32 spacing."""
    f = np.float32(float(v))
    cand = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    err = [abs(mpmath.mpf(float(c)) - v) for c in cand]
    best = cand[min(range(3), key=lambda k: err[k])]
    dn, up = np.nextafter(best, np.float32(-np.inf)), np.nextafter(best, np.float32(np.inf))
    b = mpmath.mpf(float(best))
    lo, hi = (b + mpmath.mpf(float(dn))) / 2, (b + mpmath.mpf(float(up))) / 2
    margin = min(abs(v - lo) / (b - mpmath.mpf(float(dn))), abs(hi - v) / (mpmath.mpf(float(up)) - b))
    return best, float(margin)


def test_gelu_and_derivative_correctly_rounded_against_45_digits():
    mpmath.mp.dps = 45
    x = ALL[TABLE]
    g, d = oracle.gelu_f32(x), oracle.gelu_grad_f32(x)
    worst = 1.0
    for i, a in enumerate(F32[TABLE]):
        am = mpmath.mpf(float(a))
        cdf = mpmath.ncdf(am)
        rg, mg = _round_f32(am * cdf)
        rd, md = _round_f32(cdf + am * mpmath.npdf(am))
        assert _bits(rg) == _bits(g[i]), ("GELU", float(a), float(rg), float(g[i]))
        assert _bits(rd) == _bits(d[i]), ("GELU'", float(a), float(rd), float(d[i]))
        worst = min(worst, mg, md)
    # measured 2^-14.5 of a unit: every exact value lies at least 2^-38
    # (relative) away from a rounding boundary, far outside the error of an
    # fp64 evaluation
    assert worst > 2.0 ** -16, worst


def test_closed_forms_outside_the_table_range():
    g, d, h = oracle.gelu_f32(ALL), oracle.gelu_grad_f32(ALL), oracle.gelu(ALL)
    # |x| < 2^-40: GELU(x) = x/2 + O(x^2) rounds to x/2 (exact in fp32),
    # GELU'(x) = 1/2 + O(x) rounds to 1/2
    assert np.array_equal(_bits(g[TINY]), _bits(np.float32(0.5) * F32[TINY]))
    assert np.all(d[TINY] == np.float32(0.5))
    # |x| >= 16: 1 - Phi(16) < 1e-57, so GELU(x) = x for x > 0 and rounds to
    # -0 for x < 0; GELU'(x) = 1 above, -0 below (x phi(x) < 0 dominates)
    pos, neg = BIG & ~NEG, BIG & NEG
    assert np.array_equal(_bits(g[pos]), _bits(F32[pos]))
    assert np.all(_bits(g[neg]) == 0x80000000)
    assert np.all(d[pos] == np.float32(1.0))
    assert np.all(_bits(d[neg]) == 0x80000000)
    # the bf16 activation of a value >= 16 is the input itself; below -16 it is -0
    assert np.array_equal(h[pos], ALL[pos]) and np.all(h[neg] == 0x8000)
    # the boundaries themselves, at 45 digits: the terms dropped above are
    # below half a unit of the results there (2^-25 relative for a normal
    # result, half the smallest subnormal 2^-150 for a zero one), and they
    # shrink further away from the table range
    mpmath.mp.dps = 45
    two = mpmath.mpf(2)
    for a in (two ** -40, -(two ** -40), two ** 4, -(two ** 4)):
        cdf = mpmath.ncdf(a)
        g, d = a * cdf, cdf + a * mpmath.npdf(a)
        tg = a / 2 if abs(a) < 1 else (a if a > 0 else 0)
        td = mpmath.mpf(0.5) if abs(a) < 1 else (1 if a > 0 else 0)
        assert abs(g - tg) < (two ** -25 * abs(tg) if tg else two ** -150)
        assert abs(d - td) < (two ** -26 if td else two ** -150)


def test_special_values():
    def one(bits):
        x = np.array([bits], np.uint16)
        return oracle.gelu(x)[0], oracle.gelu_grad_f32(x)[0]
    assert one(0x0000) == (0x0000, np.float32(0.5))
    assert one(0x8000)[0] == 0x8000                        # GELU(-0) = -0
    assert one(0x7F80)[0] == 0x7F80                        # GELU(+Inf) = +Inf
    assert one(0xFF80)[0] == 0x7FC0                        # -Inf * Phi(-Inf) = -Inf * 0
    assert one(0x7FC1)[0] == 0x7FC0 and one(0xFFC0)[0] == 0x7FC0   # any NaN -> canonical
    for b in (0x7F80, 0xFF80, 0x7FC0):
        assert np.isnan(one(b)[1])                         # Phi(+-Inf) + (+-Inf) * 0
    x = ALL[~np.isnan(F32)]
    assert not np.any(np.isnan(oracle.gelu_f32(x[x != 0xFF80])))


def test_standard_normal_table_values():
    # Phi(1) = 0.8413447461, Phi(2) = 0.9772498681, phi(1) = 0.2419707245,
    # phi(2) = 0.0539909665 (standard normal tables)
    x = np.array([0x3F80, 0x4000, 0xBF80], np.uint16)      # 1, 2, -1
    g, d = oracle.gelu_f32(x), oracle.gelu_grad_f32(x)
    assert abs(g[0] - 0.8413447461) < 1e-7
    assert abs(g[1] - 2 * 0.9772498681) < 2e-7
    assert abs(g[2] - (0.8413447461 - 1)) < 1e-7           # GELU(-x) = GELU(x) - x
    assert abs(d[0] - (0.8413447461 + 0.2419707245)) < 1e-7
    assert abs(d[1] - (0.9772498681 + 2 * 0.0539909665)) < 2e-7
    assert abs(d[2] - (1 - 0.8413447461 - 0.2419707245)) < 1e-7   # GELU'(-x) = 1 - GELU'(x)


def test_against_torch_float32_gelu():
    x = ALL[np.isfinite(F32) & (np.abs(F32) < 64)]
    t = torch.from_numpy(((x.astype(np.uint32) << 16).view(np.float32)).copy())
    tg = torch.nn.functional.gelu(t, approximate="none").numpy()
    g = oracle.gelu_f32(x)
    ulp = np.spacing(np.abs(g)).astype(np.float64)
    diff = np.abs(tg.astype(np.float64) - g.astype(np.float64))
    # torch forms 1 + erf(x / sqrt 2), which cancels for negative x: its
    # error there is absolute, a few units of erf's last place times |x| / 2
    # (it returns 0 below x = -6)
    xf = np.abs(t.numpy().astype(np.float64))
    assert np.all(diff <= 4 * ulp + xf * 2.0 ** -21), float(np.max(diff - 4 * ulp - xf * 2.0 ** -21))
    t.requires_grad_(True)
    torch.nn.functional.gelu(t, approximate="none").backward(torch.ones_like(t))
    td = t.grad.numpy()
    d = oracle.gelu_grad_f32(x)
    diff = np.abs(td.astype(np.float64) - d.astype(np.float64))
    # GELU'(x) crosses zero near x = -0.75, where fp32 cancellation in the
    # two-term sum costs torch absolute, not relative, accuracy
    assert np.all(diff <= 8 * np.spacing(np.maximum(np.abs(d), np.float32(0.25)))), float(np.max(diff))


def test_gelu_bf16_is_rounded_fp32():
    x = ALL
    g = oracle.gelu_f32(x)
    expect = np.where(np.isnan(g), np.uint16(0x7FC0), oracle.bf16_rne(g))
    assert np.array_equal(oracle.gelu(x), expect)


def test_dgelu_is_one_fp32_product_then_bf16():
    rng = np.random.default_rng(11)
    n = 200000
    x = rng.integers(0, 65536, n).astype(np.uint16)
    dy = oracle.bf16_rne((rng.standard_normal(n) * 1e-3).astype(np.float32))
    # a few special gradients: +-0, +-Inf, NaN, subnormal
    dy[:6] = [0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0x0001]
    with np.errstate(invalid="ignore"):
        p = oracle.dec_bf16(dy) * oracle.gelu_grad_f32(x)   # numpy: IEEE fp32 multiply
    expect = np.where(np.isnan(p), np.uint16(0x7FC0), oracle.bf16_rne(p))
    assert np.array_equal(oracle.dgelu(dy, x), expect)


@pytest.mark.parametrize("scaling", ["tensor", "1x128"])
def test_quant_gelu_is_quantize_of_the_activation(scaling):
    rng = np.random.default_rng(5)
    a = oracle.bf16_rne((rng.standard_normal((256, 384)) * 0.45).astype(np.float32))
    dh = oracle.bf16_rne((rng.standard_normal((256, 384)) * 1e-3).astype(np.float32))
    q = oracle.quant_gelu(a, "e4m3", scaling)
    r = oracle.quantize(oracle.gelu(a), "e4m3", scaling)
    assert np.array_equal(q["q_row"], r["q_row"]) and np.array_equal(q["q_col"], r["q_col"])
    q = oracle.quant_dgelu(dh, a, "e5m2", scaling)
    r = oracle.quantize(oracle.dgelu(dh, a), "e5m2", scaling)
    assert np.array_equal(q["q_row"], r["q_row"]) and np.array_equal(q["q_col"], r["q_col"])
