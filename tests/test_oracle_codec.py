"""Pins of the oracle's element codecs (FP8 encode/decode, bf16 rounding).

Each pin compares the oracle against something other than itself:
  * torch's CPU float8_e4m3fn / float8_e5m2 dtypes (library decode tables and
    library round-to-nearest-even casts, which differ from the oracle only in
    the overflow mode),
  * a brute-force nearest-value search over the 256-code table,
  * worked values from the OCP FP8 format tables (tests/golden),
  * torch's fp32 -> bf16 conversion.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_worked_values.txt")
TORCH_DT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
FMT_FMAX = {"e4m3": 448.0, "e5m2": 57344.0}


def torch_table(fmt):
    return torch.arange(256, dtype=torch.uint8).view(TORCH_DT[fmt]).float().numpy()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_decode_matches_torch_table(fmt):
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.dec(codes, fmt)
    ref = torch_table(fmt)
    both_nan = np.isnan(mine) & np.isnan(ref)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.all(both_nan | (mine.view(np.uint32) == ref.view(np.uint32)))


@pytest.mark.parametrize("fmt,finite,fmax,min_sub,min_norm",
                         [("e4m3", 254, 448.0, 2.0 ** -9, 2.0 ** -6),
                          ("e5m2", 248, 57344.0, 2.0 ** -16, 2.0 ** -14)])
def test_format_constants(fmt, finite, fmax, min_sub, min_norm):
    v = oracle.dec(np.arange(256, dtype=np.uint8), fmt)
    assert np.isfinite(v).sum() == finite
    assert np.nanmax(np.where(np.isfinite(v), v, np.nan)) == fmax
    assert oracle.fmax(fmt) == fmax
    pos = v[np.isfinite(v) & (v > 0)]
    assert pos.min() == min_sub
    # smallest value with a non-zero exponent field
    assert oracle.dec(np.array([1 << (3 if fmt == "e4m3" else 2)], np.uint8), fmt)[0] == min_norm


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_roundtrip_all_codes(fmt):
    codes = np.arange(256, dtype=np.uint8)
    v = oracle.dec(codes, fmt)
    back = oracle.enc(v, fmt)
    for c in range(256):
        if np.isnan(v[c]):
            assert back[c] == 0x7F
        elif np.isinf(v[c]):            # E5M2 infinities saturate
            assert back[c] == (0x7B | (c & 0x80))
        else:
            assert back[c] == c, (fmt, hex(c), v[c], hex(back[c]))


def brute_force_encode(v, fmt):
    """Nearest finite FP8 value by exhaustive search over torch's decode
    table; ties go to the code with an even mantissa LSB (an even code);
    values beyond the largest finite magnitude clamp to it; NaN -> 0x7F.
    Zero results keep the sign of the input."""
    tab = torch_table(fmt).astype(np.float64)
    finite = np.where(np.isfinite(tab))[0]
    vals = tab[finite]
    order = np.argsort(vals, kind="stable")
    finite, vals = finite[order], vals[order]
    v = np.asarray(v, np.float32)
    with np.errstate(invalid="ignore"):   # NaN patterns among the inputs
        vd = v.astype(np.float64)
    out = np.empty(v.shape, np.uint8)
    flat_v = vd.reshape(-1)
    flat_o = out.reshape(-1)
    chunk = 1 << 14
    for s in range(0, flat_v.size, chunk):
        x = flat_v[s:s + chunk]
        neg = np.signbit(x)
        isnan = np.isnan(x)
        x = np.clip(np.where(isnan, 0.0, x), vals[0], vals[-1])   # saturate first
        d = np.abs(x[:, None] - vals[None, :])
        best = d.min(axis=1, keepdims=True)
        cand = d == best
        # among equally near codes prefer the even code
        even = (finite % 2 == 0)[None, :]
        pick_even = cand & even
        has_even = pick_even.any(axis=1)
        idx = np.where(has_even, pick_even.argmax(axis=1), cand.argmax(axis=1))
        codes = finite[idx].astype(np.uint8)
        # +0 and -0 are both in the table; keep the input's sign on zero
        zero = vals[idx] == 0.0
        codes = np.where(zero & neg, 0x80, np.where(zero, 0x00, codes))
        codes = np.where(isnan, 0x7F, codes)
        flat_o[s:s + chunk] = codes
    return out


def structured_fp32(fmt, rng):
    """Every FP8 value, every midpoint between neighbours, one fp32 ulp either
    side of each, the format's limits, specials, all bf16 patterns, and random
    fp32 bit patterns."""
    tab = torch_table(fmt).astype(np.float64)
    fin = np.unique(tab[np.isfinite(tab)])
    mids = (fin[1:] + fin[:-1]) / 2.0
    pts = np.concatenate([fin, mids, [FMT_FMAX[fmt] * 1.03, FMT_FMAX[fmt] * 1.0715, 1e30, -1e30]])
    p32 = pts.astype(np.float32)
    vals = [p32, np.nextafter(p32, np.float32(np.inf)), np.nextafter(p32, np.float32(-np.inf))]
    vals.append(np.array([np.inf, -np.inf, np.nan, -np.nan, 0.0, -0.0, 1e-45, -1e-45,
                          np.finfo(np.float32).max, -np.finfo(np.float32).max], np.float32))
    bf = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    vals.append(bf)
    vals.append(rng.integers(0, 2 ** 32, size=1 << 17, dtype=np.uint64).astype(np.uint32).view(np.float32))
    # random values concentrated on the format's range
    vals.append((rng.standard_normal(1 << 16) * FMT_FMAX[fmt] / 8).astype(np.float32))
    return np.concatenate(vals)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_encode_matches_brute_force(fmt):
    rng = np.random.default_rng(1234)
    v = structured_fp32(fmt, rng)
    mine = oracle.enc(v, fmt)
    ref = brute_force_encode(v, fmt)
    bad = np.where(mine != ref)[0]
    assert bad.size == 0, [(float(v[i]), hex(mine[i]), hex(ref[i])) for i in bad[:10]]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_encode_matches_torch_cast_in_range(fmt):
    """torch's CPU cast rounds to nearest even but overflows to NaN/Inf; in the
    range where no overflow happens both must agree bit for bit."""
    rng = np.random.default_rng(99)
    v = structured_fp32(fmt, rng)
    lim = 464.0 if fmt == "e4m3" else 61440.0
    with np.errstate(invalid="ignore"):   # NaN patterns among the inputs
        keep = np.isfinite(v) & (np.abs(v.astype(np.float64)) < lim)
    v = v[keep]
    mine = oracle.enc(v, fmt)
    ref = torch.from_numpy(v).to(TORCH_DT[fmt]).view(torch.uint8).numpy()
    bad = np.where(mine != ref)[0]
    assert bad.size == 0, [(float(v[i]), hex(mine[i]), hex(ref[i])) for i in bad[:10]]


def test_golden_worked_values():
    n = 0
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fmt, bits, code = line.split()[:3]
            v = np.array([int(bits, 16)], np.uint32).view(np.float32)
            got = oracle.enc(v, fmt)[0]
            assert got == int(code, 16), line
            n += 1
    assert n >= 25


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(7)
    r = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    # exact ties (low 16 bits = 0x8000) with both parities, and one off either side
    ties = (r & 0xFFFF0000) | 0x8000
    v = np.concatenate([r, ties, ties + 1, ties - 1]).view(np.float32)
    v = v[~np.isnan(v)]
    mine = oracle.bf16_rne(v)
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    nan = oracle.bf16_rne(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def test_bf16_decode_is_exact():
    bits = np.arange(65536, dtype=np.uint16)
    v = oracle.dec_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    ok = (v.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(v) & np.isnan(ref))
    assert ok.all()
