"""Amax hand-off (producer-side amax), tensorwise recipe, through the C ABI.

A GEMM that writes a bf16 tensor can emit its amax as partial maxima; the
tensorwise quantize of that tensor then skips its amax pass.  Pinned here:
  - the partials reduce to exactly max |C| of the GEMM's own output (amax is
    an exact, order-free maximum of bf16 magnitudes), unused slots are zero,
    and C itself is bitwise the plain GEMM's;
  - the cast-only quantize from those partials gives bytes, scales and amax
    bitwise equal to the two-pass quantize of the same tensor (whose parity
    with the oracle the quantize tests establish);
  - a two-layer chain (forward: Y1 -> X2; backward: dX2 -> dY1) with the
    hand-off gives every output bitwise equal to the same calls without it.
Each of these is also held against the oracle: the partials against the
oracle's amax of the GPU's bf16 output, the cast-only quantize against the
oracle's quantize of that output, and the chain layer by layer (the oracle
fed the GPU's bf16 layer inputs Y1 and dX2).
"""
import numpy as np
import pytest
import torch

import oracle
from _util import check_gemm, to_np_u16, to_np_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    import fp8_mixed_precision_amax_amd as m
    m.lib()
    return m


def _mag_max(bf16):
    """max |x| of a bf16 tensor as magnitude bits (NaN above +Inf)."""
    bits = bf16.view(torch.int16).to(torch.int32) & 0x7FFF
    return int(bits.max().item())


def _slots(partials):
    return partials.view(torch.int16).to(torch.int32) & 0xFFFF


def _codes(shape, seed, dev):
    g = torch.Generator(device="cpu").manual_seed(seed)
    # E4M3 codes without NaN (0x7F / 0xFF excluded), random signs
    c = torch.randint(0, 0x7F, shape, generator=g, dtype=torch.int32)
    c |= torch.randint(0, 2, shape, generator=g, dtype=torch.int32) << 7
    return c.to(torch.uint8).to(dev)


# I, J, K: one tile, a ragged tile count, split-K (small output, long contraction),
# the bench's forward shape
SHAPES = [(256, 256, 512), (640, 384, 1024), (256, 256, 16384), (131072, 2048, 512)]


@pytest.mark.parametrize("I,J,K", SHAPES)
def test_gemm_emits_amax_of_its_output(fp8, I, J, K):
    dev = torch.device("cuda")
    a, b = _codes((I, K), 1 + I, dev), _codes((J, K), 2 + J, dev)
    s = torch.tensor([1.0 / 512], device=dev)
    plain = fp8.gemm(a, fp8.E4M3, fp8.gemm_scale(s), b, fp8.E4M3, fp8.gemm_scale(s))
    part = fp8.amax_partials(dev)
    part.fill_(0xAB)   # every slot must be written
    c = fp8.gemm(a, fp8.E4M3, fp8.gemm_scale(s), b, fp8.E4M3, fp8.gemm_scale(s), amax_out=part)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), plain.view(torch.int16)), "C differs from fp8_gemm's"
    slots = _slots(part)
    assert int(slots.max().item()) == _mag_max(c), "partials do not reduce to max |C|"
    amax_ref = np.float32(oracle.amax_bf16(to_np_u16(c)))
    assert int(slots.max().item()) == int(amax_ref.view(np.uint32) >> 16), "partials differ from the oracle's amax"
    # one slot per workgroup (the GEMM's grid or the split-K reduce's), the rest zero
    nz = int((slots != 0).sum().item())
    assert nz <= 2048 and bool((slots[nz:] == 0).all().item()), "slots after the written ones must be zero"


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quantize_from_gemm_partials_matches_two_pass(fp8, fmt):
    dev = torch.device("cuda")
    I, J, K = 4096, 1024, 2048
    a, b = _codes((I, K), 11, dev), _codes((J, K), 12, dev)
    s = torch.tensor([1.0 / 64], device=dev)
    part = fp8.amax_partials(dev)
    x = fp8.gemm(a, fp8.E4M3, fp8.gemm_scale(s), b, fp8.E4M3, fp8.gemm_scale(s), amax_out=part)
    F = fp8.E4M3 if fmt == "e4m3" else fp8.E5M2
    ref = fp8.quantize(x, F)
    got = fp8.quantize(x, F, amax_partials=part)
    torch.cuda.synchronize()
    for name in ("q_row", "q_col", "scale", "scale_inv", "amax"):
        assert torch.equal(getattr(got, name), getattr(ref, name)), name
    o = oracle.quant_tensor(to_np_u16(x), fmt)
    assert np.array_equal(to_np_u8(got.q_row), o["q_row"]) and np.array_equal(to_np_u8(got.q_col), o["q_col"])
    f = lambda t: t.cpu().numpy().view(np.uint32)[0]
    assert f(got.scale) == np.float32(o["scale"]).view(np.uint32)
    assert f(got.scale_inv) == np.float32(o["scale_inv"]).view(np.uint32)
    assert f(got.amax) == np.float32(o["amax"]).view(np.uint32)


def test_linear_chain_handoff_is_bitwise(fp8):
    """Two stacked linears 512 -> 1024 -> 512, N = 8192: the hand-off moves
    amaxes between the layers (Y1 -> X2 forward, dX2 -> dY1 backward) and
    changes no byte of any output."""
    dev = torch.device("cuda")
    N, D, H = 8192, 512, 1024
    g = torch.Generator(device="cpu").manual_seed(5)
    x1 = torch.randn(N, D, generator=g).to(torch.bfloat16).to(dev)
    w1 = (torch.randn(H, D, generator=g) * 0.02).to(torch.bfloat16).to(dev)
    w2 = (torch.randn(D, H, generator=g) * 0.02).to(torch.bfloat16).to(dev)
    dy2 = (torch.randn(N, D, generator=g) * 1e-3).to(torch.bfloat16).to(dev)

    def run(handoff):
        l1 = fp8.Fp8Linear(N, D, H, device=dev)
        l2 = fp8.Fp8Linear(N, H, D, device=dev)
        p_y1, p_dx2 = (fp8.amax_partials(dev), fp8.amax_partials(dev)) if handoff else (None, None)
        y1 = l1.forward(x1, w1, y_amax=p_y1)
        y2 = l2.forward(y1, w2, x_amax=p_y1)
        dx2, dw2 = l2.backward(dy2, dx_amax=p_dx2)
        dx1, dw1 = l1.backward(dx2, dy_amax=p_dx2)
        torch.cuda.synchronize()
        q = {"x2_row": l2.saved_x.q_row, "x2_col": l2.saved_x.q_col, "x2_scale": l2.saved_x.scale,
             "x2_scale_inv": l2.saved_x.scale_inv,
             "dy1_row": l1.dy_q.q_row, "dy1_col": l1.dy_q.q_col, "dy1_scale": l1.dy_q.scale,
             "dy1_scale_inv": l1.dy_q.scale_inv}
        return {"y1": y1, "y2": y2, "dx2": dx2, "dw2": dw2, "dx1": dx1, "dw1": dw1, **{k: v.clone() for k, v in q.items()}}

    plain, chained = run(False), run(True)
    for k in plain:
        a, b = plain[k], chained[k]
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b), k

    # the chained run against the oracle, layer by layer, fed the GPU's Y1 and dX2
    c = chained
    y1b, dx2b = to_np_u16(c["y1"]), to_np_u16(c["dx2"])
    y2r, ctx2 = oracle.linear_fwd(y1b, to_np_u16(w2), "tensor")
    x2q = ctx2["xq"]
    assert np.array_equal(to_np_u8(c["x2_row"]), x2q["q_row"]) and np.array_equal(to_np_u8(c["x2_col"]), x2q["q_col"])
    assert c["x2_scale_inv"].cpu().numpy().view(np.uint32)[0] == np.float32(x2q["scale_inv"]).view(np.uint32)
    _, ctx1 = oracle.linear_fwd(to_np_u16(x1), to_np_u16(w1), "tensor")
    dx1r, dw1r, dy1q = oracle.linear_bwd(dx2b, ctx1)
    assert np.array_equal(to_np_u8(c["dy1_row"]), dy1q["q_row"]) and np.array_equal(to_np_u8(c["dy1_col"]), dy1q["q_col"])
    assert c["dy1_scale_inv"].cpu().numpy().view(np.uint32)[0] == np.float32(dy1q["scale_inv"]).view(np.uint32)
    rng = np.random.default_rng(6)
    w2q, w1q, x1q = ctx2["wq"], ctx1["wq"], ctx1["xq"]
    for name, got, ref, A, fa, B, fb, t, Kc in [
        ("Y2", c["y2"], y2r, x2q["q_row"], "e4m3", w2q["q_row"], "e4m3", x2q["scale_inv"] * w2q["scale_inv"], H),
        ("dX1", c["dx1"], dx1r, dy1q["q_row"], "e5m2", w1q["q_col"], "e4m3", dy1q["scale_inv"] * w1q["scale_inv"], H),
        ("dW1", c["dw1"], dw1r, dy1q["q_col"], "e5m2", x1q["q_col"], "e4m3", dy1q["scale_inv"] * x1q["scale_inv"], N),
    ]:
        g_ = to_np_u16(got)
        ii = rng.integers(0, g_.shape[0], 4096)
        jj = rng.integers(0, g_.shape[1], 4096)
        print(check_gemm(g_[ii, jj], ref[ii, jj], A, fa, B, fb, np.float32(t), Kc, "chain " + name, ii, jj),
              flush=True)
