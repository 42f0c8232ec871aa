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
"""
import numpy as np
import pytest
import torch

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
             "dy1_row": l1.dy_q.q_row, "dy1_col": l1.dy_q.q_col, "dy1_scale": l1.dy_q.scale}
        return {"y1": y1, "y2": y2, "dx2": dx2, "dw2": dw2, "dx1": dx1, "dw1": dw1, **{k: v.clone() for k, v in q.items()}}

    plain, chained = run(False), run(True)
    for k in plain:
        a, b = plain[k], chained[k]
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b), k
