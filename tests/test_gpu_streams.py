"""The Python binding on a stream other than torch's current one: quantize,
GEMM and the linear layer launched on a side stream give bitwise the results
of the same calls on the current stream, with the temporaries (workspace,
outputs) allocated on the launch stream so the caching allocator cannot hand
them out while the side stream still uses them."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_mixed_precision_amax_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("scaling", [0, 1])
def test_side_stream_quantize_and_gemm(fp8, scaling):
    N, K, M = 2048, 1024, 512
    x, w, _ = synth.operands(N, K, M, seed=21)
    x, w = x.cuda(), w.cuda()
    sw = fp8.SCALE_TENSOR if scaling == 0 else fp8.SCALE_128x128
    sx = fp8.SCALE_TENSOR if scaling == 0 else fp8.SCALE_1x128

    def run(stream):
        qx = fp8.quantize(x, fp8.E4M3, sx, stream=stream)
        qw = fp8.quantize(w, fp8.E4M3, sw, stream=stream)
        if scaling == 0:
            sa, sb = fp8.gemm_scale(qx.scale_inv), fp8.gemm_scale(qw.scale_inv)
        else:
            sa, sb = fp8.block_gemm_scale(qx.scale_inv, 1), fp8.block_gemm_scale(qw.scale_inv, 128)
        y = fp8.gemm(qx.q_row, fp8.E4M3, sa, qw.q_row, fp8.E4M3, sb, stream=stream)
        return qx, qw, y

    ref = run(None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = run(side)
    # churn the allocator on the current stream while the side stream works
    junk = [torch.empty(1 << 20, dtype=torch.uint8, device="cuda").fill_(0xAB) for _ in range(8)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del junk
    for a, b in ((ref[0].q_row, got[0].q_row), (ref[0].q_col, got[0].q_col), (ref[1].q_row, got[1].q_row),
                 (ref[0].scale_inv, got[0].scale_inv), (ref[1].scale_inv, got[1].scale_inv), (ref[2], got[2])):
        assert torch.equal(a, b)


def test_side_stream_linear(fp8):
    N, K, M = 1024, 512, 1024
    x, w, dy = (t.cuda() for t in synth.operands(N, K, M, seed=22))
    a = fp8.Fp8Linear(N, K, M, fp8.RECIPE_TENSOR)
    b = fp8.Fp8Linear(N, K, M, fp8.RECIPE_TENSOR)
    y1 = a.forward(x, w)
    dx1, dw1 = a.backward(dy)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    y2 = b.forward(x, w, stream=side)
    dx2, dw2 = b.backward(dy, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(dx1, dx2) and torch.equal(dw1, dw2)
