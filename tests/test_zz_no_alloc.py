"""fp8_linear_fwd_noalloc (the forward for callers that cannot allocate)
through the C ABI against fp8_linear_fwd on the same inputs: Y, the saved
X codes and scales and the quantized weight bitwise equal, over calls in a
row whose sizes shrink (the device scratch keeps the previous call's
contents), both recipes, a shape whose forward GEMM splits its contraction
(partial sums in the scratch), and the weight cache."""
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


def _q_equal(a, b):
    for n in ("q_row", "q_col", "scale", "scale_inv", "scale_col", "scale_inv_col"):
        ta, tb = getattr(a, n), getattr(b, n)
        if ta is None and tb is None:
            continue
        assert torch.equal(ta.contiguous().view(torch.uint8), tb.contiguous().view(torch.uint8)), n


def _both(fp8, N, K, M, recipe, seed, flag=None, cache=False):
    print("noalloc case N=%d K=%d M=%d recipe=%d seed=%d" % (N, K, M, recipe, seed), flush=True)
    x, w, _ = synth.operands(N, K, M, seed=seed, sigma_w=0.02 if recipe == 0 else 1.0,
                             outlier_frac=0.0 if recipe == 0 else 0.01)
    x, w = x.cuda(), w.cuda()
    ref = fp8.Fp8Linear(N, K, M, recipe)
    got = fp8.Fp8Linear(N, K, M, recipe, cache=cache)
    y_ref = ref.forward(x, w)
    y = torch.full((N, M), float("nan"), dtype=torch.bfloat16, device="cuda")
    got.forward_noalloc(x, w, y, is_first_microbatch=flag)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    _q_equal(got.saved_x, ref.saved_x)
    _q_equal(got.weight_q(), ref.w_q)
    return got, x, w, y_ref


@pytest.mark.parametrize("recipe", [0, 1])
def test_noalloc_forward_equals_forward_shrinking(fp8, recipe):
    _both(fp8, 4096, 1024, 2048, recipe, seed=61)
    _both(fp8, 1024, 512, 512, recipe, seed=62)        # smaller: stale scratch from the call before


def test_noalloc_forward_split_contraction(fp8):
    """N = 256, K = 4096, M = 512: the forward GEMM splits its contraction
    in 4 (2 MiB of partial sums in the scratch); then a smaller call."""
    _both(fp8, 256, 4096, 512, 0, seed=63)
    _both(fp8, 128, 2048, 256, 0, seed=64)


def test_noalloc_forward_weight_cache(fp8):
    N, K, M = 1024, 512, 1024
    lin, x, w, y_ref = _both(fp8, N, K, M, 0, seed=65, flag=True, cache=True)
    y2 = torch.empty((N, M), dtype=torch.bfloat16, device="cuda")
    lin.forward_noalloc(x, None, y2, is_first_microbatch=False)
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16), y_ref.view(torch.int16))
    assert lin.cache.fills == 1


def test_noalloc_forward_rejects_large_scratch(fp8):
    N, K, M = 256, 8192, 8192
    lin = fp8.Fp8Linear(N, K, M, 0)
    x = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    y = torch.full((N, M), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fp8.Fp8Error):
        lin.forward_noalloc(x, w, y)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())                       # untouched
