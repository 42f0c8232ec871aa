"""The linear's forward + backward captured into a HIP graph (torch's graph
capture around the library calls, which allocate nothing and record no
memset) and replayed: every replay equals the eager result bitwise.  Between
replays the captured input buffers are refilled with one of two input sets,
the outputs cleared, other eager library work runs and the host
synchronizes, so a replay that skipped a pass, read stale amax partials or
split-K slices, or wrote outside its outputs would show."""
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


def _inputs(N, K, M, seed):
    x, w, dy = synth.operands(N, K, M, seed=seed)
    return x.cuda(), w.cuda(), dy.cuda()


@pytest.mark.parametrize("recipe", ["tensor", "block"])
def test_graph_replay_matches_eager(fp8, recipe):
    # the weight gradient (1024 x 512 output, contraction 8192) runs split-K
    N, K, M = 8192, 512, 1024
    R = fp8.RECIPE_TENSOR if recipe == "tensor" else fp8.RECIPE_BLOCK
    sets = [_inputs(N, K, M, 40), _inputs(N, K, M, 41)]
    ref = fp8.Fp8Linear(N, K, M, R)
    want = []
    for x, w, dy in sets:
        y = ref.forward(x, w)
        dx, dw = ref.backward(dy)
        want.append((y.clone(), dx.clone(), dw.clone()))
    torch.cuda.synchronize()

    lin = fp8.Fp8Linear(N, K, M, R)
    x, w, dy = (t.clone() for t in sets[0])
    y = torch.empty((N, M), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")

    def step():
        lin.forward(x, w, y=y)
        lin.backward(dy, dx=dx, dw=dw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for r, which in enumerate((1, 0, 1, 1)):
        for dst, src in zip((x, w, dy), sets[which]):
            dst.copy_(src)
        for t in (y, dx, dw):
            t.zero_()
        # other eager work of the library between replays
        other = sets[1 - which]
        ref.forward(other[0], other[1])
        ref.backward(other[2])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, exp in zip(("Y", "dX", "dW"), (y, dx, dw), want[which]):
            assert torch.equal(got, exp), (recipe, r, name)
