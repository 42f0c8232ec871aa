"""The remaining workloads at full size, through the C ABI, against the oracle.

- block scaling 512 -> 8192 at N = 131072 with 1% outliers (x100);
- the square 8192 x 8192 weight at N = 16384 and 512 -> 8192 at N = 262144,
  tensorwise and block-scaled;
- the 8-layer MLP stack (16 linears, d = 512 -> 2048 -> 512, GELU between) at
  131072 tokens per microbatch with gradient accumulation over 4
  microbatches: weight cache (quantize on microbatch 1, reuse on 2-4) against
  requantizing every microbatch, bitwise.

Every quantized byte and scale of X, W and dY is compared with the oracle
(bit-exact); Y, dX and dW are compared on 4096 sampled outputs each, to the
BF16 tolerance plus the FP8 matrix-core window bound, and to the emulation of
the matrix cores' accumulation (tests/_util.py).  Operands are drawn
with the seeded device generator (synth.workload_on_device)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _util import check_gemm_rows, to_np_u16, to_np_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_mixed_precision_amax_amd as m
    m.lib()
    return m


def _u32(t):
    return t.detach().cpu().numpy().view(np.uint32)


def check_q(q, ref, kind):
    assert np.array_equal(to_np_u8(q.q_row), ref["q_row"]), "row codes"
    assert np.array_equal(to_np_u8(q.q_col), ref["q_col"]), "col codes"
    if kind == "tensor":
        assert _u32(q.scale)[0] == np.float32(ref["scale"]).view(np.uint32)
        assert _u32(q.scale_inv)[0] == np.float32(ref["scale_inv"]).view(np.uint32)
    elif kind == "1x128":
        assert np.array_equal(_u32(q.scale), ref["scale_row"].view(np.uint32))
        assert np.array_equal(_u32(q.scale_inv), ref["scale_inv_row"].view(np.uint32))
        assert np.array_equal(_u32(q.scale_col), ref["scale_col"].view(np.uint32))
        assert np.array_equal(_u32(q.scale_inv_col), ref["scale_inv_col"].view(np.uint32))
    else:
        assert np.array_equal(_u32(q.scale), ref["scale"].view(np.uint32))
        assert np.array_equal(_u32(q.scale_inv), ref["scale_inv"].view(np.uint32))


def block_row_factors(name, q1, q2, ii, jj, N, K, M):
    """Per-row factors of every contraction block for sampled rows ii of the
    GEMM's A operand and jj of its B operand (block recipe)."""
    if name == "Y":
        return q1["scale_inv_row"][ii], q2["scale_inv"][jj // 128]
    if name == "dX":
        return q1["scale_inv_row"][ii], q2["scale_inv"].T[jj // 128]
    return q1["scale_inv_col"][ii], q2["scale_inv_col"][jj]


CONFIGS = ["linear_512x8192_n131072_block",
           "linear_8192x8192_n16384", "linear_8192x8192_n16384_block",
           "linear_512x8192_n262144", "linear_512x8192_n262144_block"]


@pytest.mark.parametrize("name", CONFIGS)
def test_config_full_size(fp8, name):
    print("config", name, flush=True)
    d = synth.workload_on_device(name, seed=0)
    N, K, M, recipe = d["N"], d["K"], d["M"], d["scaling"]
    R = fp8.RECIPE_TENSOR if recipe == "tensor" else fp8.RECIPE_BLOCK
    lin = fp8.Fp8Linear(N, K, M, R)
    y = lin.forward(d["x"], d["w"])
    dx, dw = lin.backward(d["dy"])
    torch.cuda.synchronize()
    act = "tensor" if recipe == "tensor" else "1x128"
    wsc = "tensor" if recipe == "tensor" else "128x128"
    xb, wb, dyb = synth.bits(d["x"]), synth.bits(d["w"]), synth.bits(d["dy"])
    del d
    xq = oracle.quantize(xb, "e4m3", act)
    check_q(lin.saved_x, xq, act)
    wq = oracle.quantize(wb, "e4m3", wsc)
    check_q(lin.w_q, wq, wsc)
    dyq = oracle.quantize(dyb, "e5m2", act)
    check_q(lin.dy_q, dyq, act)
    del xb, wb, dyb
    rng = np.random.default_rng(1)
    n = 4096
    for gname, (A, sA, B, sB), fa, fb, I, J, Kc, out, q1, q2 in [
        ("Y", oracle.fprop_operands(xq, wq, recipe, N, K, M), "e4m3", "e4m3", N, M, K, y, xq, wq),
        ("dX", oracle.dgrad_operands(dyq, wq, recipe, N, K, M), "e5m2", "e4m3", N, K, M, dx, dyq, wq),
        ("dW", oracle.wgrad_operands(dyq, xq, recipe, N, K, M), "e5m2", "e4m3", M, K, N, dw, dyq, xq),
    ]:
        ii = rng.integers(0, I, n)
        jj = rng.integers(0, J, n)
        if recipe == "tensor":
            ref = oracle.gemm_tensor_sampled(A, fa, B, fb, sA.s[0], sB.s[0], ii, jj)
            t = np.float32(sA.s[0] * sB.s[0])
        else:
            ref = oracle.gemm_block_sampled(A, fa, sA, B, fb, sB, ii, jj)
            t = block_row_factors(gname, q1, q2, ii, jj, N, K, M)
        got = to_np_u16(out)[ii, jj]
        rep = check_gemm_rows(got, ref, A[ii], fa, B[jj], fb, t, Kc, name + " " + gname)
        print(name, gname, rep, flush=True)


def _gelu(a):
    x = a.float()
    return (0.5 * x * (1.0 + torch.erf(x * 0.7071067811865476))).to(torch.bfloat16)


def _dgelu(a, g):
    x = a.float()
    cdf = 0.5 * (1.0 + torch.erf(x * 0.7071067811865476))
    pdf = torch.exp(-0.5 * x * x) * 0.3989422804014327
    return (g.float() * (cdf + x * pdf)).to(torch.bfloat16)


def _run_stack(fp8, lins, weights, xs, dys, cached):
    """Forward + backward of the stack over the microbatches (linear 2p is
    the up projection, 2p+1 the down projection, GELU between); returns the
    outputs, the input gradients and the fp32-accumulated dW of each linear."""
    pairs = len(lins) // 2
    acc = [torch.zeros(w.shape, dtype=torch.float32, device="cuda") for w in weights]
    outs, dxs = [], []
    for mb, (x, dy) in enumerate(zip(xs, dys)):
        flag = (mb == 0) if cached else None
        wsel = (lambda l: weights[l] if (not cached or mb == 0) else None)
        h, pre = x, []
        for p in range(pairs):
            a = lins[2 * p].forward(h, wsel(2 * p), is_first_microbatch=flag)
            pre.append(a)
            h = lins[2 * p + 1].forward(_gelu(a), wsel(2 * p + 1), is_first_microbatch=flag)
        outs.append(h.clone())
        dh = dy
        for p in reversed(range(pairs)):
            dg, dw_down = lins[2 * p + 1].backward(dh)
            acc[2 * p + 1] += dw_down.float()
            dh, dw_up = lins[2 * p].backward(_dgelu(pre[p], dg))
            acc[2 * p] += dw_up.float()
        dxs.append(dh.clone())
    torch.cuda.synchronize()
    return outs, dxs, acc


def test_mlp_stack_weight_cache_bitwise(fp8):
    N, d, h, layers, mbs = 131072, 512, 2048, 8, 4
    print("mlp stack", N, d, h, layers, mbs, flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(4)
    weights = []
    for _ in range(layers):
        weights.append(synth.normal_bf16((h, d), 0.02, g, device="cuda"))
        weights.append(synth.normal_bf16((d, h), 0.02, g, device="cuda"))
    xs = [synth.normal_bf16((N, d), 1.0, g, device="cuda") for _ in range(mbs)]
    dys = [synth.normal_bf16((N, d), 1e-3, g, device="cuda") for _ in range(mbs)]
    shapes = [(d, h), (h, d)] * layers      # (K, M) of each linear
    res = {}
    for cached in (True, False):
        lins = [fp8.Fp8Linear(N, K, M, fp8.RECIPE_TENSOR, cache=cached) for K, M in shapes]
        res[cached] = _run_stack(fp8, lins, weights, xs, dys, cached)
        if cached:
            assert all(l.cache.fills == 1 and l.cache.valid for l in lins)
        del lins
        torch.cuda.empty_cache()
    (o1, x1, a1), (o2, x2, a2) = res[True], res[False]
    for mb in range(mbs):
        assert torch.equal(o1[mb], o2[mb]), ("output", mb)
        assert torch.equal(x1[mb], x2[mb]), ("input gradient", mb)
    for l in range(2 * layers):
        assert torch.equal(a1[l], a2[l]), ("dW", l)
        assert torch.isfinite(a1[l]).all()
