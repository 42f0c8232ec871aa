"""GELU amax hand-off (the producer-side amax for the MLP block's GELU), tensorwise,
through the C ABI.

The up projection's GEMM writes four 16-bit keys per workgroup about its bf16
output A (fp8_linear.h, "GELU amax hand-off"); the quantize of GELU(A) turns
them into amax(GELU(A)) and runs the cast pass alone.  Pinned here:
  - producer: for every shape (one tile, ragged tiles, split-K, the MLP
    block's 131072 x 2048 x 512) the keys reduce exactly to the keys of the
    GEMM's own output as the header defines them, unused slots are zero, and
    C is bitwise fp8_gemm's;
  - consumer: keys built on the host from that definition for bf16 tensors
    chosen to exercise every case (every bf16 pattern, NaN and -Inf, only
    values in [-0.75, 0), only values below -0.75, single values around
    GELU's minimum, normal pre-activations) give codes, scales and amax
    bit-exact with the oracle's quantize of GELU(x);
  - end to end: GEMM keys -> quantize equals the oracle on the GEMM's output;
  - fp8_mlp_fwd equals the two linear calls bitwise (both recipes, with the
    weight cache), and its second linear matches the oracle fed the GPU's A.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _util import check_gemm, linear_gemms, oracle_sampled, to_np_u16, to_np_u8

pytestmark = pytest.mark.gpu

SLOTS = 2048


@pytest.fixture(scope="module")
def fp8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_mixed_precision_amax_amd as m
    m.lib()
    return m


def keys_of(bits):
    """The four keys of a bf16 tensor (bit patterns), by the header's
    definition, each in its max-reducible stored form."""
    b = np.asarray(bits, np.uint16).reshape(-1)
    v = b.astype(np.int64)
    p = int(b.view(np.int16).max())
    d = (v + 0x40BF) & 0xFFFF
    return [(p & 0xFFFF) ^ 0x8000, int(v.max()), int(d.max()), (~int(d.min())) & 0xFFFF]


def key_buffer(keys, dev):
    buf = np.zeros(4 * SLOTS, np.uint16)
    for q in range(4):
        buf[q * SLOTS] = keys[q]
    return torch.from_numpy(buf.view(np.uint8).copy()).to(dev)


def _codes(shape, seed, dev):
    g = torch.Generator(device="cpu").manual_seed(seed)
    c = torch.randint(0, 0x7F, shape, generator=g, dtype=torch.int32)
    c |= torch.randint(0, 2, shape, generator=g, dtype=torch.int32) << 7
    return c.to(torch.uint8).to(dev)


def _check_quant(q, ref):
    assert np.array_equal(to_np_u8(q.q_row), ref["q_row"]), "row codes"
    assert np.array_equal(to_np_u8(q.q_col), ref["q_col"]), "col codes"
    f = lambda t: t.cpu().numpy().view(np.uint32)[0]
    assert f(q.scale) == np.float32(ref["scale"]).view(np.uint32), "scale"
    assert f(q.scale_inv) == np.float32(ref["scale_inv"]).view(np.uint32), "scale_inv"
    assert f(q.amax) == np.float32(ref["amax"]).view(np.uint32), "amax"


SHAPES = [(256, 256, 512), (640, 384, 1024), (256, 256, 16384), (131072, 2048, 512)]


@pytest.mark.parametrize("I,J,K", SHAPES)
def test_gemm_emits_gelu_keys_of_its_output(fp8, I, J, K):
    print("gelu keys gemm", I, J, K, flush=True)
    dev = torch.device("cuda")
    a, b = _codes((I, K), 3 + I, dev), _codes((J, K), 4 + J, dev)
    # outputs spread like pre-activations (|C| mostly below a few units)
    s = torch.tensor([1.0 / 4096], device=dev)
    t = torch.tensor([1.0 / 64 / np.sqrt(K / 512)], device=dev, dtype=torch.float32)
    plain = fp8.gemm(a, fp8.E4M3, fp8.gemm_scale(s), b, fp8.E4M3, fp8.gemm_scale(t))
    keys = fp8.gelu_amax_partials(dev)
    keys.fill_(0xAB)   # every slot must be written
    c = fp8.gemm(a, fp8.E4M3, fp8.gemm_scale(s), b, fp8.E4M3, fp8.gemm_scale(t), gelu_amax_out=keys)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), plain.view(torch.int16)), "C differs from fp8_gemm's"
    slots = keys.cpu().numpy().view(np.uint16).reshape(4, SLOTS).astype(np.int64)
    cb = to_np_u16(c)
    assert list(slots.max(axis=1)) == keys_of(cb)
    used = int((slots != 0).any(axis=0).sum())
    assert (slots[:, max(used, 1):] == 0).all(), "slots after the written ones must be zero"
    # the cast-only quantize of GELU(C) from these keys against the oracle
    for fmt, F in (("e4m3", fp8.E4M3), ("e5m2", fp8.E5M2)):
        q = fp8.quantize_gelu(c, F, gelu_amax_partials=keys)
        torch.cuda.synchronize()
        _check_quant(q, oracle.quant_gelu(cb, fmt, "tensor"))


def _pad(bits, cols=128):
    """bf16 patterns -> [R, 128] with R a multiple of 128, padded with +0."""
    b = np.asarray(bits, np.uint16).reshape(-1)
    n = -(-b.size // (128 * cols)) * 128 * cols
    out = np.zeros(n, np.uint16)
    out[:b.size] = b
    return out.reshape(-1, cols)


def _bf16(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _consumer_cases():
    allp = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(7)
    finite = allp[(allp & 0x7F80) != 0x7F80]
    cases = {
        "every pattern": rng.permutation(allp),
        "finite": rng.permutation(finite),
        "finite and +Inf": np.concatenate([finite, [0x7F80]]),
        "finite and -Inf": np.concatenate([finite, [0xFF80]]),
        "negative NaN only": np.array([0xFFC1], np.uint16),
        "[-0.75, 0) only": np.arange(0x8000, 0xBF41, dtype=np.uint32).astype(np.uint16),
        "below -0.75 only": np.arange(0xBF41, 0xFF80, dtype=np.uint32).astype(np.uint16),
        "positives only": np.arange(0x0001, 0x7F80, dtype=np.uint32).astype(np.uint16),
        "pre-activations": synth.bits(synth.normal_bf16((4096, 128), 0.45, torch.Generator().manual_seed(3))),
    }
    for v in (-0.75, -0.75390625, -0.74609375, -0.7578125, -3.0, -100.0, -1e-30, 1e-30, 0.5, 20.0, -20.0):
        cases["single %g" % v] = _bf16([v])
        cases["%g with -3 and 0.1" % v] = _bf16([v, -3.0, 0.1])
    cases["+0 only"] = np.array([0], np.uint16)
    cases["-0 only"] = np.array([0x8000], np.uint16)
    return cases


CONSUMER = _consumer_cases()


@pytest.mark.parametrize("case", list(CONSUMER))
def test_quantize_from_host_keys_matches_oracle(fp8, case):
    dev = torch.device("cuda")
    x = _pad(CONSUMER[case])
    keys = key_buffer(keys_of(x), dev)
    xt = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    for fmt, F in (("e4m3", fp8.E4M3), ("e5m2", fp8.E5M2)):
        q = fp8.quantize_gelu(xt, F, gelu_amax_partials=keys)
        torch.cuda.synchronize()
        _check_quant(q, oracle.quant_gelu(x, fmt, "tensor"))


@pytest.mark.parametrize("recipe", ["tensor", "block"])
def test_mlp_forward_equals_two_calls_and_oracle(fp8, recipe):
    N, D, H = 4096, 512, 2048
    print("mlp fwd", recipe, N, D, H, flush=True)
    R = fp8.RECIPE_TENSOR if recipe == "tensor" else fp8.RECIPE_BLOCK
    g = torch.Generator().manual_seed(71)
    x = synth.normal_bf16((N, D), 1.0, g).cuda()
    w1 = synth.normal_bf16((H, D), 0.02, g).cuda()
    w2 = synth.normal_bf16((D, H), 0.02, g).cuda()
    dy = synth.normal_bf16((N, D), 1e-3, g).cuda()
    mlp = fp8.Fp8Mlp(N, D, H, R, cache=True)
    l1, l2 = fp8.Fp8Linear(N, D, H, R), fp8.Fp8Linear(N, H, D, R)
    for mb, flag in enumerate((True, False)):
        y = mlp.forward(x, w1 if flag else None, w2 if flag else None, is_first_microbatch=flag)
        a_ref = l1.forward(x, w1)
        y_ref = l2.forward(a_ref, w2, gelu=True)
        dx, dw1, dw2 = mlp.backward(dy)
        dh_ref, dw2_ref = l2.backward(dy)
        dx_ref, dw1_ref = l1.backward(dh_ref, gelu_input=a_ref)
        torch.cuda.synchronize()
        for name, p_, q_ in (("A", mlp.a, a_ref), ("Y", y, y_ref), ("dX", dx, dx_ref), ("dW1", dw1, dw1_ref),
                             ("dW2", dw2, dw2_ref)):
            assert torch.equal(p_.view(torch.int16), q_.view(torch.int16)), (mb, name)
        for n in ("q_row", "q_col", "scale_inv"):
            assert torch.equal(getattr(mlp.down.saved_x, n), getattr(l2.saved_x, n)), (mb, n)
            assert torch.equal(getattr(mlp.up.weight_q(), n), getattr(l1.w_q, n)), (mb, n)
            assert torch.equal(getattr(mlp.down.weight_q(), n), getattr(l2.w_q, n)), (mb, n)
    # the down projection against the oracle, fed the GPU's A
    A = to_np_u16(mlp.a)
    yr_ctx = oracle.linear_fwd_gelu(A, synth.bits(w2), recipe)
    ctx = yr_ctx[1]
    act = "tensor" if recipe == "tensor" else "1x128"
    xq = ctx["xq"]
    assert np.array_equal(to_np_u8(mlp.down.saved_x.q_row), xq["q_row"])
    assert np.array_equal(to_np_u8(mlp.down.saved_x.q_col), xq["q_col"])
    dyq = oracle.quantize(synth.bits(dy.cpu()), "e5m2", act)
    name, Aq, fa, Bq, fb, t, Kc = linear_gemms(xq, ctx["wq"], dyq, recipe, N, H, D)[0]
    rng = np.random.default_rng(8)
    ii = rng.integers(0, N, 2048)
    jj = rng.integers(0, D, 2048)
    ref = oracle_sampled(Aq, fa, Bq, fb, t, ii, jj)
    print(check_gemm(to_np_u16(y)[ii, jj], ref, Aq, fa, Bq, fb, t, Kc, "mlp Y", ii, jj), flush=True)
    assert np.array_equal(ref, yr_ctx[0][ii, jj])
