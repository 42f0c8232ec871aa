"""CPU oracle for the FP8 linear layer's forward and backward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The
product (the HIP library and its Python binding) never imports, links or
calls it, and this package imports nothing from the product.

The arithmetic lives in ``fp8_oracle.c`` (plain C, compiled with
``-ffp-contract=off``); this module marshals numpy arrays through ctypes and
composes the per-step functions into the linear layer exactly as the method
orders them:

  forward   Xq = quant(X, E4M3), Wq = quant(W, E4M3), Y = GEMM(Xq_row, Wq_row)
  backward  dYq = quant(dY, E5M2) with its own current amax,
            dX = GEMM(dYq_row, Wq_col), dW = GEMM(dYq_col, Xq_col)

The recipe is the one of "Native FP8 MLP reconstruction" (implementation
paragraph): each tensor is scaled by its own amax taken on the current call;
activations and weights are encoded as E4M3, the incoming gradient as E5M2;
one cast pass produces both the ordinary and the transposed layout; every GEMM
writes BF16; the backward pass reuses the X and W codes of the forward pass
and quantizes the gradient by itself.  Block scaling follows the
Float8BlockScaling recipe named in TransformerEngine issue 2852 (opening
post): 1x128 blocks for activations and gradients, 128x128 for weights.

Arrays: bf16 tensors are numpy ``uint16`` bit patterns, FP8 tensors are
``uint8`` codes, scales are ``float32``.  Formats: ``"e4m3"`` / ``"e5m2"``.
Scalings: ``"tensor"``, ``"1x128"``, ``"128x128"``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

FORMATS = {"e4m3": 0, "e5m2": 1}


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.path.join(_HERE, "liboracle.so")
    if not os.path.exists(path):
        _build.build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    F = ctypes.c_float
    sig = {
        "orc_fmax": (F, [I]),
        "orc_dec": (F, [ctypes.c_uint8, I]),
        "orc_enc": (ctypes.c_uint8, [F, I]),
        "orc_enc_array": (None, [P, I64, I, P]),
        "orc_dec_array": (None, [P, I64, I, P]),
        "orc_dec_bf16": (F, [ctypes.c_uint16]),
        "orc_bf16_rne": (ctypes.c_uint16, [F]),
        "orc_bf16_rne_array": (None, [P, I64, P]),
        "orc_amax_bf16": (F, [P, I64]),
        "orc_scale_from_amax": (None, [F, I, P, P]),
        "orc_quant_tensor": (None, [P, I64, I64, I, P, P, P, P, P]),
        "orc_quant_delayed": (None, [P, I64, I64, I, P, I64, P, P, P, P, P]),
        "orc_quant_block_1x128": (None, [P, I64, I64, I, P, P, P, P, P, P]),
        "orc_quant_block_128x128": (None, [P, I64, I64, I, P, P, P, P]),
        "orc_gemm_tensor": (None, [P, I, P, I, I64, I64, I64, F, F, P, P, P]),
        "orc_gemm_block": (None, [P, I, P, I64, I64, I64, P, I, P, I64, I64, I64,
                                  I64, I64, I64, P, P, P]),
        "orc_gemm_tensor_sampled": (None, [P, I, P, I, I64, F, F, P, P, I64, P, P]),
        "orc_gemm_block_sampled": (None, [P, I, P, I64, I64, I64, P, I, P, I64, I64, I64,
                                          I64, P, P, I64, P, P]),
        "orc_gelu_f32": (F, [ctypes.c_uint16]),
        "orc_gelu_grad_f32": (F, [ctypes.c_uint16]),
        "orc_gelu_array": (None, [P, I64, P]),
        "orc_gelu_f32_array": (None, [P, I64, P]),
        "orc_gelu_grad_f32_array": (None, [P, I64, P]),
        "orc_dgelu_array": (None, [P, P, I64, P]),
        "orc_gemm_bf16": (None, [P, P, I64, I64, I64, P, P, P]),
        "orc_gemm_bf16_sampled": (None, [P, P, I64, P, P, I64, P, P]),
        "orc_num_threads": (I, []),
        "orc_set_num_threads": (None, [I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads():
    return _load().orc_num_threads()


def set_num_threads(n):
    _load().orc_set_num_threads(int(n))


# --------------------------------------------------------------------------
# Element codecs
# --------------------------------------------------------------------------

def fmax(fmt):
    return float(np.float32(_load().orc_fmax(FORMATS[fmt])))


def enc(v, fmt):
    """Saturating round-to-nearest-even encode of fp32 values to FP8 codes."""
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().orc_enc_array(_p(v), v.size, FORMATS[fmt], _p(out))
    return out


def dec(codes, fmt):
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, np.float32)
    _load().orc_dec_array(_p(codes), codes.size, FORMATS[fmt], _p(out))
    return out


def dec_bf16(bits):
    return (_c(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_rne(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint16)
    _load().orc_bf16_rne_array(_p(v), v.size, _p(out))
    return out


# --------------------------------------------------------------------------
# amax, scale, quantize
# --------------------------------------------------------------------------

def amax_bf16(x):
    x = _c(x, np.uint16)
    return np.float32(_load().orc_amax_bf16(_p(x), x.size))


def scale_from_amax(amax, fmt):
    s = np.zeros(1, np.float32)
    si = np.zeros(1, np.float32)
    _load().orc_scale_from_amax(ctypes.c_float(float(amax)), FORMATS[fmt], _p(s), _p(si))
    return s[0], si[0]


def quant_tensor(x, fmt, row=True, col=True):
    """Current tensorwise scaling.  x: uint16 [R, C]."""
    x = _c(x, np.uint16)
    R, C = x.shape
    q_row = np.empty((R, C), np.uint8) if row else None
    q_col = np.empty((C, R), np.uint8) if col else None
    amax = np.zeros(1, np.float32)
    s = np.zeros(1, np.float32)
    si = np.zeros(1, np.float32)
    _load().orc_quant_tensor(_p(x), R, C, FORMATS[fmt], _p(q_row), _p(q_col),
                             _p(amax), _p(s), _p(si))
    return {"q_row": q_row, "q_col": q_col, "amax": amax[0], "scale": s[0], "scale_inv": si[0]}


def quant_delayed(x, fmt, history, row=True, col=True):
    """Delayed tensorwise scaling: scale from max(history) (previous calls'
    amaxes, most recent first), then this call's amax is pushed in front.
    x: uint16 [R, C]; history: float32 [H].  Returns the codes, scales, this
    call's amax and the new history (the argument is not modified)."""
    x = _c(x, np.uint16)
    R, C = x.shape
    h = np.array(history, dtype=np.float32, copy=True)
    q_row = np.empty((R, C), np.uint8) if row else None
    q_col = np.empty((C, R), np.uint8) if col else None
    amax = np.zeros(1, np.float32)
    s = np.zeros(1, np.float32)
    si = np.zeros(1, np.float32)
    _load().orc_quant_delayed(_p(x), R, C, FORMATS[fmt], _p(h), h.size, _p(q_row), _p(q_col),
                              _p(amax), _p(s), _p(si))
    return {"q_row": q_row, "q_col": q_col, "amax": amax[0], "scale": s[0], "scale_inv": si[0], "history": h}


def quant_block_1x128(x, fmt, row=True, col=True):
    """1x128 blocks: row layout blocks run along columns, col layout blocks
    along rows (the contraction dimension of the GEMM consuming each)."""
    x = _c(x, np.uint16)
    R, C = x.shape
    assert R % 128 == 0 and C % 128 == 0
    out = {"q_row": None, "q_col": None}
    q_row = s_row = si_row = q_col = s_col = si_col = None
    if row:
        q_row = np.empty((R, C), np.uint8)
        s_row = np.empty((R, C // 128), np.float32)
        si_row = np.empty((R, C // 128), np.float32)
    if col:
        q_col = np.empty((C, R), np.uint8)
        s_col = np.empty((C, R // 128), np.float32)
        si_col = np.empty((C, R // 128), np.float32)
    _load().orc_quant_block_1x128(_p(x), R, C, FORMATS[fmt], _p(q_row), _p(s_row), _p(si_row),
                                  _p(q_col), _p(s_col), _p(si_col))
    out.update(q_row=q_row, scale_row=s_row, scale_inv_row=si_row,
               q_col=q_col, scale_col=s_col, scale_inv_col=si_col)
    return out


def quant_block_128x128(x, fmt, row=True, col=True):
    x = _c(x, np.uint16)
    R, C = x.shape
    assert R % 128 == 0 and C % 128 == 0
    q_row = np.empty((R, C), np.uint8) if row else None
    q_col = np.empty((C, R), np.uint8) if col else None
    s = np.empty((R // 128, C // 128), np.float32)
    si = np.empty((R // 128, C // 128), np.float32)
    _load().orc_quant_block_128x128(_p(x), R, C, FORMATS[fmt], _p(q_row), _p(q_col), _p(s), _p(si))
    return {"q_row": q_row, "q_col": q_col, "scale": s, "scale_inv": si}


def quantize(x, fmt, scaling, row=True, col=True):
    if scaling == "tensor":
        return quant_tensor(x, fmt, row, col)
    if scaling == "1x128":
        return quant_block_1x128(x, fmt, row, col)
    if scaling == "128x128":
        return quant_block_128x128(x, fmt, row, col)
    raise ValueError(scaling)


# --------------------------------------------------------------------------
# GEMMs: C[i][j] = sum_k A[i][k] B[j][k]
# --------------------------------------------------------------------------

class BlockScale:
    """Scale of operand row r in contraction block kb:
    s[(r // group) * stride_r + kb * stride_kb] (s flattened)."""

    def __init__(self, s, group, stride_r, stride_kb):
        self.s = _c(s, np.float32).reshape(-1)
        self.group, self.stride_r, self.stride_kb = int(group), int(stride_r), int(stride_kb)

    def args(self):
        return [_p(self.s), self.group, self.stride_r, self.stride_kb]


def gemm_tensor(A, fa, B, fb, sinvA, sinvB, want_f32=False):
    A = _c(A, np.uint8)
    B = _c(B, np.uint8)
    I, K = A.shape
    J, K2 = B.shape
    assert K == K2
    C = np.empty((I, J), np.uint16)
    C32 = np.empty((I, J), np.float32) if want_f32 else None
    work = np.empty((I + J) * K, np.float32)
    _load().orc_gemm_tensor(_p(A), FORMATS[fa], _p(B), FORMATS[fb], I, J, K,
                            ctypes.c_float(float(sinvA)), ctypes.c_float(float(sinvB)),
                            _p(C), _p(C32), _p(work))
    return (C, C32) if want_f32 else C


def gemm_block(A, fa, sA, B, fb, sB, want_f32=False):
    A = _c(A, np.uint8)
    B = _c(B, np.uint8)
    I, K = A.shape
    J, K2 = B.shape
    assert K == K2 and K % 128 == 0
    C = np.empty((I, J), np.uint16)
    C32 = np.empty((I, J), np.float32) if want_f32 else None
    work = np.empty((I + J) * K, np.float32)
    _load().orc_gemm_block(_p(A), FORMATS[fa], *sA.args(), _p(B), FORMATS[fb], *sB.args(),
                           I, J, K, _p(C), _p(C32), _p(work))
    return (C, C32) if want_f32 else C


def gemm_tensor_sampled(A, fa, B, fb, sinvA, sinvB, ii, jj, want_f32=False):
    A = _c(A, np.uint8)
    B = _c(B, np.uint8)
    K = A.shape[1]
    ii = _c(ii, np.int64)
    jj = _c(jj, np.int64)
    out = np.empty(ii.shape, np.uint16)
    out32 = np.empty(ii.shape, np.float32) if want_f32 else None
    _load().orc_gemm_tensor_sampled(_p(A), FORMATS[fa], _p(B), FORMATS[fb], K,
                                    ctypes.c_float(float(sinvA)), ctypes.c_float(float(sinvB)),
                                    _p(ii), _p(jj), ii.size, _p(out), _p(out32))
    return (out, out32) if want_f32 else out


def gemm_block_sampled(A, fa, sA, B, fb, sB, ii, jj, want_f32=False):
    A = _c(A, np.uint8)
    B = _c(B, np.uint8)
    K = A.shape[1]
    ii = _c(ii, np.int64)
    jj = _c(jj, np.int64)
    out = np.empty(ii.shape, np.uint16)
    out32 = np.empty(ii.shape, np.float32) if want_f32 else None
    _load().orc_gemm_block_sampled(_p(A), FORMATS[fa], *sA.args(), _p(B), FORMATS[fb], *sB.args(),
                                   K, _p(ii), _p(jj), ii.size, _p(out), _p(out32))
    return (out, out32) if want_f32 else out


# --------------------------------------------------------------------------
# The linear layer.  Shapes follow nn.Linear: X [N, K], W [M, K], Y [N, M].
# scaling: "tensor" (every operand tensorwise) or "block" (X and dY in 1x128
# blocks, W in 128x128 blocks).
# --------------------------------------------------------------------------

_ACT = {"tensor": "tensor", "block": "1x128"}
_WGT = {"tensor": "tensor", "block": "128x128"}


def _gemm_operands_fprop(xq, wq, scaling, N, K, M):
    if scaling == "tensor":
        return (xq["q_row"], BlockScale(np.array([xq["scale_inv"]]), N, 0, 0),
                wq["q_row"], BlockScale(np.array([wq["scale_inv"]]), M, 0, 0))
    return (xq["q_row"], BlockScale(xq["scale_inv_row"], 1, K // 128, 1),
            wq["q_row"], BlockScale(wq["scale_inv"], 128, K // 128, 1))


def _gemm_operands_dgrad(dyq, wq, scaling, N, K, M):
    if scaling == "tensor":
        return (dyq["q_row"], BlockScale(np.array([dyq["scale_inv"]]), N, 0, 0),
                wq["q_col"], BlockScale(np.array([wq["scale_inv"]]), K, 0, 0))
    # W's col layout [K, M]: row k, contraction block mb -> s[mb][k // 128]
    return (dyq["q_row"], BlockScale(dyq["scale_inv_row"], 1, M // 128, 1),
            wq["q_col"], BlockScale(wq["scale_inv"], 128, 1, K // 128))


def _gemm_operands_wgrad(dyq, xq, scaling, N, K, M):
    if scaling == "tensor":
        return (dyq["q_col"], BlockScale(np.array([dyq["scale_inv"]]), M, 0, 0),
                xq["q_col"], BlockScale(np.array([xq["scale_inv"]]), K, 0, 0))
    return (dyq["q_col"], BlockScale(dyq["scale_inv_col"], 1, N // 128, 1),
            xq["q_col"], BlockScale(xq["scale_inv_col"], 1, N // 128, 1))


def fprop_operands(xq, wq, scaling, N, K, M):
    """(A, sA, B, sB) of Y = X W^T as gemm_block / gemm_block_sampled take them."""
    return _gemm_operands_fprop(xq, wq, scaling, N, K, M)


def dgrad_operands(dyq, wq, scaling, N, K, M):
    """(A, sA, B, sB) of dX = dY W."""
    return _gemm_operands_dgrad(dyq, wq, scaling, N, K, M)


def wgrad_operands(dyq, xq, scaling, N, K, M):
    """(A, sA, B, sB) of dW = dY^T X."""
    return _gemm_operands_wgrad(dyq, xq, scaling, N, K, M)


def _gemm(a, fa, sa, b, fb, sb, scaling):
    if scaling == "tensor":
        return gemm_tensor(a, fa, b, fb, sa.s[0], sb.s[0])
    return gemm_block(a, fa, sa, b, fb, sb)


def quantize_weight(w, scaling):
    return quantize(w, "e4m3", _WGT[scaling])


def linear_fwd(x, w, scaling="tensor", wq=None):
    """Y = X W^T.  ``wq`` is a previously quantized weight (the cache); when
    None the weight is quantized here.  Returns Y (uint16 bf16 bits) and the
    context the backward pass consumes."""
    N, K = x.shape
    M = w.shape[0] if w is not None else wq["q_row"].shape[0]
    xq = quantize(x, "e4m3", _ACT[scaling])
    if wq is None:
        wq = quantize_weight(w, scaling)
    a, sa, b, sb = _gemm_operands_fprop(xq, wq, scaling, N, K, M)
    y = _gemm(a, "e4m3", sa, b, "e4m3", sb, scaling)
    return y, {"xq": xq, "wq": wq, "N": N, "K": K, "M": M, "scaling": scaling}


def linear_bwd(dy, ctx):
    N, K, M, scaling = ctx["N"], ctx["K"], ctx["M"], ctx["scaling"]
    dyq = quantize(dy, "e5m2", _ACT[scaling])
    a, sa, b, sb = _gemm_operands_dgrad(dyq, ctx["wq"], scaling, N, K, M)
    dx = _gemm(a, "e5m2", sa, b, "e4m3", sb, scaling)
    a, sa, b, sb = _gemm_operands_wgrad(dyq, ctx["xq"], scaling, N, K, M)
    dw = _gemm(a, "e5m2", sa, b, "e4m3", sb, scaling)
    return dx, dw, dyq


# --------------------------------------------------------------------------
# GELU between the two linears of an MLP block (exact erf form, fp64
# evaluation rounded once to fp32; see fp8_oracle.c)
# --------------------------------------------------------------------------

def gelu_f32(x):
    """fl32(GELU(x)) of bf16 bit patterns."""
    x = _c(x, np.uint16)
    out = np.empty(x.shape, np.float32)
    _load().orc_gelu_f32_array(_p(x), x.size, _p(out))
    return out


def gelu_grad_f32(x):
    """fl32(GELU'(x)) of bf16 bit patterns."""
    x = _c(x, np.uint16)
    out = np.empty(x.shape, np.float32)
    _load().orc_gelu_grad_f32_array(_p(x), x.size, _p(out))
    return out


def gelu(x):
    """The activation passed to the next linear: bf16(fl32(GELU(x)))."""
    x = _c(x, np.uint16)
    out = np.empty(x.shape, np.uint16)
    _load().orc_gelu_array(_p(x), x.size, _p(out))
    return out


def dgelu(dy, x):
    """The gradient passed back through GELU: bf16(fl32(dy * fl32(GELU'(x))))."""
    dy, x = _c(dy, np.uint16), _c(x, np.uint16)
    assert dy.shape == x.shape
    out = np.empty(x.shape, np.uint16)
    _load().orc_dgelu_array(_p(dy), _p(x), x.size, _p(out))
    return out


def quant_gelu(a, fmt, scaling, row=True, col=True):
    """Quantize GELU(a) as the next linear's input: the activation first,
    then the current-scaling quantizer on its bf16 values."""
    return quantize(gelu(a), fmt, scaling, row, col)


def quant_dgelu(dh, a, fmt, scaling, row=True, col=True):
    """Quantize dGELU(dh, a) as the previous linear's incoming gradient."""
    return quantize(dgelu(dh, a), fmt, scaling, row, col)


def linear_fwd_gelu(a, w, scaling="tensor", wq=None):
    """The second linear of an MLP block: Y = GELU(A) W^T."""
    return linear_fwd(gelu(a), w, scaling, wq)


def linear_bwd_dgelu(dh, a, ctx):
    """The first linear of an MLP block, backward: its incoming gradient is
    dGELU(dH, A), dH the gradient of GELU's output, A its pre-activation."""
    return linear_bwd(dgelu(dh, a), ctx)


# --------------------------------------------------------------------------
# The BF16 comparator linear (the pages' baseline: the same linears without
# FP8, "Native FP8 MLP reconstruction", isolated-linear table).  Every GEMM
# multiplies bf16 values exactly and sums in fp32 with k ascending; outputs
# are rounded to bf16.  Transposed operands are plain numpy transposes.
# --------------------------------------------------------------------------

def gemm_bf16(A, B, want_f32=False):
    """C[i][j] = bf16(sum_k A[i][k] B[j][k]); A [I, K], B [J, K] bf16 bits."""
    A = _c(A, np.uint16)
    B = _c(B, np.uint16)
    I, K = A.shape
    J, K2 = B.shape
    assert K == K2
    C = np.empty((I, J), np.uint16)
    C32 = np.empty((I, J), np.float32) if want_f32 else None
    work = np.empty((I + J) * K, np.float32)
    _load().orc_gemm_bf16(_p(A), _p(B), I, J, K, _p(C), _p(C32), _p(work))
    return (C, C32) if want_f32 else C


def gemm_bf16_sampled(A, B, ii, jj, want_f32=False):
    A = _c(A, np.uint16)
    B = _c(B, np.uint16)
    K = A.shape[1]
    ii = _c(ii, np.int64)
    jj = _c(jj, np.int64)
    out = np.empty(ii.shape, np.uint16)
    out32 = np.empty(ii.shape, np.float32) if want_f32 else None
    _load().orc_gemm_bf16_sampled(_p(A), _p(B), K, _p(ii), _p(jj), ii.size, _p(out), _p(out32))
    return (out, out32) if want_f32 else out


def linear_bf16_fwd(x, w):
    """Y = X W^T in BF16: x [N, K], w [M, K] bf16 bits."""
    return gemm_bf16(x, w)


def linear_bf16_bwd(dy, x, w):
    """dX = dY W (contraction over M), dW = dY^T X (over N)."""
    dx = gemm_bf16(dy, np.ascontiguousarray(np.asarray(w).T))
    dw = gemm_bf16(np.ascontiguousarray(np.asarray(dy).T), np.ascontiguousarray(np.asarray(x).T))
    return dx, dw
