"""MI355X (gfx950) FP8 linear layer: current amax scaling, fused dual-layout
FP8 casts, FP8 matrix-core GEMMs and a weight cache, behind a C ABI.

Python side = argument marshalling over ``libfp8linear.so``.  torch is used
for device memory and the current stream only.

    quantize(x, fmt, scaling)          -> QTensor (row + col layouts, scales)
    gemm(a, b, ...)                    -> bf16 [I, J]
    Fp8Linear(M, K, recipe)            forward / backward with optional cache
"""
import contextlib
import ctypes

import torch

from . import _lib
from ._lib import (E4M3, E5M2, LAYOUT_COL, LAYOUT_ROW, RECIPE_BLOCK, RECIPE_TENSOR, SCALE_1x128,
                   SCALE_128x128, SCALE_TENSOR, Fp8Error)

__all__ = ["block_gemm_scale", "E4M3", "E5M2", "SCALE_TENSOR", "SCALE_1x128", "SCALE_128x128", "RECIPE_TENSOR",
           "RECIPE_BLOCK", "LAYOUT_ROW", "LAYOUT_COL", "Fp8Error", "QTensor", "quantize",
           "gemm", "WeightCache", "Fp8Linear", "linear_workspace", "lib", "amax_partials",
           "AMAX_PARTIALS_BYTES", "quantize_delayed"]


def lib():
    return _lib.load()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocate temporaries (workspace, contiguous copies, outputs) on the
    stream the library launches on: the caching allocator then reuses them
    only after that stream's work, and any copy torch makes runs on it too."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _dev(x):
    if not x.is_cuda:
        raise ValueError("tensor must be on the GPU")
    return x.device


class QTensor:
    """Quantized tensor buffers (torch tensors on the device) for a source of
    shape [rows, cols] under the given scaling."""

    def __init__(self, rows, cols, scaling, device, row=True, col=True):
        self.rows, self.cols, self.scaling = rows, cols, scaling
        u8, f32 = torch.uint8, torch.float32
        self.q_row = torch.empty((rows, cols), dtype=u8, device=device) if row else None
        self.q_col = torch.empty((cols, rows), dtype=u8, device=device) if col else None
        # 1x128 scales are stored block-major ([cols/128, rows] and
        # [rows/128, cols]); the attributes are transposed views with the
        # logical shapes [rows, cols/128] and [cols, rows/128]
        if scaling == SCALE_TENSOR:
            shp = (1,)
        elif scaling == SCALE_1x128:
            shp = (rows, cols // 128)
        else:
            shp = (rows // 128, cols // 128)
        if scaling == SCALE_1x128:
            self.scale = torch.empty((cols // 128, rows), dtype=f32, device=device).t()
            self.scale_inv = torch.empty((cols // 128, rows), dtype=f32, device=device).t()
        else:
            self.scale = torch.empty(shp, dtype=f32, device=device)
            self.scale_inv = torch.empty(shp, dtype=f32, device=device)
        if scaling == SCALE_1x128 and col:
            self.scale_col = torch.empty((rows // 128, cols), dtype=f32, device=device).t()
            self.scale_inv_col = torch.empty((rows // 128, cols), dtype=f32, device=device).t()
        else:
            self.scale_col = self.scale_inv_col = None
        self.amax = torch.empty((1,), dtype=f32, device=device) if scaling == SCALE_TENSOR else None

    def c(self):
        return _lib.QTensorC(*(None if t is None else t.data_ptr() for t in
                               (self.q_row, self.q_col, self.scale, self.scale_inv,
                                self.scale_col, self.scale_inv_col, self.amax)))


AMAX_PARTIALS_BYTES = 4096         # FP8_AMAX_PARTIALS_BYTES
GELU_AMAX_PARTIALS_BYTES = 16384   # FP8_GELU_AMAX_PARTIALS_BYTES


def amax_partials(device):
    """Device buffer for the amax hand-off (2048 16-bit partial maxima)."""
    return torch.empty(AMAX_PARTIALS_BYTES, dtype=torch.uint8, device=device)


def gelu_amax_partials(device):
    """Device buffer for the GELU amax hand-off (four arrays of 2048 16-bit
    keys, see fp8_linear.h)."""
    return torch.empty(GELU_AMAX_PARTIALS_BYTES, dtype=torch.uint8, device=device)


def quantize(x, fmt, scaling=SCALE_TENSOR, layouts=LAYOUT_ROW | LAYOUT_COL, out=None, stream=None,
             amax_partials=None):
    """Current-scaling FP8 quantization of a bf16 [rows, cols] device tensor.
    amax_partials (tensorwise only): x's amax partials from its producer
    (fp8_quantize_from_amax: the cast pass alone)."""
    with _on(stream):
        return _quantize(x, fmt, scaling, layouts, out, stream, amax_partials)


def _quantize(x, fmt, scaling, layouts, out, stream, amax_partials):
    L = lib()
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    x = x.contiguous()
    R, C = x.shape
    if out is None:
        out = QTensor(R, C, scaling, _dev(x), row=bool(layouts & LAYOUT_ROW), col=bool(layouts & LAYOUT_COL))
    if amax_partials is not None:
        if scaling != SCALE_TENSOR:
            raise ValueError("amax partials serve the tensorwise quantize")
        oc = out.c()
        _lib.check(L.fp8_quantize_from_amax(_ptr(x), R, C, fmt, layouts, ctypes.byref(oc), _ptr(amax_partials),
                                            _stream(stream)))
        return out
    wsb = L.fp8_quantize_workspace_bytes(R, C, scaling)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=x.device)
    oc = out.c()
    _lib.check(L.fp8_quantize(_ptr(x), R, C, fmt, scaling, layouts, ctypes.byref(oc), _ptr(ws), wsb,
                              _stream(stream)))
    return out


def quantize_delayed(x, fmt, history, layouts=LAYOUT_ROW | LAYOUT_COL, out=None, stream=None):
    """Delayed tensorwise scaling: encode with FMAX / max(history), then roll
    the fp32 device tensor `history` (most recent amax first) and store
    amax(x) in front.  Returns the QTensor (out.amax = amax(x))."""
    with _on(stream):
        return _quantize_delayed(x, fmt, history, layouts, out, stream)


def _quantize_delayed(x, fmt, history, layouts, out, stream):
    L = lib()
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    if history.dtype != torch.float32 or history.dim() != 1 or not history.is_contiguous():
        raise ValueError("history must be a contiguous 1-D float32 tensor")
    x = x.contiguous()
    R, C = x.shape
    if out is None:
        out = QTensor(R, C, SCALE_TENSOR, _dev(x), row=bool(layouts & LAYOUT_ROW), col=bool(layouts & LAYOUT_COL))
    wsb = L.fp8_quantize_delayed_workspace_bytes(R, C)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=x.device)
    oc = out.c()
    _lib.check(L.fp8_quantize_delayed(_ptr(x), R, C, fmt, layouts, ctypes.byref(oc), _ptr(history), history.numel(),
                                      _ptr(ws), wsb, _stream(stream)))
    return out


def _bf16_pair(name, *ts):
    for t in ts:
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(name + ": tensors must be contiguous bfloat16")
    if any(t.shape != ts[0].shape for t in ts):
        raise ValueError(name + ": shapes differ")


def gelu(x, out=None, stream=None):
    """GELU(x) elementwise (exact erf form), bf16 in and out (fp8_gelu)."""
    _bf16_pair("gelu", x)
    with _on(stream):
        if out is None:
            out = torch.empty_like(x)
        _lib.check(lib().fp8_gelu(_ptr(x), _ptr(out), x.numel(), _stream(stream)))
    return out


def dgelu(dy, x, out=None, stream=None):
    """dy * GELU'(x) elementwise, bf16 in and out (fp8_dgelu): dy is the
    gradient of GELU's output, x GELU's input."""
    _bf16_pair("dgelu", dy, x)
    with _on(stream):
        if out is None:
            out = torch.empty_like(x)
        _lib.check(lib().fp8_dgelu(_ptr(dy), _ptr(x), _ptr(out), x.numel(), _stream(stream)))
    return out


def _act_quantize(name, fn, xs, fmt, scaling, layouts, out, stream):
    with _on(stream):
        return _act_quantize_on(name, fn, xs, fmt, scaling, layouts, out, stream)


def _act_quantize_on(name, fn, xs, fmt, scaling, layouts, out, stream):
    L = lib()
    _bf16_pair(name, *xs)
    if xs[0].dim() != 2:
        raise ValueError(name + ": tensors must be 2-D")
    R, C = xs[0].shape
    if out is None:
        out = QTensor(R, C, scaling, _dev(xs[0]), row=bool(layouts & LAYOUT_ROW), col=bool(layouts & LAYOUT_COL))
    wsb = L.fp8_quantize_workspace_bytes(R, C, scaling)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=xs[0].device)
    oc = out.c()
    _lib.check(fn(*[_ptr(t) for t in xs], R, C, fmt, scaling, layouts, ctypes.byref(oc), _ptr(ws), wsb,
                  _stream(stream)))
    return out


def quantize_gelu(x, fmt, scaling=SCALE_TENSOR, layouts=LAYOUT_ROW | LAYOUT_COL, out=None, stream=None,
                  gelu_amax_partials=None):
    """Quantize GELU(x) without writing the activation (fp8_quantize_gelu);
    tensorwise or 1x128 scaling.  gelu_amax_partials (tensorwise only): the
    GELU amax keys x's producer wrote (fp8_quantize_gelu_from_amax: the
    cast pass alone)."""
    if gelu_amax_partials is None:
        return _act_quantize("quantize_gelu", lib().fp8_quantize_gelu, (x,), fmt, scaling, layouts, out, stream)
    if scaling != SCALE_TENSOR:
        raise ValueError("GELU amax partials serve the tensorwise quantize")
    L = lib()
    _bf16_pair("quantize_gelu", x)
    R, C = x.shape
    with _on(stream):
        if out is None:
            out = QTensor(R, C, scaling, _dev(x), row=bool(layouts & LAYOUT_ROW), col=bool(layouts & LAYOUT_COL))
        oc = out.c()
        _lib.check(L.fp8_quantize_gelu_from_amax(_ptr(x), R, C, fmt, layouts, ctypes.byref(oc),
                                                 _ptr(gelu_amax_partials), _stream(stream)))
    return out


def quantize_dgelu(dy, x, fmt, scaling=SCALE_TENSOR, layouts=LAYOUT_ROW | LAYOUT_COL, out=None, stream=None):
    """Quantize dy * GELU'(x) without writing it (fp8_quantize_dgelu)."""
    return _act_quantize("quantize_dgelu", lib().fp8_quantize_dgelu, (dy, x), fmt, scaling, layouts, out, stream)


def gemm_scale(sinv, group=0, stride_r=0, stride_kb=0):
    """Scale descriptor of a GEMM operand; keeps a reference to the tensor so
    the device memory stays alive as long as the descriptor does."""
    s = _lib.GemmScaleC(sinv.data_ptr(), group, stride_r, stride_kb)
    s._keep = sinv
    return s


def block_gemm_scale(sinv, group):
    """Scale descriptor of a block-scaled operand whose factors are the 2-D
    tensor sinv [operand rows / group, contraction blocks] (any strides, e.g.
    the views a QTensor holds)."""
    return gemm_scale(sinv, group, sinv.stride(0), sinv.stride(1))


def gemm(a, fa, sa, b, fb, sb, out=None, stream=None, amax_out=None, gelu_amax_out=None):
    """C[i][j] = bf16(sum_k A[i][k] B[j][k] * scales); a [I, K], b [J, K]
    uint8 FP8 codes; sa / sb are GemmScaleC (see gemm_scale).  amax_out
    (tensorwise only): receives C's amax partials (fp8_gemm_amax);
    gelu_amax_out (tensorwise E4M3 x E4M3): receives C's GELU amax partials
    (fp8_gemm_gelu_amax)."""
    with _on(stream):
        return _gemm(a, fa, sa, b, fb, sb, out, stream, amax_out, gelu_amax_out)


def _gemm(a, fa, sa, b, fb, sb, out, stream, amax_out, gelu_amax_out=None):
    L = lib()
    I, K = a.shape
    J, K2 = b.shape
    if K != K2:
        raise ValueError("contraction sizes differ")
    if out is None:
        out = torch.empty((I, J), dtype=torch.bfloat16, device=a.device)
    wsb = L.fp8_gemm_workspace_bytes(I, J, K)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=a.device)
    if gelu_amax_out is not None:
        if amax_out is not None:
            raise ValueError("one hand-off per GEMM")
        _lib.check(L.fp8_gemm_gelu_amax(_ptr(a), fa, sa, _ptr(b), fb, sb, I, J, K, _ptr(out), _ptr(gelu_amax_out),
                                        _ptr(ws), wsb, _stream(stream)))
    elif amax_out is not None:
        _lib.check(L.fp8_gemm_amax(_ptr(a), fa, sa, _ptr(b), fb, sb, I, J, K, _ptr(out), _ptr(amax_out), _ptr(ws),
                                   wsb, _stream(stream)))
    else:
        _lib.check(L.fp8_gemm(_ptr(a), fa, sa, _ptr(b), fb, sb, I, J, K, _ptr(out), _ptr(ws), wsb,
                              _stream(stream)))
    return out


class WeightCache:
    """Weight cache for the is_first_microbatch protocol.  Owns the device
    buffers of the quantized weight; the library handle references them."""

    def __init__(self, M, K, recipe, device):
        self.M, self.K, self.recipe = M, K, recipe
        self.q = QTensor(M, K, SCALE_TENSOR if recipe == RECIPE_TENSOR else SCALE_128x128, device)
        self._qc = self.q.c()
        h = ctypes.c_void_p()
        _lib.check(lib().fp8_wcache_create(M, K, recipe, ctypes.byref(self._qc), ctypes.byref(h)))
        self.handle = h

    def invalidate(self):
        _lib.check(lib().fp8_wcache_invalidate(self.handle))

    @property
    def valid(self):
        return lib().fp8_wcache_valid(self.handle) == 1

    @property
    def fills(self):
        return lib().fp8_wcache_fills(self.handle)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            try:
                lib().fp8_wcache_destroy(h)
            except Exception:
                pass
            self.handle = None


def linear_workspace(N, K, M, recipe, device):
    n = lib().fp8_linear_workspace_bytes(N, K, M, recipe)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device), n


class Fp8Linear:
    """FP8 linear layer Y = X W^T with current scaling.  Holds the buffers of
    one forward/backward (saved X, quantized W or the cache, quantized dY)
    for token count N, so repeated calls allocate nothing."""

    def __init__(self, N, K, M, recipe=RECIPE_TENSOR, device="cuda", cache=False):
        self.N, self.K, self.M, self.recipe = N, K, M, recipe
        act = SCALE_TENSOR if recipe == RECIPE_TENSOR else SCALE_1x128
        wsc = SCALE_TENSOR if recipe == RECIPE_TENSOR else SCALE_128x128
        self.saved_x = QTensor(N, K, act, device)
        self.dy_q = QTensor(N, M, act, device)
        self.w_q = QTensor(M, K, wsc, device)
        self.cache = WeightCache(M, K, recipe, device) if cache else None
        self.ws, self.ws_bytes = linear_workspace(N, K, M, recipe, device)
        self._sx, self._dq, self._wq = self.saved_x.c(), self.dy_q.c(), self.w_q.c()

    def forward(self, x, w, y=None, is_first_microbatch=None, stream=None, x_amax=None, y_amax=None, gelu=False):
        """x_amax: X's amax partials from its producer (skips X's amax pass);
        y_amax: receives Y's partials (tensorwise recipe).  gelu=True: x is
        the pre-activation and the layer's input is GELU(x), applied by X's
        quantize (fp8_linear_fwd_gelu; no x_amax)."""
        flag = -1 if is_first_microbatch is None else int(bool(is_first_microbatch))
        if y is None:
            with _on(stream):
                y = torch.empty((self.N, self.M), dtype=torch.bfloat16, device=x.device)
        cache = self.cache.handle if (self.cache is not None and flag != -1) else None
        if gelu:
            if x_amax is not None:
                raise ValueError("no X amax hand-off with the GELU input")
            _lib.check(lib().fp8_linear_fwd_gelu(_ptr(x), _ptr(w), self.N, self.K, self.M, self.recipe, cache, flag,
                                                 _ptr(y), ctypes.byref(self._sx), ctypes.byref(self._wq),
                                                 _ptr(y_amax), _ptr(self.ws), self.ws_bytes, _stream(stream)))
        else:
            _lib.check(lib().fp8_linear_fwd(_ptr(x), _ptr(w), self.N, self.K, self.M, self.recipe, cache, flag,
                                            _ptr(y), ctypes.byref(self._sx), ctypes.byref(self._wq),
                                            _ptr(x_amax), _ptr(y_amax), _ptr(self.ws), self.ws_bytes,
                                            _stream(stream)))
        self._last_flag = flag
        return y

    def forward_noalloc(self, x, w, y, is_first_microbatch=None, stream=None, x_amax=None, y_amax=None):
        """forward() through fp8_linear_fwd_noalloc: the library's per-device
        scratch instead of this layer's workspace; y must be given (nothing
        is allocated here either)."""
        flag = -1 if is_first_microbatch is None else int(bool(is_first_microbatch))
        cache = self.cache.handle if (self.cache is not None and flag != -1) else None
        _lib.check(lib().fp8_linear_fwd_noalloc(_ptr(x), _ptr(w), self.N, self.K, self.M, self.recipe, cache, flag,
                                                _ptr(y), ctypes.byref(self._sx), ctypes.byref(self._wq),
                                                _ptr(x_amax), _ptr(y_amax), _stream(stream)))
        self._last_flag = flag
        return y

    def backward(self, dy, dx=None, dw=None, need_dx=True, need_dw=True, stream=None, dy_amax=None,
                 dx_amax=None, gelu_input=None):
        """dy_amax: dY's amax partials from its producer (skips dY's amax
        pass); dx_amax: receives dX's partials (tensorwise recipe).
        gelu_input: GELU's input (this layer's forward output); dy is then the
        gradient of GELU's output and the incoming gradient is
        dy * GELU'(gelu_input), applied by dY's quantize
        (fp8_linear_bwd_dgelu; no dy_amax)."""
        with _on(stream):
            if need_dx and dx is None:
                dx = torch.empty((self.N, self.K), dtype=torch.bfloat16, device=dy.device)
            if need_dw and dw is None:
                dw = torch.empty((self.M, self.K), dtype=torch.bfloat16, device=dy.device)
        use_cache = self.cache is not None and getattr(self, "_last_flag", -1) != -1
        cache = self.cache.handle if use_cache else None
        dxp, dwp = (_ptr(dx) if need_dx else None), (_ptr(dw) if need_dw else None)
        if gelu_input is not None:
            if dy_amax is not None:
                raise ValueError("no dY amax hand-off through GELU")
            _lib.check(lib().fp8_linear_bwd_dgelu(_ptr(dy), _ptr(gelu_input), self.N, self.K, self.M, self.recipe,
                                                  ctypes.byref(self._sx), cache, ctypes.byref(self._wq),
                                                  ctypes.byref(self._dq), dxp, dwp, _ptr(dx_amax), _ptr(self.ws),
                                                  self.ws_bytes, _stream(stream)))
        else:
            _lib.check(lib().fp8_linear_bwd(_ptr(dy), self.N, self.K, self.M, self.recipe,
                                            ctypes.byref(self._sx), cache, ctypes.byref(self._wq),
                                            ctypes.byref(self._dq), dxp, dwp, _ptr(dy_amax), _ptr(dx_amax),
                                            _ptr(self.ws), self.ws_bytes, _stream(stream)))
        return dx, dw

    def weight_q(self):
        """The quantized weight the last forward used (cache or w_q)."""
        use_cache = self.cache is not None and getattr(self, "_last_flag", -1) != -1
        return self.cache.q if use_cache else self.w_q


class Fp8Mlp:
    """The MLP block X [N, D] -> A = X W1^T [N, H] -> Y = GELU(A) W2^T [N, D]
    in FP8: forward in one library call (fp8_mlp_fwd: the up projection hands
    the GELU amax keys of A to the down projection's input quantize),
    backward through the two linears' entry points (the up projection's
    gradient quantize applies GELU')."""

    def __init__(self, N, D, H, recipe=RECIPE_TENSOR, device="cuda", cache=False, up=None, down=None):
        """up / down: existing Fp8Linear objects of the two linears (their
        buffers and caches are then shared with direct calls on them)."""
        self.N, self.D, self.H, self.recipe = N, D, H, recipe
        self.up = up if up is not None else Fp8Linear(N, D, H, recipe, device, cache)
        self.down = down if down is not None else Fp8Linear(N, H, D, recipe, device, cache)
        n = lib().fp8_mlp_workspace_bytes(N, D, H, recipe)
        self.ws, self.ws_bytes = torch.empty(max(n, 16), dtype=torch.uint8, device=device), n
        self.a = None

    def forward(self, x, w1, w2, y=None, a=None, is_first_microbatch=None, stream=None, x_amax=None, y_amax=None):
        flag = -1 if is_first_microbatch is None else int(bool(is_first_microbatch))
        with _on(stream):
            if a is None:
                a = torch.empty((self.N, self.H), dtype=torch.bfloat16, device=x.device)
            if y is None:
                y = torch.empty((self.N, self.D), dtype=torch.bfloat16, device=x.device)
        use_cache = self.up.cache is not None and flag != -1
        c1 = self.up.cache.handle if use_cache else None
        c2 = self.down.cache.handle if use_cache else None
        _lib.check(lib().fp8_mlp_fwd(_ptr(x), _ptr(w1), _ptr(w2), self.N, self.D, self.H, self.recipe, c1, c2, flag,
                                     _ptr(a), _ptr(y), ctypes.byref(self.up._sx), ctypes.byref(self.up._wq),
                                     ctypes.byref(self.down._sx), ctypes.byref(self.down._wq), _ptr(x_amax),
                                     _ptr(y_amax), _ptr(self.ws), self.ws_bytes, _stream(stream)))
        self.up._last_flag = self.down._last_flag = flag
        self.a = a
        return y

    def backward(self, dy, stream=None):
        """(dX, dW1, dW2) of the last forward."""
        dh, dw2 = self.down.backward(dy, stream=stream)
        dx, dw1 = self.up.backward(dh, stream=stream, gelu_input=self.a)
        return dx, dw1, dw2


# ------------------------------ BF16 comparator ------------------------------

def bf16_gemm(a, b, a_layout=0, b_layout=0, I=None, J=None, out=None, stream=None):
    """C [I, J] = bf16(sum_k A[i][k] B[j][k]) on the BF16 matrix cores
    (fp8_bf16_gemm).  layout 0: the tensor is [rows, K] (contraction-major);
    1: the tensor is [K, rows] (output-major)."""
    L = lib()
    for t in (a, b):
        if t.dtype != torch.bfloat16 or t.dim() != 2 or not t.is_contiguous():
            raise ValueError("operands must be contiguous 2-D bfloat16 tensors")
    I = a.shape[0] if a_layout == 0 else a.shape[1]
    K = a.shape[1] if a_layout == 0 else a.shape[0]
    J = b.shape[0] if b_layout == 0 else b.shape[1]
    Kb = b.shape[1] if b_layout == 0 else b.shape[0]
    if K != Kb:
        raise ValueError("contraction sizes differ")
    with _on(stream):
        if out is None:
            out = torch.empty((I, J), dtype=torch.bfloat16, device=a.device)
        wsb = L.fp8_bf16_gemm_workspace_bytes(I, J, K)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=a.device)
        _lib.check(L.fp8_bf16_gemm(_ptr(a), a_layout, _ptr(b), b_layout, I, J, K, _ptr(out), _ptr(ws), wsb,
                                   _stream(stream)))
    return out


class Bf16Linear:
    """The BF16 comparator linear Y = X W^T (fp8_bf16_linear_fwd / _bwd):
    no quantization, hand-written BF16 matrix-core GEMMs."""

    def __init__(self, N, K, M, device="cuda"):
        self.N, self.K, self.M = N, K, M
        n = lib().fp8_bf16_linear_workspace_bytes(N, K, M)
        self.ws, self.ws_bytes = torch.empty(max(n, 16), dtype=torch.uint8, device=device), n

    def forward(self, x, w, y=None, stream=None):
        with _on(stream):
            if y is None:
                y = torch.empty((self.N, self.M), dtype=torch.bfloat16, device=x.device)
        _lib.check(lib().fp8_bf16_linear_fwd(_ptr(x), _ptr(w), self.N, self.K, self.M, _ptr(y), _ptr(self.ws),
                                             self.ws_bytes, _stream(stream)))
        return y

    def backward(self, dy, x, w, dx=None, dw=None, stream=None):
        with _on(stream):
            if dx is None:
                dx = torch.empty((self.N, self.K), dtype=torch.bfloat16, device=dy.device)
            if dw is None:
                dw = torch.empty((self.M, self.K), dtype=torch.bfloat16, device=dy.device)
        _lib.check(lib().fp8_bf16_linear_bwd(_ptr(dy), _ptr(x), _ptr(w), self.N, self.K, self.M, _ptr(dx), _ptr(dw),
                                             _ptr(self.ws), self.ws_bytes, _stream(stream)))
        return dx, dw
