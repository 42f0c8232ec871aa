"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/fp8_linear.h declares, and rejects bad arguments with
the documented status before touching any device memory.  The pointers below
are fake addresses: every call here must fail validation (no call may pass it
and reach a kernel launch), so none is ever dereferenced."""
import ctypes
import os
import re

import pytest

from fp8_mixed_precision_amax_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8_linear.h")

OK, NULL, SHAPE, ALIGN, ENUM, WORKSPACE, CACHE_EMPTY, CACHE_MISMATCH = range(8)
A = 0x7F0000000000          # a fake, 16-byte aligned "device" address
U = A + 4                   # 4-byte aligned, not 16


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(fp8_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    return _lib.load()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 15
    assert sorted(names) == sorted(_lib.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.fp8_version().startswith(b"fp8linear")
    for code, name in _lib.STATUS.items():
        assert L.fp8_status_string(code).decode() == name


def qt(**kw):
    base = dict(q_row=A, q_col=A + 4096, scale=A + 8192, scale_inv=A + 8208, scale_col=A + 8224,
                scale_inv_col=A + 8240, amax=None)
    base.update(kw)
    return _lib.QTensorC(**base)


def quant(L, x=A, R=256, C=256, fmt=0, sc=0, lay=3, out=None, ws=A, wsb=4096):
    out = qt() if out is None else out
    return L.fp8_quantize(x, R, C, fmt, sc, lay, ctypes.byref(out), ws, wsb, None)


def test_quantize_argument_errors(L):
    assert quant(L, x=None) == NULL
    assert quant(L, x=U) == ALIGN
    assert quant(L, R=200) == SHAPE
    assert quant(L, C=0) == SHAPE
    assert quant(L, R=-128) == SHAPE
    assert quant(L, fmt=2) == ENUM
    assert quant(L, sc=3) == ENUM
    assert quant(L, lay=0) == ENUM
    assert quant(L, lay=4) == ENUM
    assert quant(L, out=qt(q_row=None)) == NULL
    assert quant(L, out=qt(q_col=A + 8)) == ALIGN
    assert quant(L, out=qt(q_row=None), lay=1) == NULL
    assert quant(L, out=qt(scale=None)) == NULL
    assert quant(L, sc=1, out=qt(scale_col=None)) == NULL
    assert quant(L, wsb=100) == WORKSPACE
    assert quant(L, ws=None) == NULL
    assert L.fp8_quantize(A, 256, 256, 0, 0, 3, None, A, 4096, None) == NULL
    # the cast-only variant: partials required and 16-byte aligned
    assert L.fp8_quantize_from_amax(A, 256, 256, 0, 3, ctypes.byref(qt()), None, None) == NULL
    assert L.fp8_quantize_from_amax(A, 256, 256, 0, 3, ctypes.byref(qt()), U, None) == ALIGN
    assert L.fp8_quantize_from_amax(A, 200, 256, 0, 3, ctypes.byref(qt()), A, None) == SHAPE
    # delayed scaling: 1 .. 1024 history entries, a history, enough workspace
    wsd = L.fp8_quantize_delayed_workspace_bytes(256, 256)
    assert wsd == 16                          # 4 tiles x 2 bytes, rounded to 16
    dq = lambda hist=A, H=16, ws=A, wsb=wsd: L.fp8_quantize_delayed(A, 256, 256, 0, 3, ctypes.byref(qt()), hist, H, ws,
                                                                     wsb, None)
    assert dq(H=0) == SHAPE and dq(H=1025) == SHAPE
    assert dq(hist=None) == NULL
    assert dq(wsb=8) == WORKSPACE


def test_last_error_message(L):
    assert quant(L, R=200) == SHAPE
    assert b"multiple" in L.fp8_last_error()
    assert quant(L, fmt=7) == ENUM
    assert b"format" in L.fp8_last_error()


def test_workspace_queries(L):
    assert L.fp8_quantize_workspace_bytes(1024, 512, 0) >= 4096
    assert L.fp8_quantize_workspace_bytes(1024, 512, 1) == 0
    # a weight gradient with a long contraction uses split-K partials
    assert L.fp8_gemm_workspace_bytes(2048, 512, 131072) > 0
    assert L.fp8_linear_workspace_bytes(131072, 512, 2048, 0) >= L.fp8_gemm_workspace_bytes(2048, 512, 131072)


def gs(p=A + 8192, group=0, sr=0, sk=0):
    return _lib.GemmScaleC(p, group, sr, sk)


def test_gemm_argument_errors(L):
    def g(a=A, b=A, c=A, I=256, J=256, K=256, fa=0, fb=0, sa=None, sb=None, ws=A, wsb=1 << 30):
        return L.fp8_gemm(a, fa, sa or gs(), b, fb, sb or gs(), I, J, K, c, ws, wsb, None)
    assert g(a=None) == NULL
    assert g(c=U) == ALIGN
    assert g(K=100) == SHAPE
    assert g(fa=5) == ENUM
    assert g(sa=gs(group=1, sr=2, sk=1)) == ENUM          # mixed tensor / block
    assert g(sa=gs(group=3), sb=gs(group=1)) == ENUM
    assert g(sa=gs(p=None)) == NULL
    assert g(I=256, J=256, K=131072, wsb=0) == WORKSPACE
    # 32-bit tile offsets: the contraction must stay below 2^23, checked
    # before the workspace
    assert g(K=1 << 23, wsb=0) == SHAPE
    assert g(K=(1 << 23) - 128, wsb=0) == WORKSPACE
    # the output-amax variant: tensorwise only, the partials buffer required
    def ga(c_amax=A, sa=None, sb=None):
        return L.fp8_gemm_amax(A, 0, sa or gs(), A, 0, sb or gs(), 256, 256, 256, A, c_amax, A, 1 << 30, None)
    assert ga(c_amax=None) == NULL
    assert ga(c_amax=U) == ALIGN
    assert ga(sa=gs(group=1, sr=1, sk=256), sb=gs(group=1, sr=1, sk=256)) == ENUM


def make_cache(L, M=256, K=256, recipe=0, bufs=None):
    h = ctypes.c_void_p()
    st = L.fp8_wcache_create(M, K, recipe, ctypes.byref(bufs or qt()), ctypes.byref(h))
    return st, h


def test_cache_lifecycle_and_errors(L):
    st, h = make_cache(L)
    assert st == OK and h.value
    assert L.fp8_wcache_valid(h) == 0 and L.fp8_wcache_fills(h) == 0
    assert L.fp8_wcache_invalidate(h) == OK
    assert L.fp8_wcache_valid(None) == -1
    assert L.fp8_wcache_invalidate(None) == NULL
    assert make_cache(L, M=100)[0] == SHAPE
    assert make_cache(L, recipe=9)[0] == ENUM
    assert make_cache(L, bufs=qt(q_col=None))[0] == NULL
    assert L.fp8_wcache_create(256, 256, 0, ctypes.byref(qt()), None) == NULL
    N, K, M = 256, 256, 256
    wsb = L.fp8_linear_workspace_bytes(N, K, M, 0)
    sx = qt()

    def fwd(x, w, N, K, M, recipe, cache, flag, wq, ws, wsb_, xa=None, ya=None):
        return L.fp8_linear_fwd(x, w, N, K, M, recipe, cache, flag, A, ctypes.byref(sx), wq, xa, ya, ws, wsb_, None)

    def bwd(N, K, M, recipe, cache, wq, dq, dx, dw, ws, wsb_, dya=None, dxa=None):
        return L.fp8_linear_bwd(A, N, K, M, recipe, ctypes.byref(sx), cache, wq, dq, dx, dw, dya, dxa, ws, wsb_, None)

    # False on an empty cache
    assert fwd(A, None, N, K, M, 0, h, 0, None, A, wsb) == CACHE_EMPTY
    # shape / recipe mismatch
    assert fwd(A, A, N, K, 512, 0, h, 1, None, A, L.fp8_linear_workspace_bytes(N, K, 512, 0)) == CACHE_MISMATCH
    assert fwd(A, A, N, K, M, 1, h, 1, None, A, L.fp8_linear_workspace_bytes(N, K, M, 1)) == CACHE_MISMATCH
    # bad flag, small workspace, None without w_q
    assert fwd(A, A, N, K, M, 0, h, 2, None, A, wsb) == ENUM
    assert fwd(A, A, N, K, M, 0, h, 1, None, A, 16) == WORKSPACE
    assert fwd(A, A, N, K, M, 0, None, -1, None, A, wsb) == NULL
    # every linear dimension is some GEMM's contraction: below 2^23
    big = 1 << 23
    assert fwd(A, A, big, K, M, 0, None, -1, ctypes.byref(qt()), A, 1 << 40) == SHAPE
    assert bwd(N, K, big, 0, None, ctypes.byref(qt()), ctypes.byref(qt()), A, A, A, 1 << 40) == SHAPE
    # amax hand-off: tensorwise recipe only, 16-byte aligned, dX partials need dX
    wsb1 = L.fp8_linear_workspace_bytes(N, K, M, 1)
    assert fwd(A, A, N, K, M, 1, None, -1, ctypes.byref(qt()), A, wsb1, xa=A) == ENUM
    assert fwd(A, A, N, K, M, 0, None, -1, ctypes.byref(qt()), A, wsb, ya=U) == ALIGN
    assert bwd(N, K, M, 1, None, ctypes.byref(qt()), ctypes.byref(qt()), A, A, A, wsb1, dya=A) == ENUM
    assert bwd(N, K, M, 0, None, ctypes.byref(qt()), ctypes.byref(qt()), None, A, A, wsb, dxa=A) == NULL
    # backward through an empty cache
    dq = qt()
    assert bwd(N, K, M, 0, h, None, ctypes.byref(dq), A, A, A, wsb) == CACHE_EMPTY
    assert bwd(N, K, M, 0, h, None, ctypes.byref(dq), None, None, A, wsb) == NULL
    assert L.fp8_wcache_valid(h) == 0          # nothing above filled it
    L.fp8_wcache_destroy(h)
    L.fp8_wcache_destroy(None)


def test_gelu_argument_errors(L):
    """GELU of the MLP block: elementwise ops, the fused quantizers and the
    two MLP-block linears validate like the plain entry points."""
    assert L.fp8_gelu(A, A, 12, None) == SHAPE
    assert L.fp8_gelu(A, A, -8, None) == SHAPE
    assert L.fp8_gelu(None, A, 8, None) == NULL
    assert L.fp8_gelu(A, U, 8, None) == ALIGN
    assert L.fp8_gelu(A, A, 0, None) == OK                 # empty: nothing is enqueued
    assert L.fp8_dgelu(A, None, A, 8, None) == NULL
    assert L.fp8_dgelu(A, A, U, 8, None) == ALIGN
    assert L.fp8_dgelu(A, A, A, 4, None) == SHAPE
    o = qt()

    def qg(x=A, R=256, C=256, sc=0, ws=A, wsb=4096):
        return L.fp8_quantize_gelu(x, R, C, 0, sc, 3, ctypes.byref(o), ws, wsb, None)

    def qd(x=A, sc=0):
        return L.fp8_quantize_dgelu(A, x, 256, 256, 1, sc, 3, ctypes.byref(o), A, 4096, None)

    assert qg(sc=2) == ENUM                                # 128x128 blocks are for weights
    assert qg(R=200) == SHAPE
    assert qg(x=U) == ALIGN
    assert qg(wsb=100) == WORKSPACE
    assert qd(x=None) == NULL and qd(x=U) == ALIGN and qd(sc=2) == ENUM
    wsb = L.fp8_linear_workspace_bytes(256, 256, 256, 0)
    sx = qt()

    def fwd(N=256, wq=True):
        return L.fp8_linear_fwd_gelu(A, A, N, 256, 256, 0, None, -1, A, ctypes.byref(sx),
                                     ctypes.byref(qt()) if wq else None, None, A, wsb, None)

    def bwd(y_pre=A):
        return L.fp8_linear_bwd_dgelu(A, y_pre, 256, 256, 256, 0, ctypes.byref(sx), None, ctypes.byref(qt()),
                                      ctypes.byref(qt()), A, A, None, A, wsb, None)

    assert fwd(N=200) == SHAPE
    assert fwd(wq=False) == NULL                           # None (-1) needs w_q
    assert bwd(y_pre=None) == NULL and bwd(y_pre=U) == ALIGN


def test_ceilings_library_exports():
    """The benchmark's ceiling probes (libfp8ceilings.so, built beside the
    library) load without a GPU and export their four entry points; the MFMA
    probe rejects a block size it cannot run before launching anything."""
    import ctypes
    path = os.path.join(ROOT, "fp8_mixed_precision_amax_amd", "libfp8ceilings.so")
    if not os.path.exists(path):
        pytest.skip("libfp8ceilings.so not built")
    C = ctypes.CDLL(path)
    for n in ("fp8c_hbm_read", "fp8c_hbm_write", "fp8c_hbm_copy", "fp8c_mfma"):
        assert hasattr(C, n), n
    C.fp8c_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                            ctypes.c_void_p]
    assert C.fp8c_mfma(1, 100, 1, None, None, None) != 0


def test_noalloc_forward_rejections(L):
    """fp8_linear_fwd_noalloc validates shape and recipe, and refuses a
    forward whose scratch would exceed the fixed device array, before it
    touches any device: a short output over a long contraction (256 x 8192
    tokens-by-weight with K = 8192 splits its GEMM 8 ways: 64 MiB of
    partial sums, above 8 MiB)."""
    assert _lib.NOALLOC_SCRATCH_BYTES == 8 << 20
    x = qt()
    w = qt()

    def call(N, K, M, recipe=0):
        return L.fp8_linear_fwd_noalloc(A, A, N, K, M, recipe, None, -1, A, ctypes.byref(x), ctypes.byref(w),
                                        None, None, None)
    assert call(100, 512, 512) == SHAPE
    assert call(256, 512, 512, recipe=5) == ENUM
    assert call(256, 8192, 8192) == WORKSPACE
    assert b"8388608-byte device scratch" in L.fp8_last_error()


def test_missing_library_fails_loudly(tmp_path):
    """Without the built library the package raises on first use; nothing
    falls back to a CPU path (run in a fresh interpreter whose package points
    at an empty directory)."""
    import subprocess
    import sys
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from fp8_mixed_precision_amax_amd import _lib\n"
        "import fp8_mixed_precision_amax_amd as fp8\n"
        "_lib.LIB_PATH = %r\n"
        "_lib._lib = None\n"
        "try:\n"
        "    fp8.lib()\n"
        "except ImportError as e:\n"
        "    print('raised:', e)\n"
        "    sys.exit(0)\n"
        "sys.exit(1)\n" % (ROOT, str(tmp_path / "libfp8linear.so")))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "not built" in r.stdout
