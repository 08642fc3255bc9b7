"""The CPU oracle for the Q8_0 GEMV / sparse-MoE hot path.

TEST INFRASTRUCTURE, NOT PRODUCT: only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It wraps
``oracle/q8s_oracle.c`` (plain C, double-precision sums) through ctypes and
shares no code with the HIP library in ``q8_gemv_sparse_amd``.

Functions take and return numpy arrays.  Each cites the passage its C
counterpart follows (see the header of q8s_oracle.c):

* ``gemv_f32``   G, struct Q8Ref dequant + fn emit_moe_forward's f64 sums
* ``quantize``   Q, llama.cpp's one-word Q8_0 activation (enum Q8MatKind)
* ``block_dots`` the exact int32 block sums of the int8 mode
* ``gemv_i8``    I, one-word int8 activations
* ``quantize_x2`` Q2, the two-word (~14-bit) activation (CudaKnobs `activations`;
  arena.rs fn quant_parts: words, low words, one scale a block)
* ``gemv_i8x2``  I2, two-word int8 activations (two exact block dots a block)
* ``add_rmsnorm``  N, forward_shim.rs module doc (add_norm)
* ``route``      R, fn emit_moe_forward (softmax, keep K, renormalise)
* ``moe``        M, fn emit_moe_forward / struct MoeWeights
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(os.path.join(_HERE, "q8s_oracle.c")):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB)
    lib.oracle_gemv_f32.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p]
    lib.oracle_quantize.argtypes = [_p, _i64, _i64, _p, _p]
    lib.oracle_block_dots.argtypes = [_p, _i64, _i64, _p, _i64, _p]
    lib.oracle_gemv_i8.argtypes = [_p, _p, _i64, _i64, _p, _p, _i64, _p]
    lib.oracle_quantize_x2.argtypes = [_p, _i64, _i64, _p, _p, _p]
    lib.oracle_gemv_i8x2.argtypes = [_p, _p, _i64, _i64, _p, _p, _p, _i64, _p]
    lib.oracle_add_rmsnorm.argtypes = [_p, _p, _p, _i64, _i64, ctypes.c_float, _p, _p]
    lib.oracle_route.argtypes = [_p, _p, _i64, _i64, _i64, _i64, _p, _p, _p]
    lib.oracle_route_q8.argtypes = [ctypes.c_int, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _p, _p, _p]
    lib.oracle_route_q8x.argtypes = [ctypes.c_int, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _p, _p, _p]
    lib.oracle_moe.argtypes = [ctypes.c_int, _p, _p, _p, _p, _p, _p, _p, _p,
                               _i64, _i64, _i64, _i64, _i64, _p, _p, _p, _p]
    lib.oracle_moe.restype = ctypes.c_int
    lib.oracle_moe_shared.argtypes = [ctypes.c_int] + [_p] * 16 + [_i64] * 6 + [_p] * 4
    lib.oracle_moe_shared.restype = ctypes.c_int
    _lib = lib
    return lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _finite(*arrays):
    """The oracle is defined on finite values only: NaN and infinity in an
    activation, a router row or a scale have no reading on the pages, so it
    refuses them rather than rank or sum them."""
    for a in arrays:
        if a is not None and a.dtype.kind == "f":
            assert np.all(np.isfinite(a)), "oracle inputs must be finite"


def _check_q8(Wq, Ws, n_in):
    assert n_in % 32 == 0, "n_in must be a multiple of 32"
    assert Wq.shape[1] == n_in and Ws.shape == (Wq.shape[0], n_in // 32)


def gemv_f32(Wq, Ws, x):
    """y[m, n_out] (float64) = dequant(W) @ x[m, n_in]^T."""
    Wq = _c(Wq, np.int8); Ws = _c(Ws, np.float32)
    x = _c(np.atleast_2d(x), np.float32)
    _finite(Ws, x)
    n_out, n_in = Wq.shape
    _check_q8(Wq, Ws, n_in)
    assert x.shape[1] == n_in
    y = np.empty((x.shape[0], n_out), np.float64)
    _load().oracle_gemv_f32(_ptr(Wq), _ptr(Ws), n_out, n_in, _ptr(x), x.shape[0], _ptr(y))
    return y


def quantize(v):
    """Q8_0 quantise rows of v[rows, n]: returns (q int8 [rows, n], d f32 [rows, n/32])."""
    v = _c(np.atleast_2d(v), np.float32)
    _finite(v)
    rows, n = v.shape
    assert n % 32 == 0
    q = np.empty((rows, n), np.int8)
    d = np.empty((rows, n // 32), np.float32)
    _load().oracle_quantize(_ptr(v), rows, n, _ptr(q), _ptr(d))
    return q, d


def block_dots(Wq, xq):
    """isum[m, n_out, n_in/32] (int32) of the int8 mode."""
    Wq = _c(Wq, np.int8); xq = _c(np.atleast_2d(xq), np.int8)
    n_out, n_in = Wq.shape
    assert xq.shape[1] == n_in and n_in % 32 == 0
    isum = np.empty((xq.shape[0], n_out, n_in // 32), np.int32)
    _load().oracle_block_dots(_ptr(Wq), n_out, n_in, _ptr(xq), xq.shape[0], _ptr(isum))
    return isum


def gemv_i8(Wq, Ws, xq, xs):
    """y[m, n_out] (float64) of the one-word int8 mode from quantised rows."""
    Wq = _c(Wq, np.int8); Ws = _c(Ws, np.float32)
    xq = _c(np.atleast_2d(xq), np.int8); xs = _c(np.atleast_2d(xs), np.float32)
    _finite(Ws, xs)
    n_out, n_in = Wq.shape
    _check_q8(Wq, Ws, n_in)
    assert xq.shape[1] == n_in and xs.shape == (xq.shape[0], n_in // 32)
    y = np.empty((xq.shape[0], n_out), np.float64)
    _load().oracle_gemv_i8(_ptr(Wq), _ptr(Ws), n_out, n_in, _ptr(xq), _ptr(xs), xq.shape[0], _ptr(y))
    return y


def quantize_x2(v):
    """Two-word quantise rows of v[rows, n]: returns (q int8 [rows, n], lo int8
    [rows, n], d f32 [rows, n/32]), v ~= d * (q + lo/128) per block."""
    v = _c(np.atleast_2d(v), np.float32)
    _finite(v)
    rows, n = v.shape
    assert n % 32 == 0
    q = np.empty((rows, n), np.int8)
    lo = np.empty((rows, n), np.int8)
    d = np.empty((rows, n // 32), np.float32)
    _load().oracle_quantize_x2(_ptr(v), rows, n, _ptr(q), _ptr(lo), _ptr(d))
    return q, lo, d


def gemv_i8x2(Wq, Ws, xq, xl, xs):
    """y[m, n_out] (float64) of the two-word int8 mode from quantised rows."""
    Wq = _c(Wq, np.int8); Ws = _c(Ws, np.float32)
    xq = _c(np.atleast_2d(xq), np.int8); xl = _c(np.atleast_2d(xl), np.int8)
    xs = _c(np.atleast_2d(xs), np.float32)
    _finite(Ws, xs)
    n_out, n_in = Wq.shape
    _check_q8(Wq, Ws, n_in)
    assert xq.shape[1] == n_in and xl.shape == xq.shape and xs.shape == (xq.shape[0], n_in // 32)
    y = np.empty((xq.shape[0], n_out), np.float64)
    _load().oracle_gemv_i8x2(_ptr(Wq), _ptr(Ws), n_out, n_in, _ptr(xq), _ptr(xl), _ptr(xs), xq.shape[0], _ptr(y))
    return y


def add_rmsnorm(h, r, w, eps):
    """Returns (sum f32 [rows, d], y float64 [rows, d])."""
    h = _c(np.atleast_2d(h), np.float32); r = _c(np.atleast_2d(r), np.float32)
    w = _c(w, np.float32)
    _finite(h, r, w)
    rows, d = h.shape
    assert r.shape == h.shape and w.shape == (d,)
    s = np.empty((rows, d), np.float32)
    y = np.empty((rows, d), np.float64)
    _load().oracle_add_rmsnorm(_ptr(h), _ptr(r), _ptr(w), rows, d, float(eps), _ptr(s), _ptr(y))
    return s, y


def route(x, Wr, k):
    """Returns (idx int32 [rows, k], wts float64 [rows, k], logits float64 [rows, E])."""
    x = _c(np.atleast_2d(x), np.float32); Wr = _c(Wr, np.float32)
    _finite(x, Wr)
    rows, d = x.shape
    E = Wr.shape[0]
    assert Wr.shape == (E, d) and 1 <= k <= E
    idx = np.empty((rows, k), np.int32)
    wts = np.empty((rows, k), np.float64)
    logits = np.empty((rows, E), np.float64)
    _load().oracle_route(_ptr(x), _ptr(Wr), rows, d, E, k, _ptr(idx), _ptr(wts), _ptr(logits))
    return idx, wts, logits


def route_q8(Wrq, Wrs, k, x=None, xq=None, xs=None, xl=None):
    """The router over Q8_0 rows (E rows of d): logits are the Q8_0 GEMV of
    `x` (float activations), of `xq`/`xs` (int8 activations, one word each) or
    of `xq`/`xl`/`xs` (two words), then the softmax top-K of `route`.  Returns
    (idx int32 [rows, k], wts float64 [rows, k], logits float64 [rows, E])."""
    Wrq = _c(Wrq, np.int8); Wrs = _c(Wrs, np.float32)
    _finite(Wrs, None if x is None else np.asarray(x), None if xs is None else np.asarray(xs))
    E, d = Wrq.shape
    act = 0 if x is not None else (2 if xl is not None else 1)
    if act == 0:
        x = _c(np.atleast_2d(x), np.float32)
        rows = x.shape[0]
        assert x.shape == (rows, d)
        xq_p = xs_p = None
        x_p = _ptr(x)
    else:
        xq = _c(np.atleast_2d(xq), np.int8); xs = _c(np.atleast_2d(xs), np.float32)
        rows = xq.shape[0]
        assert xq.shape == (rows, d) and xs.shape == (rows, d // 32)
        x_p = None
        xq_p, xs_p = _ptr(xq), _ptr(xs)
    assert Wrs.shape == (E, d // 32) and d % 32 == 0 and 1 <= k <= E
    idx = np.empty((rows, k), np.int32)
    wts = np.empty((rows, k), np.float64)
    logits = np.empty((rows, E), np.float64)
    xl_p = None
    if act == 2:
        xl = _c(np.atleast_2d(xl), np.int8)
        assert xl.shape == xq.shape
        xl_p = _ptr(xl)
    _load().oracle_route_q8x(act, x_p, xq_p, xl_p, xs_p, _ptr(Wrq), _ptr(Wrs), rows, d, E, k,
                             _ptr(idx), _ptr(wts), _ptr(logits))
    return idx, wts, logits


def moe(x, Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds, k, act):
    """The MoE FFN block.  Returns (idx, wts, h f32 [rows, k, dff], y float64 [rows, d])."""
    x = _c(np.atleast_2d(x), np.float32); Wr = _c(Wr, np.float32)
    Wgq = _c(Wgq, np.int8); Wgs = _c(Wgs, np.float32)
    Wuq = _c(Wuq, np.int8); Wus = _c(Wus, np.float32)
    Wdq = _c(Wdq, np.int8); Wds = _c(Wds, np.float32)
    _finite(x, Wr, Wgs, Wus, Wds)
    rows, d = x.shape
    E = Wr.shape[0]
    dff = Wgq.shape[0] // E
    assert Wgq.shape == (E * dff, d) and Wuq.shape == (E * dff, d)
    assert Wdq.shape == (E * d, dff) and d % 32 == 0 and dff % 32 == 0
    assert Wgs.shape == (E * dff, d // 32) and Wus.shape == Wgs.shape and Wds.shape == (E * d, dff // 32)
    idx = np.empty((rows, k), np.int32)
    wts = np.empty((rows, k), np.float64)
    h = np.empty((rows, k, dff), np.float32)
    y = np.empty((rows, d), np.float64)
    rc = _load().oracle_moe(int(act), _ptr(x), _ptr(Wr), _ptr(Wgq), _ptr(Wgs), _ptr(Wuq), _ptr(Wus),
                            _ptr(Wdq), _ptr(Wds), rows, d, dff, E, k, _ptr(idx), _ptr(wts), _ptr(h), _ptr(y))
    assert rc == 0, "oracle_moe: unknown activation mode"
    return idx, wts, h, y


def moe_shared(x, Wgq, Wgs, Wuq, Wus, Wdq, Wds, k, act, Wr=None, Wrq=None, Wrs=None, shared=None):
    """The MoE FFN block with its variants: the router as float rows ``Wr``
    or Q8_0 rows ``Wrq``/``Wrs``; ``shared`` = (Sgq, Sgs, Suq, Sus, Sdq, Sds)
    an always-on expert added unweighted.  Returns (idx, wts, h f32
    [rows, k*dff + sdff], y float64 [rows, d])."""
    x = _c(np.atleast_2d(x), np.float32)
    Wgq = _c(Wgq, np.int8); Wgs = _c(Wgs, np.float32)
    Wuq = _c(Wuq, np.int8); Wus = _c(Wus, np.float32)
    Wdq = _c(Wdq, np.int8); Wds = _c(Wds, np.float32)
    _finite(x, Wgs, Wus, Wds, None if Wr is None else np.asarray(Wr), None if Wrs is None else np.asarray(Wrs))
    rows, d = x.shape
    assert (Wr is None) != (Wrq is None)
    if Wr is not None:
        Wr = _c(Wr, np.float32)
        E = Wr.shape[0]
        assert Wr.shape == (E, d)
    else:
        Wrq = _c(Wrq, np.int8); Wrs = _c(Wrs, np.float32)
        E = Wrq.shape[0]
        assert Wrq.shape == (E, d) and Wrs.shape == (E, d // 32)
    dff = Wgq.shape[0] // E
    assert Wgq.shape == (E * dff, d) and Wuq.shape == (E * dff, d) and Wdq.shape == (E * d, dff)
    assert d % 32 == 0 and dff % 32 == 0 and 1 <= k <= E
    sp = [None] * 6
    sdff = 0
    if shared is not None:
        Sgq, Sgs, Suq, Sus, Sdq, Sds = shared
        sdff = Sgq.shape[0]
        assert sdff % 32 == 0 and Sgq.shape == (sdff, d) and Suq.shape == (sdff, d) and Sdq.shape == (d, sdff)
        assert Sgs.shape == (sdff, d // 32) and Sus.shape == Sgs.shape and Sds.shape == (d, sdff // 32)
        keep = [_c(Sgq, np.int8), _c(Sgs, np.float32), _c(Suq, np.int8), _c(Sus, np.float32),
                _c(Sdq, np.int8), _c(Sds, np.float32)]
        sp = [_ptr(a) for a in keep]
    idx = np.empty((rows, k), np.int32)
    wts = np.empty((rows, k), np.float64)
    h = np.empty((rows, k * dff + sdff), np.float32)
    y = np.empty((rows, d), np.float64)
    rc = _load().oracle_moe_shared(int(act), _ptr(x), _ptr(Wr) if Wr is not None else None,
                                   _ptr(Wrq) if Wrq is not None else None, _ptr(Wrs) if Wrs is not None else None,
                                   _ptr(Wgq), _ptr(Wgs), _ptr(Wuq), _ptr(Wus), _ptr(Wdq), _ptr(Wds), *sp,
                                   sdff, rows, d, dff, E, k, _ptr(idx), _ptr(wts), _ptr(h), _ptr(y))
    assert rc == 0, "oracle_moe_shared: unknown activation mode"
    return idx, wts, h, y
