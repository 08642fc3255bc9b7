"""Python binding of libq8s.so, the Q8_0 GEMV / sparse-MoE library for MI355X.

The functions carry the C entry points' names (include/q8s.h) and only
marshal arguments: they check that tensors are contiguous device tensors of
the right dtype, read sizes off their shapes, pass ``data_ptr()`` and the
current HIP stream, and raise ``Q8sError`` with the library's message when a
call is refused.  Every step of the computation runs in the HIP kernels;
there is no fallback.  PyTorch supplies device memory and streams only.

Importing this package loads ``libq8s.so`` from this directory and fails
loudly if it has not been built (``python q8_gemv_sparse_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "ACT_F32", "ACT_INT8", "FN_ROUTE", "FN_DOWN", "FN_BLOCK", "Q8sError", "LIB_PATH",
    "q8_gemv", "q8_quantize_rows", "add_rmsnorm_q8", "moe_route_topk",
    "moe_gate_up", "moe_down_combine", "moe_ffn_block", "add_rmsnorm_router", "moe_topk_gate_up",
    "add_rmsnorm_gemv", "moe_route_topk_q8", "add_rmsnorm_router_q8", "moe_ffn_block_ex",
    "moe_topk_gate_up_ex", "moe_down_combine_ex",
    "q8s_scratch_bytes", "q8s_block_scratch_bytes", "q8s_last_error",
    "q8s_version", "q8s_stream_read", "STREAM_WGS", "library", "q8_quantize_rows_x2", "q8_gemv_x2",
    "add_rmsnorm_gemv_x2", "moe_topk_gate_up_x2", "ACT_X2", "moe_ffn_block_noalloc", "NOALLOC_SCRATCH_BYTES",
    "moe_ffn_stack", "FN_STACK", "moe_gate_up_x2", "moe_down_combine_x2", "q8s_moe_path", "PATH_ROWS",
    "PATH_GROUPED", "PATH_GROUPED_MFMA", "moe_route_topk_gemv", "add_rmsnorm_q8_x2",
]

ACT_F32 = 0
ACT_INT8 = 1
ACT_X2 = 2  # two-word int8 activations (the *_x2 calls, and moe_ffn_block)
FN_ROUTE = 1
FN_DOWN = 2
FN_BLOCK = 3
FN_STACK = 4
PATH_ROWS = 0          # q8s_moe_path: the decode kernels, row by row
PATH_GROUPED = 1       # choices grouped by expert, on the vector units
PATH_GROUPED_MFMA = 2  # choices grouped by expert, on the matrix cores
STREAM_WGS = 2048  # Q8S_STREAM_WGS: words q8s_stream_read writes
NOALLOC_SCRATCH_BYTES = 32 << 20  # Q8S_NOALLOC_SCRATCH_BYTES: moe_ffn_block_noalloc's static scratch per GPU

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libq8s.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libq8s.so is not built at %s; build it with `python q8_gemv_sparse_amd/build.py`" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)
_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t

_SIGS = {
    "q8_gemv": [_p, _p, _i64, _i64, _p, _p, _p, _i64, _p, ctypes.c_int, _p],
    "q8_quantize_rows": [_p, _i64, _i64, _p, _p, _p],
    "add_rmsnorm_q8": [_p, _p, _p, _i64, _i64, ctypes.c_float, _p, _p, _p, _p, _p],
    "add_rmsnorm_q8_x2": [_p, _p, _p, _i64, _i64, ctypes.c_float, _p, _p, _p, _p, _p, _p],
    "moe_route_topk": [_p, _p, _i64, _i64, _i64, _i64, _p, _p, _p, _sz, _p],
    "moe_route_topk_gemv": [_p, _p, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _i64, _p, _p, _p, _p, ctypes.c_int, _p,
                            _sz, _p],
    "moe_gate_up": [_p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _p, _p, _p, ctypes.c_int, _p],
    "moe_down_combine": [_p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _p, ctypes.c_int, _p, _sz, _p],
    "moe_ffn_block": [_p, _p, _p, ctypes.c_float, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _p, _p,
                      _p, _p, ctypes.c_int, _p, _sz, _p],
    "moe_gate_up_x2": [_p] * 8 + [_i64] * 5 + [_p] * 5,
    "moe_down_combine_x2": [_p] * 7 + [_i64] * 5 + [_p, _p, _sz, _p],
    "moe_ffn_stack": [_p, _p, _i64] + [_p] * 8 + [_i64] * 5 + [ctypes.c_float, _p, _p, _p, ctypes.c_int, _p, _sz, _p],
    "moe_ffn_block_noalloc": [_p, _p, _p, ctypes.c_float, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64,
                              _p, _p, _p, _p, ctypes.c_int, _p],
    "add_rmsnorm_gemv": [_p, _p, _p, ctypes.c_float, _p, _p, _i64, _i64, _i64, _p, _p, _p, _p, _p, ctypes.c_int, _p],
    "add_rmsnorm_router": [_p, _p, _p, ctypes.c_float, _p, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p],
    "moe_topk_gate_up": [_p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _p,
                         ctypes.c_int, _p],
    "moe_route_topk_q8": [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _p, _p, ctypes.c_int, _p, _sz, _p],
    "add_rmsnorm_router_q8": [_p, _p, _p, ctypes.c_float, _p, _p, _i64, _i64, _i64, _p, _p, _p, _p, _p,
                              ctypes.c_int, _p],
    "moe_ffn_block_ex": [_p, _p, _p, ctypes.c_float] + [_p] * 15 + [_i64] * 6 + [_p] * 4 + [ctypes.c_int, _p, _sz,
                                                                                           _p],
    "moe_topk_gate_up_ex": [_p] * 12 + [_i64] * 6 + [_p] * 5 + [ctypes.c_int, _p],
    "moe_down_combine_ex": [_p] * 7 + [_i64, _p, _p] + [_i64] * 5 + [_p, ctypes.c_int, _p],
    "q8s_scratch_bytes": [ctypes.c_int, _i64, _i64, _i64, _i64, _i64, ctypes.c_int],
    "q8s_block_scratch_bytes": [_i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int],
    "q8s_moe_path": [_i64, _i64, _i64, _i64, _i64, ctypes.c_int],
    "q8s_stream_read": [_p, _i64, _p, _p],
    "q8_quantize_rows_x2": [_p, _i64, _i64, _p, _p, _p, _p],
    "q8_gemv_x2": [_p, _p, _i64, _i64, _p, _p, _p, _i64, _p, _p],
    "add_rmsnorm_gemv_x2": [_p, _p, _p, ctypes.c_float, _p, _p, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p],
    "moe_topk_gate_up_x2": [_p] * 8 + [_i64] * 5 + [_p] * 5 + [_p],
}
for _name, _args in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_int
_lib.q8s_scratch_bytes.restype = _sz
_lib.q8s_block_scratch_bytes.restype = _sz
_lib.q8s_last_error.restype = ctypes.c_char_p
_lib.q8s_last_error.argtypes = []
_lib.q8s_version.restype = ctypes.c_char_p
_lib.q8s_version.argtypes = []


def library():
    """The loaded ctypes library (for callers that marshal raw pointers)."""
    return _lib


class Q8sError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("q8s error %d: %s" % (code, msg))
        self.code = code


def q8s_last_error():
    return _lib.q8s_last_error().decode()


def q8s_version():
    return _lib.q8s_version().decode()


def q8s_scratch_bytes(fn, rows, d, dff, E, k, act=ACT_F32):
    return int(_lib.q8s_scratch_bytes(fn, rows, d, dff, E, k, act))


def q8s_block_scratch_bytes(rows, d, dff, sdff, E, k, act=ACT_F32):
    return int(_lib.q8s_block_scratch_bytes(rows, d, dff, sdff, E, k, act))


def q8s_moe_path(rows, d, dff, E, k, act=ACT_INT8):
    """Which kernels the mixture's expert stages run for these sizes:
    PATH_ROWS, PATH_GROUPED or PATH_GROUPED_MFMA (host logic, no device call)."""
    rc = int(_lib.q8s_moe_path(rows, d, dff, E, k, act))
    if rc < 0:
        raise Q8sError(rc, "q8s_moe_path: invalid sizes")
    return rc


def q8s_stream_read(buf, out=None, nbytes=None, stream=None):
    """Reads ``nbytes`` (default: all) of the device tensor ``buf`` once with
    the library's plain streaming reader, writing one uint32 word per
    workgroup into ``out`` (int32 [STREAM_WGS]); returns ``out``.  A
    measuring stick, not part of the method."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise TypeError("buf must be a contiguous device tensor")
    n = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    if n > buf.numel() * buf.element_size():
        raise ValueError("nbytes exceeds the buffer")
    if out is None:
        out = torch.empty(STREAM_WGS, dtype=torch.int32, device=buf.device)
    out = _dev(out, torch.int32, "out")
    if out.numel() < STREAM_WGS:
        raise ValueError("out must hold STREAM_WGS words")
    _check(_lib.q8s_stream_read(buf.data_ptr(), n, out.data_ptr(), _stream(stream)))
    return out


def _check(rc):
    if rc != 0:
        raise Q8sError(rc, q8s_last_error())


def _dev(t, dtype, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def q8_gemv(Wq, Ws, x=None, xq=None, xs=None, y=None, act=ACT_F32, stream=None):
    """y[m, n_out] = Q8_0(Wq, Ws) @ activations; f32 ``x`` or Q8_0 ``xq``/``xs``."""
    _dev(Wq, torch.int8, "Wq"); _dev(Ws, torch.float32, "Ws")
    n_out, n_in = Wq.shape
    if act == ACT_F32:
        _dev(x, torch.float32, "x")
        m = x.numel() // n_in
    else:
        _dev(xq, torch.int8, "xq"); _dev(xs, torch.float32, "xs")
        m = xq.numel() // n_in
    if y is None:
        y = torch.empty((m, n_out), dtype=torch.float32, device=Wq.device)
    _dev(y, torch.float32, "y")
    _check(_lib.q8_gemv(_ptr(Wq), _ptr(Ws), n_out, n_in, _ptr(x), _ptr(xq), _ptr(xs), m, _ptr(y), act,
                        _stream(stream)))
    return y


def q8_quantize_rows(x, xq=None, xs=None, stream=None):
    """Q8_0 form of f32 rows ``x [rows, n]``: (xq int8 [rows, n], xs f32 [rows, n/32])."""
    _dev(x, torch.float32, "x")
    n = x.shape[-1]
    rows = x.numel() // n
    if xq is None:
        xq = torch.empty((rows, n), dtype=torch.int8, device=x.device)
    if xs is None:
        xs = torch.empty((rows, n // 32), dtype=torch.float32, device=x.device)
    _dev(xq, torch.int8, "xq"); _dev(xs, torch.float32, "xs")
    _check(_lib.q8_quantize_rows(_ptr(x), rows, n, _ptr(xq), _ptr(xs), _stream(stream)))
    return xq, xs


def q8_quantize_rows_x2(x, xq=None, xl=None, xs=None, stream=None):
    """Two-word Q8_0 form of x[rows, n]: returns (xq, xl, xs), the words, the
    low words and the block scales, x ~= xs * (xq + xl/128) per block."""
    _dev(x, torch.float32, "x")
    rows, n = x.shape
    if xq is None:
        xq = torch.empty((rows, n), dtype=torch.int8, device=x.device)
    if xl is None:
        xl = torch.empty((rows, n), dtype=torch.int8, device=x.device)
    if xs is None:
        xs = torch.empty((rows, n // 32), dtype=torch.float32, device=x.device)
    _dev(xq, torch.int8, "xq"); _dev(xl, torch.int8, "xl"); _dev(xs, torch.float32, "xs")
    _check(_lib.q8_quantize_rows_x2(x.data_ptr(), rows, n, xq.data_ptr(), xl.data_ptr(), xs.data_ptr(),
                                    _stream(stream)))
    return xq, xl, xs


def q8_gemv_x2(Wq, Ws, xq, xl, xs, y=None, stream=None):
    """y[m, n_out] = Q8_0 W times two-word int8 rows (xq, xl, xs)."""
    _dev(Wq, torch.int8, "Wq"); _dev(Ws, torch.float32, "Ws")
    _dev(xq, torch.int8, "xq"); _dev(xl, torch.int8, "xl"); _dev(xs, torch.float32, "xs")
    n_out, n_in = Wq.shape
    m = xq.shape[0]
    if y is None:
        y = torch.empty((m, n_out), dtype=torch.float32, device=Wq.device)
    _dev(y, torch.float32, "y")
    _check(_lib.q8_gemv_x2(Wq.data_ptr(), Ws.data_ptr(), n_out, n_in, xq.data_ptr(), xl.data_ptr(), xs.data_ptr(),
                           m, y.data_ptr(), _stream(stream)))
    return y


def add_rmsnorm_gemv_x2(h, r, w, eps, Wq, Ws, sum=None, y=None, yq=None, yl=None, ys=None, out=None, stream=None):
    """add_rmsnorm_q8 feeding q8_gemv_x2 (one launch for one row of d <=
    4096).  Returns (sum, y, yq, yl, ys, out)."""
    for t, n in ((h, "h"), (r, "r"), (w, "w"), (Ws, "Ws")):
        _dev(t, torch.float32, n)
    _dev(Wq, torch.int8, "Wq")
    rows, d = h.shape
    n_out = Wq.shape[0]
    f = lambda t, shape, dt: t if t is not None else torch.empty(shape, dtype=dt, device=h.device)
    sum = f(sum, (rows, d), torch.float32); y = f(y, (rows, d), torch.float32)
    yq = f(yq, (rows, d), torch.int8); yl = f(yl, (rows, d), torch.int8)
    ys = f(ys, (rows, d // 32), torch.float32); out = f(out, (rows, n_out), torch.float32)
    for t, n, dt in ((sum, "sum", torch.float32), (y, "y", torch.float32), (yq, "yq", torch.int8),
                     (yl, "yl", torch.int8), (ys, "ys", torch.float32), (out, "out", torch.float32)):
        _dev(t, dt, n)
    _check(_lib.add_rmsnorm_gemv_x2(h.data_ptr(), r.data_ptr(), w.data_ptr(), eps, Wq.data_ptr(), Ws.data_ptr(), rows,
                                    d, n_out, sum.data_ptr(), y.data_ptr(), yq.data_ptr(), yl.data_ptr(),
                                    ys.data_ptr(), out.data_ptr(), _stream(stream)))
    return sum, y, yq, yl, ys, out


def moe_topk_gate_up_x2(logits, Wgq, Wgs, Wuq, Wus, k, xq, xl, xs, idx=None, wts=None, hq=None, hl=None, hs=None,
                        stream=None):
    """The two-word mixture's gate-up launch: top-K from `logits` inside each
    workgroup, the two-word row (xq, xl, xs), hidden rows written in two words.
    Returns (idx, wts, hq, hl, hs)."""
    _dev(logits, torch.float64, "logits")
    for t, n in ((Wgq, "Wgq"), (Wuq, "Wuq"), (xq, "xq"), (xl, "xl")):
        _dev(t, torch.int8, n)
    for t, n in ((Wgs, "Wgs"), (Wus, "Wus"), (xs, "xs")):
        _dev(t, torch.float32, n)
    rows, E = logits.shape
    d = Wgq.shape[1]
    dff = Wgq.shape[0] // E
    dev = Wgq.device
    f = lambda t, shape, dt: t if t is not None else torch.empty(shape, dtype=dt, device=dev)
    idx = f(idx, (rows, k), torch.int32); wts = f(wts, (rows, k), torch.float32)
    hq = f(hq, (rows, k, dff), torch.int8); hl = f(hl, (rows, k, dff), torch.int8)
    hs = f(hs, (rows, k, dff // 32), torch.float32)
    _check(_lib.moe_topk_gate_up_x2(_ptr(logits), _ptr(xq), _ptr(xl), _ptr(xs), _ptr(Wgq), _ptr(Wgs), _ptr(Wuq),
                                    _ptr(Wus), rows, d, dff, E, k, _ptr(idx), _ptr(wts), _ptr(hq), _ptr(hl),
                                    _ptr(hs), _stream(stream)))
    return idx, wts, hq, hl, hs


def add_rmsnorm_q8(h, r, w, eps, sum=None, y=None, yq=None, ys=None, want_f32=True, want_q8=True, stream=None):
    """sum = h + r; y = RMSNorm(sum) * w; Q8_0(y).  Returns (sum, y or None, yq or None, ys or None)."""
    _dev(h, torch.float32, "h"); _dev(r, torch.float32, "r"); _dev(w, torch.float32, "w")
    d = h.shape[-1]
    rows = h.numel() // d
    dev = h.device
    if sum is None:
        sum = torch.empty((rows, d), dtype=torch.float32, device=dev)
    if want_f32 and y is None:
        y = torch.empty((rows, d), dtype=torch.float32, device=dev)
    if want_q8 and yq is None:
        yq = torch.empty((rows, d), dtype=torch.int8, device=dev)
        ys = torch.empty((rows, d // 32), dtype=torch.float32, device=dev)
    for t, dt, n in ((sum, torch.float32, "sum"), (y, torch.float32, "y"), (yq, torch.int8, "yq"),
                     (ys, torch.float32, "ys")):
        _dev(t, dt, n)
    _check(_lib.add_rmsnorm_q8(_ptr(h), _ptr(r), _ptr(w), rows, d, float(eps), _ptr(sum), _ptr(y), _ptr(yq),
                               _ptr(ys), _stream(stream)))
    return sum, y, yq, ys


def add_rmsnorm_q8_x2(h, r, w, eps, sum=None, y=None, yq=None, yl=None, ys=None, want_f32=True, stream=None):
    """sum = h + r; y = RMSNorm(sum) * w; its two-word form in the same launch.
    Returns (sum, y or None, yq, yl, ys)."""
    _dev(h, torch.float32, "h"); _dev(r, torch.float32, "r"); _dev(w, torch.float32, "w")
    d = h.shape[-1]
    rows = h.numel() // d
    f = lambda t, shape, dt: t if t is not None else torch.empty(shape, dtype=dt, device=h.device)
    sum = f(sum, (rows, d), torch.float32)
    if want_f32:
        y = f(y, (rows, d), torch.float32)
    yq = f(yq, (rows, d), torch.int8); yl = f(yl, (rows, d), torch.int8); ys = f(ys, (rows, d // 32), torch.float32)
    for t, dt, n in ((sum, torch.float32, "sum"), (y, torch.float32, "y"), (yq, torch.int8, "yq"),
                     (yl, torch.int8, "yl"), (ys, torch.float32, "ys")):
        _dev(t, dt, n)
    _check(_lib.add_rmsnorm_q8_x2(_ptr(h), _ptr(r), _ptr(w), rows, d, float(eps), _ptr(sum), _ptr(y), _ptr(yq),
                                  _ptr(yl), _ptr(ys), _stream(stream)))
    return sum, y, yq, yl, ys


def moe_route_topk(x, Wr, k, idx=None, wts=None, scratch=None, stream=None):
    """Router + top-K: (idx int32 [rows, k], wts f32 [rows, k]).  ``scratch`` is a
    uint8 device tensor of at least q8s_scratch_bytes(FN_ROUTE, ...) bytes (the
    logits); one is allocated when none is given."""
    _dev(x, torch.float32, "x"); _dev(Wr, torch.float32, "Wr")
    E, d = Wr.shape
    rows = x.numel() // d
    dev = x.device
    if idx is None:
        idx = torch.empty((rows, k), dtype=torch.int32, device=dev)
    if wts is None:
        wts = torch.empty((rows, k), dtype=torch.float32, device=dev)
    if scratch is None:
        scratch = torch.empty(q8s_scratch_bytes(FN_ROUTE, rows, d, 32, E, k), dtype=torch.uint8, device=dev)
    _dev(idx, torch.int32, "idx"); _dev(wts, torch.float32, "wts"); _dev(scratch, torch.uint8, "scratch")
    _check(_lib.moe_route_topk(_ptr(x), _ptr(Wr), rows, d, E, k, _ptr(idx), _ptr(wts), _ptr(scratch),
                               scratch.numel(), _stream(stream)))
    return idx, wts


def moe_route_topk_gemv(x, Wr, k, Dq, Ds, xq, xs, xl=None, idx=None, wts=None, y=None, scratch=None, stream=None):
    """moe_route_topk(x, Wr, k) and the dense projection of the same rows' Q8_0
    form (q8_gemv in one word, or q8_gemv_x2 when the low words ``xl`` are
    given) in one call: (idx, wts, y)."""
    _dev(x, torch.float32, "x"); _dev(Wr, torch.float32, "Wr")
    _dev(Dq, torch.int8, "Dq"); _dev(Ds, torch.float32, "Ds")
    _dev(xq, torch.int8, "xq"); _dev(xs, torch.float32, "xs")
    if xl is not None:
        _dev(xl, torch.int8, "xl")
    E, d = Wr.shape
    rows = x.numel() // d
    n_out = Dq.shape[0]
    dev = x.device
    f = lambda t, shape, dt: t if t is not None else torch.empty(shape, dtype=dt, device=dev)
    idx = f(idx, (rows, k), torch.int32); wts = f(wts, (rows, k), torch.float32)
    y = f(y, (rows, n_out), torch.float32)
    if scratch is None:
        scratch = torch.empty(q8s_scratch_bytes(FN_ROUTE, rows, d, 32, E, k), dtype=torch.uint8, device=dev)
    _dev(idx, torch.int32, "idx"); _dev(wts, torch.float32, "wts"); _dev(y, torch.float32, "y")
    _dev(scratch, torch.uint8, "scratch")
    act = ACT_X2 if xl is not None else ACT_INT8
    _check(_lib.moe_route_topk_gemv(_ptr(x), _ptr(Wr), rows, d, E, k, _ptr(idx), _ptr(wts), _ptr(Dq), _ptr(Ds),
                                    n_out, _ptr(xq), _ptr(xl), _ptr(xs), _ptr(y), act, _ptr(scratch),
                                    scratch.numel(), _stream(stream)))
    return idx, wts, y


def moe_gate_up(Wgq, Wgs, Wuq, Wus, idx, E, x=None, xq=None, xs=None, h=None, hq=None, hs=None, act=ACT_F32,
                want_h=True, want_q8=True, stream=None):
    """h[rows, k, dff] = SiLU(Wg[e] x) * (Wu[e] x) for each kept expert e.
    Returns (h, hq, hs): INT8 also writes the hidden row's Q8_0 form; h may be
    skipped there for one row (want_h=False); with several rows it is the
    chunk kernels' staging and is always written, and want_q8=False leaves
    out the Q8_0 form (hq, hs returned None)."""
    for t, n in ((Wgq, "Wgq"), (Wuq, "Wuq")):
        _dev(t, torch.int8, n)
    for t, n in ((Wgs, "Wgs"), (Wus, "Wus")):
        _dev(t, torch.float32, n)
    _dev(idx, torch.int32, "idx")
    rows, k = idx.shape
    d = Wgq.shape[1]
    dff = Wgq.shape[0] // E
    dev = Wgq.device
    if act == ACT_F32:
        _dev(x, torch.float32, "x")
    else:
        _dev(xq, torch.int8, "xq"); _dev(xs, torch.float32, "xs")
        if hq is None and want_q8:
            hq = torch.empty((rows, k, dff), dtype=torch.int8, device=dev)
        if hs is None and want_q8:
            hs = torch.empty((rows, k, dff // 32), dtype=torch.float32, device=dev)
    if h is None and (want_h or act == ACT_F32 or rows > 1):  # several int8 rows stage h
        h = torch.empty((rows, k, dff), dtype=torch.float32, device=dev)
    _dev(h, torch.float32, "h"); _dev(hq, torch.int8, "hq"); _dev(hs, torch.float32, "hs")
    _check(_lib.moe_gate_up(_ptr(x), _ptr(xq), _ptr(xs), _ptr(Wgq), _ptr(Wgs), _ptr(Wuq), _ptr(Wus), _ptr(idx),
                            rows, d, dff, E, k, _ptr(h), _ptr(hq), _ptr(hs), act, _stream(stream)))
    return h, hq, hs


def moe_down_combine(Wdq, Wds, idx, wts, E, h=None, hq=None, hs=None, y=None, act=ACT_F32, scratch=None,
                     stream=None):
    """y[rows, d] = sum_j wts[:, j] * (Wd[idx[:, j]] @ h[:, j]); INT8 reads hq/hs."""
    _dev(Wdq, torch.int8, "Wdq"); _dev(Wds, torch.float32, "Wds")
    _dev(idx, torch.int32, "idx"); _dev(wts, torch.float32, "wts")
    rows, k = idx.shape
    dff = Wdq.shape[1]
    d = Wdq.shape[0] // E
    dev = Wdq.device
    if act == ACT_F32:
        _dev(h, torch.float32, "h")
    else:
        _dev(hq, torch.int8, "hq"); _dev(hs, torch.float32, "hs")
    if y is None:
        y = torch.empty((rows, d), dtype=torch.float32, device=dev)
    _dev(y, torch.float32, "y")
    need = q8s_scratch_bytes(FN_DOWN, rows, d, dff, E, k, act)
    if need and scratch is None:
        scratch = torch.empty(need, dtype=torch.uint8, device=dev)
    _dev(scratch, torch.uint8, "scratch")
    _check(_lib.moe_down_combine(_ptr(h), _ptr(hq), _ptr(hs), _ptr(Wdq), _ptr(Wds), _ptr(idx), _ptr(wts), rows, d,
                                 dff, E, k, _ptr(y), act, _ptr(scratch), 0 if scratch is None else scratch.numel(),
                                 _stream(stream)))
    return y


def moe_ffn_block(h, r, w, eps, Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds, k, act=ACT_F32, sum=None, idx=None, wts=None,
                  out=None, scratch=None, stream=None):
    """The whole mixture block of a layer: sum = h + r, x = RMSNorm(sum) * w,
    then the router, top-K, gate-up and down-combine over x.  Returns
    (sum, idx, wts, out).  ``scratch`` is a uint8 device tensor of at least
    q8s_scratch_bytes(FN_BLOCK, ...) bytes; one is allocated when none is given."""
    for t, n in ((h, "h"), (r, "r"), (w, "w"), (Wr, "Wr"), (Wgs, "Wgs"), (Wus, "Wus"), (Wds, "Wds")):
        _dev(t, torch.float32, n)
    for t, n in ((Wgq, "Wgq"), (Wuq, "Wuq"), (Wdq, "Wdq")):
        _dev(t, torch.int8, n)
    E, d = Wr.shape
    rows = h.numel() // d
    dff = Wgq.shape[0] // E
    dev = h.device
    if sum is None:
        sum = torch.empty((rows, d), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((rows, k), dtype=torch.int32, device=dev)
    if wts is None:
        wts = torch.empty((rows, k), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((rows, d), dtype=torch.float32, device=dev)
    if scratch is None:
        scratch = torch.empty(max(q8s_scratch_bytes(FN_BLOCK, rows, d, dff, E, k, act), 1), dtype=torch.uint8,
                              device=dev)
    _dev(sum, torch.float32, "sum"); _dev(idx, torch.int32, "idx"); _dev(wts, torch.float32, "wts")
    _dev(out, torch.float32, "out"); _dev(scratch, torch.uint8, "scratch")
    _check(_lib.moe_ffn_block(_ptr(h), _ptr(r), _ptr(w), float(eps), _ptr(Wr), _ptr(Wgq), _ptr(Wgs), _ptr(Wuq),
                              _ptr(Wus), _ptr(Wdq), _ptr(Wds), rows, d, dff, E, k, _ptr(sum), _ptr(idx), _ptr(wts),
                              _ptr(out), act, _ptr(scratch), scratch.numel(), _stream(stream)))
    return sum, idx, wts, out


def moe_gate_up_x2(Wgq, Wgs, Wuq, Wus, idx, E, xq, xl, xs, h=None, hq=None, hl=None, hs=None, want_q8=True,
                   stream=None):
    """moe_gate_up in two-word numerics.  Returns (h or None, hq, hl, hs); a
    chunk of rows stages the float32 hidden rows in h (allocated when not
    given) and, with want_q8=False, leaves out their two-word form."""
    for t, n in ((Wgq, "Wgq"), (Wuq, "Wuq"), (xq, "xq"), (xl, "xl")):
        _dev(t, torch.int8, n)
    for t, n in ((Wgs, "Wgs"), (Wus, "Wus"), (xs, "xs")):
        _dev(t, torch.float32, n)
    _dev(idx, torch.int32, "idx")
    rows, k = idx.shape
    d = Wgq.shape[1]
    dff = Wgq.shape[0] // E
    dev = Wgq.device
    if h is None and rows > 1:
        h = torch.empty((rows, k, dff), dtype=torch.float32, device=dev)
    if want_q8:
        if hq is None:
            hq = torch.empty((rows, k, dff), dtype=torch.int8, device=dev)
        if hl is None:
            hl = torch.empty((rows, k, dff), dtype=torch.int8, device=dev)
        if hs is None:
            hs = torch.empty((rows, k, dff // 32), dtype=torch.float32, device=dev)
    _dev(h, torch.float32, "h"); _dev(hq, torch.int8, "hq"); _dev(hl, torch.int8, "hl"); _dev(hs, torch.float32, "hs")
    _check(_lib.moe_gate_up_x2(_ptr(xq), _ptr(xl), _ptr(xs), _ptr(Wgq), _ptr(Wgs), _ptr(Wuq), _ptr(Wus), _ptr(idx),
                               rows, d, dff, E, k, _ptr(h), _ptr(hq), _ptr(hl), _ptr(hs), _stream(stream)))
    return h, hq, hl, hs


def moe_down_combine_x2(Wdq, Wds, idx, wts, E, hq, hl, hs, y=None, scratch=None, stream=None):
    """moe_down_combine in two-word numerics: y[rows, d]."""
    _dev(Wdq, torch.int8, "Wdq"); _dev(Wds, torch.float32, "Wds")
    _dev(idx, torch.int32, "idx"); _dev(wts, torch.float32, "wts")
    _dev(hq, torch.int8, "hq"); _dev(hl, torch.int8, "hl"); _dev(hs, torch.float32, "hs")
    rows, k = idx.shape
    dff = Wdq.shape[1]
    d = Wdq.shape[0] // E
    dev = Wdq.device
    if y is None:
        y = torch.empty((rows, d), dtype=torch.float32, device=dev)
    _dev(y, torch.float32, "y")
    need = q8s_scratch_bytes(FN_DOWN, rows, d, dff, E, k, ACT_X2)
    if need and scratch is None:
        scratch = torch.empty(need, dtype=torch.uint8, device=dev)
    _dev(scratch, torch.uint8, "scratch")
    _check(_lib.moe_down_combine_x2(_ptr(hq), _ptr(hl), _ptr(hs), _ptr(Wdq), _ptr(Wds), _ptr(idx), _ptr(wts), rows,
                                    d, dff, E, k, _ptr(y), _ptr(scratch), 0 if scratch is None else scratch.numel(),
                                    _stream(stream)))
    return y


def moe_ffn_stack(h, r, layers, k, eps, act=ACT_F32, out=None, idx=None, wts=None, scratch=None, stream=None):
    """``len(layers)`` mixture blocks in a row: ``layers`` is a list of per-layer
    tuples (w, Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds) of device tensors.  Returns
    (out, idx [L, rows, k], wts [L, rows, k]); out is the residual stream after
    the last layer."""
    _dev(h, torch.float32, "h"); _dev(r, torch.float32, "r")
    L = len(layers)
    cols = list(zip(*layers)) if L else [()] * 8
    dts = (torch.float32, torch.float32, torch.int8, torch.float32, torch.int8, torch.float32, torch.int8,
           torch.float32)
    names = ("w", "Wr", "Wgq", "Wgs", "Wuq", "Wus", "Wdq", "Wds")
    for col, dt, nm in zip(cols, dts, names):
        for t in col:
            _dev(t, dt, nm)
    E, d = layers[0][1].shape
    dff = layers[0][2].shape[0] // E
    rows = h.numel() // d
    dev = h.device
    if out is None:
        out = torch.empty((rows, d), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((L, rows, k), dtype=torch.int32, device=dev)
    if wts is None:
        wts = torch.empty((L, rows, k), dtype=torch.float32, device=dev)
    if scratch is None:
        scratch = torch.empty(max(q8s_scratch_bytes(FN_STACK, rows, d, dff, E, k, act), 1), dtype=torch.uint8,
                              device=dev)
    _dev(out, torch.float32, "out"); _dev(idx, torch.int32, "idx"); _dev(wts, torch.float32, "wts")
    _dev(scratch, torch.uint8, "scratch")
    arrs = [(ctypes.c_void_p * L)(*[t.data_ptr() for t in col]) for col in cols]
    _check(_lib.moe_ffn_stack(_ptr(h), _ptr(r), L, *arrs, rows, d, dff, E, k, float(eps), _ptr(out), _ptr(idx),
                              _ptr(wts), act, _ptr(scratch), scratch.numel(), _stream(stream)))
    return out, idx, wts


def moe_ffn_block_noalloc(h, r, w, eps, Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds, k, sum, idx, wts, out, act=ACT_F32,
                          stream=None):
    """moe_ffn_block on the library's static scratch: no scratch argument and
    no allocation by the library.  The outputs are the caller's (sum, idx,
    wts, out, as moe_ffn_block); returns them."""
    for t, n in ((h, "h"), (r, "r"), (w, "w"), (Wr, "Wr"), (Wgs, "Wgs"), (Wus, "Wus"), (Wds, "Wds"),
                 (sum, "sum"), (wts, "wts"), (out, "out")):
        _dev(t, torch.float32, n)
    for t, n in ((Wgq, "Wgq"), (Wuq, "Wuq"), (Wdq, "Wdq")):
        _dev(t, torch.int8, n)
    _dev(idx, torch.int32, "idx")
    E, d = Wr.shape
    rows = h.numel() // d
    dff = Wgq.shape[0] // E
    _check(_lib.moe_ffn_block_noalloc(_ptr(h), _ptr(r), _ptr(w), float(eps), _ptr(Wr), _ptr(Wgq), _ptr(Wgs),
                                      _ptr(Wuq), _ptr(Wus), _ptr(Wdq), _ptr(Wds), rows, d, dff, E, k, _ptr(sum),
                                      _ptr(idx), _ptr(wts), _ptr(out), act, _stream(stream)))
    return sum, idx, wts, out


def add_rmsnorm_router(h, r, w, eps, Wr, sum=None, x=None, xq=None, xs=None, logits=None, want_f32=True,
                       want_q8=True, stream=None):
    """add_rmsnorm_q8 with the router's logits fused in.  Returns
    (sum, x or None, xq or None, xs or None, logits float64 [rows, E])."""
    _dev(h, torch.float32, "h"); _dev(r, torch.float32, "r"); _dev(w, torch.float32, "w")
    _dev(Wr, torch.float32, "Wr")
    E, d = Wr.shape
    rows = h.numel() // d
    dev = h.device
    if sum is None:
        sum = torch.empty((rows, d), dtype=torch.float32, device=dev)
    if want_f32 and x is None:
        x = torch.empty((rows, d), dtype=torch.float32, device=dev)
    if want_q8 and xq is None:
        xq = torch.empty((rows, d), dtype=torch.int8, device=dev)
        xs = torch.empty((rows, d // 32), dtype=torch.float32, device=dev)
    if logits is None:
        logits = torch.empty((rows, E), dtype=torch.float64, device=dev)
    for t, dt, n in ((sum, torch.float32, "sum"), (x, torch.float32, "x"), (xq, torch.int8, "xq"),
                     (xs, torch.float32, "xs"), (logits, torch.float64, "logits")):
        _dev(t, dt, n)
    _check(_lib.add_rmsnorm_router(_ptr(h), _ptr(r), _ptr(w), float(eps), _ptr(Wr), rows, d, E, _ptr(sum), _ptr(x),
                                   _ptr(xq), _ptr(xs), _ptr(logits), _stream(stream)))
    return sum, x, xq, xs, logits


def moe_topk_gate_up(logits, Wgq, Wgs, Wuq, Wus, k, x=None, xq=None, xs=None, idx=None, wts=None, h=None, hq=None,
                     hs=None, act=ACT_F32, want_h=True, stream=None):
    """moe_gate_up taking each row's top-K from ``logits`` itself.  Returns
    (idx, wts, h, hq, hs)."""
    _dev(logits, torch.float64, "logits")
    for t, n in ((Wgq, "Wgq"), (Wuq, "Wuq")):
        _dev(t, torch.int8, n)
    for t, n in ((Wgs, "Wgs"), (Wus, "Wus")):
        _dev(t, torch.float32, n)
    rows, E = logits.shape
    d = Wgq.shape[1]
    dff = Wgq.shape[0] // E
    dev = Wgq.device
    if idx is None:
        idx = torch.empty((rows, k), dtype=torch.int32, device=dev)
    if wts is None:
        wts = torch.empty((rows, k), dtype=torch.float32, device=dev)
    if act == ACT_F32:
        _dev(x, torch.float32, "x")
    else:
        _dev(xq, torch.int8, "xq"); _dev(xs, torch.float32, "xs")
        if hq is None:
            hq = torch.empty((rows, k, dff), dtype=torch.int8, device=dev)
        if hs is None:
            hs = torch.empty((rows, k, dff // 32), dtype=torch.float32, device=dev)
    if h is None and (want_h or act == ACT_F32):
        h = torch.empty((rows, k, dff), dtype=torch.float32, device=dev)
    _dev(idx, torch.int32, "idx"); _dev(wts, torch.float32, "wts")
    _dev(h, torch.float32, "h"); _dev(hq, torch.int8, "hq"); _dev(hs, torch.float32, "hs")
    _check(_lib.moe_topk_gate_up(_ptr(logits), _ptr(x), _ptr(xq), _ptr(xs), _ptr(Wgq), _ptr(Wgs), _ptr(Wuq),
                                 _ptr(Wus), rows, d, dff, E, k, _ptr(idx), _ptr(wts), _ptr(h), _ptr(hq), _ptr(hs), act,
                                 _stream(stream)))
    return idx, wts, h, hq, hs


def add_rmsnorm_gemv(h, r, w, eps, Wq, Ws, act=ACT_F32, sum=None, y=None, yq=None, ys=None, out=None,
                     want_f32=None, want_q8=None, stream=None):
    """add_rmsnorm_q8 feeding q8_gemv in one call.  Returns (sum, y or None,
    yq or None, ys or None, out).  By default the normed row is written in the
    form the projection reads (f32 for ACT_F32, Q8_0 for ACT_INT8)."""
    _dev(h, torch.float32, "h"); _dev(r, torch.float32, "r"); _dev(w, torch.float32, "w")
    _dev(Wq, torch.int8, "Wq"); _dev(Ws, torch.float32, "Ws")
    n_out, d = Wq.shape
    rows = h.numel() // d
    dev = h.device
    want_f32 = (act == ACT_F32) if want_f32 is None else want_f32
    want_q8 = (act == ACT_INT8) if want_q8 is None else want_q8
    if sum is None:
        sum = torch.empty((rows, d), dtype=torch.float32, device=dev)
    if want_f32 and y is None:
        y = torch.empty((rows, d), dtype=torch.float32, device=dev)
    if want_q8 and yq is None:
        yq = torch.empty((rows, d), dtype=torch.int8, device=dev)
        ys = torch.empty((rows, d // 32), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((rows, n_out), dtype=torch.float32, device=dev)
    for t, dt, n in ((sum, torch.float32, "sum"), (y, torch.float32, "y"), (yq, torch.int8, "yq"),
                     (ys, torch.float32, "ys"), (out, torch.float32, "out")):
        _dev(t, dt, n)
    _check(_lib.add_rmsnorm_gemv(_ptr(h), _ptr(r), _ptr(w), float(eps), _ptr(Wq), _ptr(Ws), rows, d, n_out, _ptr(sum),
                                 _ptr(y), _ptr(yq), _ptr(ys), _ptr(out), act, _stream(stream)))
    return sum, y, yq, ys, out


def moe_route_topk_q8(Wrq, Wrs, k, x=None, xq=None, xs=None, act=ACT_F32, idx=None, wts=None, scratch=None,
                      stream=None):
    """Router over Q8_0 rows + top-K: (idx int32 [rows, k], wts f32 [rows, k]).
    F32 reads ``x``; INT8 reads ``xq``/``xs``.  ``scratch`` as moe_route_topk."""
    _dev(Wrq, torch.int8, "Wrq"); _dev(Wrs, torch.float32, "Wrs")
    _dev(x, torch.float32, "x"); _dev(xq, torch.int8, "xq"); _dev(xs, torch.float32, "xs")
    E, d = Wrq.shape
    a = x if act == ACT_F32 else xq
    rows = a.numel() // d
    dev = Wrq.device
    if idx is None:
        idx = torch.empty((rows, k), dtype=torch.int32, device=dev)
    if wts is None:
        wts = torch.empty((rows, k), dtype=torch.float32, device=dev)
    if scratch is None:
        scratch = torch.empty(q8s_scratch_bytes(FN_ROUTE, rows, d, 32, E, k), dtype=torch.uint8, device=dev)
    _dev(idx, torch.int32, "idx"); _dev(wts, torch.float32, "wts"); _dev(scratch, torch.uint8, "scratch")
    _check(_lib.moe_route_topk_q8(_ptr(x), _ptr(xq), _ptr(xs), _ptr(Wrq), _ptr(Wrs), rows, d, E, k, _ptr(idx),
                                  _ptr(wts), act, _ptr(scratch), scratch.numel(), _stream(stream)))
    return idx, wts


def add_rmsnorm_router_q8(h, r, w, eps, Wrq, Wrs, act=ACT_F32, sum=None, x=None, xq=None, xs=None, logits=None,
                          want_f32=True, want_q8=True, stream=None):
    """add_rmsnorm_router over Q8_0 router rows.  Returns
    (sum, x or None, xq or None, xs or None, logits float64 [rows, E])."""
    _dev(h, torch.float32, "h"); _dev(r, torch.float32, "r"); _dev(w, torch.float32, "w")
    _dev(Wrq, torch.int8, "Wrq"); _dev(Wrs, torch.float32, "Wrs")
    E, d = Wrq.shape
    rows = h.numel() // d
    dev = h.device
    if sum is None:
        sum = torch.empty((rows, d), dtype=torch.float32, device=dev)
    if want_f32 and x is None:
        x = torch.empty((rows, d), dtype=torch.float32, device=dev)
    if want_q8 and xq is None:
        xq = torch.empty((rows, d), dtype=torch.int8, device=dev)
        xs = torch.empty((rows, d // 32), dtype=torch.float32, device=dev)
    if logits is None:
        logits = torch.empty((rows, E), dtype=torch.float64, device=dev)
    for t, dt, n in ((sum, torch.float32, "sum"), (x, torch.float32, "x"), (xq, torch.int8, "xq"),
                     (xs, torch.float32, "xs"), (logits, torch.float64, "logits")):
        _dev(t, dt, n)
    _check(_lib.add_rmsnorm_router_q8(_ptr(h), _ptr(r), _ptr(w), float(eps), _ptr(Wrq), _ptr(Wrs), rows, d, E,
                                      _ptr(sum), _ptr(x), _ptr(xq), _ptr(xs), _ptr(logits), act, _stream(stream)))
    return sum, x, xq, xs, logits


def moe_ffn_block_ex(h, r, w, eps, Wgq, Wgs, Wuq, Wus, Wdq, Wds, k, E, act=ACT_F32, Wr=None, Wrq=None, Wrs=None,
                     shared=None, sum=None, idx=None, wts=None, out=None, scratch=None, stream=None):
    """moe_ffn_block with the router as float rows ``Wr`` or Q8_0 rows
    ``Wrq``/``Wrs``, and ``shared`` = (Sgq, Sgs, Suq, Sus, Sdq, Sds), an
    always-on expert added unweighted (None: no shared expert).  Returns
    (sum, idx, wts, out).  ``scratch`` is a uint8 device tensor of at least
    q8s_block_scratch_bytes(...) bytes; one is allocated when none is given."""
    for t, n in ((h, "h"), (r, "r"), (w, "w"), (Wr, "Wr"), (Wrs, "Wrs"), (Wgs, "Wgs"), (Wus, "Wus"), (Wds, "Wds")):
        _dev(t, torch.float32, n)
    for t, n in ((Wrq, "Wrq"), (Wgq, "Wgq"), (Wuq, "Wuq"), (Wdq, "Wdq")):
        _dev(t, torch.int8, n)
    d = h.shape[-1]
    rows = h.numel() // d
    dff = Wgq.shape[0] // E
    sh = [None] * 6
    sdff = 0
    if shared is not None:
        sh = list(shared)
        for i, n in enumerate(("Sgq", "Sgs", "Suq", "Sus", "Sdq", "Sds")):
            _dev(sh[i], torch.int8 if i % 2 == 0 else torch.float32, n)
        sdff = sh[0].shape[0]
    dev = h.device
    if sum is None:
        sum = torch.empty((rows, d), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((rows, k), dtype=torch.int32, device=dev)
    if wts is None:
        wts = torch.empty((rows, k), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((rows, d), dtype=torch.float32, device=dev)
    if scratch is None:
        scratch = torch.empty(max(q8s_block_scratch_bytes(rows, d, dff, sdff, E, k, act), 1), dtype=torch.uint8,
                              device=dev)
    _dev(sum, torch.float32, "sum"); _dev(idx, torch.int32, "idx"); _dev(wts, torch.float32, "wts")
    _dev(out, torch.float32, "out"); _dev(scratch, torch.uint8, "scratch")
    _check(_lib.moe_ffn_block_ex(_ptr(h), _ptr(r), _ptr(w), float(eps), _ptr(Wr), _ptr(Wrq), _ptr(Wrs), _ptr(Wgq),
                                 _ptr(Wgs), _ptr(Wuq), _ptr(Wus), _ptr(Wdq), _ptr(Wds), *[_ptr(t) for t in sh], sdff,
                                 rows, d, dff, E, k, _ptr(sum), _ptr(idx), _ptr(wts), _ptr(out), act, _ptr(scratch),
                                 scratch.numel(), _stream(stream)))
    return sum, idx, wts, out


def _shared4(shared, names):
    if shared is None:
        return [None] * len(names), 0
    for t, n in zip(shared, names):
        _dev(t, torch.int8 if n.endswith("q") else torch.float32, n)
    return list(shared), shared[0].shape[0] if names[0] != "Sdq" else shared[0].shape[1]


def moe_topk_gate_up_ex(logits, Wgq, Wgs, Wuq, Wus, k, shared=None, x=None, xq=None, xs=None, idx=None, wts=None,
                        h=None, hq=None, hs=None, act=ACT_F32, want_h=True, stream=None):
    """moe_topk_gate_up with a shared expert's gate and up, ``shared`` =
    (Sgq, Sgs, Suq, Sus): the hidden rows hold k*dff + sdff values.  Returns
    (idx, wts, h or None, hq or None, hs or None)."""
    _dev(logits, torch.float64, "logits")
    for t, n in ((Wgs, "Wgs"), (Wus, "Wus"), (x, "x"), (xs, "xs")):
        _dev(t, torch.float32, n)
    for t, n in ((Wgq, "Wgq"), (Wuq, "Wuq"), (xq, "xq")):
        _dev(t, torch.int8, n)
    sh, sdff = _shared4(shared, ("Sgq", "Sgs", "Suq", "Sus"))
    rows, E = logits.shape
    d = Wgq.shape[1]
    dff = Wgq.shape[0] // E
    dev = logits.device
    hw = k * dff + sdff
    if idx is None:
        idx = torch.empty((rows, k), dtype=torch.int32, device=dev)
    if wts is None:
        wts = torch.empty((rows, k), dtype=torch.float32, device=dev)
    if (act == ACT_F32 or want_h) and h is None:
        h = torch.empty((rows, hw), dtype=torch.float32, device=dev)
    if act == ACT_INT8 and hq is None:
        hq = torch.empty((rows, hw), dtype=torch.int8, device=dev)
        hs = torch.empty((rows, hw // 32), dtype=torch.float32, device=dev)
    for t, dt, n in ((idx, torch.int32, "idx"), (wts, torch.float32, "wts"), (h, torch.float32, "h"),
                     (hq, torch.int8, "hq"), (hs, torch.float32, "hs")):
        _dev(t, dt, n)
    _check(_lib.moe_topk_gate_up_ex(_ptr(logits), _ptr(x), _ptr(xq), _ptr(xs), _ptr(Wgq), _ptr(Wgs), _ptr(Wuq),
                                    _ptr(Wus), *[_ptr(t) for t in sh], sdff, rows, d, dff, E, k, _ptr(idx),
                                    _ptr(wts), _ptr(h), _ptr(hq), _ptr(hs), act, _stream(stream)))
    return idx, wts, h, hq, hs


def moe_down_combine_ex(Wdq, Wds, idx, wts, E, shared=None, h=None, hq=None, hs=None, y=None, act=ACT_F32,
                        stream=None):
    """moe_down_combine with a shared expert's down row added, ``shared`` =
    (Sdq, Sds); h (or hq/hs) hold k*dff + sdff values a row.  Returns y."""
    _dev(Wdq, torch.int8, "Wdq"); _dev(Wds, torch.float32, "Wds")
    _dev(idx, torch.int32, "idx"); _dev(wts, torch.float32, "wts")
    _dev(h, torch.float32, "h"); _dev(hq, torch.int8, "hq"); _dev(hs, torch.float32, "hs")
    sh, sdff = _shared4(shared, ("Sdq", "Sds"))
    rows, k = idx.shape
    dff = Wdq.shape[1]
    d = Wdq.shape[0] // E
    if y is None:
        y = torch.empty((rows, d), dtype=torch.float32, device=Wdq.device)
    _dev(y, torch.float32, "y")
    _check(_lib.moe_down_combine_ex(_ptr(h), _ptr(hq), _ptr(hs), _ptr(Wdq), _ptr(Wds), *[_ptr(t) for t in sh], sdff,
                                    _ptr(idx), _ptr(wts), rows, d, dff, E, k, _ptr(y), act, _stream(stream)))
    return y
