"""The C ABI on the host: the library loads, exports every entry point that
include/q8s.h declares, and refuses bad arguments by naming the rule -- all
before any HIP call, so these run without a GPU (pointers here are fake,
never dereferenced)."""
import ctypes
import os
import re

import pytest

import q8_gemv_sparse_amd as q8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8s.h")
LIB = q8.library()

A = 0x10000  # fake, 16-byte aligned device addresses, far apart
B = 0x20000000
C = 0x40000000
D = 0x60000000
F = 0x80000000
G = 0xA0000000
H = 0xC0000000
J = 0xE0000000


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"Q8S_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) >= {"q8_gemv", "add_rmsnorm_q8", "moe_route_topk", "moe_gate_up", "moe_down_combine",
                          "q8_quantize_rows", "q8s_scratch_bytes", "q8s_last_error"}
    for n in names:
        assert hasattr(LIB, n), n
    assert q8.q8s_version().startswith("q8s")


def _err():
    return q8.q8s_last_error()


def gemv(n_out=64, n_in=64, m=1, act=0, Wq=A, Ws=B, x=C, xq=D, xs=F, y=G):
    return LIB.q8_gemv(Wq, Ws, n_out, n_in, x, xq, xs, m, y, act, None)


def test_gemv_refusals():
    assert gemv(n_in=48) == -1 and "multiple of 32" in _err()
    assert gemv(n_in=0) == -1
    assert gemv(n_out=0) == -1 and "n_out" in _err()
    assert gemv(m=0) == -1
    assert gemv(act=2) == -2 and "two-word" in _err()
    assert gemv(act=7) == -2 and "unknown activation" in _err()
    assert gemv(x=None) == -1 and "`x` is null" in _err()
    assert gemv(act=1, xq=None) == -1 and "`xq` is null" in _err()
    assert gemv(Wq=A + 8) == -3 and "16-byte aligned" in _err()
    assert gemv(n_in=65536 * 2) == -2 and "longest row" in _err()
    # output overlapping an input: y placed inside x
    assert gemv(y=C + 64) == -1 and "overlaps input `x`" in _err()


def test_quantize_refusals():
    assert LIB.q8_quantize_rows(A, 2, 40, B, C, None) == -1 and "multiple of 32" in _err()
    assert LIB.q8_quantize_rows(A, 2, 64, A + 256, C, None) == -1 and "overlaps" in _err()


def norm(rows=1, d=64, eps=1e-6, h=A, r=B, w=C, s=D, y=F, yq=G, ys=H):
    return LIB.add_rmsnorm_q8(h, r, w, rows, d, ctypes.c_float(eps), s, y, yq, ys, None)


def test_norm_refusals():
    assert norm(d=20) == -1
    assert norm(yq=None) == -1 and "together" in _err()
    assert norm(y=None, yq=None, ys=None) == -1 and "neither" in _err()
    assert norm(eps=-1.0) == -1 and "eps" in _err()
    assert norm(eps=float("nan")) == -1
    assert norm(s=None) == -1 and "`sum` is null" in _err()
    assert norm(y=A) == -1 and "overlaps input `h`" in _err()
    assert norm(y=D) == -1 and "outputs `sum` and `y` overlap" in _err()


def norm_x2(rows=1, d=64, eps=1e-6, h=A, r=B, w=C, s=D, y=F, yq=G, yl=H, ys=J):
    return LIB.add_rmsnorm_q8_x2(h, r, w, rows, d, ctypes.c_float(eps), s, y, yq, yl, ys, None)


def test_norm_x2_refusals():
    assert norm_x2(d=20) == -1 and "multiple of 32" in _err()
    assert norm_x2(yl=None) == -1 and "`yl` is null" in _err()
    assert norm_x2(yq=None) == -1 and "`yq` is null" in _err()
    assert norm_x2(s=None) == -1 and "`sum` is null" in _err()
    assert norm_x2(eps=-1.0) == -1 and "eps" in _err()
    assert norm_x2(yl=G + 32) == -1 and "overlap" in _err()
    assert norm_x2(y=A) == -1 and "overlaps input `h`" in _err()


def route(rows=1, d=64, E=8, k=2, sb=None, scratch=J, x=A, Wr=B, idx=C, wts=D):
    if sb is None:
        sb = q8.q8s_scratch_bytes(q8.FN_ROUTE, rows, d, 32, E, k)
    return LIB.moe_route_topk(x, Wr, rows, d, E, k, idx, wts, scratch, sb, None)


def test_route_refusals_and_scratch():
    assert q8.q8s_scratch_bytes(q8.FN_ROUTE, 1, 2048, 768, 128, 8) >= 128 * 8  # the f64 logits
    assert q8.q8s_scratch_bytes(99, 1, 2048, 768, 128, 8) == 0
    assert route(k=0) == -1 and "1 <= k <= E" in _err()
    assert route(k=9) == -1
    assert route(E=64, k=33) == -2 and "32 experts kept" in _err()
    assert route(E=8193, k=8) == -2
    assert route(d=100) == -1
    assert route(sb=8) == -4 and "scratch" in _err()
    assert route(scratch=None) == -4
    assert route(scratch=J + 16) == -3 and "256-byte" in _err()
    assert route(scratch=A) == -1 and "overlaps input `x`" in _err()


def gate_up(act=0, rows=1, d=64, dff=64, E=4, k=2, x=A, xq=A, xs=B, h=J, hq=H, hs=0xF0000000):
    return LIB.moe_gate_up(x, xq, xs, C, D, F, G, 0xD0000000, rows, d, dff, E, k, h, hq, hs, act, None)


def route_gemv(rows=8, d=64, E=8, k=2, n_out=32, act=1, xl=None, sb=None, scratch=0x100000000, x=A, Wr=B, idx=C,
               wts=D, Dq=F, Ds=G, xq=H, xs=J, y=0x110000000):
    if sb is None:
        sb = q8.q8s_scratch_bytes(q8.FN_ROUTE, rows, d, 32, E, k)
    return LIB.moe_route_topk_gemv(x, Wr, rows, d, E, k, idx, wts, Dq, Ds, n_out, xq, xl, xs, y, act, scratch, sb,
                                   None)


def test_route_gemv_refusals():
    assert route_gemv(act=0) == -2 and "Q8_0 form" in _err()
    assert route_gemv(act=3) == -1
    assert route_gemv(act=1, xl=0x120000000) == -1 and "`xl`" in _err()
    assert route_gemv(act=2) == -1 and "`xl`" in _err()
    assert route_gemv(k=9) == -1 and "1 <= k <= E" in _err()
    assert route_gemv(n_out=0) == -1
    assert route_gemv(d=40) == -1 and "multiple of 32" in _err()
    assert route_gemv(sb=8) == -4 and "scratch" in _err()
    assert route_gemv(y=H) == -1 and "overlaps input `xq`" in _err()


def test_gate_up_refusals():
    assert gate_up(dff=48) == -1 and "dff" in _err()
    assert gate_up(k=5) == -1
    assert gate_up(act=1, xq=None) == -1 and "`xq` is null" in _err()
    assert gate_up(act=1, hq=None) == -1 and "`hq` is null" in _err()
    assert gate_up(act=0, h=None) == -1 and "`h` is null" in _err()
    assert gate_up(act=2) == -2
    assert gate_up(h=C) == -1 and "overlaps input `Wgq`" in _err()
    # several int8 rows stage the float32 hidden rows in h
    assert gate_up(act=1, rows=2, h=None) == -1 and "`h` is required" in _err()


def test_down_refusals():
    assert q8.q8s_scratch_bytes(q8.FN_DOWN, 1, 64, 64, 4, 2) == 0  # a decode row needs none
    assert q8.q8s_scratch_bytes(q8.FN_DOWN, 4, 64, 64, 4, 2, q8.ACT_F32) == 0  # f32 rows run one by one
    need = q8.q8s_scratch_bytes(q8.FN_DOWN, 4, 64, 64, 4, 2, q8.ACT_INT8)
    assert need >= 4 * 2 * 64 * 4  # a chunk's per-choice results
    r = LIB.moe_down_combine(None, A, B, C, D, F, J, 4, 64, 64, 4, 2, G, 1, None, 0, None)
    assert r == -4 and "scratch" in _err()
    r = LIB.moe_down_combine(None, A, B, C, D, F, J, 4, 64, 64, 4, 2, G, 1, 0x30000008, need, None)
    assert r == -3 and "256-byte" in _err()
    r = LIB.moe_down_combine(A, None, None, B, C, D, F, 1, 64, 64, 4, 2, A, 0, None, 0, None)
    assert r == -1 and "overlaps" in _err()
    r = LIB.moe_down_combine(None, A, None, B, C, D, F, 1, 64, 64, 4, 2, G, 1, None, 0, None)
    assert r == -1 and "`hs` is null" in _err()


def block(act=0, rows=1, d=64, dff=64, E=4, k=2, eps=1e-6, sb=None, scratch=0x3000000, **over):
    # inputs h r w Wr Wgq Wgs Wuq Wus Wdq Wds, outputs sum idx wts out: 1 MiB apart
    names = ["h", "r", "w", "Wr", "Wgq", "Wgs", "Wuq", "Wus", "Wdq", "Wds", "sum", "idx", "wts", "out"]
    p = {n: 0x100000 * (i + 1) for i, n in enumerate(names)}
    p.update(over)
    if sb is None:
        sb = q8.q8s_scratch_bytes(q8.FN_BLOCK, rows, d, dff, E, k, act)
    return LIB.moe_ffn_block(p["h"], p["r"], p["w"], ctypes.c_float(eps), p["Wr"], p["Wgq"], p["Wgs"], p["Wuq"],
                             p["Wus"], p["Wdq"], p["Wds"], rows, d, dff, E, k, p["sum"], p["idx"], p["wts"], p["out"],
                             act, scratch, sb, None)


def test_block_scratch_and_refusals():
    # the logits, the normed row, the hidden rows: at least their bytes
    f32 = q8.q8s_scratch_bytes(q8.FN_BLOCK, 1, 2048, 768, 128, 8, q8.ACT_F32)
    assert f32 >= 128 * 8 + 2048 * 4 + 8 * 768 * 4
    i8 = q8.q8s_scratch_bytes(q8.FN_BLOCK, 1, 2048, 768, 128, 8, q8.ACT_INT8)
    assert i8 >= 128 * 8 + 2048 * (4 + 1) + 8 * 768 * (1 + 4 / 32)
    # a chunk in int8 also holds the down-combine's per-choice results
    chunk = q8.q8s_scratch_bytes(q8.FN_BLOCK, 64, 2048, 768, 128, 8, q8.ACT_INT8)
    assert chunk >= q8.q8s_scratch_bytes(q8.FN_DOWN, 64, 2048, 768, 128, 8, q8.ACT_INT8) + 64 * 128 * 8
    assert block(k=0) == -1 and "1 <= k <= E" in _err()
    assert block(d=40) == -1 and "multiple of 32" in _err()
    assert block(act=3) == -2 and "unknown activation" in _err()
    assert block(eps=-1.0) == -1 and "eps" in _err()
    assert block(Wr=None) == -1 and "`Wr` is null" in _err()
    assert block(out=0x100000 * 14 + 8) == -3 and "16-byte" in _err()
    assert block(sb=64) == -4 and "scratch" in _err()
    assert block(scratch=None) == -4
    assert block(scratch=0x3000010) == -3 and "256-byte" in _err()
    assert block(out=0x100000 * 1) == -1 and "overlaps input `h`" in _err()
    assert block(scratch=0x100000 * 11) == -1 and "overlap" in _err()


def norm_router(rows=1, d=64, E=4, eps=1e-6, h=A, r=B, w=C, Wr=D, s=F, x=G, xq=H, xs=J, logits=0x30000000):
    return LIB.add_rmsnorm_router(h, r, w, ctypes.c_float(eps), Wr, rows, d, E, s, x, xq, xs, logits, None)


def test_norm_router_refusals():
    assert norm_router(d=8192 + 32) == -2 and "add_rmsnorm_q8 then moe_route_topk" in _err()
    assert norm_router(E=0) == -1
    assert norm_router(xs=None) == -1 and "together" in _err()
    assert norm_router(x=None, xq=None, xs=None) == -1 and "neither" in _err()
    assert norm_router(logits=None) == -1 and "`logits` is null" in _err()
    assert norm_router(logits=A + 64) == -1 and "overlaps input `h`" in _err()
    assert norm_router(eps=float("inf")) == -1 or norm_router(eps=-2.0) == -1


def topk_gate_up(act=0, rows=1, d=64, dff=64, E=4, k=2, logits=A, x=B, xq=B, xs=C, h=J, hq=H, hs=0xF0000000):
    return LIB.moe_topk_gate_up(logits, x, xq, xs, D, F, G, 0x30000000, rows, d, dff, E, k, 0x38000000, 0x3C000000,
                                h, hq, hs, act, None)


def test_topk_gate_up_refusals():
    assert topk_gate_up(E=257, k=2) == -2 and "moe_route_topk then moe_gate_up" in _err()
    assert topk_gate_up(k=5) == -1
    assert topk_gate_up(logits=None) == -1 and "`logits` is null" in _err()
    assert topk_gate_up(act=1, hq=None) == -1 and "`hq` is null" in _err()
    assert topk_gate_up(act=0, h=None) == -1 and "`h` is null" in _err()
    assert topk_gate_up(h=B) == -1 and "overlaps input" in _err()


def norm_gemv(act=0, rows=1, d=64, n_out=64, eps=1e-6, h=A, r=B, w=C, Wq=D, Ws=F, s=G, y=H, yq=J, ys=0x30000000,
              out=0x38000000):
    return LIB.add_rmsnorm_gemv(h, r, w, ctypes.c_float(eps), Wq, Ws, rows, d, n_out, s, y, yq, ys, out, act, None)


def test_norm_gemv_refusals():
    assert norm_gemv(d=48) == -1 and "multiple of 32" in _err()
    assert norm_gemv(act=0, y=None) == -1 and "`y` is required" in _err()
    assert norm_gemv(act=1, yq=None, ys=None) == -1 and "`yq`/`ys` are required" in _err()
    assert norm_gemv(ys=None) == -1 and "together" in _err()
    assert norm_gemv(eps=-1.0) == -1 and "eps" in _err()
    assert norm_gemv(out=None) == -1 and "`out` is null" in _err()
    assert norm_gemv(out=D + 64) == -1 and "overlaps input `Wq`" in _err()
    assert norm_gemv(act=2) == -2


def route_q8(act=0, rows=1, d=64, E=4, k=2, x=A, xq=A, xs=B, Wrq=C, Wrs=D, idx=F, wts=G, scratch=0x30000000,
             sb=None):
    if sb is None:
        sb = q8.q8s_scratch_bytes(q8.FN_ROUTE, rows, d, 32, E, k)
    return LIB.moe_route_topk_q8(x, xq, xs, Wrq, Wrs, rows, d, E, k, idx, wts, act, scratch, sb, None)


def test_route_q8_refusals():
    assert route_q8(k=5) == -1 and "1 <= k <= E" in _err()
    assert route_q8(d=48) == -1 and "multiple of 32" in _err()
    assert route_q8(act=2) == -2 and "two-word" in _err()
    assert route_q8(x=None) == -1 and "`x` is null" in _err()
    assert route_q8(act=1, xq=None) == -1 and "`xq` is null" in _err()
    assert route_q8(Wrs=None) == -1 and "`Wrs` is null" in _err()
    assert route_q8(sb=8) == -4 and "scratch" in _err()
    assert route_q8(scratch=0x30000010) == -3 and "256-byte" in _err()
    assert route_q8(idx=C + 32) == -1 and "overlaps input `Wrq`" in _err()


def norm_router_q8(act=0, rows=1, d=64, E=4, eps=1e-6, Wrq=D, Wrs=0x34000000, x=G, xq=H, xs=J):
    return LIB.add_rmsnorm_router_q8(A, B, C, ctypes.c_float(eps), Wrq, Wrs, rows, d, E, F, x, xq, xs, 0x30000000,
                                     act, None)


def test_norm_router_q8_refusals():
    assert norm_router_q8(act=3) == -2 and "unknown activation" in _err()
    assert norm_router_q8(Wrq=None) == -1 and "`Wrq` is null" in _err()
    assert norm_router_q8(Wrs=None) == -1 and "`Wrs` is null" in _err()
    assert norm_router_q8(d=8192 + 32) == -2
    assert norm_router_q8(x=None, xq=None, xs=None) == -1 and "neither" in _err()
    assert norm_router_q8(x=D + 16) == -1 and "overlaps input `Wrq`" in _err()


def block_ex(act=0, rows=1, d=64, dff=64, sdff=0, E=4, k=2, eps=1e-6, sb=None, scratch=0x3000000, **over):
    names = ["h", "r", "w", "Wr", "Wrq", "Wrs", "Wgq", "Wgs", "Wuq", "Wus", "Wdq", "Wds",
             "Sgq", "Sgs", "Suq", "Sus", "Sdq", "Sds", "sum", "idx", "wts", "out"]
    p = {n: 0x100000 * (i + 1) for i, n in enumerate(names)}
    p["Wrq"] = p["Wrs"] = None
    if sdff == 0:
        for n in ("Sgq", "Sgs", "Suq", "Sus", "Sdq", "Sds"):
            p[n] = None
    p.update(over)
    if sb is None:
        sb = q8.q8s_block_scratch_bytes(rows, d, dff, sdff, E, k, act)
    return LIB.moe_ffn_block_ex(p["h"], p["r"], p["w"], ctypes.c_float(eps), p["Wr"], p["Wrq"], p["Wrs"], p["Wgq"],
                                p["Wgs"], p["Wuq"], p["Wus"], p["Wdq"], p["Wds"], p["Sgq"], p["Sgs"], p["Suq"],
                                p["Sus"], p["Sdq"], p["Sds"], sdff, rows, d, dff, E, k, p["sum"], p["idx"], p["wts"],
                                p["out"], act, scratch, sb, None)


def test_block_ex_scratch_and_refusals():
    # no shared expert: the same scratch as moe_ffn_block
    for act in (0, 1):
        for rows in (1, 64):
            assert q8.q8s_block_scratch_bytes(rows, 2048, 768, 0, 128, 8, act) == \
                q8.q8s_scratch_bytes(q8.FN_BLOCK, rows, 2048, 768, 128, 8, act)
    # a shared expert's hidden row: f32 values, or their Q8_0 form
    base = q8.q8s_block_scratch_bytes(1, 2048, 768, 0, 128, 8, 0)
    assert q8.q8s_block_scratch_bytes(1, 2048, 768, 1024, 128, 8, 0) >= base + 1024 * 4
    base = q8.q8s_block_scratch_bytes(64, 2048, 768, 0, 128, 8, 1)
    assert q8.q8s_block_scratch_bytes(64, 2048, 768, 1024, 128, 8, 1) >= base + 64 * 1024 * (1 + 4 / 32)
    assert q8.q8s_block_scratch_bytes(1, 2048, 768, -32, 128, 8, 0) == 0
    assert block_ex(Wr=None) == -1 and "exactly one" in _err()
    assert block_ex(Wrq=0x100000 * 5, Wrs=0x100000 * 6) == -1 and "exactly one" in _err()
    assert block_ex(Wr=None, Wrq=0x100000 * 5) == -1 and "`Wrs` is null" in _err()
    assert block_ex(sdff=48) == -1 and "sdff" in _err()
    assert block_ex(sdff=-32) == -1 and "negative" in _err()
    assert block_ex(Sgq=0x100000 * 13) == -1 and "sdff = 0" in _err()
    assert block_ex(sdff=64, Sds=None) == -1 and "`Sds` is null" in _err()
    assert block_ex(sdff=64, out=0x100000 * 17 + 64) == -1 and "overlaps input `Sdq`" in _err()
    # a shared expert too wide for the down-combine's partials
    assert block_ex(d=64, dff=65536, k=32, E=32, sdff=32) == -2 and "512" in _err()
    assert block_ex(sdff=64, sb=64) == -4 and "scratch" in _err()


def test_shared_stage_refusals():
    # moe_topk_gate_up_ex: logits x xq xs Wgq Wgs Wuq Wus Sgq Sgs Suq Sus sdff rows d dff E k idx wts h hq hs act
    def gu(sdff=64, Sgq=0x31000000, act=0, h=J, **kw):
        a = dict(rows=1, d=64, dff=64, E=4, k=2)
        a.update(kw)
        return LIB.moe_topk_gate_up_ex(A, B, B, C, D, F, G, 0x30000000, Sgq, 0x32000000, 0x33000000, 0x34000000,
                                       sdff, a["rows"], a["d"], a["dff"], a["E"], a["k"], 0x38000000, 0x3C000000,
                                       h, H, 0xF0000000, act, None)
    assert gu(sdff=40) == -1 and "sdff" in _err()
    assert gu(sdff=0) == -1 and "sdff = 0" in _err()
    assert gu(Sgq=None) == -1 and "`Sgq` is null" in _err()
    assert gu(E=257) == -2 and "moe_route_topk then moe_gate_up" in _err()
    assert gu(h=0x33000000 + 64) == -1 and "overlaps input `Suq`" in _err()
    # moe_down_combine_ex: h hq hs Wdq Wds Sdq Sds sdff idx wts rows d dff E k y act
    def dn(sdff=64, Sdq=0x31000000, y=G, act=0):
        return LIB.moe_down_combine_ex(A, None, None, B, C, Sdq, 0x32000000, sdff, D, F, 1, 64, 64, 4, 2, y, act,
                                       None)
    assert dn(sdff=-32) == -1 and "negative" in _err()
    assert dn(Sdq=None) == -1 and "`Sdq` is null" in _err()
    assert dn(y=0x31000000) == -1 and "overlaps input `Sdq`" in _err()
    assert dn(act=1) == -1 and "`hq` is null" in _err()


def test_stream_read_refusals():
    assert LIB.q8s_stream_read(A, 0, B, None) == -1 and "multiple of 16" in _err()
    assert LIB.q8s_stream_read(A, 40, B, None) == -1 and "multiple of 16" in _err()
    assert LIB.q8s_stream_read(None, 64, B, None) == -1 and "`buf` is null" in _err()
    assert LIB.q8s_stream_read(A + 4, 64, B, None) == -3
    assert LIB.q8s_stream_read(A, 1 << 20, A + 4096, None) == -1 and "overlaps" in _err()


def test_two_word_refusals():
    # the quantiser: whole blocks, disjoint outputs
    assert LIB.q8_quantize_rows_x2(A, 2, 40, B, C, D, None) == -1 and "multiple of 32" in _err()
    assert LIB.q8_quantize_rows_x2(A, 2, 64, B, B + 64, D, None) == -1 and "overlap" in _err()
    assert LIB.q8_quantize_rows_x2(A, 2, 64, B, None, D, None) == -1 and "`xl` is null" in _err()
    # the GEMV: every array present and aligned, whole blocks
    gemv2 = lambda n_out=64, n_in=64, m=1, xq=D, xl=F, xs=G, y=H: LIB.q8_gemv_x2(A, B, n_out, n_in, xq, xl, xs, m, y,
                                                                                 None)
    assert gemv2(xl=None) == -1 and "`xl` is null" in _err()
    assert gemv2(n_in=48) == -1 and "multiple of 32" in _err()
    assert gemv2(m=0) == -1
    assert gemv2(xq=D + 8) == -3
    assert gemv2(y=F + 16) == -1 and "overlaps input `xl`" in _err()
    # the one-word entry points name the two-word ones
    assert gemv(act=2) == -2 and "q8_gemv_x2" in _err()


def test_norm_gemv_x2_refusals():
    f = lambda d=64, yl=J, y=F, eps=1e-6: LIB.add_rmsnorm_gemv_x2(A, B, C, ctypes.c_float(eps), D, 0xF0000000, 1, d,
                                                                   64, G, y, H, yl, 0xD0000000, 0xB0000000, None)
    assert f(yl=None) == -1 and "`yl` is null" in _err()
    assert f(y=None) == -1 and "`y` is null" in _err()
    assert f(d=40) == -1 and "multiple of 32" in _err()
    assert f(eps=-1.0) == -1 and "eps" in _err()


def test_block_two_word_limits():
    # two words: the float router without a shared expert, E <= 256, d <= 8192
    blk = lambda E=4, d=64, act=2: LIB.moe_ffn_block(A, B, C, ctypes.c_float(1e-6), D, F, G, H, J, 0xB0000000,
                                                      0xC8000000, 1, d, 64, E, 2, 0xD0000000, 0xD8000000,
                                                      0xE8000000, 0xF0000000, act, 0xF8000000, 1 << 24, None)
    assert blk(E=300) == -2 and "two-word" in _err()
    assert blk(d=16384) == -2 and "two-word" in _err()
    assert blk(act=3) == -2
    # the stage calls stay one-word
    assert gate_up(act=2) == -2 and "two-word" in _err()


def test_block_scratch_holds_the_two_word_rows():
    # two words need the one-word arrays (x and the hidden rows in Q8_0 form)
    # plus their low words; a scratch sized for float32 rows would leave the
    # int8 arrays unplaced
    al = lambda n: -(-n // 256) * 256
    for rows, d, dff, E, k in ((1, 2048, 768, 128, 8), (1, 96, 160, 5, 3)):  # decode rows (no chunk scratch)
        one = q8.q8s_scratch_bytes(q8.FN_BLOCK, rows, d, dff, E, k, q8.ACT_INT8)
        two = q8.q8s_scratch_bytes(q8.FN_BLOCK, rows, d, dff, E, k, 2)
        assert two == one + al(rows * d) + al(rows * k * dff)


def test_gate_up_without_q8_form_only_for_chunks():
    # one row (the decode kernels quantise in their epilogue): hq/hs required
    assert gate_up(act=1, rows=1, hq=None, hs=None) == -1 and "only a chunk" in _err()
    # a chunk may leave both out, not one of them
    assert gate_up(act=1, rows=4, hq=None) == -1 and "`hq` is null" in _err()


def test_block_noalloc_refusals_before_any_hip_call():
    # the allocation-free block refuses shapes and sizes beyond its static
    # scratch before touching a device (fake pointers, never dereferenced)
    f = LIB.moe_ffn_block_noalloc

    def call(rows=1, d=2048, dff=768, E=128, k=8, act=1):
        return f(A, A + 0x1000000, A + 0x2000000, ctypes.c_float(1e-6), B, C, D, F, G, H, J, rows, d, dff, E, k,
                 0x8000000, 0x9000000, 0xA000000, 0xB000000, act, None)
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_float] + [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 5 + \
        [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p]
    assert call(rows=512) == -2 and "static scratch holds" in _err()
    assert q8.q8s_scratch_bytes(q8.FN_BLOCK, 512, 2048, 768, 128, 8, 1) > q8.NOALLOC_SCRATCH_BYTES
    assert call(act=3) == -2 and "unknown activation" in _err()
    assert call(k=0) == -1 and "1 <= k <= E" in _err()
    assert call(d=40) == -1 and "multiple of 32" in _err()


def test_stack_refusals_before_any_hip_call():
    f = LIB.moe_ffn_stack
    P = ctypes.c_void_p
    f.argtypes = [P, P, ctypes.c_int64] + [P] * 8 + [ctypes.c_int64] * 5 + [ctypes.c_float, P, P, P, ctypes.c_int, P,
                                                                          ctypes.c_size_t, P]
    d, dff, E, k, rows = 256, 96, 8, 2, 1
    need = q8.q8s_scratch_bytes(q8.FN_STACK, rows, d, dff, E, k, 1)
    assert need >= q8.q8s_scratch_bytes(q8.FN_BLOCK, rows, d, dff, E, k, 1) + 3 * rows * d * 4

    def arrays(L, hole=None):
        out = []
        for i in range(8):  # w, Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds of each layer, far apart
            vals = [0x1000000 * (1 + 8 * l + i) for l in range(L)]
            if hole == (i, 1):
                vals[1] = 0
            out.append((P * L)(*vals))
        return out

    def call(L=2, hole=None, arrs=None, sb=None, out=0x7000000000, scratch=0x7100000000):
        a = arrs if arrs is not None else arrays(L, hole)
        return f(0x6000000000, 0x6100000000, L, *a, rows, d, dff, E, k, ctypes.c_float(1e-6), out,
                 0x7200000000, 0x7300000000, 1, scratch, need if sb is None else sb, None)
    assert call(L=0) == -1 and "layers" in _err()
    assert call(L=2000) == -2 and "1024" in _err()
    assert call(hole=(2, 1)) == -1 and "`Wgq[1]` is null" in _err()
    nulls = arrays(2)
    nulls[5] = None
    assert call(arrs=nulls) == -1 and "pointer array" in _err()
    assert call(sb=64) == -4 and "scratch" in _err()
    assert call(scratch=0x7100000010) == -3 and "256-byte" in _err()
    assert call(out=0x1000000 * 2) == -1 and "overlaps input `Wr[0]`" in _err()


def test_two_word_stage_refusals_before_any_hip_call():
    P = ctypes.c_void_p
    gu = LIB.moe_gate_up_x2
    gu.argtypes = [P] * 8 + [ctypes.c_int64] * 5 + [P] * 5
    dn = LIB.moe_down_combine_x2
    dn.argtypes = [P] * 7 + [ctypes.c_int64] * 5 + [P, P, ctypes.c_size_t, P]
    base = [0x1000000 * (i + 1) for i in range(8)]  # xq, xl, xs, Wgq, Wgs, Wuq, Wus, idx

    def g(rows=1, d=256, dff=96, E=8, k=2, h=None, hq=0x20000000, hl=0x21000000, hs=0x22000000):
        return gu(*base, rows, d, dff, E, k, h, hq, hl, hs, None)
    assert g(rows=4) == -1 and "`h` is required" in _err()
    assert g(hq=None, hl=None, hs=None) == -1 and "hq`/`hl`/`hs` are required" in _err()
    assert g(d=40) == -1 and "multiple of 32" in _err()
    assert g(hl=None) == -1 and "`hl` is null" in _err()
    need = q8.q8s_scratch_bytes(q8.FN_DOWN, 4, 256, 96, 8, 2, q8.ACT_X2)
    assert need >= 4 * 2 * 256 * 4  # the per-choice results of a chunk

    def dcall(rows=4, sb=None, scratch=0x30000000):
        return dn(*[0x1000000 * (i + 1) for i in range(7)], rows, 256, 96, 8, 2, 0x40000000, scratch,
                  need if sb is None else sb, None)
    assert dcall(sb=64) == -4 and "per-choice" in _err()
    assert dcall(scratch=0x30000010) == -3
    assert dcall(rows=0) == -1


def test_moe_path_rule():
    # which kernels the mixture's expert stages run: one row or float32
    # activations row by row; chunks grouped by expert, on the matrix cores
    # from 8 choices an expert with d, dff multiples of 256 whose 16 staged
    # rows fit 64 KiB
    path = q8.q8s_moe_path
    R, G, M = q8.PATH_ROWS, q8.PATH_GROUPED, q8.PATH_GROUPED_MFMA
    assert path(1, 2048, 768, 128, 8, 1) == R
    assert path(64, 2048, 768, 128, 8, 0) == R
    assert path(64, 4096, 768, 128, 8, 1) == R          # d past the grouped kernels
    assert path(64, 2048, 768, 128, 8, 1) == G          # 4 choices an expert
    assert path(127, 2048, 768, 128, 8, 1) == G         # 7.9
    assert path(128, 2048, 768, 128, 8, 1) == M         # 8
    assert path(256, 2048, 768, 128, 8, 2) == M         # two words, 32 KiB rows of 2048
    assert path(128, 1056, 768, 128, 8, 1) == G         # d not a multiple of 256
    assert path(150, 128, 96, 2, 1, 1) == G             # rows of 128
    assert path(40, 512, 4096, 4, 2, 1) == M            # 16 rows of 4096 = 64 KiB
    assert path(40, 512, 4096, 4, 2, 2) == G            # twice that in two words
    # the GPU tests' wide cases take the matrix cores
    for rows, E, k, d, dff in [(150, 2, 1, 256, 256), (200, 3, 3, 512, 256), (70, 5, 2, 256, 512),
                               (32, 4, 2, 2048, 512), (40, 4, 2, 512, 4096), (12, 2, 2, 256, 256)]:
        assert path(rows, d, dff, E, k, 1) == M
    for d, dff, E, k, rows in [(2048, 768, 128, 8, 128), (256, 256, 2, 1, 150), (512, 2048, 4, 2, 40)]:
        assert path(rows, d, dff, E, k, 2) == M
    for bad in [(0, 64, 64, 2, 1, 1), (2, 64, 64, 2, 3, 1), (2, 64, 64, 2, 1, 3), (2, 64, 0, 2, 1, 1)]:
        with pytest.raises(q8.Q8sError):
            path(*bad)
