"""The mixture's linked variants on the GPU -- the router as Q8_0 rows
(moe_route_topk_q8, add_rmsnorm_router_q8) and the shared expert
(moe_ffn_block_ex) -- against the oracle's route_q8 and moe_shared on the
same seeded inputs.

Tolerances as the other parity tests: 1e-5 (f32 numerics) and 2e-3 (int8
numerics) on the block's output; the sum and the routing choices bit-exact
(rows whose deciding logits are closer than double rounding can separate
are reported, and none of these seeds has one); logits to double rounding.
"""
import numpy as np
import pytest
import torch

import oracle
import q8_gemv_sparse_amd as q8
import synthetic
from gpu_helpers import dev, host, rel_err, route_ambiguous

pytestmark = pytest.mark.gpu

TOL = {0: 1e-5, 1: 2e-3}
EPS = 1e-6


def banner(msg):
    print("[case] " + msg, flush=True)


# ---------------------------------------------------------------------------
# the router over Q8_0 rows


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("rows,d,E,k", [
    (1, 2048, 128, 8),     # the 128-expert decode router
    (1, 4096, 8, 2),       # the 8-expert decode router
    (3, 96, 5, 3),         # ragged: 6 chunks, most threads idle
    (64, 2048, 128, 8),    # a 64-row chunk: tiles of 4 rows
    (5, 8192, 16, 4),      # two passes of 256 chunks; a ragged row tile
    (2, 256, 300, 6),      # past the top-K's LDS: arg-max rounds
])
def test_route_q8_matches_oracle(rows, d, E, k, act):
    banner("moe_route_topk_q8 rows=%d d=%d E=%d k=%d act=%d" % (rows, d, E, k, act))
    v = synthetic.variant_inputs(30, d, 64, E, k, rows)
    x = synthetic.normal(np.random.default_rng(31), rows, d)
    Wrq, Wrs = dev(v.Wrq), dev(v.Wrs)
    if act == 0:
        idx, wts = q8.moe_route_topk_q8(Wrq, Wrs, k, x=dev(x), act=0)
        ridx, rw, logits = oracle.route_q8(v.Wrq, v.Wrs, k, x=x)
    else:
        xq, xs = oracle.quantize(x)
        idx, wts = q8.moe_route_topk_q8(Wrq, Wrs, k, xq=dev(xq), xs=dev(xs), act=1)
        ridx, rw, logits = oracle.route_q8(v.Wrq, v.Wrs, k, xq=xq, xs=xs)
    assert not route_ambiguous(logits, k).any()
    assert np.array_equal(host(idx), ridx)
    assert rel_err(host(wts), rw) <= 1e-6


@pytest.mark.parametrize("act", [0, 1])
def test_route_q8_ties_go_to_the_lower_index(act):
    # identical router rows give exactly equal logits: ranks by index
    banner("moe_route_topk_q8 ties act=%d" % act)
    d, E, k = 256, 12, 5
    v = synthetic.variant_inputs(32, d, 64, E, k, 1)
    Wrq, Wrs = v.Wrq.copy(), v.Wrs.copy()
    for e in (3, 7, 9):
        Wrq[e], Wrs[e] = Wrq[2], Wrs[2]
    x = synthetic.normal(np.random.default_rng(33), 1, d)
    xq, xs = oracle.quantize(x)
    kw = dict(x=dev(x), act=0) if act == 0 else dict(xq=dev(xq), xs=dev(xs), act=1)
    idx, wts = q8.moe_route_topk_q8(dev(Wrq), dev(Wrs), k, **kw)
    okw = dict(x=x) if act == 0 else dict(xq=xq, xs=xs)
    ridx, rw, _ = oracle.route_q8(Wrq, Wrs, k, **okw)
    assert np.array_equal(host(idx), ridx)
    assert rel_err(host(wts), rw) <= 1e-6


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("rows,d,E", [(1, 2048, 128), (1, 4096, 8), (3, 96, 5), (2, 2080, 7), (1, 8192, 16)])
def test_norm_router_q8(rows, d, E, act):
    banner("add_rmsnorm_router_q8 rows=%d d=%d E=%d act=%d" % (rows, d, E, act))
    v = synthetic.variant_inputs(34, d, 64, E, 1, rows)
    b = v.block
    h, r, w = dev(b.h), dev(b.r), dev(b.w)
    s, x, xq, xs, logits = q8.add_rmsnorm_router_q8(h, r, w, EPS, dev(v.Wrq), dev(v.Wrs), act=act)
    s2, y2, q2, d2 = q8.add_rmsnorm_q8(h, r, w, EPS)
    for a, c in ((s, s2), (x, y2), (xq, q2), (xs, d2)):
        assert torch.equal(a, c)
    # the logits as the oracle forms them from that normed row (or its Q8_0
    # form), to double rounding of the sums
    okw = dict(x=host(x)) if act == 0 else dict(xq=host(xq), xs=host(xs))
    _, _, ref = oracle.route_q8(v.Wrq, v.Wrs, 1, **okw)
    W = v.Wrq.astype(np.float64) * np.repeat(v.Wrs.astype(np.float64), 32, axis=1)
    xx = host(x) if act == 0 else host(xq) * np.repeat(host(xs), 32, axis=1)
    mag = np.abs(xx.astype(np.float64)) @ np.abs(W).T
    assert np.all(np.abs(host(logits) - ref) <= 1e-13 * mag)
    # without xq requested, the int8 router still quantises the row itself
    _, _, q3, _, l3 = q8.add_rmsnorm_router_q8(h, r, w, EPS, dev(v.Wrq), dev(v.Wrs), act=act, want_q8=False)
    assert q3 is None and torch.equal(l3, logits)


# ---------------------------------------------------------------------------
# the whole block with its variants


def run_ex(v, act, q8_router, shared, scratch=None):
    b, m = v.block, v.block.moe
    W = [dev(a) for a in (m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds)]
    rk = dict(Wrq=dev(v.Wrq), Wrs=dev(v.Wrs)) if q8_router else dict(Wr=dev(m.Wr))
    sh = tuple(dev(a) for a in (v.Sgq, v.Sgs, v.Suq, v.Sus, v.Sdq, v.Sds)) if shared else None
    s, idx, wts, out = q8.moe_ffn_block_ex(dev(b.h), dev(b.r), dev(b.w), EPS, *W, m.k, m.E, act=act, shared=sh,
                                           scratch=scratch, **rk)
    return host(s), host(idx), host(wts), host(out)


def oracle_ex(v, act, q8_router, shared):
    b, m = v.block, v.block.moe
    s, y64 = oracle.add_rmsnorm(b.h, b.r, b.w, EPS)
    x = y64.astype(np.float32)
    rk = dict(Wrq=v.Wrq, Wrs=v.Wrs) if q8_router else dict(Wr=m.Wr)
    sh = (v.Sgq, v.Sgs, v.Suq, v.Sus, v.Sdq, v.Sds) if shared else None
    idx, wts, _, y = oracle.moe_shared(x, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, m.k, act, shared=sh, **rk)
    if q8_router:
        okw = dict(x=x) if act == 0 else dict(zip(("xq", "xs"), oracle.quantize(x)))
        _, _, logits = oracle.route_q8(v.Wrq, v.Wrs, m.k, **okw)
    else:
        _, _, logits = oracle.route(x, m.Wr, m.k)
    return s, idx, wts, y, logits


def check_ex(v, act, q8_router, shared, got):
    s, idx, wts, out = got
    rs, ridx, rw, ry, logits = oracle_ex(v, act, q8_router, shared)
    assert np.array_equal(s, rs)
    assert not route_ambiguous(logits, v.block.moe.k).any()
    assert np.array_equal(idx, ridx)
    assert rel_err(wts, rw) <= 1e-5
    for r in range(out.shape[0]):
        assert rel_err(out[r], ry[r]) <= TOL[act], r


EX_CASES = [
    # (d, dff, sdff, E, k, rows)
    (2048, 768, 0, 128, 8, 1),       # Q8_0 router alone, the 128-expert decode block
    (2048, 768, 1024, 128, 8, 1),    # + a shared expert wider than a slice of dff
    (2048, 768, 768, 128, 8, 1),     # a shared expert as wide as the routed ones
    (4096, 1408, 5632, 16, 4, 1),    # a shared expert four times dff, int8 rows in 4 slices
    (2048, 1408, 5632, 60, 4, 1),    # the 60-expert shared block: 352 int8 tiles, the 8-wave gate-up shape
    (96, 160, 96, 5, 3, 1),          # ragged lane groups of 16; sdff < dff
    (256, 64, 800, 6, 2, 3),         # 3 rows: per-row f32; int8 grouped chunk kernels + shared pass
    (128, 64, 128, 300, 4, 1),       # E > 256: separate norm, router, top-K, gate-up
    (16384, 64, 96, 4, 2, 1),        # a row past the fused norm: separate launches
]


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("d,dff,sdff,E,k,rows", EX_CASES)
def test_block_ex_matches_oracle(d, dff, sdff, E, k, rows, act):
    for q8_router in (True, False):
        if sdff == 0 and not q8_router:
            continue  # moe_ffn_block's case
        banner("moe_ffn_block_ex d=%d dff=%d sdff=%d E=%d k=%d rows=%d act=%d q8_router=%s"
               % (d, dff, sdff, E, k, rows, act, q8_router))
        v = synthetic.variant_inputs(35, d, dff, E, k, rows, sdff)
        check_ex(v, act, q8_router, sdff > 0, run_ex(v, act, q8_router, sdff > 0))


def test_block_ex_chunk_64_rows_with_shared_expert():
    banner("moe_ffn_block_ex 64-row chunk, int8, Q8_0 router, shared expert")
    v = synthetic.variant_inputs(36, 2048, 768, 128, 8, 64, 1024)
    check_ex(v, 1, True, True, run_ex(v, 1, True, True))


@pytest.mark.parametrize("act", [0, 1])
def test_block_ex_without_variants_is_moe_ffn_block(act):
    # the float router and no shared expert: moe_ffn_block's launches, bit
    # for bit
    banner("moe_ffn_block_ex == moe_ffn_block act=%d" % act)
    v = synthetic.variant_inputs(37, 2048, 768, 128, 8, 1)
    b, m = v.block, v.block.moe
    W = [dev(a) for a in (m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds)]
    a = q8.moe_ffn_block(dev(b.h), dev(b.r), dev(b.w), EPS, *W, m.k, act=act)
    c = q8.moe_ffn_block_ex(dev(b.h), dev(b.r), dev(b.w), EPS, *W[1:], m.k, m.E, act=act, Wr=W[0])
    for x, y in zip(a, c):
        assert torch.equal(x, y)


@pytest.mark.parametrize("act", [0, 1])
def test_shared_expert_fused_equals_separate(act):
    # the shared expert inside the gate-up and down launches gives the output
    # of the block without it plus the shared expert's own down row (computed
    # here by q8_gemv calls on the block's normed row), to float rounding
    banner("shared expert fused vs separate act=%d" % act)
    d, dff, sdff = 2048, 768, 1024
    v = synthetic.variant_inputs(38, d, dff, 128, 8, 1, sdff)
    b, m = v.block, v.block.moe
    _, _, _, with_sh = run_ex(v, act, True, True)
    _, _, _, without = run_ex(v, act, True, False)
    s, x, xq, xs = q8.add_rmsnorm_q8(dev(b.h), dev(b.r), dev(b.w), EPS)
    kw = dict(x=x, act=0) if act == 0 else dict(xq=xq, xs=xs, act=1)
    g = q8.q8_gemv(dev(v.Sgq), dev(v.Sgs), **kw)
    u = q8.q8_gemv(dev(v.Suq), dev(v.Sus), **kw)
    hid = torch.nn.functional.silu(g) * u
    if act == 0:
        dn = q8.q8_gemv(dev(v.Sdq), dev(v.Sds), x=hid, act=0)
    else:
        hq, hs = q8.q8_quantize_rows(hid)
        dn = q8.q8_gemv(dev(v.Sdq), dev(v.Sds), xq=hq, xs=hs, act=1)
    ref = without + host(dn)
    assert rel_err(with_sh, ref) <= TOL[act]


def test_block_ex_scratch_reuse_and_determinism():
    banner("moe_ffn_block_ex scratch reuse")
    big = synthetic.variant_inputs(39, 2048, 768, 128, 8, 64, 1024)
    one = synthetic.variant_inputs(39, 2048, 768, 128, 8, 1, 1024)
    need = q8.q8s_block_scratch_bytes(64, 2048, 768, 1024, 128, 8, q8.ACT_INT8)
    assert need >= q8.q8s_block_scratch_bytes(1, 2048, 768, 1024, 128, 8, q8.ACT_INT8)
    scratch = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    first = run_ex(one, 1, True, True, scratch)
    run_ex(big, 1, True, True, scratch)
    again = run_ex(one, 1, True, True, scratch)
    for a, c in zip(first, again):
        assert np.array_equal(a, c)
    check_ex(one, 1, True, True, again)


@pytest.mark.parametrize("act", [0, 1])
def test_block_ex_equals_its_stage_calls(act):
    # moe_ffn_block_ex's three launches are add_rmsnorm_router_q8,
    # moe_topk_gate_up_ex and moe_down_combine_ex: the same values, bit for bit
    banner("moe_ffn_block_ex vs stage calls act=%d" % act)
    d, dff, sdff, E, k = 2048, 768, 1024, 128, 8
    v = synthetic.variant_inputs(40, d, dff, E, k, 1, sdff)
    b, m = v.block, v.block.moe
    Wgq, Wgs, Wuq, Wus, Wdq, Wds = (dev(a) for a in (m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds))
    Sgq, Sgs, Suq, Sus, Sdq, Sds = (dev(a) for a in (v.Sgq, v.Sgs, v.Suq, v.Sus, v.Sdq, v.Sds))
    Wrq, Wrs = dev(v.Wrq), dev(v.Wrs)
    s, x, xq, xs, logits = q8.add_rmsnorm_router_q8(dev(b.h), dev(b.r), dev(b.w), EPS, Wrq, Wrs, act=act)
    kw = dict(x=x) if act == 0 else dict(xq=xq, xs=xs, want_h=False)
    idx, wts, h, hq, hs = q8.moe_topk_gate_up_ex(logits, Wgq, Wgs, Wuq, Wus, k, shared=(Sgq, Sgs, Suq, Sus),
                                                 act=act, **kw)
    y = q8.moe_down_combine_ex(Wdq, Wds, idx, wts, E, shared=(Sdq, Sds), h=h, hq=hq, hs=hs, act=act)
    bs, bidx, bw, bout = q8.moe_ffn_block_ex(dev(b.h), dev(b.r), dev(b.w), EPS, Wgq, Wgs, Wuq, Wus, Wdq, Wds, k, E,
                                             act=act, Wrq=Wrq, Wrs=Wrs, shared=(Sgq, Sgs, Suq, Sus, Sdq, Sds))
    for a, c in ((s, bs), (idx, bidx), (wts, bw), (y, bout)):
        assert torch.equal(a, c)
    # the stage calls without a shared expert are the plain ones
    i2, w2, h2, _, _ = q8.moe_topk_gate_up(logits, Wgq, Wgs, Wuq, Wus, k, x=x, act=0)
    i3, w3, h3, _, _ = q8.moe_topk_gate_up_ex(logits, Wgq, Wgs, Wuq, Wus, k, x=x, act=0)
    assert torch.equal(i2, i3) and torch.equal(w2, w3) and torch.equal(h2.reshape(h3.shape), h3)
    assert torch.equal(q8.moe_down_combine(Wdq, Wds, i2, w2, E, h=h2, act=0),
                       q8.moe_down_combine_ex(Wdq, Wds, i2, w2, E, h=h2, act=0))
