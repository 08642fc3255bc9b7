"""moe_ffn_block -- the whole mixture block of a layer in one call (add +
norm, router + top-K, gate-up, down-combine) -- against the oracle's chain
add_rmsnorm -> moe on the same seeded inputs, and against the separate C
calls it stands for.

Tolerances as the parity tests: 1e-5 (f32 numerics), 2e-3 (int8 numerics,
against the oracle's int8 mode); the sum and the routing choices bit-exact
(except rows whose deciding logits are closer than double rounding can
separate, which none of these seeds has).
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


def weights(b):
    m = b.moe
    return [dev(a) for a in (m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds)]


def run_block(b, act, W=None, scratch=None):
    W = W or weights(b)
    s, idx, wts, out = q8.moe_ffn_block(dev(b.h), dev(b.r), dev(b.w), EPS, *W, b.moe.k, act=act, scratch=scratch)
    return host(s), host(idx), host(wts), host(out)


def oracle_block(b, act):
    s, y64 = oracle.add_rmsnorm(b.h, b.r, b.w, EPS)
    x = y64.astype(np.float32)
    m = b.moe
    idx, wts, h, y = oracle.moe(x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, m.k, act)
    _, _, logits = oracle.route(x, m.Wr, m.k)
    return s, idx, wts, y, logits


def check(b, act, got):
    s, idx, wts, out = got
    rs, ridx, rw, ry, logits = oracle_block(b, act)
    assert np.array_equal(s, rs)
    amb = route_ambiguous(logits, b.moe.k)
    assert not amb.any()
    assert np.array_equal(idx, ridx)
    assert rel_err(wts, rw) <= 1e-5
    for r in range(out.shape[0]):
        assert rel_err(out[r], ry[r]) <= TOL[act], r


BLOCK_CASES = [
    # (d, dff, E, k, rows): which launches run is noted
    (2048, 768, 128, 8, 1),     # the 128-expert decode block: fused launches
    (4096, 14336, 8, 2, 1),     # the 8-expert decode block: fused, int8 rows in 4 slices
    (2080, 4096, 4, 4, 1),      # int8 rows of 130 chunks: 3 slices, the last of 2 chunks
    (1056, 8320, 3, 2, 1),      # 520 gate-up tiles, rows of 66 chunks
    (96, 160, 5, 3, 1),         # ragged: lane groups of 16, tiles past dff
    (2080, 96, 7, 2, 1),        # a partial second 2048-value segment in the fused norm
    (256, 64, 5, 5, 1),         # K = E
    (64, 64, 1, 1, 1),          # one expert
    (512, 96, 256, 32, 1),      # the most experts the gate-up ranks itself, the most kept
    (128, 64, 300, 4, 1),       # more: separate norm, router and top-K launches
    (16384, 64, 4, 2, 1),       # a row past the fused norm's registers: separate launches
    (256, 96, 6, 2, 3),         # 3 rows: f32 fused per row; int8 grouped chunk kernels
]


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("d,dff,E,k,rows", BLOCK_CASES)
def test_block_matches_oracle(d, dff, E, k, rows, act):
    banner("block d=%d dff=%d E=%d k=%d rows=%d act=%d" % (d, dff, E, k, rows, act))
    b = synthetic.block_inputs(20, d, dff, E, k, rows)
    check(b, act, run_block(b, act))


@pytest.mark.parametrize("rows", [64, 128, 256])
def test_block_chunk_rows(rows):
    # 4 choices an expert at 64 rows (the vector-unit grouped kernels); 8 and
    # 16 at 128 and 256 (the matrix-core grouped kernels)
    banner("block %d-row chunk, int8" % rows)
    want = q8.PATH_GROUPED if rows == 64 else q8.PATH_GROUPED_MFMA
    assert q8.q8s_moe_path(rows, 2048, 768, 128, 8, q8.ACT_INT8) == want
    b = synthetic.block_inputs(21, 2048, 768, 128, 8, rows)
    check(b, 1, run_block(b, 1))


@pytest.mark.parametrize("rows", [64, 128])
def test_chunk_block_equals_stage_calls(rows):
    # a chunk in int8 numerics: add_rmsnorm_q8 -> moe_route_topk ->
    # moe_gate_up -> moe_down_combine compute bit for bit what moe_ffn_block
    # computes (the same grouped kernels: the vector-unit ones at 64 rows,
    # the matrix-core ones at 128)
    banner("chunk block vs stage calls rows=%d" % rows)
    b = synthetic.block_inputs(27, 2048, 768, 128, 8, rows)
    W = weights(b)
    Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds = W
    s, x, xq, xs = q8.add_rmsnorm_q8(dev(b.h), dev(b.r), dev(b.w), EPS)
    idx, wts = q8.moe_route_topk(x, Wr, 8)
    _, hq, hs = q8.moe_gate_up(Wgq, Wgs, Wuq, Wus, idx, 128, xq=xq, xs=xs, act=1)
    y = q8.moe_down_combine(Wdq, Wds, idx, wts, 128, hq=hq, hs=hs, act=1)
    bs, bidx, bw, bout = run_block(b, 1, W)
    assert np.array_equal(bs, host(s))
    assert np.array_equal(bidx, host(idx))
    assert np.array_equal(bw, host(wts))
    assert np.array_equal(bout, host(y))


@pytest.mark.parametrize("act", [0, 1])
def test_block_equals_separate_calls(act):
    # the fused launches compute what add_rmsnorm_q8 -> moe_route_topk ->
    # moe_gate_up -> moe_down_combine compute: the sum and the normed row's
    # encodings bit for bit, the same choices, outputs to float rounding of
    # the routing weights
    banner("block vs separate calls act=%d" % act)
    b = synthetic.block_inputs(22, 2048, 768, 128, 8, 1)
    W = weights(b)
    Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds = W
    s, x, xq, xs = q8.add_rmsnorm_q8(dev(b.h), dev(b.r), dev(b.w), EPS)
    idx, wts = q8.moe_route_topk(x, Wr, 8)
    if act == 0:
        h, _, _ = q8.moe_gate_up(Wgq, Wgs, Wuq, Wus, idx, 128, x=x, act=0)
        y = q8.moe_down_combine(Wdq, Wds, idx, wts, 128, h=h, act=0)
    else:
        _, hq, hs = q8.moe_gate_up(Wgq, Wgs, Wuq, Wus, idx, 128, xq=xq, xs=xs, act=1, want_h=False)
        y = q8.moe_down_combine(Wdq, Wds, idx, wts, 128, hq=hq, hs=hs, act=1)
    bs, bidx, bw, bout = run_block(b, act, W)
    assert np.array_equal(bs, host(s))
    assert np.array_equal(bidx, host(idx))
    assert rel_err(bw, host(wts)) <= 1e-6
    assert rel_err(bout, host(y)) <= 1e-6


def test_block_scratch_reuse_and_determinism():
    # one scratch sized for the largest call serves smaller ones; repeated
    # calls give identical results
    banner("block scratch reuse")
    big = synthetic.block_inputs(23, 2048, 768, 128, 8, 64)
    one = synthetic.block_inputs(24, 2048, 768, 128, 8, 1)
    W = weights(big)
    one.moe = big.moe
    need = q8.q8s_scratch_bytes(q8.FN_BLOCK, 64, 2048, 768, 128, 8, q8.ACT_INT8)
    assert need >= q8.q8s_scratch_bytes(q8.FN_BLOCK, 1, 2048, 768, 128, 8, q8.ACT_INT8)
    scratch = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    first = run_block(one, 1, W, scratch)
    run_block(big, 1, W, scratch)
    again = run_block(one, 1, W, scratch)
    for a, c in zip(first, again):
        assert np.array_equal(a, c)
    check(one, 1, again)


# ---------------------------------------------------------------------------
# the two fused stages on their own


@pytest.mark.parametrize("rows,d,E", [(1, 2048, 128), (1, 4096, 8), (3, 96, 5), (2, 2080, 7), (1, 8192, 16)])
def test_norm_router(rows, d, E):
    banner("add_rmsnorm_router rows=%d d=%d E=%d" % (rows, d, E))
    b = synthetic.block_inputs(25, d, 64, E, 1, rows)
    h, r, w, Wr = dev(b.h), dev(b.r), dev(b.w), dev(b.moe.Wr)
    s, x, xq, xs, logits = q8.add_rmsnorm_router(h, r, w, EPS, Wr)
    s2, y2, q2, d2 = q8.add_rmsnorm_q8(h, r, w, EPS)
    # the norm's outputs are add_rmsnorm_q8's, bit for bit
    for a, c in ((s, s2), (x, y2), (xq, q2), (xs, d2)):
        assert torch.equal(a, c)
    # the logits: double sums of the router row times the float32 normed row
    xx = host(x).astype(np.float64)
    ref = xx @ b.moe.Wr.astype(np.float64).T
    mag = np.abs(xx) @ np.abs(b.moe.Wr.astype(np.float64)).T
    assert np.all(np.abs(host(logits) - ref) <= 1e-13 * mag)
    # f32-only and q8-only forms write the same values
    _, x3, q3, _, l3 = q8.add_rmsnorm_router(h, r, w, EPS, Wr, want_q8=False)
    _, x4, q4, s4, l4 = q8.add_rmsnorm_router(h, r, w, EPS, Wr, want_f32=False)
    assert q3 is None and x4 is None
    assert torch.equal(x3, x) and torch.equal(q4, xq) and torch.equal(s4, xs)
    assert torch.equal(l3, logits) and torch.equal(l4, logits)


def host_topk(logits, k):
    """The K largest of each row (ties to the lower index) in rank order and
    their renormalised softmax weights, in float64."""
    idx = np.stack([np.lexsort((np.arange(l.size), -l))[:k] for l in logits]).astype(np.int32)
    kept = np.take_along_axis(logits, idx, axis=1)
    p = np.exp(kept - kept[:, :1])
    return idx, p / p.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("act", [0, 1])
# E <= 16 ranks in each wave's registers, more experts in LDS: both orders
# are checked on exact ties, near-ties (equal upper 32 bits) and signed zeros
@pytest.mark.parametrize("E,k,ties", [(128, 8, ""), (8, 2, ""), (256, 32, "exact"), (5, 5, "exact"), (1, 1, ""),
                                        (128, 8, "near"), (256, 32, "near"), (16, 4, "near"), (16, 16, "exact"),
                                        (12, 8, "near")])
def test_topk_gate_up(E, k, ties, act):
    banner("moe_topk_gate_up E=%d k=%d ties=%s act=%d" % (E, k, ties, act))
    rows, d, dff = 2, 256, 96
    m = synthetic.moe_inputs(26, d, dff, E, k, rows)
    rng = np.random.default_rng(27)
    logits = rng.standard_normal((rows, E))
    if ties == "exact":
        logits = np.round(logits * 2) / 2  # many exact ties
    elif ties == "near":
        # logits equal in their upper 32 bits and apart in the lower ones,
        # exact ties among them, and signed zeros (equal logits)
        logits = 1.0 + rng.integers(0, 6, (rows, E)) * 2.0**-40
        logits[:, 1::7] = np.where(rng.random((rows, logits[:, 1::7].shape[1])) < 0.5, 0.0, -0.0)
        logits[:, 3] = 1.0 + 9 * 2.0**-40
    Wgq, Wgs, Wuq, Wus = (dev(a) for a in (m.Wgq, m.Wgs, m.Wuq, m.Wus))
    x = dev(m.x)
    xq, xs = q8.q8_quantize_rows(x)
    kw = dict(x=x, act=0) if act == 0 else dict(xq=xq, xs=xs, act=1)
    idx, wts, h, hq, hs = q8.moe_topk_gate_up(dev(logits), Wgq, Wgs, Wuq, Wus, k, **kw)
    ridx, rw = host_topk(logits, k)
    assert np.array_equal(host(idx), ridx)
    assert rel_err(host(wts), rw) <= 1e-6
    # the hidden rows are moe_gate_up's for those choices: bit for bit in f32
    # numerics (the same row-by-row kernels); in int8 numerics moe_gate_up
    # groups the two rows by expert on the matrix cores, whose block sums are
    # exact but whose float sum over blocks runs in another order, so h agrees
    # to float rounding and each side's hq/hs is the Q8_0 form of its own h
    h2, hq2, hs2 = q8.moe_gate_up(Wgq, Wgs, Wuq, Wus, idx, E, **kw)
    if act == 0:
        assert torch.equal(h, h2)
    else:
        assert rel_err(host(h), host(h2)) <= 1e-5
        for hh, qq, ss in ((h, hq, hs), (h2, hq2, hs2)):
            rq, rs = q8.q8_quantize_rows(hh.reshape(rows * k, dff))
            assert torch.equal(qq.reshape(rq.shape), rq) and torch.equal(ss.reshape(rs.shape), rs)


def test_topk_gate_up_many_tiles():
    # 8 x 1408 hidden outputs at d 2048 make 352 int8 tiles, more than the
    # 256 CUs, so the fused gate-up takes its 8-wave shape; the choices are
    # the host ranking's and the hidden rows agree with moe_gate_up's
    banner("moe_topk_gate_up 352 tiles")
    rows, d, dff, E, k = 1, 2048, 1408, 12, 8
    m = synthetic.moe_inputs(30, d, dff, E, k, rows)
    logits = np.random.default_rng(31).standard_normal((rows, E))
    Wgq, Wgs, Wuq, Wus = (dev(a) for a in (m.Wgq, m.Wgs, m.Wuq, m.Wus))
    xq, xs = q8.q8_quantize_rows(dev(m.x))
    idx, wts, h, hq, hs = q8.moe_topk_gate_up(dev(logits), Wgq, Wgs, Wuq, Wus, k, xq=xq, xs=xs, act=1)
    ridx, rw = host_topk(logits, k)
    assert np.array_equal(host(idx), ridx)
    assert rel_err(host(wts), rw) <= 1e-6
    # moe_gate_up's 8-wave shape meets the oracle in test_moe_block_small
    h2, hq2, hs2 = q8.moe_gate_up(Wgq, Wgs, Wuq, Wus, idx, E, xq=xq, xs=xs, act=1)
    assert torch.equal(h, h2) and torch.equal(hq, hq2) and torch.equal(hs, hs2)


@pytest.mark.parametrize("E", [128, 12])
def test_topk_gate_up_nan_logits(E):
    # NaN logits: a NaN with the sign bit clear ranks above every number, one
    # with it set below; the choices stay K distinct experts in range (128
    # experts ranked in LDS, 12 in registers)
    banner("moe_topk_gate_up NaN logits E=%d" % E)
    rows, d, dff, k = 2, 256, 96, 8
    m = synthetic.moe_inputs(26, d, dff, E, k, rows)
    rng = np.random.default_rng(28)
    logits = rng.standard_normal((rows, E))
    pos, neg = np.float64(np.nan), -np.float64(np.nan)
    assert not np.signbit(pos) and np.signbit(neg)
    hi = E - 3
    logits[0, [5, hi]] = pos
    logits[0, [1, 2, 3]] = neg
    logits[1, :] = neg
    logits[1, 9] = 0.5
    Wgq, Wgs, Wuq, Wus = (dev(a) for a in (m.Wgq, m.Wgs, m.Wuq, m.Wus))
    idx, wts, h, hq, hs = q8.moe_topk_gate_up(dev(logits), Wgq, Wgs, Wuq, Wus, k, x=dev(m.x), act=0)
    idx = host(idx)
    for r in range(rows):
        assert len(set(idx[r].tolist())) == k and idx[r].min() >= 0 and idx[r].max() < E
    # row 0: the two positive NaNs by index, then the six largest numbers
    finite = [e for e in np.lexsort((np.arange(E), -np.nan_to_num(logits[0], nan=-np.inf))) if not np.isnan(logits[0, e])]
    assert list(idx[0]) == [5, hi] + finite[:k - 2]
    # row 1: the one number, then negative NaNs by index
    assert list(idx[1]) == [9, 0, 1, 2, 3, 4, 5, 6]


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("d,E", [(4096, 8), (2048, 16), (96, 3)])
def test_block_few_experts_equals_stage_calls(d, E, act):
    # the block with few experts is add_rmsnorm_router -> moe_topk_gate_up ->
    # moe_down_combine: the same sum, choices and output
    banner("block few experts vs stage calls d=%d E=%d act=%d" % (d, E, act))
    b = synthetic.block_inputs(29, d, 1024, E, 2, 1)
    W = weights(b)
    Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds = W
    s, x, xq, xs, logits = q8.add_rmsnorm_router(dev(b.h), dev(b.r), dev(b.w), EPS, Wr)
    kw = dict(x=x) if act == 0 else dict(xq=xq, xs=xs, want_h=False)
    idx, wts, h, hq, hs = q8.moe_topk_gate_up(logits, Wgq, Wgs, Wuq, Wus, 2, act=act, **kw)
    y = q8.moe_down_combine(Wdq, Wds, idx, wts, E, h=h, hq=hq, hs=hs, act=act)
    bs, bidx, bw, bout = run_block(b, act, W)
    assert np.array_equal(bs, host(s))
    assert np.array_equal(bidx, host(idx))
    assert rel_err(bw, host(wts)) <= 1e-6
    assert rel_err(bout, host(y)) <= 1e-6
    check(b, act, (bs, bidx, bw, bout))
