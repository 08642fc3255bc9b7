"""The two-word (~14-bit) int8 activation on the GPU against the oracle: the
quantiser bit-exact (words, low words, scales); the GEMV within 1e-5 of the
oracle's same-mode result (float32 block partials, as the float32 mode) and
bit-exact where every float step is exact; the fused norm + GEMV bit-exact
against the separate calls; the mixture block (moe_ffn_block, its gate-up
stage, and moe_ffn_block_ex with the Q8_0 router and the shared expert)
within 2.5e-4 of the oracle's two-word block, routing bit-exact."""
import numpy as np
import pytest

import oracle
import q8_gemv_sparse_amd as q8
import synthetic
from gpu_helpers import dev, host, rel_err

pytestmark = pytest.mark.gpu

TOL = 1e-5


def banner(msg):
    print("[case] " + msg, flush=True)


@pytest.mark.parametrize("rows,n", [(1, 32), (3, 96), (1, 2048), (2, 2080), (1, 6144)])
def test_quantize_rows_x2_bit_exact(rows, n):
    banner("q8_quantize_rows_x2 rows %d n %d" % (rows, n))
    rng = np.random.default_rng(n + rows)
    x = synthetic.normal(rng, rows, n)
    if n >= 64:
        x[0, :32] = 0.0                                    # a zero block
        x[0, 32:64] = np.linspace(-127, 127, 32)           # integer-ish block
    if n >= 96:
        x[0, 64:96] = np.round(synthetic.normal(rng, 1, 32) * 512) / 128  # many exact 128ths
    xq, xl, xs = q8.q8_quantize_rows_x2(dev(x))
    rq, rl, rs = oracle.quantize_x2(x)
    assert np.array_equal(host(xq), rq) and np.array_equal(host(xl), rl) and np.array_equal(host(xs), rs)


# (n_out, n_in, m): batch 1 at the 512x256 and 4096x2048 shapes, rows cut into
# slices (n_in > 2048), several rows, ragged n_out, the longest row, the least
GEMV_CASES = [(512, 256, 1), (4096, 2048, 1), (96, 4096, 3), (50, 9216, 1), (33, 96, 5), (8, 65536, 1),
              (1, 32, 1), (70, 768, 4), (130, 2048, 9),
              # five rows and more: the matrix-core GEMM, two MFMAs a block
              (4096, 2048, 16), (4096, 2048, 64), (100, 2080, 20), (16, 65536, 5), (4096, 2048, 33)]


@pytest.mark.parametrize("n_out,n_in,m", GEMV_CASES)
def test_gemv_x2(n_out, n_in, m):
    banner("q8_gemv_x2 n_out %d n_in %d m %d" % (n_out, n_in, m))
    rng = np.random.default_rng(7 * n_out + n_in + m)
    Wq, Ws = synthetic.q8_matrix(rng, n_out, n_in)
    x = synthetic.normal(rng, m, n_in)
    xq, xl, xs = oracle.quantize_x2(x)
    y = q8.q8_gemv_x2(dev(Wq), dev(Ws), dev(xq), dev(xl), dev(xs))
    ref = oracle.gemv_i8x2(Wq, Ws, xq, xl, xs)
    assert rel_err(host(y), ref) <= TOL


@pytest.mark.parametrize("m", [2, 20])
def test_gemv_x2_exact_special_case(m):
    # small integers and power-of-two scales: every float step exact, so the
    # GPU equals the oracle bit for bit (pins the two block dots and the 1/128,
    # on the vector units at 2 rows and on the matrix cores at 20)
    banner("q8_gemv_x2 exact special case m=%d" % m)
    n_out, n_in = 40, 256
    Wq = synthetic.fill_pattern(n_out * n_in).reshape(n_out, n_in).astype(np.int8)
    xq = synthetic.fill_pattern(m * n_in + 3)[3:].reshape(m, n_in).astype(np.int8)
    xl = synthetic.fill_pattern(m * n_in + 5)[5:].reshape(m, n_in).astype(np.int8)
    nb = n_in // 32
    # block values are multiples of 2^-10 below 2^9: the float32 sums are exact
    Ws = np.array([[2.0 ** -((o + b) % 3) for b in range(nb)] for o in range(n_out)], np.float32)
    xs = np.array([[2.0 ** -((r + b) % 2) for b in range(nb)] for r in range(m)], np.float32)
    y = host(q8.q8_gemv_x2(dev(Wq), dev(Ws), dev(xq), dev(xl), dev(xs)))
    ref = oracle.gemv_i8x2(Wq, Ws, xq, xl, xs)
    assert np.array_equal(y.astype(np.float64), ref)


def test_quantize_then_gemv_x2_at_the_norm_gemv_shape():
    # the device quantiser feeding the device GEMV, 2048 -> 4096, against the
    # oracle's quantiser feeding the oracle's GEMV; and closer to the float32
    # GEMV than the one-word mode
    banner("q8_quantize_rows_x2 -> q8_gemv_x2 4096 x 2048")
    rng = np.random.default_rng(5)
    Wq, Ws = synthetic.q8_matrix(rng, 4096, 2048)
    x = synthetic.normal(rng, 1, 2048)
    Wd, Sd = dev(Wq), dev(Ws)
    xq, xl, xs = q8.q8_quantize_rows_x2(dev(x))
    y2 = host(q8.q8_gemv_x2(Wd, Sd, xq, xl, xs))
    rq, rl, rs = oracle.quantize_x2(x)
    assert rel_err(y2, oracle.gemv_i8x2(Wq, Ws, rq, rl, rs)) <= TOL
    yf = oracle.gemv_f32(Wq, Ws, x)
    q1, s1 = oracle.quantize(x)
    assert rel_err(y2, yf) < rel_err(oracle.gemv_i8(Wq, Ws, q1, s1), yf) / 16


# (d, n_out, rows): one launch for one row of d <= 4096, else the separate calls
NORM_CASES = [(2048, 4096, 1), (4096, 1000, 1), (1024, 130, 1), (768, 97, 1), (256, 33, 1), (32, 5, 1),
              (2080, 64, 1), (2048, 512, 3), (8192, 96, 1)]


@pytest.mark.parametrize("d,n_out,rows", NORM_CASES)
def test_norm_gemv_x2(d, n_out, rows):
    # against the separate calls bit for bit (the same normed row, its same
    # two-word form, the same dots), and against the oracle's chain
    banner("add_rmsnorm_gemv_x2 d=%d n_out=%d rows=%d" % (d, n_out, rows))
    import torch
    inp = synthetic.norm_gemv_inputs(40, d, n_out, rows)
    h, r, w, Wq, Ws = dev(inp.h), dev(inp.r), dev(inp.w), dev(inp.Wq), dev(inp.Ws)
    s, y, yq, yl, ys, out = q8.add_rmsnorm_gemv_x2(h, r, w, 1e-6, Wq, Ws)
    s2, y2, _, _ = q8.add_rmsnorm_q8(h, r, w, 1e-6, want_q8=False)
    q2, l2, d2 = q8.q8_quantize_rows_x2(y2)
    o2 = q8.q8_gemv_x2(Wq, Ws, q2, l2, d2)
    for a, b in ((s, s2), (y, y2), (yq, q2), (yl, l2), (ys, d2), (out, o2)):
        assert torch.equal(a, b)
    rs, ry = oracle.add_rmsnorm(inp.h, inp.r, inp.w, 1e-6)
    assert np.array_equal(host(s), rs)
    ref = oracle.gemv_i8x2(inp.Wq, inp.Ws, *oracle.quantize_x2(ry.astype(np.float32)))
    got = host(out)
    for i in range(rows):
        assert rel_err(got[i], ref[i]) <= TOL, i


# ---------------------------------------------------------------------------
# the mixture block in two words: moe_ffn_block(act=2) against the oracle's
# chain add_rmsnorm -> moe(act=2).  The hidden rows are float32 on both sides
# but summed in different orders, so a low word can round the other way where
# the two float32 values straddle a 128th of a step: each such flip moves one
# value by 1/128 of a one-word flip, so the one-word tolerance of 2e-3 scales
# to 2e-3 * 16 / 128 = 2.5e-4 (a margin of 16 flips' worth).
TOL_X2_BLOCK = 2.5e-4

BLOCK_X2_CASES = [
    # (d, dff, E, k, rows)
    (2048, 768, 128, 8, 1),     # the 128-expert decode block
    (4096, 14336, 8, 2, 1),     # the 8-expert decode block: rows in 4 slices
    (2080, 4096, 4, 4, 1),      # rows of 130 chunks: 3 slices, the last of 2 chunks
    (96, 160, 5, 3, 1),         # ragged: lane groups of 16, tiles past dff
    (256, 64, 5, 5, 1),         # K = E
    (64, 64, 1, 1, 1),          # one expert
    (512, 96, 256, 32, 1),      # the most experts ranked in the gate-up, the most kept
    (256, 96, 6, 2, 3),         # several rows: the grouped chunk kernels in two words
    (2048, 768, 128, 8, 64),    # the 64-row chunk of the 128-expert block, each expert read once
    (1024, 2048, 16, 4, 8),     # hidden rows of 2048: the chunk down projection a lane group a row
    (96, 160, 5, 3, 4),         # ragged rows in the chunk kernels
    # 8 and more choices an expert: the matrix-core grouped kernels, two
    # MFMAs a block
    (2048, 768, 128, 8, 128),   # gate-up tiles of 16 rows (two-word token rows of 2 KB)
    (256, 256, 2, 1, 150),      # 75 choices an expert: three tiles of 32 rows, the last ragged
    (512, 2048, 4, 2, 40),      # down tiles of 16 rows
]


@pytest.mark.parametrize("d,dff,E,k,rows", BLOCK_X2_CASES)
def test_block_x2_matches_oracle(d, dff, E, k, rows):
    banner("block x2 d=%d dff=%d E=%d k=%d rows=%d" % (d, dff, E, k, rows))
    b = synthetic.block_inputs(20, d, dff, E, k, rows)
    m = b.moe
    W = [dev(a) for a in (m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds)]
    s, idx, wts, out = q8.moe_ffn_block(dev(b.h), dev(b.r), dev(b.w), 1e-6, *W, k, act=2)
    rs, y64 = oracle.add_rmsnorm(b.h, b.r, b.w, 1e-6)
    x = y64.astype(np.float32)
    ridx, rw, rh, ry = oracle.moe(x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, k, 2)
    assert np.array_equal(host(s), rs)
    assert np.array_equal(host(idx), ridx)
    assert rel_err(host(wts), rw) <= 1e-5
    got = host(out)
    for r in range(rows):
        assert rel_err(got[r], ry[r]) <= TOL_X2_BLOCK, r
    # closer to the f32 mode than the one-word block is
    _, _, _, yf = oracle.moe(x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, k, 0)
    _, _, _, y1 = oracle.moe(x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, k, 1)
    assert rel_err(got, yf) < rel_err(y1, yf) / 8


@pytest.mark.parametrize("d,dff,E,k", [(2048, 768, 128, 8), (4096, 14336, 8, 2), (96, 160, 5, 3)])
def test_topk_gate_up_x2(d, dff, E, k):
    # the stage alone: choices as the oracle's, and hidden rows whose two-word
    # form reads back within half a low-word step of the oracle's float32 rows
    banner("moe_topk_gate_up_x2 d=%d dff=%d E=%d k=%d" % (d, dff, E, k))
    b = synthetic.block_inputs(22, d, dff, E, k, 1)
    m = b.moe
    rs, y64 = oracle.add_rmsnorm(b.h, b.r, b.w, 1e-6)
    x = y64.astype(np.float32)
    ridx, rw, logits = oracle.route(x, m.Wr, k)
    rq, rl, rsc = oracle.quantize_x2(x)
    idx, wts, hq, hl, hs = q8.moe_topk_gate_up_x2(dev(logits), dev(m.Wgq), dev(m.Wgs), dev(m.Wuq), dev(m.Wus), k,
                                                  dev(rq), dev(rl), dev(rsc))
    _, _, rh, _ = oracle.moe(x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, k, 2)
    assert np.array_equal(host(idx), ridx)
    assert rel_err(host(wts), rw) <= 1e-5
    step = np.repeat(host(hs).reshape(1, k, dff // 32).astype(np.float64), 32, axis=2)
    back = step * (host(hq).astype(np.float64) + host(hl).astype(np.float64) / 128.0)
    ref = rh.astype(np.float64)
    assert np.all(np.abs(back - ref) <= step / 256.0 * (1 + 1e-6) + 1e-5 * np.max(np.abs(ref)))


# the block's linked variants in two words: moe_ffn_block_ex(act=2) with the
# Q8_0 router (two exact dots a block over the row's two words) and/or the
# shared expert, against oracle.moe_shared(act=2)
X2_EX_CASES = [
    # (d, dff, sdff, E, k, rows, q8_router)
    (2048, 768, 0, 128, 8, 1, True),       # the Q8_0 router alone
    (2048, 768, 1024, 128, 8, 1, True),    # + a shared expert wider than a slice of dff
    (2048, 1408, 5632, 60, 4, 1, True),    # the shared-expert block's shape
    (4096, 1408, 5632, 16, 4, 1, True),    # int8 rows in 4 slices
    (96, 160, 96, 5, 3, 1, False),         # the float router with a shared expert, ragged
    (256, 64, 800, 6, 2, 3, True),         # several rows
]


@pytest.mark.parametrize("d,dff,sdff,E,k,rows,q8_router", X2_EX_CASES)
def test_block_ex_x2_matches_oracle(d, dff, sdff, E, k, rows, q8_router):
    banner("moe_ffn_block_ex x2 d=%d dff=%d sdff=%d E=%d k=%d rows=%d q8_router=%s"
           % (d, dff, sdff, E, k, rows, q8_router))
    from gpu_helpers import route_ambiguous
    v = synthetic.variant_inputs(35, d, dff, E, k, rows, sdff)
    b, m = v.block, v.block.moe
    W = [dev(a) for a in (m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds)]
    rk = dict(Wrq=dev(v.Wrq), Wrs=dev(v.Wrs)) if q8_router else dict(Wr=dev(m.Wr))
    sh = tuple(dev(a) for a in (v.Sgq, v.Sgs, v.Suq, v.Sus, v.Sdq, v.Sds)) if sdff else None
    s, idx, wts, out = q8.moe_ffn_block_ex(dev(b.h), dev(b.r), dev(b.w), 1e-6, *W, k, E, act=2, shared=sh, **rk)
    rs, y64 = oracle.add_rmsnorm(b.h, b.r, b.w, 1e-6)
    x = y64.astype(np.float32)
    ork = dict(Wrq=v.Wrq, Wrs=v.Wrs) if q8_router else dict(Wr=m.Wr)
    osh = (v.Sgq, v.Sgs, v.Suq, v.Sus, v.Sdq, v.Sds) if sdff else None
    ridx, rw, _, ry = oracle.moe_shared(x, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, k, 2, shared=osh, **ork)
    if q8_router:
        xq, xl, xs = oracle.quantize_x2(x)
        _, _, logits = oracle.route_q8(v.Wrq, v.Wrs, k, xq=xq, xs=xs, xl=xl)
    else:
        _, _, logits = oracle.route(x, m.Wr, k)
    assert np.array_equal(host(s), rs)
    assert not route_ambiguous(logits, k).any()
    assert np.array_equal(host(idx), ridx)
    assert rel_err(host(wts), rw) <= 1e-5
    got = host(out)
    for r in range(rows):
        assert rel_err(got[r], ry[r]) <= TOL_X2_BLOCK, r


def test_block_x2_scratch_needs_no_initial_contents_and_repeats():
    # the block's scratch holds nothing between calls: a scratch full of
    # garbage gives the same bits as a fresh one, and calls repeat exactly
    banner("block x2 scratch reuse and determinism")
    import torch
    b = synthetic.block_inputs(23, 2048, 768, 128, 8, 1)
    m = b.moe
    W = [dev(a) for a in (m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds)]
    h, r, w = dev(b.h), dev(b.r), dev(b.w)
    nbytes = q8.q8s_scratch_bytes(q8.FN_BLOCK, 1, 2048, 768, 128, 8, q8.ACT_X2)
    scratch = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
    first = q8.moe_ffn_block(h, r, w, 1e-6, *W, m.k, act=q8.ACT_X2, scratch=scratch)
    for _ in range(3):
        again = q8.moe_ffn_block(h, r, w, 1e-6, *W, m.k, act=q8.ACT_X2, scratch=scratch)
        for a, c in zip(first, again):
            assert torch.equal(a, c)
    fresh = q8.moe_ffn_block(h, r, w, 1e-6, *W, m.k, act=q8.ACT_X2)
    for a, c in zip(first, fresh):
        assert torch.equal(a, c)


@pytest.mark.parametrize("rows", [1, 64, 128])
def test_x2_stage_calls_equal_block(rows):
    # add_rmsnorm_q8 -> q8_quantize_rows_x2 -> moe_route_topk -> moe_gate_up_x2
    # -> moe_down_combine_x2 compute what moe_ffn_block(act 2) computes: bit
    # for bit for a chunk (the block runs these very kernels: the vector-unit
    # ones at 64 rows, the matrix-core ones at 128), and for one row within
    # float rounding of the routing weights (the block's fused launches form
    # the logits in another order)
    banner("x2 stage calls vs block rows=%d" % rows)
    import torch
    b = synthetic.block_inputs(31, 2048, 768, 128, 8, rows)
    m = b.moe
    W = [dev(a) for a in (m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds)]
    Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds = W
    s, x, _, _ = q8.add_rmsnorm_q8(dev(b.h), dev(b.r), dev(b.w), 1e-6, want_q8=False)
    xq, xl, xs = q8.q8_quantize_rows_x2(x)
    idx, wts = q8.moe_route_topk(x, Wr, 8)
    _, hq, hl, hs = q8.moe_gate_up_x2(Wgq, Wgs, Wuq, Wus, idx, 128, xq, xl, xs)
    y = q8.moe_down_combine_x2(Wdq, Wds, idx, wts, 128, hq, hl, hs)
    bs, bidx, bw, bout = q8.moe_ffn_block(dev(b.h), dev(b.r), dev(b.w), 1e-6, *W, 8, act=2)
    assert torch.equal(bs, s) and torch.equal(bidx, idx)
    if rows > 1:
        assert torch.equal(bw, wts) and torch.equal(bout, y)
    else:
        assert rel_err(host(bw), host(wts)) <= 1e-6 and rel_err(host(bout), host(y)) <= 1e-6
    rs, y64 = oracle.add_rmsnorm(b.h, b.r, b.w, 1e-6)
    ridx, _, _, ry = oracle.moe(y64.astype(np.float32), m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 8, 2)
    assert np.array_equal(host(idx), ridx)
    got = host(y)
    for r in range(rows):
        assert rel_err(got[r], ry[r]) <= TOL_X2_BLOCK, r


@pytest.mark.parametrize("rows,d", [(1, 2048), (64, 2048), (3, 96), (2, 2080), (1, 4096), (2, 16384)])
def test_add_rmsnorm_q8_x2_equals_norm_then_quantiser(rows, d):
    # the two-word epilogue writes exactly what add_rmsnorm_q8 followed by
    # q8_quantize_rows_x2 writes, every byte, and its words and scales are
    # add_rmsnorm_q8's one-word form
    banner("add_rmsnorm_q8_x2 rows=%d d=%d" % (rows, d))
    rng = np.random.default_rng(31)
    h, r = synthetic.normal(rng, rows, d), synthetic.normal(rng, rows, d)
    w = rng.uniform(0.5, 1.5, d).astype(np.float32)
    hd, rd, wd = dev(h), dev(r), dev(w)
    s1, y1, q1, l1, s1c = q8.add_rmsnorm_q8_x2(hd, rd, wd, 1e-6)
    s0, y0, _, _ = q8.add_rmsnorm_q8(hd, rd, wd, 1e-6, want_q8=False)
    q0, l0, c0 = q8.q8_quantize_rows_x2(y0)
    _, _, q1w, c1w = q8.add_rmsnorm_q8(hd, rd, wd, 1e-6)
    for a, b in ((s1, s0), (y1, y0), (q1, q0), (l1, l0), (s1c, c0), (q1, q1w), (s1c, c1w)):
        assert np.array_equal(host(a).view(np.uint8), host(b).view(np.uint8))
    # without the float32 rows
    _, none_y, q2, l2, c2 = q8.add_rmsnorm_q8_x2(hd, rd, wd, 1e-6, want_f32=False)
    assert none_y is None
    for a, b in ((q2, q0), (l2, l0), (c2, c0)):
        assert np.array_equal(host(a).view(np.uint8), host(b).view(np.uint8))
