"""moe_route_topk_gemv: the router's top-K carried by the dense projection's
launch.  Its routing must equal moe_route_topk's and its projection
q8_gemv's (or q8_gemv_x2's) bit for bit, and both must match the oracle as
those calls do: the choices exactly (up to near-equal logits a different
double summation order may rank the other way), the weights within 1e-5 and
the projection within 2e-3 of the oracle's int8 result.

Cases span the fused path (5 rows and more, E <= 256) -- with more rows than
the projection has workgroups (the rows past them ranked after the
contraction), 16-row and 32-row tiles, a ragged last output tile, k = 32 at
E = 256 -- and the calls it falls back to (fewer than 5 rows, E > 256)."""
import numpy as np
import pytest

import oracle
import q8_gemv_sparse_amd as q8
import synthetic
from gpu_helpers import dev, host, rel_err, route_ambiguous

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_I8 = 2e-3

# rows, d, E, k, n_out, act
CASES = [
    (64, 2048, 128, 8, 4096, 1),   # the 64-row chunk's router and dense projection
    (64, 2048, 128, 8, 4096, 2),
    (128, 2048, 128, 8, 4096, 1),  # 4 row tiles
    (20, 512, 60, 4, 256, 1),      # 16 workgroups for 20 rows: 4 ranked at the end
    (7, 256, 256, 32, 48, 2),      # 16-row tiles, 3 workgroups for 7 rows, k = 32 at E = 256
    (16, 4096, 8, 2, 130, 2),      # ragged last output tile, 9 workgroups for 16 rows
    (5, 64, 3, 3, 16, 1),          # the fewest rows the fused path takes, one workgroup
    (3, 256, 16, 2, 64, 1),        # below 5 rows: the two calls' launches in turn
    (40, 1024, 300, 6, 512, 1),    # E > 256: the two calls' launches in turn
]


def banner(msg):
    print("[case] " + msg, flush=True)


def _inputs(rows, d, E, n_out, act, seed=11):
    rng = np.random.default_rng(seed)
    Wr = (0.02 * synthetic.normal(rng, E, d)).astype(np.float32)
    x = synthetic.normal(rng, rows, d)
    Dq, Ds = synthetic.q8_matrix(rng, n_out, d)
    xd = dev(x)
    if act == 2:
        xq, xl, xs = q8.q8_quantize_rows_x2(xd)
    else:
        (xq, xs), xl = q8.q8_quantize_rows(xd), None
    return Wr, x, xd, Dq, Ds, xq, xl, xs


@pytest.mark.parametrize("rows,d,E,k,n_out,act", CASES)
def test_route_topk_gemv(rows, d, E, k, n_out, act):
    banner("route_topk_gemv rows=%d d=%d E=%d k=%d n_out=%d act=%d" % (rows, d, E, k, n_out, act))
    Wr, x, xd, Dq, Ds, xq, xl, xs = _inputs(rows, d, E, n_out, act)
    Wrd, Dqd, Dsd = dev(Wr), dev(Dq), dev(Ds)
    idx, wts, y = q8.moe_route_topk_gemv(xd, Wrd, k, Dqd, Dsd, xq, xs, xl=xl)
    # the two calls it stands for, bit for bit
    idx2, wts2 = q8.moe_route_topk(xd, Wrd, k)
    if act == 2:
        y2 = q8.q8_gemv_x2(Dqd, Dsd, xq, xl, xs)
    else:
        y2 = q8.q8_gemv(Dqd, Dsd, xq=xq, xs=xs, act=q8.ACT_INT8)
    idx, wts, y = host(idx), host(wts), host(y)
    assert np.array_equal(idx, host(idx2))
    assert np.array_equal(wts.view(np.uint32), host(wts2).view(np.uint32))
    assert np.array_equal(y.view(np.uint32), host(y2).view(np.uint32))
    # and the oracle
    ridx, rw, logits = oracle.route(x, Wr, k)
    amb = route_ambiguous(logits, k)
    assert amb.sum() <= max(1, rows // 16)
    assert np.array_equal(idx[~amb], ridx[~amb])
    assert rel_err(wts[~amb], rw[~amb]) <= TOL_F32
    for row in idx:
        assert len(set(row.tolist())) == k and row.min() >= 0 and row.max() < E
    if act == 2:
        ref = oracle.gemv_i8x2(Dq, Ds, host(xq), host(xl), host(xs))
    else:
        ref = oracle.gemv_i8(Dq, Ds, host(xq), host(xs))
    assert rel_err(y, ref) <= TOL_I8


def test_route_topk_gemv_ties_and_repeat():
    # a zero router gives every expert the same logit: each row keeps experts
    # 0 .. k-1 with equal weights; a second call on the same outputs (and
    # scratch) with other rows overwrites them whole
    banner("route_topk_gemv ties, repeated call")
    rows, d, E, k, n_out = 24, 256, 40, 5, 64
    _, x, xd, Dq, Ds, xq, _, xs = _inputs(rows, d, E, n_out, 1, seed=12)
    Dqd, Dsd = dev(Dq), dev(Ds)
    idx, wts, y = q8.moe_route_topk_gemv(xd, dev(np.zeros((E, d), np.float32)), k, Dqd, Dsd, xq, xs)
    assert (host(idx) == np.arange(k)).all() and np.allclose(host(wts), 1.0 / k)
    assert rel_err(host(y), oracle.gemv_i8(Dq, Ds, host(xq), host(xs))) <= TOL_I8
    Wr, x2, xd2, _, _, xq2, _, xs2 = _inputs(rows, d, E, n_out, 1, seed=13)
    q8.moe_route_topk_gemv(xd2, dev(Wr), k, Dqd, Dsd, xq2, xs2, idx=idx, wts=wts, y=y)
    ridx, rw, logits = oracle.route(x2, Wr, k)
    amb = route_ambiguous(logits, k)
    assert np.array_equal(host(idx)[~amb], ridx[~amb])
    assert rel_err(host(y), oracle.gemv_i8(Dq, Ds, host(xq2), host(xs2))) <= TOL_I8


def test_route_topk_gemv_refusals():
    banner("route_topk_gemv refusals")
    rows, d, E, k, n_out = 8, 64, 4, 2, 16
    Wr, x, xd, Dq, Ds, xq, _, xs = _inputs(rows, d, E, n_out, 1, seed=14)
    Wrd = dev(Wr)
    with pytest.raises(q8.Q8sError):  # low words for one-word numerics
        q8._check(q8._lib.moe_route_topk_gemv(xd.data_ptr(), Wrd.data_ptr(), rows, d, E, k, 0, 0, 0, 0, n_out,
                                              xq.data_ptr(), xq.data_ptr(), xs.data_ptr(), 0, 1, 0, 0, None))
    with pytest.raises(q8.Q8sError):  # f32 numerics
        q8._check(q8._lib.moe_route_topk_gemv(xd.data_ptr(), Wrd.data_ptr(), rows, d, E, k, 0, 0, 0, 0, n_out,
                                              xq.data_ptr(), None, xs.data_ptr(), 0, 0, 0, 0, None))
    with pytest.raises(q8.Q8sError):  # k > E
        q8.moe_route_topk_gemv(xd, Wrd, E + 1, dev(Dq), dev(Ds), xq, xs)
