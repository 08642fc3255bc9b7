"""The kernels at the library's stated limits, against the oracle: the longest
reduced dimension (65536 values, cut into the most slices), the longest rows
of the mixture in both directions (d or dff of 65536), and a router row too
long for the fused norm + router launch.

Tolerances as the parity tests: 1e-5 (f32 numerics), 2e-3 (int8 numerics);
routing bit-exact.
"""
import numpy as np
import pytest

import oracle
import q8_gemv_sparse_amd as q8
import synthetic
from gpu_helpers import dev, host, rel_err, route_ambiguous

pytestmark = pytest.mark.gpu

TOL = {0: 1e-5, 1: 2e-3}
EPS = 1e-6
MAX_NIN = 65536


def banner(msg):
    print("[case] " + msg, flush=True)


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("n_out,m", [(24, 1), (9, 3), (5, 6)])
def test_gemv_longest_rows(n_out, m, act):
    # 65536 values a row: the most slices along k; m = 6 runs on the matrix
    # cores in int8 numerics
    banner("gemv n_in=%d n_out=%d m=%d act=%d" % (MAX_NIN, n_out, m, act))
    rng = np.random.default_rng(40 + m)
    Wq, Ws = synthetic.q8_matrix(rng, n_out, MAX_NIN)
    x = synthetic.normal(rng, m, MAX_NIN)
    if act == 0:
        y = host(q8.q8_gemv(dev(Wq), dev(Ws), x=dev(x), act=0))
        ref = oracle.gemv_f32(Wq, Ws, x)
    else:
        xq, xs = oracle.quantize(x)
        y = host(q8.q8_gemv(dev(Wq), dev(Ws), xq=dev(xq), xs=dev(xs), act=1))
        ref = oracle.gemv_i8(Wq, Ws, xq, xs)
    for r in range(m):
        assert rel_err(y[r], ref[r]) <= TOL[act], r


def _block_check(b, act):
    m = b.moe
    W = [dev(a) for a in (m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds)]
    s, idx, wts, out = q8.moe_ffn_block(dev(b.h), dev(b.r), dev(b.w), EPS, *W, m.k, act=act)
    rs, y64 = oracle.add_rmsnorm(b.h, b.r, b.w, EPS)
    x = y64.astype(np.float32)
    ridx, rw, _, ry = oracle.moe(x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, m.k, act)
    _, _, logits = oracle.route(x, m.Wr, m.k)
    assert np.array_equal(host(s), rs)
    assert not route_ambiguous(logits, m.k).any()
    assert np.array_equal(host(idx), ridx)
    assert rel_err(host(wts), rw) <= 1e-5
    out = host(out)
    for r in range(out.shape[0]):
        assert rel_err(out[r], ry[r]) <= TOL[act], r


@pytest.mark.parametrize("act", [0, 1])
def test_block_longest_model_dimension(act):
    # d = 65536: the norm past its register rows, the router and gate-up rows
    # cut into the most slices (separate launches)
    banner("block d=%d act=%d" % (MAX_NIN, act))
    _block_check(synthetic.block_inputs(41, MAX_NIN, 64, 3, 2, 1), act)


@pytest.mark.parametrize("act", [0, 1])
def test_block_longest_hidden_rows(act):
    # dff = 65536: the down-combine's rows cut into 16 slices for each of the
    # two kept experts; two rows (per-row kernels, no grouping at this width)
    banner("block dff=%d act=%d" % (MAX_NIN, act))
    _block_check(synthetic.block_inputs(42, 64, MAX_NIN, 3, 2, 2), act)
