"""The two-word (~14-bit) int8 activation on the GPU against the oracle: the
quantiser bit-exact (words, low words, scales), the GEMV within 1e-5 of the
oracle's same-mode result (float32 block partials, as the float32 mode), and
bit-exact where every float step is exact."""
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
              (1, 32, 1), (70, 768, 4), (130, 2048, 9)]


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


def test_gemv_x2_exact_special_case():
    # small integers and power-of-two scales: every float step exact, so the
    # GPU equals the oracle bit for bit (pins the two block dots and the 1/128)
    banner("q8_gemv_x2 exact special case")
    n_out, n_in, m = 40, 256, 2
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
