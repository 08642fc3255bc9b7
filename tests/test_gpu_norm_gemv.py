"""add_rmsnorm_gemv -- the residual add + RMSNorm feeding a Q8_0 projection
in one call -- against the separate calls add_rmsnorm_q8 -> q8_gemv (bit for
bit: the same normed row, the same per-row dot in the same lane order) and
against the oracle's chain add_rmsnorm -> gemv (1e-5 in f32 numerics, 2e-3 in
int8 numerics against the oracle's int8 mode)."""
import numpy as np
import pytest
import torch

import oracle
import q8_gemv_sparse_amd as q8
import synthetic
from gpu_helpers import dev, host, rel_err

pytestmark = pytest.mark.gpu

EPS = 1e-6


def banner(msg):
    print("[case] " + msg, flush=True)


CASES = [
    # (d, n_out, rows): the fused launch covers one row of d <= 4096
    (2048, 4096, 1),    # the 2048 -> 4096 batch-1 workload
    (4096, 1000, 1),    # two 2048-value segments, lane groups of 64 with 4 chunks
    (1024, 130, 1),     # lane groups of 64 with 1 chunk, ragged outputs
    (768, 97, 1),       # lane groups of 16 with 3 chunks
    (256, 33, 1),       # lane groups of 16 with 1 chunk
    (32, 5, 1),         # one block
    (2080, 64, 1),      # a partial second segment
    (2048, 512, 3),     # several rows: add_rmsnorm_q8 then q8_gemv
    (8192, 96, 1),      # past one wave's slice: add_rmsnorm_q8 then q8_gemv
]


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("d,n_out,rows", CASES)
def test_norm_gemv(d, n_out, rows, act):
    banner("add_rmsnorm_gemv d=%d n_out=%d rows=%d act=%d" % (d, n_out, rows, act))
    inp = synthetic.norm_gemv_inputs(30, d, n_out, rows)
    h, r, w, Wq, Ws = dev(inp.h), dev(inp.r), dev(inp.w), dev(inp.Wq), dev(inp.Ws)
    s, y, yq, ys, out = q8.add_rmsnorm_gemv(h, r, w, EPS, Wq, Ws, act=act, want_f32=True, want_q8=True)
    # the separate calls, bit for bit
    s2, y2, q2, d2 = q8.add_rmsnorm_q8(h, r, w, EPS)
    if act == 0:
        o2 = q8.q8_gemv(Wq, Ws, x=y2, act=0)
    else:
        o2 = q8.q8_gemv(Wq, Ws, xq=q2, xs=d2, act=1)
    for a, b in ((s, s2), (y, y2), (yq, q2), (ys, d2), (out, o2)):
        assert torch.equal(a, b)
    # the oracle's chain
    rs, ry = oracle.add_rmsnorm(inp.h, inp.r, inp.w, EPS)
    assert np.array_equal(host(s), rs)
    x = ry.astype(np.float32)
    if act == 0:
        ref = oracle.gemv_f32(inp.Wq, inp.Ws, x)
        tol = 1e-5
    else:
        ref = oracle.gemv_i8(inp.Wq, inp.Ws, *oracle.quantize(x))
        tol = 2e-3
    got = host(out)
    for i in range(rows):
        assert rel_err(got[i], ref[i]) <= tol, i


def test_norm_gemv_only_the_form_read():
    # int8 numerics with no f32 row requested, f32 numerics with no Q8_0 form
    banner("add_rmsnorm_gemv optional outputs")
    inp = synthetic.norm_gemv_inputs(31, 2048, 256, 1)
    h, r, w, Wq, Ws = dev(inp.h), dev(inp.r), dev(inp.w), dev(inp.Wq), dev(inp.Ws)
    _, y, yq, ys, o1 = q8.add_rmsnorm_gemv(h, r, w, EPS, Wq, Ws, act=1)
    assert y is None and yq is not None
    _, _, _, _, o1b = q8.add_rmsnorm_gemv(h, r, w, EPS, Wq, Ws, act=1, want_f32=True)
    assert torch.equal(o1, o1b)
    _, y0, yq0, _, o0 = q8.add_rmsnorm_gemv(h, r, w, EPS, Wq, Ws, act=0)
    assert yq0 is None and y0 is not None
    _, _, _, _, o0b = q8.add_rmsnorm_gemv(h, r, w, EPS, Wq, Ws, act=0, want_q8=True)
    assert torch.equal(o0, o0b)
