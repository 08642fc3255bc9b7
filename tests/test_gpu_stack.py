"""moe_ffn_stack -- several mixture blocks in a row, each layer's residual add
deferred into the next layer's add + norm launch and the last one's folded
into the down-combine epilogue -- against (1) the chain of moe_ffn_block
calls it stands for (h = m_{l-1}, r = s_{l-1}) and one float32 add at the
end, bit for bit, and (2) the oracle's chain add_rmsnorm -> moe per layer
(routing exact; the residual stream within the numerics' tolerance a layer,
summed over the layers)."""
import numpy as np
import pytest
import torch

import oracle
import q8_gemv_sparse_amd as q8
import synthetic
from gpu_helpers import dev, host, rel_err

pytestmark = pytest.mark.gpu

EPS = 1e-6
TOL = {0: 1e-5, 1: 2e-3, 2: 2.5e-4}


def banner(msg):
    print("[case] " + msg, flush=True)


def make_layers(seed, L, d, dff, E, k, rows):
    """L layers' weights (each drawn as block_inputs draws a block), and the
    stack's input rows h, r from the first draw."""
    blocks = [synthetic.block_inputs(seed + l, d, dff, E, k, rows) for l in range(L)]
    return blocks, blocks[0].h, blocks[0].r


def dev_layer(b):
    m = b.moe
    return tuple(dev(a) for a in (b.w, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds))


CASES = [
    # (L, d, dff, E, k, rows, act)
    (3, 2048, 768, 128, 8, 1, 0),     # the 128-expert decode block, three numerics
    (3, 2048, 768, 128, 8, 1, 1),
    (3, 2048, 768, 128, 8, 1, 2),
    (4, 1024, 512, 32, 4, 1, 1),
    (2, 2048, 768, 128, 8, 64, 1),    # a 64-row chunk: the grouped kernels, the add in the combine
    (2, 2048, 768, 128, 8, 64, 2),    # the same in two words
    (2, 2048, 768, 128, 8, 128, 1),   # a 128-row chunk: the matrix-core grouped kernels
    (2, 256, 96, 6, 2, 3, 0),         # 3 rows of float32 numerics
    (1, 512, 128, 8, 2, 1, 1),        # one layer: out = s_0 + m_0
]


@pytest.mark.parametrize("L,d,dff,E,k,rows,act", CASES)
def test_stack_equals_chained_blocks(L, d, dff, E, k, rows, act):
    banner("stack vs chained blocks L=%d d=%d dff=%d E=%d k=%d rows=%d act=%d" % (L, d, dff, E, k, rows, act))
    blocks, h, r = make_layers(60, L, d, dff, E, k, rows)
    layers = [dev_layer(b) for b in blocks]
    out, idx, wts = q8.moe_ffn_stack(dev(h), dev(r), layers, k, EPS, act=act)
    hh, rr = dev(h), dev(r)
    for l, lw in enumerate(layers):
        s, bidx, bw, m = q8.moe_ffn_block(hh, rr, lw[0], EPS, *lw[1:], k, act=act)
        assert torch.equal(idx[l], bidx) and torch.equal(wts[l], bw), l
        hh, rr = m, s
    assert torch.equal(out, rr + hh)
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("act", [0, 1, 2])
def test_stack_matches_oracle_chain(act):
    L, d, dff, E, k, rows = 3, 512, 256, 16, 4, 2
    banner("stack vs oracle chain act=%d" % act)
    blocks, h, r = make_layers(70, L, d, dff, E, k, rows)
    layers = [dev_layer(b) for b in blocks]
    out, idx, wts = q8.moe_ffn_stack(dev(h), dev(r), layers, k, EPS, act=act)
    hh, rr = h, r
    for l, b in enumerate(blocks):
        s, y64 = oracle.add_rmsnorm(hh, rr, b.w, EPS)
        m = b.moe
        ridx, rw, _, ry = oracle.moe(y64.astype(np.float32), m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, k, act)
        assert np.array_equal(host(idx[l]), ridx), l
        # layer 0 reads the same input on both sides; a later layer reads the
        # previous layer's output, which differs within that numerics'
        # tolerance, and the difference carries into its routing weights
        assert rel_err(host(wts[l]), rw) <= (1e-5 if l == 0 else l * TOL[act]), l
        hh, rr = ry.astype(np.float32), s
    ref = rr.astype(np.float64) + hh.astype(np.float64)
    assert rel_err(host(out), ref) <= L * TOL[act]


def test_stack_scratch_reuse():
    # one scratch for a 64-row stack serves a 1-row one; repeated calls repeat
    banner("stack scratch reuse")
    blocks, h, r = make_layers(80, 2, 2048, 768, 128, 8, 64)
    layers = [dev_layer(b) for b in blocks]
    scratch = torch.full((q8.q8s_scratch_bytes(q8.FN_STACK, 64, 2048, 768, 128, 8, 1),), 0x5A, dtype=torch.uint8,
                         device="cuda")
    a = q8.moe_ffn_stack(dev(h[:1]), dev(r[:1]), layers, 8, EPS, act=1, scratch=scratch)
    q8.moe_ffn_stack(dev(h), dev(r), layers, 8, EPS, act=1, scratch=scratch)
    b = q8.moe_ffn_stack(dev(h[:1]), dev(r[:1]), layers, 8, EPS, act=1, scratch=scratch)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
