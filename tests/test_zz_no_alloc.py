"""moe_ffn_block_noalloc -- the mixture block on the library's static
scratch, no scratch argument and no allocation -- against moe_ffn_block with
a scratch of the caller's (the same kernels, so bit-exact), two calls in a
row, the second with a smaller input, and against the oracle's chain
add_rmsnorm -> moe (1e-5 f32, 2e-3 int8, 2.5e-4 two words; routing exact)."""
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


def outputs(rows, d, k):
    z = lambda *s, dt=torch.float32: torch.full(s, -7, dtype=dt, device="cuda")
    return z(rows, d), z(rows, k, dt=torch.int32), z(rows, k), z(rows, d)


def both(b, act):
    """(no-alloc outputs, moe_ffn_block outputs) on the same inputs."""
    m = b.moe
    W = [dev(a) for a in (m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds)]
    h, r, w = dev(b.h), dev(b.r), dev(b.w)
    rows, d = b.h.shape
    got = q8.moe_ffn_block_noalloc(h, r, w, EPS, *W, m.k, *outputs(rows, d, m.k), act=act)
    got = [host(t) for t in got]
    ref = q8.moe_ffn_block(h, r, w, EPS, *W, m.k, act=act)
    ref = [host(t) for t in ref]
    return got, ref


def check_oracle(b, act, got):
    s, y64 = oracle.add_rmsnorm(b.h, b.r, b.w, EPS)
    m = b.moe
    ridx, rw, _, ry = oracle.moe(y64.astype(np.float32), m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, m.k, act)
    assert np.array_equal(got[0], s)
    assert np.array_equal(got[1], ridx)
    assert rel_err(got[2], rw) <= 1e-5
    for i in range(got[3].shape[0]):
        assert rel_err(got[3][i], ry[i]) <= TOL[act], i


def test_noalloc_two_calls_second_smaller():
    # a 64-row chunk in int8 numerics (the grouped kernels: 6.6 MiB of the
    # static scratch), then one decode row of the same block: the second call
    # reuses what the first left in the array
    banner("moe_ffn_block_noalloc: 64-row chunk int8, then one row")
    big = synthetic.block_inputs(41, 2048, 768, 128, 8, 64)
    got, ref = both(big, q8.ACT_INT8)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)
    check_oracle(big, q8.ACT_INT8, got)
    small = synthetic.block_inputs(42, 2048, 768, 128, 8, 1)
    got, ref = both(small, q8.ACT_INT8)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)
    check_oracle(small, q8.ACT_INT8, got)


@pytest.mark.parametrize("act", [1, 2])
def test_noalloc_wide_chunk_then_smaller(act):
    # a 128-row chunk (8 choices an expert: the matrix-core grouped kernels)
    # bit for bit against moe_ffn_block, then a 64-row chunk on the vector
    # units in the array the first call left
    banner("moe_ffn_block_noalloc: 128-row chunk act=%d, then 64 rows" % act)
    assert q8.q8s_moe_path(128, 2048, 768, 128, 8, act) == q8.PATH_GROUPED_MFMA
    for rows, seed in ((128, 45), (64, 46)):
        got, ref = both(synthetic.block_inputs(seed, 2048, 768, 128, 8, rows), act)
        for g, r in zip(got, ref):
            assert np.array_equal(g, r)


@pytest.mark.parametrize("act", [0, 1, 2])
def test_noalloc_each_numerics(act):
    # a 3-row block, then a smaller 1-row block of another shape, in each
    # numerics
    banner("moe_ffn_block_noalloc act=%d" % act)
    for b in (synthetic.block_inputs(43, 1024, 256, 32, 4, 3), synthetic.block_inputs(44, 256, 128, 16, 2, 1)):
        got, ref = both(b, act)
        for g, r in zip(got, ref):
            assert np.array_equal(g, r)
        check_oracle(b, act, got)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    # 512 rows of the 128-expert block need more than the 32 MiB array; the
    # call is refused before any launch and names the limit
    banner("moe_ffn_block_noalloc refusal")
    need = q8.q8s_scratch_bytes(q8.FN_BLOCK, 512, 2048, 768, 128, 8, q8.ACT_INT8)
    assert need > q8.NOALLOC_SCRATCH_BYTES
    z = lambda *s, dt=torch.float32: torch.zeros(s, dtype=dt, device="cuda")
    E, d, dff, k, rows = 128, 2048, 768, 8, 512
    W = [z(E, d), z(E * dff, d, dt=torch.int8), z(E * dff, d // 32), z(E * dff, d, dt=torch.int8),
         z(E * dff, d // 32), z(E * d, dff, dt=torch.int8), z(E * d, dff // 32)]
    out = z(rows, d)
    with pytest.raises(q8.Q8sError, match="static scratch holds"):
        q8.moe_ffn_block_noalloc(z(rows, d), z(rows, d), z(d), EPS, *W, k, z(rows, d), z(rows, k, dt=torch.int32),
                                 z(rows, k), out, act=q8.ACT_INT8)
    torch.cuda.synchronize()
    assert not out.any()
