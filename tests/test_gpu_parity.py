"""Parity of the HIP path with the CPU oracle, element by element, on seeded
inputs: small shapes spanning several tiles and ragged tails, edge cases, and
the full sizes of the five workloads in the launch shapes the benchmark uses.

Tolerances (max |gpu - oracle| / max |oracle|, float64):
  * f32-activation mode: 1e-5;
  * int8-activation mode: 2e-3 against the oracle's int8 mode;
  * integer results (quantised codes, routing choices, exact block dots):
    bit-exact, except where the oracle's own float64 value sits on a float32
    rounding boundary (flagged, counted, and checked for validity instead).
"""
import numpy as np
import pytest
import torch

import oracle
import q8_gemv_sparse_amd as q8
import synthetic
from gpu_helpers import dev, f32_ambiguous, host, rel_err, route_ambiguous

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_I8 = 2e-3


def banner(msg):
    print("[case] " + msg, flush=True)


# ---------------------------------------------------------------------------
# q8_gemv, f32 activations

GEMV_F32_CASES = [
    (512, 256, 1),      # the 512x256 batch-1 workload
    (4096, 2048, 1),    # the 2048 -> 4096 batch-1 projection
    (97, 160, 1),       # ragged rows, a row shorter than a lane group's reach
    (130, 768, 3),      # lane groups of 16 with 3 chunks, 3 activation rows
    (64, 1024, 2),
    (33, 4096, 4),
    (40, 8192, 1),      # cut along k across 2 waves
    (19, 14336, 2),     # cut along k across 4 waves, last slice partial
    (5, 32, 1),         # one block
    (300, 2048, 7),     # more activation rows than a register pass holds
]


@pytest.mark.parametrize("n_out,n_in,m", GEMV_F32_CASES)
def test_gemv_f32(n_out, n_in, m):
    banner("gemv f32 %dx%d m=%d" % (n_out, n_in, m))
    g = synthetic.gemv_inputs(1, n_out, n_in, m)
    ref = oracle.gemv_f32(g.Wq, g.Ws, g.x)
    y = q8.q8_gemv(dev(g.Wq), dev(g.Ws), x=dev(g.x), act=q8.ACT_F32)
    assert rel_err(host(y), ref) <= TOL_F32


def test_gemv_f32_fill_closed_form_exact():
    banner("gemv f32 closed form")
    n_in = 2048
    Wq = np.ones((70, n_in), np.int8)
    Ws = np.full((70, n_in // 32), 1.0, np.float32)
    x = synthetic.fill_pattern(n_in)[None, :]
    y = host(q8.q8_gemv(dev(Wq), dev(Ws), x=dev(x)))
    assert np.all(y == -6.0)  # tests/golden/fill_closed_forms.txt, n_in = 2048


# ---------------------------------------------------------------------------
# q8_gemv, int8 activations

GEMV_I8_CASES = [
    (4096, 2048, 1), (512, 256, 1), (97, 160, 2), (130, 768, 4), (19, 14336, 1),
    (100, 2048, 5), (4096, 2048, 64), (77, 96, 16), (33, 512, 65), (16, 4096, 130),
    # matrix-core path with an odd number of 32-block passes, the last one
    # short (65 blocks: three passes; 97 blocks: four)
    (50, 2080, 24), (40, 3104, 9),
]


@pytest.mark.parametrize("n_out,n_in,m", GEMV_I8_CASES)
def test_gemv_int8(n_out, n_in, m):
    banner("gemv int8 %dx%d m=%d" % (n_out, n_in, m))
    rng = np.random.default_rng(2)
    Wq, Ws = synthetic.q8_matrix(rng, n_out, n_in)
    xq, xs = synthetic.q8_matrix(rng, m, n_in)
    ref = oracle.gemv_i8(Wq, Ws, xq, xs)
    y = q8.q8_gemv(dev(Wq), dev(Ws), xq=dev(xq), xs=dev(xs), act=q8.ACT_INT8)
    assert rel_err(host(y), ref) <= TOL_I8


@pytest.mark.parametrize("n_out,n_in,m", [(64, 256, 1), (200, 2048, 3), (48, 4096, 20), (50, 9216, 1)])
def test_gemv_int8_block_dots_bit_exact(n_out, n_in, m):
    # Power-of-two scales and small integers make every float step exact: the
    # result is then the exact integer block dots, on both sides, bit for bit
    # (register path for m <= 4, MFMA path above).
    banner("gemv int8 exact %dx%d m=%d" % (n_out, n_in, m))
    Wq = synthetic.fill_pattern(n_out * n_in).reshape(n_out, n_in).astype(np.int8)
    xq = synthetic.fill_pattern(m * n_in + 5)[5:].reshape(m, n_in).astype(np.int8)
    nb = n_in // 32
    Ws = np.array([[2.0 ** -((o + b) % 4) for b in range(nb)] for o in range(n_out)], np.float32)
    xs = np.array([[2.0 ** -((r * 3 + b) % 3) for b in range(nb)] for r in range(m)], np.float32)
    ref = oracle.gemv_i8(Wq, Ws, xq, xs)
    y = host(q8.q8_gemv(dev(Wq), dev(Ws), xq=dev(xq), xs=dev(xs), act=q8.ACT_INT8))
    assert np.array_equal(y.astype(np.float64), ref)


def test_gemv_int8_extreme_block_dots():
    # every block dot at its extreme, -516128 (int32 headroom), both paths
    banner("gemv int8 extremes")
    for m in (1, 16):
        Wq = np.full((32, 256), 127, np.int8)
        xq = np.full((m, 256), -127, np.int8)
        Ws = np.ones((32, 8), np.float32)
        xs = np.ones((m, 8), np.float32)
        y = host(q8.q8_gemv(dev(Wq), dev(Ws), xq=dev(xq), xs=dev(xs), act=q8.ACT_INT8))
        assert np.all(y == -516128.0 * 8)


# ---------------------------------------------------------------------------
# quantiser and fused add + RMSNorm


def _quant_edge_rows(n):
    rng = np.random.default_rng(3)
    rows = [synthetic.normal(rng, n), 1e-4 * synthetic.normal(rng, n), 1e4 * synthetic.normal(rng, n),
            np.zeros(n, np.float32)]
    ties = np.zeros(n, np.float32)
    ties[0::32] = 127.0
    ties[1::32] = 2.5
    ties[2::32] = -2.5
    ties[3::32] = 0.5
    ties[4::32] = -126.5
    rows.append(ties)
    ints = np.round(synthetic.normal(rng, n) * 30).astype(np.float32)
    rows.append(ints)
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("n", [32, 96, 2048, 2080, 6144])
def test_quantize_rows_bit_exact(n):
    banner("quantize n=%d" % n)
    x = _quant_edge_rows(n)
    rq, rs = oracle.quantize(x)
    xq, xs = q8.q8_quantize_rows(dev(x))
    assert np.array_equal(host(xq), rq)
    assert np.array_equal(host(xs), rs)


@pytest.mark.parametrize("rows,d", [(1, 2048), (3, 96), (2, 2080), (64, 2048), (1, 4096), (1, 32), (2, 16384)])
def test_add_rmsnorm_q8(rows, d):
    banner("add_rmsnorm rows=%d d=%d" % (rows, d))
    inp = synthetic.norm_gemv_inputs(4, d, 32, rows)
    eps = 1e-6
    rsum, y64 = oracle.add_rmsnorm(inp.h, inp.r, inp.w, eps)
    s, y, yq, ys = q8.add_rmsnorm_q8(dev(inp.h), dev(inp.r), dev(inp.w), eps)
    s, y, yq, ys = host(s), host(y), host(yq), host(ys)
    assert np.array_equal(s, rsum)
    assert rel_err(y, y64) <= TOL_F32
    y32 = y64.astype(np.float32)
    # The two sides sum the mean square in different orders: float64 values
    # agree to ~d * 2^-53 relative (~2.3e-13 at d = 2048, the worst case);
    # elements within 4e-13 of a float32 rounding boundary may round either way.
    amb = f32_ambiguous(y64, rel=4e-13)
    # codes are decided by the float32 y: exact wherever the oracle's float32
    # y is fixed by its float64 value
    rq, rs = oracle.quantize(y32)
    blocks_amb = amb.reshape(rows, d // 32, 32).any(axis=2)
    ok = ~blocks_amb
    assert blocks_amb.mean() <= 0.01
    assert np.array_equal(ys[ok], rs[ok])
    assert np.array_equal(yq.reshape(rows, d // 32, 32)[ok], rq.reshape(rows, d // 32, 32)[ok])
    # y itself to the nearest float32 where unambiguous, one ulp where not
    assert np.array_equal(y[~amb], y32[~amb])
    assert np.all(np.abs(y[amb].astype(np.float64) - y64[amb]) <= np.spacing(np.abs(y32[amb])))
    # ambiguous blocks: still a valid Q8_0 encoding of the GPU's own y, codes
    # within one step of the oracle's
    qb = yq.reshape(rows, d // 32, 32)[blocks_amb].astype(np.int32)
    assert np.all(np.abs(qb - rq.reshape(rows, d // 32, 32)[blocks_amb].astype(np.int32)) <= 1)
    assert np.all(np.abs(ys[blocks_amb] - rs[blocks_amb]) <= np.spacing(rs[blocks_amb]))


def test_add_rmsnorm_modes_and_fusion():
    # the fused kernel equals the unfused chain add -> norm -> quantise
    banner("add_rmsnorm fusion")
    inp = synthetic.norm_gemv_inputs(5, 2048, 32, 2)
    h, r, w = dev(inp.h), dev(inp.r), dev(inp.w)
    s1, y1, q1, d1 = q8.add_rmsnorm_q8(h, r, w, 1e-6)
    s2, y2, _, _ = q8.add_rmsnorm_q8(h, r, w, 1e-6, want_q8=False)
    s3, _, q3, d3 = q8.add_rmsnorm_q8(h, r, w, 1e-6, want_f32=False)
    qx, dx = q8.q8_quantize_rows(y1)
    for a, b in ((s1, s2), (s1, s3), (y1, y2), (q1, q3), (d1, d3), (q1, qx), (d1, dx)):
        assert torch.equal(a, b)
    # no residual: the norm of h alone
    s4, y4, _, _ = q8.add_rmsnorm_q8(s1, torch.zeros_like(s1), w, 1e-6, want_q8=False)
    assert torch.equal(y4, y1)


# ---------------------------------------------------------------------------
# router + top-K

ROUTE_CASES = [
    (1, 2048, 128, 8),   # the 128-expert decode router
    (1, 4096, 8, 2),     # the 8-expert decode router
    (64, 2048, 128, 8),  # a 64-row chunk
    (5, 96, 6, 6),       # K = E
    (3, 64, 1, 1),       # one expert
    (2, 128, 300, 1),    # E not a multiple of the workgroup's 4 experts
    (1, 256, 8192, 32),  # the limits
    (7, 32, 40, 32),
    # from 16 rows up the logits run as 4-expert x 8-row tiles: ragged rows
    # and experts, rows shorter than the 2048 values a pass covers, and rows
    # of two passes, the second one short
    (16, 64, 6, 2), (37, 4096, 130, 8), (20, 2080, 9, 3),
]


@pytest.mark.parametrize("rows,d,E,k", ROUTE_CASES)
def test_route_topk(rows, d, E, k):
    banner("route rows=%d d=%d E=%d k=%d" % (rows, d, E, k))
    rng = np.random.default_rng(6)
    Wr = (0.02 * synthetic.normal(rng, E, d)).astype(np.float32)
    x = synthetic.normal(rng, rows, d)
    ridx, rw, logits = oracle.route(x, Wr, k)
    idx, wts = q8.moe_route_topk(dev(x), dev(Wr), k)
    idx, wts = host(idx), host(wts)
    amb = route_ambiguous(logits, k)
    assert amb.sum() == 0 or rows > 1
    assert np.array_equal(idx[~amb], ridx[~amb])
    assert rel_err(wts[~amb], rw[~amb]) <= TOL_F32
    assert np.allclose(wts.sum(axis=1), 1.0, atol=1e-6)
    # every row's choices are distinct valid experts
    for row in idx:
        assert len(set(row.tolist())) == k and row.min() >= 0 and row.max() < E


def test_route_ties_and_zero_router():
    banner("route ties")
    d = 64
    x = synthetic.normal(np.random.default_rng(7), 2, d)
    idx, wts = q8.moe_route_topk(dev(x), dev(np.zeros((16, d), np.float32)), 4)
    assert (host(idx) == np.arange(4)).all() and np.allclose(host(wts), 0.25)
    Wr = np.zeros((6, d), np.float32)
    Wr[3] = Wr[1] = x[0] / 8
    Wr[5] = x[0] / 16
    idx, _ = q8.moe_route_topk(dev(x[:1]), dev(Wr), 3)
    assert list(host(idx)[0]) == [1, 3, 5]


def test_route_ties_many_rows():
    # the tiled logits: experts 1 and 3 share a router row (equal logits in
    # every row, ranked by index) and expert 5's row is exactly half of it
    banner("route ties, 24 rows")
    d = 160
    rng = np.random.default_rng(8)
    x = np.abs(synthetic.normal(rng, 24, d)).astype(np.float32)
    Wr = np.zeros((7, d), np.float32)
    Wr[1] = Wr[3] = np.abs(synthetic.normal(rng, d)) / 8
    Wr[5] = Wr[1] / 2
    idx, wts = q8.moe_route_topk(dev(x), dev(Wr), 3)
    assert (host(idx) == np.array([1, 3, 5])).all()
    _, rw, _ = oracle.route(x, Wr, 3)
    assert rel_err(host(wts), rw) <= TOL_F32


@pytest.mark.parametrize("E", [200, 300])
def test_route_near_ties(E):
    # a one-hot row makes each logit exactly its router entry; entries one to
    # three float32 ulps above 1.0 share the upper 32 bits of their double
    # code, so the ranking is settled by the lower halves and, on equal
    # entries, by the index (E 300 takes the arg-max rounds instead)
    banner("route near ties E=%d" % E)
    d, k = 64, 8
    rng = np.random.default_rng(9)
    x = np.zeros((1, d), np.float32)
    x[0, 5] = 1.0
    Wr = (0.01 * synthetic.normal(rng, E, d)).astype(np.float32)
    col = np.float32(1.0) + rng.integers(0, 4, E).astype(np.float32) * np.float32(2.0 ** -23)
    col[::9] = np.float32(0.5)
    Wr[:, 5] = col
    idx, wts = q8.moe_route_topk(dev(x), dev(Wr), k)
    logits = col.astype(np.float64)
    want = np.lexsort((np.arange(E), -logits))[:k]
    assert list(host(idx)[0]) == list(want)
    p = np.exp(logits[want] - logits[want[0]])
    assert rel_err(host(wts)[0], p / p.sum()) <= TOL_F32


def _code_order(l):
    """The documented rank of logits that may hold NaN or infinity: the
    order-preserving code of each double (-0 as +0; a NaN above +inf when its
    sign bit is clear, below -inf when set), ties to the lower index."""
    b = np.where(l == 0.0, 0.0, l).view(np.uint64)
    sign = (b >> np.uint64(63)).astype(bool)
    code = np.where(sign, ~b, b | np.uint64(1 << 63))
    return sorted(range(len(l)), key=lambda e: (-int(code[e]), e))


@pytest.mark.parametrize("E", [200, 300])
@pytest.mark.parametrize("with_nan", [False, True])
def test_route_non_finite_logits(E, with_nan):
    # a one-hot row makes each logit its router entry: -inf everywhere but a
    # few finite entries (and NaNs of both signs).  The choices are K distinct
    # experts in the documented rank, at E 200 (the one-pass rank) and E 300
    # (the arg-max rounds), where a retired expert must not come back.
    banner("route non-finite logits E=%d nan=%s" % (E, with_nan))
    d, k = 64, 8
    x = np.zeros((1, d), np.float32)
    x[0, 5] = 1.0
    Wr = np.zeros((E, d), np.float32)
    col = np.full(E, -np.inf, np.float32)
    col[[3, 100, E - 1, 150]] = [0.25, 1.5, -3.0, 1.5]
    if with_nan:
        col[[7, 180]] = np.float32(np.nan)
        col[11] = -np.float32(np.nan)
    Wr[:, 5] = col
    scratch = torch.zeros(q8.q8s_scratch_bytes(q8.FN_ROUTE, 1, d, 32, E, k), dtype=torch.uint8, device="cuda")
    idx, wts = q8.moe_route_topk(dev(x), dev(Wr), k, scratch=scratch)
    logits = host(scratch)[:E * 8].view(np.float64)
    got = host(idx)[0]
    assert len(set(got.tolist())) == k and got.min() >= 0 and got.max() < E
    assert list(got) == _code_order(logits)[:k]
    w = host(wts)[0]
    if with_nan:
        # a kept NaN (a NaN whose sign bit is clear ranks first) makes every
        # kept weight NaN
        assert np.isnan(logits[got]).any() and np.isnan(w).all()
    else:
        assert list(got[:4]) == [100, 150, 3, E - 1] and list(got[4:]) == [0, 1, 2, 4]
        p = np.exp(logits[got] - logits[got[0]])
        assert rel_err(w, p / p.sum()) <= TOL_F32 and (w[4:] == 0).all()


def test_route_scratch_reuse():
    # one scratch sized for 64 rows serves calls of any smaller size
    banner("route scratch reuse")
    rng = np.random.default_rng(8)
    Wr = (0.02 * synthetic.normal(rng, 128, 2048)).astype(np.float32)
    xs = [synthetic.normal(rng, r, 2048) for r in (1, 64, 1, 3)]
    scratch = torch.zeros(q8.q8s_scratch_bytes(q8.FN_ROUTE, 64, 2048, 32, 128, 8), dtype=torch.uint8, device="cuda")
    for x in xs:
        ridx, _, _ = oracle.route(x, Wr, 8)
        idx, _ = q8.moe_route_topk(dev(x), dev(Wr), 8, scratch=scratch)
        assert np.array_equal(host(idx), ridx)


# ---------------------------------------------------------------------------
# the MoE block


def run_moe_gpu(m, act):
    """The GPU pipeline: route (f32 x), [quantise x], gate-up, down-combine."""
    x = dev(m.x)
    Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds = (dev(a) for a in (m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds))
    idx, wts = q8.moe_route_topk(x, Wr, m.k)
    if act == q8.ACT_F32:
        h, _, _ = q8.moe_gate_up(Wgq, Wgs, Wuq, Wus, idx, m.E, x=x, act=act)
        y = q8.moe_down_combine(Wdq, Wds, idx, wts, m.E, h=h, act=act)
    else:
        xq, xs = q8.q8_quantize_rows(x)
        h, hq, hs = q8.moe_gate_up(Wgq, Wgs, Wuq, Wus, idx, m.E, xq=xq, xs=xs, act=act)
        # the hidden row's Q8_0 form is the quantiser's encoding of h
        rq, rs = q8.q8_quantize_rows(h.reshape(-1, h.shape[-1]))
        assert torch.equal(hq.reshape(rq.shape), rq) and torch.equal(hs.reshape(rs.shape), rs)
        y = q8.moe_down_combine(Wdq, Wds, idx, wts, m.E, hq=hq, hs=hs, act=act)
    return host(idx), host(wts), host(h), host(y)


MOE_SMALL = [
    dict(d=96, dff=160, E=5, k=3, rows=1),
    dict(d=768, dff=256, E=6, k=2, rows=1),
    dict(d=256, dff=96, E=4, k=4, rows=2),
    dict(d=2048, dff=768, E=16, k=8, rows=3),
    dict(d=64, dff=14336 // 4, E=3, k=1, rows=1),
    # 352 int8 tiles of 32 hidden outputs, more than the 256 CUs: the gate-up
    # takes its 8-wave shape
    dict(d=2048, dff=1408, E=12, k=8, rows=1),
]


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("shape", MOE_SMALL, ids=lambda s: "d%(d)d_dff%(dff)d_E%(E)d_k%(k)d_r%(rows)d" % s)
def test_moe_block_small(shape, act):
    banner("moe small %s act=%d" % (shape, act))
    m = synthetic.moe_inputs(9, shape["d"], shape["dff"], shape["E"], shape["k"], shape["rows"])
    ridx, rw, rh, ry = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, m.k, act)
    idx, wts, h, y = run_moe_gpu(m, act)
    tol = TOL_F32 if act == 0 else TOL_I8
    assert np.array_equal(idx, ridx)
    assert rel_err(wts, rw) <= TOL_F32
    assert rel_err(h, rh) <= tol
    assert rel_err(y, ry) <= tol


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("name", ["moe_d2048_dff768_e128_k8", "moe_d4096_dff14336_e8_k2"])
def test_moe_block_full_size(name, act):
    cfg = synthetic.CONFIGS[name]
    banner("moe full %s act=%d" % (name, act))
    m = synthetic.moe_inputs(0, cfg["d"], cfg["dff"], cfg["E"], cfg["k"], 1)
    ridx, rw, rh, ry = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, m.k, act)
    idx, wts, h, y = run_moe_gpu(m, act)
    tol = TOL_F32 if act == 0 else TOL_I8
    assert np.array_equal(idx, ridx)
    assert rel_err(h, rh) <= tol
    assert rel_err(y, ry) <= tol


def test_moe_invalid_expert_index_contributes_zero():
    banner("moe invalid idx")
    m = synthetic.moe_inputs(10, 64, 64, 4, 2, 1)
    Wgq, Wgs, Wuq, Wus, Wdq, Wds = (dev(a) for a in (m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds))
    idx = dev(np.array([[-1, 7]], np.int32))
    wts = dev(np.array([[0.5, 0.5]], np.float32))
    h, _, _ = q8.moe_gate_up(Wgq, Wgs, Wuq, Wus, idx, 4, x=dev(m.x))
    y = q8.moe_down_combine(Wdq, Wds, idx, wts, 4, h=h)
    assert not host(h).any() and not host(y).any()
    hq = dev(np.ones((1, 2, 64), np.int8))
    hs = dev(np.ones((1, 2, 2), np.float32))
    y = q8.moe_down_combine(Wdq, Wds, idx, wts, 4, hq=hq, hs=hs, act=q8.ACT_INT8)
    assert not host(y).any()


@pytest.mark.parametrize("rows,E,k", [(150, 2, 1), (200, 3, 3), (70, 5, 2)])
def test_chunk_many_choices_per_expert(rows, E, k):
    # more than 64 choices of one expert: the grouped kernels take several
    # passes over the expert's list
    banner("chunk passes rows=%d E=%d k=%d" % (rows, E, k))
    m = synthetic.moe_inputs(12, 128, 96, E, k, rows)
    ridx, rw, rh, ry = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, m.k, 1)
    idx, wts, h, y = run_moe_gpu(m, 1)
    assert np.array_equal(idx, ridx)
    assert rel_err(h, rh) <= TOL_I8
    for r in range(rows):
        assert rel_err(y[r], ry[r]) <= TOL_I8, r


@pytest.mark.parametrize("k", [12, 32])
def test_chunk_combine_many_slots(k):
    # the per-row combine takes the slots in batches of 8 (k = 12: a full
    # batch and a ragged one; k = 32: the most kept, four batches); the sum
    # still runs in slot order
    banner("chunk combine k=%d" % k)
    m = synthetic.moe_inputs(13, 128, 96, 40, k, 24)
    ridx, rw, rh, ry = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, m.k, 1)
    idx, wts, h, y = run_moe_gpu(m, 1)
    assert np.array_equal(idx, ridx)
    assert rel_err(h, rh) <= TOL_I8
    for r in range(m.x.shape[0]):
        assert rel_err(y[r], ry[r]) <= TOL_I8, r


# Chunks of 8 and more choices an expert on average, in rows of whole
# 256-byte groups, run their gate-up and down projection on the matrix cores:
# 16 weight rows a wave against tiles of 32 staged choice rows (16 where 32
# would not fit the staging LDS), several tiles for an expert with more.
WIDE_CASES = [
    (150, 2, 1, 256, 256),     # 75 choices an expert: three tiles, the last ragged
    (200, 3, 3, 512, 256),     # 200 an expert: seven tiles
    (70, 5, 2, 256, 512),      # 28 an expert, unevenly spread: one tile, some experts two
    (32, 4, 2, 2048, 512),     # token rows of 2 KB, 16 choices an expert
    (40, 4, 2, 512, 4096),     # hidden rows of 4 KB: down tiles of 16 rows
]


@pytest.mark.parametrize("rows,E,k,d,dff", WIDE_CASES)
def test_chunk_wide_matches_oracle(rows, E, k, d, dff):
    banner("chunk wide rows=%d E=%d k=%d d=%d dff=%d" % (rows, E, k, d, dff))
    assert q8.q8s_moe_path(rows, d, dff, E, k, q8.ACT_INT8) == q8.PATH_GROUPED_MFMA
    m = synthetic.moe_inputs(14, d, dff, E, k, rows)
    ridx, rw, rh, ry = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, m.k, 1)
    idx, wts, h, y = run_moe_gpu(m, 1)
    assert np.array_equal(idx, ridx)
    assert rel_err(h, rh) <= TOL_I8
    for r in range(rows):
        assert rel_err(y[r], ry[r]) <= TOL_I8, r


@pytest.mark.parametrize("case", ["quarter", "most", "one_expert", "k1"])
def test_chunk_wide_invalid_expert_index(case):
    # choices given directly to the matrix-core path (8 and more an expert):
    #   quarter     24 choices over 2 experts, a quarter invalid
    #   most        48 choices, 40 invalid: the invalid row's workgroups
    #               take two tiles of 32
    #   one_expert  every valid choice on expert 1 of 4: experts 0, 2, 3
    #               have none (their workgroups only scan the list)
    #   k1          one choice a row
    # An invalid choice gets a zero hidden row and adds nothing to y.
    banner("chunk wide invalid idx: %s" % case)
    rows, E, k, d, dff = {"quarter": (12, 2, 2, 256, 256), "most": (24, 2, 2, 256, 256),
                          "one_expert": (24, 4, 2, 256, 512), "k1": (40, 4, 1, 512, 256)}[case]
    assert q8.q8s_moe_path(rows, d, dff, E, k, q8.ACT_INT8) == q8.PATH_GROUPED_MFMA
    m = synthetic.moe_inputs(15, d, dff, E, k, rows)
    Wgq, Wgs, Wuq, Wus, Wdq, Wds = (dev(a) for a in (m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds))
    xq, xs = q8.q8_quantize_rows(dev(m.x))
    rng = np.random.default_rng(16)
    idx = rng.integers(0, E, (rows, k)).astype(np.int32)
    if case == "quarter":
        idx[::4, 0] = -1
        idx[1::4, 1] = 9
    elif case == "most":
        flat = idx.reshape(-1)
        bad = rng.permutation(flat.size)[:40]
        flat[bad] = np.where(rng.random(40) < 0.5, -3, E + 5)
        assert (~((idx >= 0) & (idx < E))).sum() == 40
    elif case == "one_expert":
        idx[:] = 1
        idx[::3, 1] = -1
    else:
        idx[::5, 0] = 77
    wts = rng.random((rows, k)).astype(np.float32)
    h, hq, hs = q8.moe_gate_up(Wgq, Wgs, Wuq, Wus, dev(idx), E, xq=xq, xs=xs, act=q8.ACT_INT8)
    y = q8.moe_down_combine(Wdq, Wds, dev(idx), dev(wts), E, hq=hq, hs=hs, act=q8.ACT_INT8)
    h, y = host(h), host(y)
    xqq, xss = oracle.quantize(m.x)
    for r in range(rows):
        yref = np.zeros(d)
        for c in range(k):
            e = idx[r, c]
            if not 0 <= e < E:
                assert not h[r, c].any(), (r, c)
                continue
            sl = slice(e * dff, (e + 1) * dff)
            g = oracle.gemv_i8(m.Wgq[sl], m.Wgs[sl], xqq[r:r + 1], xss[r:r + 1])
            u = oracle.gemv_i8(m.Wuq[sl], m.Wus[sl], xqq[r:r + 1], xss[r:r + 1])
            hid = (g / (1 + np.exp(-g)) * u)
            assert rel_err(h[r, c], hid[0]) <= TOL_I8, (r, c)
            hqq, hss = oracle.quantize(h[r, c][None])
            yref += wts[r, c] * oracle.gemv_i8(m.Wdq[e * d:(e + 1) * d], m.Wds[e * d:(e + 1) * d], hqq, hss)[0]
        assert rel_err(y[r], yref) <= TOL_I8, r


def test_chunk_invalid_expert_index():
    banner("chunk invalid idx")
    m = synthetic.moe_inputs(13, 64, 64, 4, 2, 3)
    Wgq, Wgs, Wuq, Wus, Wdq, Wds = (dev(a) for a in (m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds))
    xq, xs = q8.q8_quantize_rows(dev(m.x))
    idx = dev(np.array([[-1, 1], [9, 4], [2, 0]], np.int32))
    wts = dev(np.full((3, 2), 0.5, np.float32))
    h, hq, hs = q8.moe_gate_up(Wgq, Wgs, Wuq, Wus, idx, 4, xq=xq, xs=xs, act=q8.ACT_INT8)
    y = q8.moe_down_combine(Wdq, Wds, idx, wts, 4, hq=hq, hs=hs, act=q8.ACT_INT8)
    h, hq, y = host(h), host(hq), host(y)
    assert not h[0, 0].any() and not h[1].any() and not hq[1].any()
    assert h[0, 1].any() and h[2].any()
    assert not y[1].any()
    # row 2 (choices 2 and 0, weights 0.5): the oracle's pieces, expert by
    # expert -- int8 gate/up dots over the stacked rows, h in float32, h
    # quantised, int8 down dots
    xr = m.x[2:3]
    g, u = (oracle.gemv_i8(W, S, *oracle.quantize(xr)) for W, S in ((m.Wgq, m.Wgs), (m.Wuq, m.Wus)))
    hid = (g / (1 + np.exp(-g)) * u).astype(np.float32).reshape(4, 64)
    yref = np.zeros(64)
    for e in (2, 0):
        hqq, hss = oracle.quantize(hid[e:e + 1])
        yref += 0.5 * oracle.gemv_i8(m.Wdq[e * 64:(e + 1) * 64], m.Wds[e * 64:(e + 1) * 64], hqq, hss)[0]
    assert rel_err(y[2], yref) <= TOL_I8


def test_moe_deterministic():
    banner("moe determinism")
    m = synthetic.moe_inputs(11, 2048, 768, 32, 8, 1)
    a = run_moe_gpu(m, 1)
    b = run_moe_gpu(m, 1)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


# ---------------------------------------------------------------------------
# the 64-row prefill chunk: MoE over expert-grouped rows + dense GEMM


def test_chunk_full_size():
    cfg = synthetic.CONFIGS["chunk64_moe_d2048_dense4096"]
    banner("chunk 64 rows, int8")
    m, Dq, Ds = synthetic.chunk_inputs(0, cfg["d"], cfg["dff"], cfg["E"], cfg["k"], cfg["rows"], cfg["n_dense"])
    ridx, rw, rh, ry = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, m.k, 1)
    idx, wts, h, y = run_moe_gpu(m, 1)
    assert np.array_equal(idx, ridx)
    for r in range(cfg["rows"]):
        assert rel_err(y[r], ry[r]) <= TOL_I8, r
    # the dense projection of the same rows' Q8_0 form
    xq, xs = q8.q8_quantize_rows(dev(m.x))
    rq, rs = oracle.quantize(m.x)
    assert np.array_equal(host(xq), rq) and np.array_equal(host(xs), rs)
    Y = host(q8.q8_gemv(dev(Dq), dev(Ds), xq=xq, xs=xs, act=q8.ACT_INT8))
    ref = oracle.gemv_i8(Dq, Ds, rq, rs)
    for r in range(cfg["rows"]):
        assert rel_err(Y[r], ref[r]) <= TOL_I8, r


def test_chunk_gate_up_without_q8_pass():
    # a chunk's gate-up may leave out the hidden rows' Q8_0 pass: the float32
    # rows are the same bits, and quantising them afterwards gives the pass's
    # words and scales
    banner("chunk gate-up without the Q8_0 pass")
    m = synthetic.moe_inputs(7, 2048, 768, 128, 8, rows=64)
    xq, xs = q8.q8_quantize_rows(dev(m.x))
    idx, _ = q8.moe_route_topk(dev(m.x), dev(m.Wr), m.k)
    W = [dev(a) for a in (m.Wgq, m.Wgs, m.Wuq, m.Wus)]
    h1, hq1, hs1 = q8.moe_gate_up(*W, idx, m.E, xq=xq, xs=xs, act=q8.ACT_INT8)
    h2, hq2, hs2 = q8.moe_gate_up(*W, idx, m.E, xq=xq, xs=xs, act=q8.ACT_INT8, want_q8=False)
    assert hq2 is None and hs2 is None
    assert torch.equal(h1, h2)
    q3, s3 = q8.q8_quantize_rows(h2.reshape(-1, 768))
    assert torch.equal(q3.reshape(hq1.shape), hq1) and torch.equal(s3.reshape(hs1.shape), hs1)
