"""Seeded synthetic inputs for the Q8_0 GEMV / sparse-MoE hot path.

This module only draws random numbers: it holds none of the method's
arithmetic (no dequantisation, no quantiser, no routing).  Both the CPU oracle
(under ``oracle/``) and the HIP path read their inputs from here, so a test can
hand the very same arrays to each side.

Distributions follow the workload recipe of the Q8_0 weight rows described on
the ``codegen_cuda::qwen_emit`` module page (struct ``Q8Ref``: int8 quants, row
major, plus one f32 scale per 32 inputs in a separate array) and the stacked
expert layout of struct ``MoeWeights`` on the same page (router ``[E, d]``,
gate/up ``[E*dff, d]``, down ``[E*d, dff]``):

* quants: uniform integers in [-127, 127];
* block scales: uniform in [1e-3, 1e-2], float32;
* activations, residuals: standard normal, float32;
* router: 0.02 * standard normal, float32;
* RMSNorm weight: uniform in [0.5, 1.5], float32.

Every generator takes a ``numpy.random.Generator`` or a seed and draws in the
order its docstring lists, so a given seed always reproduces the same arrays.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

QBLOCK = 32


def _rng(seed_or_rng):
    if isinstance(seed_or_rng, np.random.Generator):
        return seed_or_rng
    return np.random.default_rng(seed_or_rng)


def quants(rng, rows, cols):
    return rng.integers(-127, 127, size=(rows, cols), endpoint=True, dtype=np.int8)


def scales(rng, rows, cols):
    assert cols % QBLOCK == 0
    return rng.uniform(1e-3, 1e-2, size=(rows, cols // QBLOCK)).astype(np.float32)


def normal(rng, *shape):
    return rng.standard_normal(shape, dtype=np.float32)


def q8_matrix(rng, rows, cols):
    """Draws quants then scales of one Q8_0 matrix ``[rows, cols]``."""
    q = quants(rng, rows, cols)
    s = scales(rng, rows, cols)
    return q, s


# ---------------------------------------------------------------------------
# workloads


@dataclass
class GemvInputs:
    Wq: np.ndarray  # int8 [n_out, n_in]
    Ws: np.ndarray  # f32 [n_out, n_in/32]
    x: np.ndarray   # f32 [m, n_in]


def gemv_inputs(seed, n_out, n_in, m=1):
    """Draw order: Wq, Ws, x."""
    rng = _rng(seed)
    Wq, Ws = q8_matrix(rng, n_out, n_in)
    x = normal(rng, m, n_in)
    return GemvInputs(Wq, Ws, x)


@dataclass
class NormGemvInputs:
    w: np.ndarray   # f32 [d]  RMSNorm weight
    h: np.ndarray   # f32 [rows, d]
    r: np.ndarray   # f32 [rows, d]
    Wq: np.ndarray  # int8 [n_out, d]
    Ws: np.ndarray  # f32 [n_out, d/32]


def norm_gemv_inputs(seed, d, n_out, rows=1):
    """Draw order: w, h, r, then the GEMV's Wq, Ws."""
    rng = _rng(seed)
    w = rng.uniform(0.5, 1.5, size=d).astype(np.float32)
    h = normal(rng, rows, d)
    r = normal(rng, rows, d)
    Wq, Ws = q8_matrix(rng, n_out, d)
    return NormGemvInputs(w, h, r, Wq, Ws)


@dataclass
class MoeInputs:
    Wr: np.ndarray   # f32 [E, d]
    Wgq: np.ndarray  # int8 [E*dff, d]
    Wgs: np.ndarray  # f32 [E*dff, d/32]
    Wuq: np.ndarray
    Wus: np.ndarray
    Wdq: np.ndarray  # int8 [E*d, dff]
    Wds: np.ndarray  # f32 [E*d, dff/32]
    x: np.ndarray    # f32 [rows, d]
    d: int
    dff: int
    E: int
    k: int


def moe_weights(rng, d, dff, E):
    """Draw order: router, gate (q, s), up (q, s), down (q, s)."""
    Wr = (0.02 * rng.standard_normal((E, d), dtype=np.float32)).astype(np.float32)
    Wgq, Wgs = q8_matrix(rng, E * dff, d)
    Wuq, Wus = q8_matrix(rng, E * dff, d)
    Wdq, Wds = q8_matrix(rng, E * d, dff)
    return Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds


def moe_inputs(seed, d, dff, E, k, rows=1):
    """Draw order: the weights as ``moe_weights`` lists, then x ``[rows, d]``."""
    rng = _rng(seed)
    Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds = moe_weights(rng, d, dff, E)
    x = normal(rng, rows, d)
    return MoeInputs(Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds, x, d, dff, E, k)


def chunk_inputs(seed, d, dff, E, k, rows, n_dense):
    """A prefill chunk: the MoE block's weights and rows ``X`` (as
    ``moe_inputs`` with ``rows`` rows), then a dense Q8_0 matrix
    ``[n_dense, d]`` (quants, scales) drawn from the same generator."""
    rng = _rng(seed)
    Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds = moe_weights(rng, d, dff, E)
    X = normal(rng, rows, d)
    Dq, Ds = q8_matrix(rng, n_dense, d)
    return MoeInputs(Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds, X, d, dff, E, k), Dq, Ds


@dataclass
class BlockInputs:
    moe: MoeInputs   # the mixture's weights (its x is unused: the block forms x)
    w: np.ndarray    # f32 [d]  RMSNorm weight
    h: np.ndarray    # f32 [rows, d]
    r: np.ndarray    # f32 [rows, d]


def block_inputs(seed, d, dff, E, k, rows=1):
    """A whole mixture block of a layer, fed by its add + norm: draw order the
    weights as ``moe_weights`` lists, then the norm weight, h, r."""
    rng = _rng(seed)
    Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds = moe_weights(rng, d, dff, E)
    w = rng.uniform(0.5, 1.5, size=d).astype(np.float32)
    h = normal(rng, rows, d)
    r = normal(rng, rows, d)
    m = MoeInputs(Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds, None, d, dff, E, k)
    return BlockInputs(m, w, h, r)


@dataclass
class VariantInputs:
    block: BlockInputs  # the block as ``block_inputs`` draws it
    Wrq: np.ndarray     # int8 [E, d]   router rows in Q8_0 form
    Wrs: np.ndarray     # f32  [E, d/32]
    Sgq: np.ndarray     # int8 [sdff, d] shared expert gate (None when sdff = 0)
    Sgs: np.ndarray
    Suq: np.ndarray     # int8 [sdff, d] shared expert up
    Sus: np.ndarray
    Sdq: np.ndarray     # int8 [d, sdff] shared expert down
    Sds: np.ndarray
    sdff: int


def variant_inputs(seed, d, dff, E, k, rows=1, sdff=0):
    """The mixture block with its variants: ``block_inputs``' draws, then
    Q8_0 router rows (quants, then scales in [2e-4, 5e-4], so the weights
    spread about as the float router's 0.02 does), then, for sdff > 0, a
    shared expert's gate, up and down Q8_0 matrices."""
    rng = _rng(seed)
    b = block_inputs(rng, d, dff, E, k, rows)
    Wrq = quants(rng, E, d)
    Wrs = rng.uniform(2e-4, 5e-4, size=(E, d // QBLOCK)).astype(np.float32)
    S = [None] * 6
    if sdff:
        S[0], S[1] = q8_matrix(rng, sdff, d)
        S[2], S[3] = q8_matrix(rng, sdff, d)
        S[4], S[5] = q8_matrix(rng, d, sdff)
    return VariantInputs(b, Wrq, Wrs, *S, sdff)


def fill_pattern(n, scale=1.0):
    """The deterministic small-integer fill ``v[p] = (p % 7) - 3`` (optionally
    scaled) that the ``emit_forward`` item of the ``codegen_cuda::qwen_emit``
    module page uses for its inputs; every value is exact in f32."""
    p = np.arange(n, dtype=np.int64)
    return (((p % 7) - 3) * scale).astype(np.float32)


# The workloads, by name; sizes as in the project's benchmark table.
CONFIGS = {
    "gemv_512x256": dict(kind="gemv", n_out=512, n_in=256, m=1),
    "norm_gemv_2048x4096": dict(kind="norm_gemv", d=2048, n_out=4096, eps=1e-6),
    "moe_d2048_dff768_e128_k8": dict(kind="moe", d=2048, dff=768, E=128, k=8),
    "moe_d4096_dff14336_e8_k2": dict(kind="moe", d=4096, dff=14336, E=8, k=2),
    "chunk64_moe_d2048_dense4096": dict(kind="chunk", d=2048, dff=768, E=128, k=8, rows=64, n_dense=4096),
    # wider prefill chunks through the same block and projection
    "chunk128_moe_d2048_dense4096": dict(kind="chunk", d=2048, dff=768, E=128, k=8, rows=128, n_dense=4096),
    "chunk256_moe_d2048_dense4096": dict(kind="chunk", d=2048, dff=768, E=128, k=8, rows=256, n_dense=4096),
    # a mixture with an always-on shared expert four experts wide and its
    # router as Q8_0 rows (the Qwen1.5-MoE-A2.7B-like FFN shape)
    "moe_shared_d2048_dff1408_e60_k4_s5632": dict(kind="moe_shared", d=2048, dff=1408, E=60, k=4, sdff=5632),
    # four layers of the 128-expert block in a row, each with weights of its own
    "stack4_moe_d2048_dff768_e128_k8": dict(kind="stack", d=2048, dff=768, E=128, k=8, layers=4),
}
