"""Helpers of the GPU parity tests: moving seeded inputs to the device and the
comparisons the tests make."""
import numpy as np
import torch


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def rel_err(got, ref):
    """max |got - ref| / max |ref|, in float64 (normalised by the largest
    reference value, so outputs near zero do not dominate)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.max(np.abs(ref))
    if scale == 0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / scale)


def f32_ambiguous(y64, rel=1e-12):
    """Elements whose float64 value lies so close to a float32 rounding
    boundary that a different (but correct) summation order may round them
    the other way."""
    y64 = np.asarray(y64, np.float64)
    lo = (y64 * (1 - rel)).astype(np.float32)
    hi = (y64 * (1 + rel)).astype(np.float32)
    return lo != hi


def route_ambiguous(logits, k, rel=1e-12):
    """Rows where two logits that decide the kept set or its order differ, but
    by no more than rel * max|l|: double sums in another order may rank them
    the other way.  Exactly equal logits are not ambiguous (both sides keep the
    lower index)."""
    out = np.zeros(logits.shape[0], bool)
    for i, l in enumerate(logits):
        order = np.lexsort((np.arange(len(l)), -l))
        top = l[order[: min(k + 1, len(l))]]
        gaps = np.abs(np.diff(top))
        # exact ties are decided the same way on both sides (lower index)
        out[i] = bool(np.any((gaps > 0) & (gaps <= rel * np.max(np.abs(l)))))
    return out
