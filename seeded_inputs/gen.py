"""Seeded input generation.

Draw order is fixed: q, k, v, then dO (when the workload has a backward), each
`standard_normal(shape, dtype=float32)` from one `numpy.random.default_rng(seed)`
stream (PCG64). For bf16 workloads every draw is rounded to bf16 with
round-to-nearest-even; the rounded values (held exactly in float32) are what
both the GPU path and the oracle consume.
"""

import numpy as np


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of float32 `x`, round-to-nearest-even.

    Inputs are finite normal draws, so no NaN handling is needed; a NaN input
    raises rather than being silently rounded.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.isfinite(x).all():
        raise ValueError("bf16_bits: non-finite input")
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 array holding the bf16-rounded (RNE) values of `x`."""
    b = bf16_bits(x).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def make_inputs(wl, seed=None, with_grad=None):
    """Return a dict of float32 arrays q, k, v (and do) for workload `wl`.

    Layout is [B, L, H, d], contiguous. For bf16 workloads the values are
    already bf16-representable.
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    with_grad = wl.backward if with_grad is None else with_grad
    shapes = [("q", wl.q_shape()), ("k", wl.kv_shape()), ("v", wl.kv_shape())]
    if with_grad:
        shapes.append(("do", wl.q_shape()))
    out = {}
    for name, shp in shapes:
        x = rng.standard_normal(shp, dtype=np.float32)
        if wl.dtype == "bf16":
            x = bf16_round(x)
        out[name] = x
    return out
