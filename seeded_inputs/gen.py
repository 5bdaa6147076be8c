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


BLOCK_PARAM_ORDER = ("wq", "wk", "wv", "wo", "aq", "ak", "av", "ao", "bq", "bk", "bv", "bo")


def make_block_inputs(wl, seed=None, scale_up=0.25):
    """x, dy and the block's weights for a BlockWorkload, rounded to bf16.

    Draw order from one default_rng(seed) stream: x, then the weights in
    BLOCK_PARAM_ORDER, then dy; all standard normals in float32.  A weight
    with fan-in n is scaled by 1/sqrt(n) before rounding, so q, k, v and y are
    O(1).  The LoRA up-projections (B) are random too, so the adapter path
    carries signal (they would start at zero in training), at `scale_up` of
    that scale: the adapters perturb the frozen projections rather than
    dominate them.
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    Dm, Nq, Nkv, r = wl.Hq * wl.d, wl.Hq * wl.d, wl.Hkv * wl.d, wl.lora_rank
    shapes = {"wq": (Nq, Dm), "wk": (Nkv, Dm), "wv": (Nkv, Dm), "wo": (Dm, Nq),
              "aq": (r, Dm), "ak": (r, Dm), "av": (r, Dm), "ao": (r, Nq),
              "bq": (Nq, r), "bk": (Nkv, r), "bv": (Nkv, r), "bo": (Dm, r)}
    out = {"x": bf16_round(rng.standard_normal((wl.B, wl.L, Dm), dtype=np.float32))}
    p = {}
    for name in BLOCK_PARAM_ORDER:
        shp = shapes[name]
        w = rng.standard_normal(shp, dtype=np.float32) * np.float32(1.0 / np.sqrt(shp[1]))
        p[name] = bf16_round(w * np.float32(scale_up if name[0] == "b" else 1.0))
    out["params"] = p
    out["dy"] = bf16_round(rng.standard_normal((wl.B, wl.L, Dm), dtype=np.float32))
    return out
