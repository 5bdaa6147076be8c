"""Helpers for the GPU parity tests: device upload, error metrics, tolerances."""

import math
import sys

import numpy as np
import torch

# bf16 outputs and gradients: relative Frobenius error and max-abs error.
BF16_REL_F = 5e-3
BF16_MAX_ABS = 2e-2
# fp32 path.
F32_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x, dtype):
    """float32 numpy -> device tensor of `dtype` (values already representable)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).cuda()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def errs(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    assert np.isfinite(x).all(), "non-finite values in GPU output"
    diff = x - ref
    nrm = np.linalg.norm(ref)
    rel = float(np.linalg.norm(diff) / nrm) if nrm > 0 else float(np.linalg.norm(diff))
    return rel, float(np.max(np.abs(diff))) if diff.size else 0.0


def bf16_half_ulp(maxabs):
    """Half a bf16 ulp at magnitude `maxabs` (the rounding floor of a bf16 store)."""
    if maxabs <= 0:
        return 0.0
    e = math.floor(math.log2(maxabs))
    return 2.0 ** (e - 7) / 2


def bf16_store_tol(ref):
    """Max-abs bound for a bf16-stored result: the 2e-2 tolerance on the computed
    value plus half a bf16 ulp at the reference's largest magnitude (the store's
    own rounding, which alone exceeds 2e-2 once |x| >= 8)."""
    return BF16_MAX_ABS + bf16_half_ulp(float(np.max(np.abs(ref))))


def check(name, x, ref, rel_tol, abs_tol):
    rel, mx = errs(x, ref)
    say(f"  {name:10s} rel_F={rel:.3e} max_abs={mx:.3e} (max|ref|={np.max(np.abs(ref)):.3f})")
    assert rel <= rel_tol, f"{name}: rel_F {rel} > {rel_tol}"
    assert mx <= abs_tol, f"{name}: max_abs {mx} > {abs_tol}"
    return rel, mx
