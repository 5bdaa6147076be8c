"""bench.py's host-side contract, on the CPU: the one-GPU guard and the
host description the CPU baseline carries."""

import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_host_info_names_cpu_numpy_and_blas():
    info = _bench_module().host_info()
    assert set(info) == {"cpu_model", "numpy", "blas"}
    assert info["numpy"]


def test_kernel_source_hash_is_stable():
    b = _bench_module()
    h = b.kernel_source_sha()
    assert h == b.kernel_source_sha() and len(h) == 16 and int(h, 16) >= 0


def test_two_step_form_is_s2attn():
    """bench.py's two-step PyTorch form (roll, fold groups into the batch, causal SDPA,
    unfold, roll back) computes S2-Attn: fp64 on the CPU it equals the oracle's group form,
    outputs and gradients, with no, some and all heads shifted."""
    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    from oracle import s2attn as ref

    two_step_form = _bench_module().two_step_form
    rng = np.random.default_rng(7)
    B, L, H, d, G = 2, 24, 4, 8, 6
    q, k, v, do = (rng.standard_normal((B, L, H, d)) for _ in range(4))
    for sh in (0, 2, 4):
        tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
        y = two_step_form(tq, tk, tv, G, sh)
        y.backward(torch.tensor(do))
        o, _ = ref.forward(q, k, v, G, sh)
        dq, dk, dv, _, _ = ref.backward(q, k, v, do, G, sh)
        for got, want in ((y.detach(), o), (tq.grad, dq), (tk.grad, dk), (tv.grad, dv)):
            np.testing.assert_allclose(got.numpy(), want, rtol=0, atol=1e-12)
