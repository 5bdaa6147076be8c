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
