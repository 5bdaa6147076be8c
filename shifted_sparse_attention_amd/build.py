"""Build libs2attn.so in-tree for gfx950.

    python -m shifted_sparse_attention_amd.build

Compiles every source under csrc/ with hipcc for gfx950 and links the shared
library against the HIP runtime that torch ships (torch/lib/libamdhip64.so),
with an rpath to it, so that a process which imports torch maps a single HIP
runtime and stream handles from torch are valid inside the library.  When
torch is not importable the ROCm install's runtime is used instead.
"""

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libs2attn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

# Packed fp32 instructions are kept out of the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]


def _hipcc():
    p = os.path.join(ROCM, "bin", "hipcc")
    return p if os.path.exists(p) else shutil.which("hipcc")


def _clangxx():
    p = os.path.join(ROCM, "lib", "llvm", "bin", "clang++")
    return p if os.path.exists(p) else shutil.which("clang++")


def hip_runtime_dir():
    """Directory of the libamdhip64.so to link against (torch's when available)."""
    try:
        import torch  # noqa: F401
        d = os.path.join(os.path.dirname(torch.__file__), "lib")
        if os.path.exists(os.path.join(d, "libamdhip64.so")):
            return d
    except Exception:
        pass
    return os.path.join(ROCM, "lib")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def build(verbose=False, extra_flags=()):
    hipcc, clangxx = _hipcc(), _clangxx()
    if hipcc is None or clangxx is None:
        raise RuntimeError("hipcc / clang++ not found under ROCM_PATH")
    rt = hip_runtime_dir()
    objs = []
    with tempfile.TemporaryDirectory(prefix="s2attn_build_") as tmp:
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmd = [hipcc, *COMMON, *DEVICE_FLAGS, *extra_flags, *lang, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            errs = [ln for ln in (res.stderr or "").splitlines()
                    if "packed-fp32-ops" not in ln]
            if res.returncode != 0:
                raise RuntimeError(f"compile failed: {src}\n" + "\n".join(errs))
            if verbose and errs:
                print("\n".join(errs), flush=True)
            objs.append(obj)
        tmp_lib = LIB_PATH + ".tmp"
        # hipBLASLt (the attention block's projection GEMMs) from the same
        # directory as the HIP runtime, so both come from one ROCm release.
        cmd = [clangxx, "-shared", "-fPIC", *objs, "-o", tmp_lib,
               f"-L{rt}", "-l:libamdhip64.so", "-l:libhipblaslt.so", f"-Wl,-rpath,{rt}",
               f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-Wl,--no-undefined",
               "-Wl,-soname," + LIB_NAME]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed\n" + res.stderr)
        os.replace(tmp_lib, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
