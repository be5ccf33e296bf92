"""Builds libgptq.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

    python -m post_weight_quantization_20_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgptq.so")
SOURCES = ["abi.hip", "runtime.hip", "gemm_f32.hip", "hessian.hip", "factor.hip", "quant.hip", "dequant.hip", "block.hip", "gemm_f16.hip", "noalloc.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed fp32 instructions (v_pk_fma_f32 and friends)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the GPTQ library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build_shared(sources, out: str, verbose: bool = False, jobs: int = 5) -> str:
    """Compiles HIP sources to objects and links a shared library at `out` (replaced atomically)."""
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="gptq_build_")
    try:
        objs = [os.path.join(tmp, f"{i}_" + os.path.basename(s).replace(".hip", ".o")) for i, s in enumerate(sources)]
        cmds = [[cc, *FLAGS, "-c", s, "-o", o] for s, o in zip(sources, objs)]
        with ThreadPoolExecutor(max(1, jobs)) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        out_tmp = out + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp, *objs], verbose)
        os.replace(out_tmp, out)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return out


def build(verbose: bool = False, jobs: int = 5) -> str:
    """Builds libgptq.so from every kernel source and the C ABI."""
    return build_shared([os.path.join(CSRC, s) for s in SOURCES], LIB, verbose, jobs)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
