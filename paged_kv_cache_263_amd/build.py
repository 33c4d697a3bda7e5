"""Build libpagedkv.so (host allocator + gfx950 kernels + C ABI) in-tree.

    python paged_kv_cache_263_amd/build.py        # or build() from Python

(Run it by path: ``python -m`` would import the package, which loads the
library this script is about to rebuild.)

Every source is compiled with hipcc for gfx950 only.  Packed fp32 arithmetic
is switched off for device code (ordinary fp32 code is compiled to scalar fp32
instructions), fp32 division is the correctly rounded one, which the fp8
quantiser relies on, and matrix-core accumulators are kept in VGPRs.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpagedkv.so")

SOURCES = ["errors.cpp", "checks.cpp", "pool.cpp", "decode.hip", "prefill.hip", "cache_ops.hip", "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # keep matrix-core accumulators in VGPRs, so the softmax rescale of the
    # accumulators needs no AGPR<->VGPR copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless.
    noise = ("packed-fp32-ops", "unknown target feature", "warning generated", "warnings generated")
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if l.strip() and not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg:
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library; returns its path."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
