"""Build libpagedkv.so (host allocator + gfx950 kernels + C ABI) in-tree.

    python paged_kv_cache_263_amd/build.py        # or build() from Python
    python paged_kv_cache_263_amd/build.py --sanitize
        # host code built with AddressSanitizer + UndefinedBehaviorSanitizer
        # into _build/sanitize/libpagedkv.so, then the CPU tests of the C ABI
        # (tests/test_abi.py) run against it (no GPU needed)

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


# Sanitizers apply to the host pass only (-Xarch_host before each option):
# the allocator, the argument checks and the launch code are host C++; device
# code is built as usual.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-g"]
SANITIZE_DIR = os.path.join(BUILD, "sanitize")


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(SANITIZE_DIR if sanitize else BUILD, src + ".o")
    cmd = [HIPCC, *FLAGS, *(SANITIZE_FLAGS if sanitize else []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless.
    noise = ("packed-fp32-ops", "unknown target feature", "warning generated", "warnings generated")
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if l.strip() and not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg:
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library; returns its
    path (with ``sanitize``, the ASan/UBSan host build under _build/sanitize)."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    out_dir = SANITIZE_DIR if sanitize else BUILD
    lib = os.path.join(SANITIZE_DIR, "libpagedkv.so") if sanitize else LIB
    os.makedirs(out_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    if sanitize:
        cmd += ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime (it carries the UBSan handlers too)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang's ASan runtime not found")
    return path


def run_sanitized_abi_tests() -> int:
    """Build the sanitized library and run the C ABI's CPU tests against it, in
    a child process with the ASan runtime preloaded (Python itself is not
    instrumented, so leak checking is off; any ASan or UBSan report aborts)."""
    lib = build(verbose=True, sanitize=True)
    env = dict(os.environ)
    env.update({
        "PKV_LIBRARY": lib,
        "LD_PRELOAD": asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi.py"),
           os.path.join(ROOT, "tests", "test_prefix_cache_traffic.py")]
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


def resource_usage() -> str:
    """Per-kernel registers, scratch, LDS and occupancy as the compiler reports
    them (-Rpass-analysis=kernel-resource-usage) for the device code of every
    .hip source, as a text table."""
    import re

    rows = []
    for src in SOURCES:
        if not src.endswith(".hip"):
            continue
        cmd = [HIPCC, *FLAGS, "--cuda-device-only", "-Rpass-analysis=kernel-resource-usage", "-c",
               os.path.join(CSRC, src), "-o", os.devnull]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        cur = None
        for line in r.stderr.splitlines():
            m = re.search(r"remark: (?:\s*)([^:]+?): (.+?) \[-Rpass-analysis", line)
            if not m:
                continue
            key, val = m.group(1).strip(), m.group(2).strip()
            if key == "Function Name":
                dem = subprocess.run(["c++filt", val], capture_output=True, text=True).stdout.strip() or val
                dem = dem.replace("pkv::(anonymous namespace)::", "").replace("(pkv::(anonymous namespace)::", "(")
                cur = {"src": src, "kernel": dem}
                rows.append(cur)
            elif cur is not None:
                cur[key] = val
    cols = [("kernel", "kernel"), ("VGPRs", "VGPR"), ("AGPRs", "AGPR"), ("TotalSGPRs", "SGPR"),
            ("ScratchSize [bytes/lane]", "scratch B/lane"), ("VGPRs Spill", "VGPR spill"),
            ("SGPRs Spill", "SGPR spill"), ("LDS Size [bytes/block]", "LDS B/block"),
            ("Occupancy [waves/SIMD]", "waves/SIMD")]
    out = ["| source | " + " | ".join(h for _, h in cols) + " |", "|---" * (len(cols) + 1) + "|"]
    for r in rows:
        out.append(f"| {r['src']} | " + " | ".join(str(r.get(k, "")) for k, _ in cols) + " |")
    return "\n".join(out)


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        sys.exit(run_sanitized_abi_tests())
    if "--resource-usage" in sys.argv[1:]:
        print(resource_usage())
        sys.exit(0)
    build(verbose=True)
