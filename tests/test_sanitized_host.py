"""The host code of the library (allocator, prefix cache, swap bookkeeping,
argument checks) under AddressSanitizer and UndefinedBehaviorSanitizer: the
library is rebuilt with both on its host pass, and the C ABI's CPU tests run
against that build in a child process (the ASan runtime preloaded; any report
aborts the child).  No GPU is used."""

import importlib.util
import os
import shutil

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
def test_abi_tests_pass_under_asan_and_ubsan():
    spec = importlib.util.spec_from_file_location("_pkv_build", os.path.join(ROOT, "paged_kv_cache_263_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert mod.run_sanitized_abi_tests() == 0
