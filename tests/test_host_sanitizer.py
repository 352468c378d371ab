"""The library's host-side validation under AddressSanitizer and UndefinedBehaviorSanitizer:
tests/test_abi.py (every entry point's argument checks, no GPU needed) rerun in a child
process against libcsahca_hostsan.so, with the ASan runtime preloaded and any report
fatal."""
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

SAN_LIB = os.path.join(ROOT, "compressed_attention_compress_amd", "libcsahca_hostsan.so")


def asan_runtime():
    try:
        out = subprocess.run(["/opt/rocm/bin/hipcc", "-print-file-name=libclang_rt.asan-x86_64.so"],
                             capture_output=True, text=True, timeout=60).stdout.strip()
    except (OSError, subprocess.SubprocessError):
        return None
    return out if out and os.path.isabs(out) and os.path.exists(out) else None


def test_abi_validation_under_asan_and_ubsan():
    if not os.path.exists(SAN_LIB):
        pytest.fail("libcsahca_hostsan.so is not built (run __graft_entry__.build())")
    rt = asan_runtime()
    assert rt, "the ASan runtime of the ROCm clang was not found"
    env = dict(os.environ, CSAHCA_LIB=SAN_LIB, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
    print(res.stdout.strip().splitlines()[-1])
