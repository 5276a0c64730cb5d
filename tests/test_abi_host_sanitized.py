"""The CPU ABI tests again, against the build whose host code (the C ABI layer:
argument validation, workspace layouts, launch set-up) is compiled with
AddressSanitizer and UndefinedBehaviorSanitizer (``build_host_sanitized``),
with the ASan runtime preloaded into a child interpreter. Any sanitizer report
fails the child (UBSan is built not to recover). No GPU is needed: the ABI
tests only pass arguments that validation rejects."""

import glob
import os
import subprocess
import sys

import pytest

from adaptive_sparse_long_amd import build as _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_under_host_sanitizers(tmp_path):
    if not os.path.exists(_build.SAN_LIB):
        pytest.skip("the host-sanitized library is not built (python -m adaptive_sparse_long_amd.build --host-sanitize)")
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this ROCm toolchain")
    log = tmp_path / "san"
    env = dict(os.environ, DASH_LIB=_build.SAN_LIB, LD_PRELOAD=rt,
               ASAN_OPTIONS=f"detect_leaks=0:log_path={log}", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = "".join(open(f).read() for f in glob.glob(str(log) + "*"))
    assert res.returncode == 0 and not reports, (res.stdout[-2000:] + res.stderr[-2000:] + reports)
