"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with its host code (argument validation, split
planning, workspace sizes, dispatch) instrumented (-fsanitize=address and
-fsanitize=undefined on the host pass only, errors fatal), and the whole of
tests/test_boundary.py runs against that build in a child process with the
sanitizer runtime preloaded.  No call there passes validation, so nothing is
launched; any out-of-bounds access, use after free or undefined arithmetic
(signed overflow, bad shifts) on the host fails the run.  This is how two
signed overflows in split planning for stream counts near the int32 limit
were found."""
import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.skipif(_asan_runtime() is None, reason="no clang AddressSanitizer runtime")
def test_boundary_suite_clean_under_host_sanitizers():
    sys.path.insert(0, ROOT)
    from vector_quantized_bit_amd import build as b

    with tempfile.TemporaryDirectory() as tmp:
        lib = b.build_host_sanitized(os.path.join(tmp, "libvqkv_hostsan.so"))
        logs = os.path.join(tmp, "san")
        env = dict(os.environ,
                   LD_PRELOAD=_asan_runtime(),
                   ASAN_OPTIONS=f"detect_leaks=0:log_path={logs}",
                   UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={logs}",
                   VQKV_LIBRARY=lib)
        r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests",
                                                                         "test_boundary.py"),
                            "-q", "-p", "no:cacheprovider"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        reports = "".join(open(f).read() for f in glob.glob(logs + "*"))
        assert r.returncode == 0 and not reports, (r.stdout[-3000:], reports[:3000])
        assert " passed" in r.stdout
