"""Host-side AddressSanitizer run of the C ABI's argument handling (CPU only).

libmxq is rebuilt with AddressSanitizer on its host code (the device code is
unchanged) and the whole C-ABI battery of test_boundary.py -- every entry point
with null, misaligned, out-of-range and too-small arguments, the workspace size
functions at extreme sizes, the status strings -- runs against it in a
subprocess with the ASan runtime preloaded.  Any heap or stack error in the
validation code fails the run.  No call reaches the GPU: each either fails
validation or is a no-op.
"""
import glob
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.slow
def test_c_abi_validation_under_host_asan(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no ASan runtime in this ROCm install")
    sys.path.insert(0, ROOT)
    from float8_quantization_moe_amd import build
    lib = build.build_host_asan(str(tmp_path))
    env = dict(os.environ, LD_PRELOAD=rt, MXQ_TEST_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:exitcode=99")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(HERE, "test_boundary.py"), "-k", "not missing_library"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
