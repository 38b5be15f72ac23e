"""The C-ABI layer's host code under AddressSanitizer and UndefinedBehavior-
Sanitizer: the library is rebuilt with both sanitizers on its host pass only
(device code is built as usual), and the host-side ABI tests -- argument
checks, workspace sizing and carving, error reporting, every exported symbol
-- run against it in a child process that preloads the sanitizer runtime.
Any sanitizer report fails the test.  No GPU is touched: every call here is
rejected or answered on the host before a launch."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_DIR = os.path.join(ROOT, "_build", "host_sanitizers")
SAN_LIB = os.path.join(SAN_DIR, "libmoe_w8a16_san.so")

# host pass only: each flag follows -Xarch_host
HOST_SAN_FLAGS = []
for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer"):
    HOST_SAN_FLAGS += ["-Xarch_host", f]

DRIVER = r"""
import sys
sys.path.insert(0, {root!r})
from block_scaled_fp8_amd import binding
binding.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu",
                      {abi!r}]))
"""


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.timeout(900)
def test_abi_layer_under_host_sanitizers():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime in this ROCm install")
    from block_scaled_fp8_amd import build
    try:
        build._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    build.build_library(extra_flags=HOST_SAN_FLAGS, lib_path=SAN_LIB, build_dir=SAN_DIR)
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = DRIVER.format(root=ROOT, lib=SAN_LIB, abi=os.path.join(ROOT, "tests", "test_abi.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
