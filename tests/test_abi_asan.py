"""The C ABI's host-side argument handling under AddressSanitizer (CPU only).

The translation unit holding every entry point (csrc/api.hip) is compiled
with host-only ASan instrumentation (the device code is compiled as usual),
linked with the library's other objects into _build/asan/libmoeglu_asan.so,
and the argument-validation calls of test_abi.py run against it in a child
Python process that preloads the ASan runtime.  Any out-of-bounds read of the
caller's host structs or a use of freed memory on those paths aborts the
child with an ASan report.  No GPU is touched: every call returns its status
before anything would launch.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_DIR = os.path.join(ROOT, "_build", "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libmoeglu_asan.so")


def _build_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_moeglu_build", os.path.join(ROOT, "grouped_gemm_glu_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _asan_runtime():
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return libs[-1] if libs else None


@pytest.fixture(scope="module")
def asan_lib():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no ASan runtime in this ROCm installation")
    b = _build_module()
    try:
        b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    return b.build_host_asan(), rt


def test_asan_library_is_instrumented(asan_lib):
    lib, _ = asan_lib
    out = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    assert out.returncode == 0, out.stderr
    assert "__asan_" in out.stdout, "the host code was not built with AddressSanitizer"


CHILD = r"""
import ctypes, sys
sys.path.insert(0, {root!r})
import grouped_gemm_glu_amd as G
lib = ctypes.CDLL({lib!r})
for name, (args, res) in G._SIGS.items():
    f = getattr(lib, name)
    f.argtypes = args
    f.restype = res
G._lib = lib
from tests import test_abi
test_abi.test_status_strings()
test_abi.test_host_argument_errors_return_before_launch()
print("asan-child-ok")
"""


def test_host_argument_checks_clean_under_asan(asan_lib):
    lib, rt = asan_lib
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=0"
    env["HIP_VISIBLE_DEVICES"] = ""
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, lib=lib)], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=300)
    assert "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0 and "asan-child-ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
