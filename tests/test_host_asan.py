"""The library's host code under AddressSanitizer (CPU only).

Builds the library with its host pass instrumented (device code as usual) and
runs the host-side checks of test_abi_host.py and the property checks of
test_abi_fuzz.py against it in a child process with the ASan runtime preloaded:
symbol lookup, every entry point's argument validation, the workspace size
queries and the workspace carving they share.
An invalid read or write, a use after free or a double free in any of them
aborts the child with an AddressSanitizer report.  Leak detection is off: the
Python interpreter itself keeps allocations alive at exit.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_lib():
    from rl_lora_linear_amd import build as B
    srcs = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC)] + \
        [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))]
    lib = B.ASAN_LIB
    if not os.path.exists(lib) or os.path.getmtime(lib) < max(os.path.getmtime(s) for s in srcs):
        B.build_host_asan()
    return lib, B.asan_runtime()


def test_host_code_clean_under_asan():
    lib, rt = _asan_lib()
    with open(lib, "rb") as f:
        assert b"__asan_report_load" in f.read(), "the host code is not instrumented"
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, LORA_MI355X_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_host.py"),
                          os.path.join(ROOT, "tests", "test_abi_fuzz.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
