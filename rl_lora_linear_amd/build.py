"""Build the gfx950 HIP library `liblora_mi355x.so` in-tree.

    python -m rl_lora_linear_amd.build             # or build() from Python
    python -m rl_lora_linear_amd.build --host-asan # host code under AddressSanitizer

Each csrc/*.hip is compiled with hipcc for gfx950 only; the objects are
linked into one shared library next to this file.  Packed-fp32 instruction
selection is disabled for all device code.

The --host-asan build instruments the host code only (argument validation,
workspace carving, launch set-up) with AddressSanitizer; device code is built
as usual.  It goes to _build/asan/liblora_mi355x.so and is loaded through
LORA_MI355X_LIB with the compiler's ASan runtime preloaded.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblora_mi355x.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++20", "-Wall", "-Wno-unused-function",
    "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "liblora_mi355x.so")
# host-only instrumentation: every sanitizer flag applies to the host pass
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The compiler's shared ASan runtime, to be preloaded into the host process."""
    res = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        llvm = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "lib", "clang")
        for root, _dirs, files in os.walk(llvm):
            if "libclang_rt.asan-x86_64.so" in files:
                return os.path.join(root, "libclang_rt.asan-x86_64.so")
        raise RuntimeError("the ASan runtime libclang_rt.asan-x86_64.so was not found")
    return path


def _compile(src: str, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _build_into(out_dir: str, lib: str, extra=(), verbose: bool = False) -> str:
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the library; returns its path."""
    return _build_into(BUILD, LIB, (), verbose)


def build_host_asan(verbose: bool = False) -> str:
    """The same library with its host code under AddressSanitizer; returns its path."""
    return _build_into(ASAN_DIR, ASAN_LIB, ASAN_FLAGS, verbose)


if __name__ == "__main__":
    if "--host-asan" in sys.argv[1:]:
        build_host_asan(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
