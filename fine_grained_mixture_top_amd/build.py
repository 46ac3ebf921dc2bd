"""Build the HIP shared library (libmoe_gfx950.so) in-tree with hipcc.

Each .hip file under csrc/ compiles to an object in ``_build/`` (in parallel),
then they link into ``fine_grained_mixture_top_amd/libmoe_gfx950.so``.
Usage: ``python -m fine_grained_mixture_top_amd.build`` (or ``build()``).

``--sanitize`` builds ``libmoe_gfx950_san.so`` instead, with AddressSanitizer
and UndefinedBehaviorSanitizer on the host code only (the C ABI's validation,
workspace and capacity arithmetic, the launch planners); the device code is
built as usual.  It is for host-side checks on a CPU machine, e.g.::

    LD_PRELOAD=$(/opt/rocm/lib/llvm/bin/clang++ -print-file-name=libclang_rt.asan-x86_64.so) \
      ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1 \
      python -c "import sys; sys.path[:0] = ['.', 'tests']; \
                 from fine_grained_mixture_top_amd import binding as B; \
                 B.LIB_PATH = B.LIB_PATH.replace('.so', '_san.so'); \
                 import pytest; sys.exit(pytest.main(['tests/test_abi_host.py', '-q']))"
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_gfx950.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    "-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions stay off: the compiler would otherwise form
    # v_pk_* fp32 ops from plain float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# host-only sanitizers: each flag applies to the host compilation only
SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
]
LIB_SAN = os.path.join(PKG, "libmoe_gfx950_san.so")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ("_san.o" if sanitize else ".o"))
    extra = SANITIZE_FLAGS if sanitize else []
    cmd = [HIPCC, *FLAGS, *extra, "-I", CSRC, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source and link the library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    workers = min(len(srcs), max(1, (os.cpu_count() or 4)), 8)
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, sanitize), srcs))
    lib = LIB_SAN if sanitize else LIB
    tmp = lib + ".tmp"
    extra = SANITIZE_FLAGS if sanitize else []
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
