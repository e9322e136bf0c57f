"""Build the HIP library ``libmoe.so`` in-tree with hipcc for gfx950.

    python -m expert_dispatch_router_amd.build        # compile + link

Each source under ``csrc/`` is compiled to an object in ``_build/`` in
parallel, then linked into ``expert_dispatch_router_amd/libmoe.so``.  The
build always recompiles (it is the "does it build" check) and replaces the
library atomically.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["router.hip", "route.hip", "dispatch.hip", "grouped_gemm.hip", "combine.hip",
           "moe_api.cpp"]

# -packed-fp32-ops: no packed fp32 VALU ops in device code (the host pass
# warns that it does not know the feature; that is harmless).
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Host code instrumented with AddressSanitizer and UndefinedBehaviorSanitizer
# (device code is not: -Xarch_host puts each flag on the host pass only), for
# `build(sanitize=True)` -> libmoe_san.so, which the binding loads when
# MOE_LIBRARY names it and the process preloads clang's ASan runtime
# (tests/sanitize_host.sh).
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
SAN_LIB = os.path.join(PKG, "libmoe_san.so")


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + (".san.o" if sanitize else ".o"))
    cmd = [HIPCC, *FLAGS, *(SAN_FLAGS if sanitize else []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip() and verbose:
        print(out, flush=True)
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), SOURCES))
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp%d" % os.getpid()
    # (a sanitized build leaves the sanitizer runtime's symbols to the
    # preloaded runtime)
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
