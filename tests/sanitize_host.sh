#!/bin/bash
# The CPU test suite against host code built with AddressSanitizer and
# UndefinedBehaviorSanitizer (no GPU needed): first the oracle (gcc's
# runtimes), then the host side of the HIP library (clang's runtime; its
# device code is not instrumented), each in its own processes.
set -euo pipefail
R=$(cd "$(dirname "$0")/.." && pwd)
cd "$R"
export ASAN_OPTIONS=detect_leaks=0:abort_on_error=1 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1
ORACLE_SANITIZE=1 python -c "import oracle; oracle.build()"
ORACLE_SANITIZE=1 LD_PRELOAD="$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so)" \
    python -m pytest tests -m "not gpu" -q -p no:cacheprovider
python -m expert_dispatch_router_amd.build --sanitize
ASANRT=$(ls /opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)
MOE_LIBRARY="$R/expert_dispatch_router_amd/libmoe_san.so" LD_PRELOAD="$ASANRT" \
    python -m pytest tests/test_abi.py tests/test_bench_host.py -q -p no:cacheprovider
