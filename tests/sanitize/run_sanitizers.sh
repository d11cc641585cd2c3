#!/bin/bash
# CPU-only sanitizer run of the host code: the C-ABI layer (ua_api.cpp, with
# stand-in kernel launchers) and the C oracle (oracle/ua_oracle.c), each built
# by the host compiler with AddressSanitizer and UndefinedBehaviorSanitizer
# (any report aborts the process), then driven by the CPU ABI tests and the
# oracle's pin battery.  Needs no GPU.  Usage: bash tests/sanitize/run_sanitizers.sh
set -euo pipefail
ROOT="$(cd "$(dirname "$0")/../.." && pwd)"
OUT="${SANITIZE_OUT:-/tmp/ua_sanitize}"
mkdir -p "$OUT"
SAN="-fsanitize=address,undefined -fno-sanitize-recover=all -fno-omit-frame-pointer -g -O1"
g++ -std=c++17 -D__HIP_PLATFORM_AMD__ -I/opt/rocm/include -I"$ROOT/include" \
    -I"$ROOT/paged_varlen_flashattention_amd/csrc" $SAN -fPIC -shared \
    "$ROOT/paged_varlen_flashattention_amd/csrc/ua_api.cpp" "$ROOT/tests/sanitize/host_stubs.cpp" \
    -o "$OUT/libua_host_sanitized.so"
gcc -std=c11 -fopenmp $SAN -fPIC -shared "$ROOT/oracle/ua_oracle.c" -lm -o "$OUT/libua_oracle_sanitized.so"
PRE="$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so)"
cd "$ROOT"
# the Python interpreter is not instrumented: leak checks off, every other
# report fatal
env LD_PRELOAD="$PRE" ASAN_OPTIONS=detect_leaks=0:abort_on_error=1 \
    UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \
    UA_TEST_LIBRARY="$OUT/libua_host_sanitized.so" UA_TEST_ORACLE_LIBRARY="$OUT/libua_oracle_sanitized.so" \
    OMP_NUM_THREADS=4 \
    python -m pytest -q -p no:cacheprovider tests/test_abi.py tests/test_oracle.py -m "not gpu" "$@"
