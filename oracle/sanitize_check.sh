#!/bin/bash
# The oracle's CPU test suite against an AddressSanitizer + UBSan build of
# oracle.c (gcc; runtimes preloaded into the test process, which is not built
# with them). Run from the repository root; CPU only.
set -euo pipefail
ROOT=$(cd "$(dirname "$0")/.." && pwd)
cd "$ROOT"
SAN=$(python3 -c "import oracle; print(oracle.build(force=True, sanitize=True))")
export ORACLE_LIB=$SAN
export LD_PRELOAD="$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so)"
export ASAN_OPTIONS=detect_leaks=0:abort_on_error=1
export UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1
python3 -m pytest tests -q -m "not gpu" -k "oracle or synth or ffn_tolerance" -p no:cacheprovider "$@"
