#!/bin/bash
# The C ABI's host-side validation under AddressSanitizer + UBSan, on the CPU:
# the library built with the sanitizers on its host code only (each one behind
# -Xarch_host; the gfx950 device code is built as usual), loaded into the ABI
# test process with clang's ASan runtime preloaded. Every call those tests make
# fails validation before the HIP runtime is used. Run from the repository root.
set -euo pipefail
ROOT=$(cd "$(dirname "$0")/.." && pwd)
cd "$ROOT"
OUT=$ROOT/_build/san
mkdir -p "$OUT"
SRC=combine_moe_route_03_amd/csrc
# the library's own source list, so that the sanitized library never misses a file
SOURCES=$(python3 -c "import sys; sys.path.insert(0, 'combine_moe_route_03_amd'); \
import _build; print(' '.join('$SRC/' + s for s in _build.SOURCES))")
/opt/rocm/bin/hipcc --offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -shared \
  -Xclang -target-feature -Xclang -packed-fp32-ops \
  -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
  -Xarch_host -fno-sanitize-recover=undefined -shared-libsan -Wl,-z,defs \
  -I include -I $SRC $SOURCES \
  -o "$OUT/libmoe_route_san.so"
export MOE_ROUTE_LIB=$OUT/libmoe_route_san.so
export LD_PRELOAD=$(ls /opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)
export ASAN_OPTIONS=detect_leaks=0:abort_on_error=1
export UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1
python3 -m pytest tests/test_abi.py -q -p no:cacheprovider "$@"
