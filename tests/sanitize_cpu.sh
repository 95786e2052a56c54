#!/bin/bash
# CPU sanitizer run: builds the C oracle and libgdn (host code only; the gfx950 device code
# is built as usual) with AddressSanitizer and UndefinedBehaviorSanitizer, then runs the
# CPU tests that exercise them -- the oracle's pins and the boundary's host-side checks --
# with the sanitizer runtime preloaded. Any report fails the run.
#   usage: tests/sanitize_cpu.sh [out_dir]       (default /tmp/gdn_sanitize)
set -euo pipefail
ROOT=$(cd "$(dirname "$0")/.." && pwd)
OUT=${1:-/tmp/gdn_sanitize}
mkdir -p "$OUT/obj"
LLVM=/opt/rocm/llvm
RT=$(ls $LLVM/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)
SAN="-fsanitize=address,undefined -fno-sanitize-recover=undefined -fno-omit-frame-pointer -g"

echo "[sanitize] oracle (clang, $SAN)"
$LLVM/bin/clang -O1 -std=c11 -fPIC -shared -pthread -fno-fast-math -ffp-contract=off $SAN \
  -o "$OUT/libgdn_oracle_san.so" "$ROOT/oracle/gdn_oracle.c" -lm

echo "[sanitize] libgdn host code (hipcc -Xarch_host ...)"
HFLAGS="-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer"
for f in "$ROOT"/gated_deltanet_prefill_gdn_amd/csrc/*.hip; do
  /opt/rocm/bin/hipcc -c "$f" -o "$OUT/obj/$(basename "$f" .hip).o" -O1 -g -std=c++17 -fPIC \
    --offload-arch=gfx950 -I "$ROOT/include" -I "$ROOT/gated_deltanet_prefill_gdn_amd/csrc" \
    -Xclang -target-feature -Xclang -packed-fp32-ops $HFLAGS &
done
wait
/opt/rocm/bin/hipcc -shared -fPIC --offload-arch=gfx950 -Xarch_host -fsanitize=address \
  -Xarch_host -fsanitize=undefined -o "$OUT/libgdn_san.so" "$OUT"/obj/*.o

echo "[sanitize] tests under $RT"
cd "$ROOT"
LD_PRELOAD="$RT" \
ASAN_OPTIONS=detect_leaks=0:abort_on_error=1:halt_on_error=1 \
UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1 \
GDN_LIBRARY="$OUT/libgdn_san.so" GDN_ORACLE_LIB="$OUT/libgdn_oracle_san.so" \
  python -m pytest -q -p no:cacheprovider -m "not gpu" \
    tests/test_abi.py tests/test_oracle_pins.py tests/test_oracle_decode.py 2>&1 | tee "$OUT/pytest.log"
