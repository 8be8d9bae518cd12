#!/bin/bash
# Host-side AddressSanitizer + UndefinedBehaviorSanitizer run of the
# library's host code (argument checks, workspace sizing, the prefill
# planner): builds libidx.so with the sanitizers on the host pass only (the
# gfx950 device code is compiled as usual) into a temporary directory and
# runs the CPU ABI tests against it.  CPU only; needs no GPU.
#   usage: tests/run_host_sanitizers.sh
set -euo pipefail
ROOT="$(cd "$(dirname "$0")/.." && pwd)"
OUT="$(mktemp -d)"
trap 'rm -rf "$OUT"' EXIT
CSRC="$ROOT/sparse_attention_indexer_decode_amd/csrc"
HIPCC="${HIPCC:-/opt/rocm/bin/hipcc}"
"$HIPCC" --offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -shared \
  -Xclang -target-feature -Xclang -packed-fp32-ops \
  -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
  -Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer \
  -shared-libsan -Wno-unused-command-line-argument \
  "$CSRC/idx_lib.hip" "$CSRC/planner.cpp" -o "$OUT/libidx_san.so"
RT="$("$HIPCC" -print-file-name=libclang_rt.asan-x86_64.so)"
echo "sanitized library: $OUT/libidx_san.so (runtime $RT)"
cd "$ROOT"
IDX_LIB_PATH="$OUT/libidx_san.so" LD_PRELOAD="$RT" \
  ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1" \
  UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1" \
  python -m pytest tests/test_abi_cpu.py -q -p no:cacheprovider
