#!/bin/bash
# CPU run of the test-suite with AddressSanitizer and UndefinedBehaviorSanitizer
# on the host code: the oracle (oracle.c) and the library's host side
# (argument validation, planning and launch set-up in api.hip and the
# launchers; device code is built without sanitizers).  Works on a copy of the
# repository in a temporary folder, so the in-tree builds are untouched.
# Usage: tests/sanitize_cpu.sh [extra pytest args]
set -euo pipefail
ROOT="$(cd "$(dirname "${BASH_SOURCE[0]}")/.." && pwd)"
WORK="$(mktemp -d /tmp/specv_asan.XXXXXX)"
trap '[ -n "${KEEP:-}" ] || rm -rf "$WORK"' EXIT
tar -C "$ROOT" --exclude=.git --exclude=_work --exclude=gpurun_out --exclude='*.so' -cf - . | tar -C "$WORK" -xf -
LLVM=/opt/rocm/llvm
RT="$(ls "$LLVM"/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)"
cd "$WORK"
export SPEC_HOST_FLAGS="-fsanitize=address -fsanitize=undefined -fno-sanitize-recover=undefined -fno-omit-frame-pointer -shared-libsan"
export ORACLE_CC="$LLVM/bin/clang"
export ORACLE_CFLAGS="-fsanitize=address -fsanitize=undefined -fno-sanitize-recover=undefined -fno-omit-frame-pointer -shared-libsan"
python -c "from speculative_decoding_verification_tree_amd import build; build.build(); import oracle; oracle.build()"
LD_PRELOAD="$RT" LD_LIBRARY_PATH="$LLVM/lib:${LD_LIBRARY_PATH:-}" \
ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1" \
UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1" \
    python -m pytest tests -m "not gpu" -x -q -s -p no:cacheprovider "$@"
