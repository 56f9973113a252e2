#!/bin/bash
# The C ABI's host code (argument checks, workspace sizing and carving) under
# AddressSanitizer and UndefinedBehaviorSanitizer: builds libattn_san.so with
# the sanitizers on the host pass only, then runs the CPU-side ABI tests
# against it with the ASan runtime loaded first.  No GPU is involved: every
# call in those tests is rejected on the host before any launch (the few with
# valid arguments stop at the device query, which finds no GPU).
#   usage: transformer_attention_causal_amd/sanitize.sh [extra pytest arguments]
set -euo pipefail
cd "$(dirname "$0")/.."
python3 -m transformer_attention_causal_amd.build --sanitized
ASAN_RT=$(ls /opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)
export ATTN_LIB=$PWD/transformer_attention_causal_amd/libattn_san.so
export ASAN_OPTIONS=detect_leaks=0:abort_on_error=1:halt_on_error=1
export UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1
LD_PRELOAD="$ASAN_RT" python3 -m pytest tests/test_abi.py -q -p no:cacheprovider "$@"
