#!/bin/bash
# The oracle's CPU pins and planted-mistake battery under AddressSanitizer and
# UndefinedBehaviorSanitizer (host code only; no GPU is involved).  Builds
# oracle/liboracle_san.so, then runs the two CPU test files with the ASan
# runtime loaded first; any sanitizer report aborts the run.
#   usage: oracle/sanitize.sh [extra pytest arguments]
set -euo pipefail
cd "$(dirname "$0")/.."
ORACLE_SANITIZE=1 python3 -c "import oracle; oracle.build()"
ASAN_LIB=$(gcc -print-file-name=libasan.so)
UBSAN_LIB=$(gcc -print-file-name=libubsan.so)
export ORACLE_SANITIZE=1
export ASAN_OPTIONS=detect_leaks=0:abort_on_error=1:halt_on_error=1
export UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1
LD_PRELOAD="$ASAN_LIB:$UBSAN_LIB" python3 -m pytest tests/test_oracle_pins.py \
    tests/test_oracle_mutants.py -q -p no:cacheprovider "$@"
