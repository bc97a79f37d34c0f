#!/bin/bash
# The CPU test tier (-m "not gpu") under AddressSanitizer and
# UndefinedBehaviorSanitizer: the oracle (C, built with clang) and libgdn's host
# code (argument validation, planning, workspace layout, launch set-up; the
# kernels are not instrumented) are rebuilt with both sanitizers into separate
# libraries, which GDN_HOST_SANITIZE=1 selects, and the clang sanitizer runtime
# is preloaded into Python.  Any report ends the run with a non-zero status.
# CPU only: nothing here runs a kernel.
set -euo pipefail
cd "$(dirname "$0")/.."
# the sanitizer builds are for this run only
trap 'rm -f gated_delta_rule_linear_amd/libgdn_hostsan.so oracle/libgdn_oracle_hostsan.so' EXIT
python -m gated_delta_rule_linear_amd.build --host-sanitize
python -c "import oracle; oracle.build(force=True, sanitize=True)"
RT=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so)
export GDN_HOST_SANITIZE=1
export ASAN_OPTIONS=detect_leaks=0:abort_on_error=1:halt_on_error=1
export UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1
LD_PRELOAD="$RT" python -m pytest tests -m "not gpu" -x -q -p no:cacheprovider "$@"
