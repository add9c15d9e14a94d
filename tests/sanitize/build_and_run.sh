#!/bin/bash
# Build the host-side C ABI (gr_attn_api.cpp), the C oracle and the test program
# with AddressSanitizer and UndefinedBehaviorSanitizer (g++ only: no device
# code), then run the test program.  Usage: build_and_run.sh OUT_DIR
set -euo pipefail
here="$(cd "$(dirname "$0")" && pwd)"
root="$(cd "$here/../.." && pwd)"
out="${1:?output folder}"
mkdir -p "$out"
flags=(-std=c++17 -O1 -g -fno-omit-frame-pointer -fsanitize=address,undefined
       -fno-sanitize-recover=all -D__HIP_PLATFORM_AMD__ -I/opt/rocm/include
       -I"$root/include" -I"$root/shared_prefix_beam_amd/csrc" -I"$here")
g++ "${flags[@]}" -c "$root/shared_prefix_beam_amd/csrc/gr_attn_api.cpp" -o "$out/api.o"
g++ "${flags[@]}" -c "$here/hip_stubs.cpp" -o "$out/stubs.o"
g++ "${flags[@]}" -c "$here/host_checks.cpp" -o "$out/checks.o"
gcc -std=c99 -O1 -g -fno-omit-frame-pointer -fsanitize=address,undefined \
    -fno-sanitize-recover=all -c "$root/oracle/oracle.c" -o "$out/oracle.o"
g++ -fsanitize=address,undefined "$out/api.o" "$out/stubs.o" "$out/checks.o" "$out/oracle.o" \
    -o "$out/host_checks" -lpthread -lm
ASAN_OPTIONS=detect_leaks=1:abort_on_error=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \
    "$out/host_checks"
