#!/bin/bash
# Host-only build of the C-ABI layer with AddressSanitizer and
# UndefinedBehaviorSanitizer (g++; no device code): libsanta_asan.so in $1.
set -e
ROOT=$(cd "$(dirname "$0")/../.." && pwd)
OUT=${1:-$ROOT/_build/asan}
mkdir -p "$OUT"
g++ -std=c++17 -O1 -g -fno-omit-frame-pointer -fsanitize=address,undefined -fno-sanitize-recover=undefined \
    -shared -fPIC -D__HIP_PLATFORM_AMD__ -I/opt/rocm/include -I"$ROOT/include" \
    -I"$ROOT/stochastic_sparse_decode_amd/csrc" \
    "$ROOT/stochastic_sparse_decode_amd/csrc/santa_api.cpp" "$ROOT/tests/asan/launch_stubs.cpp" \
    -L/opt/rocm/lib -lamdhip64 -Wl,-rpath,/opt/rocm/lib -o "$OUT/libsanta_asan.so"
echo "$OUT/libsanta_asan.so"
