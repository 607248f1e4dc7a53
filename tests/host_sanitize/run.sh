#!/bin/bash
# Runs the host-sanitized driver (build it first: python tests/host_sanitize/build.py)
# in a process of its own on an MI355X.  It must be the only process using the GPU:
# the cooperative launches it makes fail while another process holds the device.
# Any AddressSanitizer or UndefinedBehaviorSanitizer report aborts it.
HERE=$(cd "$(dirname "$0")" && pwd)
RT=$(ls -d /opt/rocm/llvm/lib/clang/*/lib/linux | tail -1)
LD_LIBRARY_PATH=$RT:$LD_LIBRARY_PATH ASAN_OPTIONS=detect_leaks=0:halt_on_error=1 \
  UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1 "$HERE/driver"
