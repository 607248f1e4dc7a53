"""Builds the host-sanitized copy of libprnn and the driver that exercises it.

Host code (the library's planning, checks and launches, and the driver) is
compiled with -fsanitize=address,undefined; device code is compiled as in the
product build.  Outputs, next to this file: libprnn_hostsan.so and driver.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
from persistent_rnn_fwd_amd import build as pkg_build  # noqa: E402

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer"]


def build() -> str:
    cc = pkg_build.hipcc()
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    flags = [f for f in pkg_build.FLAGS if f != "-O3"] + ["-O1", "-g"] + SAN
    jobs = []
    for src in pkg_build.SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        jobs.append([cc, *flags, "-c", os.path.join(pkg_build.CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        list(ex.map(lambda c: subprocess.run(c, check=True, capture_output=True), jobs))
    lib = os.path.join(HERE, "libprnn_hostsan.so")
    objs = [j[-1] for j in jobs]
    subprocess.run([cc, "-shared", "-fPIC", "--offload-arch=gfx950", *SAN, "-shared-libasan", "-o", lib, *objs],
                   check=True, capture_output=True)
    exe = os.path.join(HERE, "driver")
    subprocess.run([cc, "-O1", "-g", "-std=c++17", "-I" + os.path.join(ROOT, "include"), *SAN, "-shared-libasan",
                    os.path.join(HERE, "driver.cpp"), "-L" + HERE, "-lprnn_hostsan", "-Wl,-rpath,$ORIGIN", "-o", exe],
                   check=True, capture_output=True)
    return exe


if __name__ == "__main__":
    print(build())
