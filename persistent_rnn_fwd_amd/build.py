"""Builds libprnn.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m persistent_rnn_fwd_amd.build        # or __graft_entry__.build()
"""
from __future__ import annotations

import json
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libprnn.so")
RESOURCES = os.path.join(BUILD, "kernel_resources.json")  # per-kernel registers, scratch, LDS, occupancy
SOURCES = ["dense_f16.hip", "dense_f32.hip", "sparse_f16.hip", "sparse_f32.hip", "team_f16.hip", "team_f32.hip", "team_half.hip",
           "team_split.hip", "team_rows.hip", "project.hip", "stack.hip", "noalloc.hip", "prnn.cpp"]

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in device code.
FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libprnn.so)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + err)
    return err


_REMARK = re.compile(r"remark:\s+(Function Name|TotalSGPRs|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Dynamic Stack|"
                     r"Occupancy \[waves/SIMD\]|SGPRs Spill|VGPRs Spill|LDS Size \[bytes/block\]): (\S+)")


def parse_resource_remarks(text: str) -> dict:
    """The compiler's kernel-resource-usage remarks, per kernel symbol."""
    out, cur = {}, None
    for m in _REMARK.finditer(text):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key.split(" [")[0]] = int(val) if val.isdigit() else val
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        extra = ["-Rpass-analysis=kernel-resource-usage"] if src.endswith(".hip") else []
        jobs.append((obj, [cc, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]))
    resources = {}
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        for out in ex.map(lambda j: _run(j[1]), jobs):
            resources.update(parse_resource_remarks(out))
            rest = "\n".join(l for l in out.splitlines() if "remark:" not in l and l.strip())
            if verbose and rest:
                print(rest)
    with open(RESOURCES, "w") as fh:
        json.dump(resources, fh, indent=0, sort_keys=True)
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *[o for o, _ in jobs]])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
