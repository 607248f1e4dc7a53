"""W is loaded once per call: evidence from the gfx950 assembly of the
persistent kernels, compiled here from this repository's sources.

For each instance of the configured N = 1792 layers the test compiles that one
kernel to assembly, finds the time loop (the backward branch whose body holds
the per-step workgroup barrier) and checks that no weight load lies inside it.
Weights arrive through plain global loads: `global_load_dwordx2` (four fp16
weights of a row) and `global_load_ushort` (single fp16 weights, or int16
column indices, on the ragged path).  Inside the loop the kernel reads only the
exchange ring (`buffer_load_dwordx4 ... sc0 sc1`), x (`buffer_load_dword`), h0
at t = 0 (`global_load_dword`) and LDS.  Nothing may touch scratch memory.
"""
import os
import re
import subprocess
import tempfile

import pytest

from persistent_rnn_fwd_amd import build as buildmod

# (explicit instantiation, mangled name, W-quad loads expected in the prologue)
INSTANCES = {
    "dense_exact_7x7": ("dense_team_kernel<_Float16, 7, 7, true, false, false>",
                        "_ZN4prnn17dense_team_kernelIDF16_Li7ELi7ELb1ELb0ELb0EEEvNS_8StepArgsE", 49),
    "dense_half_7x7": ("dense_team_kernel<_Float16, 7, 7, false, false, true>",
                       "_ZN4prnn17dense_team_kernelIDF16_Li7ELi7ELb0ELb0ELb1EEEvNS_8StepArgsE", 49),
    "sparse_7x3": ("sparse_team_kernel<_Float16, 7, 3, false, 8>",
                   "_ZN4prnn18sparse_team_kernelIDF16_Li7ELi3ELb0ELi8ELb0EEEvNS_8StepArgsE", 0),
    # rows of unequal length (the unbalanced 10 % layer at N = 2304)
    "sparse_rows_6x10": ("sparse_team_kernel<_Float16, 6, 10, false, 12, true>",
                         "_ZN4prnn18sparse_team_kernelIDF16_Li6ELi10ELb0ELi12ELb1EEEvNS_8StepArgsE", 0),
}
WEIGHT_LOADS = ("global_load_dwordx2", "global_load_ushort", "global_load_short_d16")
LABEL = re.compile(r"^(\.LBB\w+):")


def kernel_asm(inst: str, name: str) -> list:
    try:
        cc = buildmod.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "k.hip")
        with open(src, "w") as fh:
            fh.write('#include "team_kernel.h"\n'
                     f"template __global__ void prnn::{inst}(prnn::StepArgs);\n")
        out = os.path.join(tmp, "k.asm")
        cmd = [cc, *[f for f in buildmod.FLAGS if f != "-fPIC"], "--cuda-device-only", "-S", src, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        text = open(out).read()
    start = text.index(name + ":")
    end = text.index(".Lfunc_end", start)
    return [l.strip() for l in text[start:end].splitlines()]


def time_loop(ins: list) -> tuple:
    labels = {m.group(1): k for k, l in enumerate(ins) for m in [LABEL.match(l)] if m}
    barriers = [k for k, l in enumerate(ins) if l.startswith("s_barrier")]
    step_barrier = barriers[-1]
    loops = []
    for k, l in enumerate(ins):
        op = l.split()[0] if l else ""
        if op.startswith(("s_branch", "s_cbranch")):
            target = labels.get(l.split()[-1])
            if target is not None and target < step_barrier < k:
                loops.append((target, k))
    assert loops, "no backward branch around the step barrier"
    return min(loops, key=lambda se: se[1] - se[0])


@pytest.mark.parametrize("key", sorted(INSTANCES))
def test_no_weight_load_inside_the_time_loop(key):
    inst, name, quads = INSTANCES[key]
    ins = kernel_asm(inst, name)
    lo, hi = time_loop(ins)
    body = ins[lo:hi + 1]
    assert any(l.startswith("buffer_load_dwordx4") and "sc0 sc1" in l for l in body), "ring polls not in the loop"
    inside = [l for l in body if l.startswith(WEIGHT_LOADS)]
    assert not inside, inside[:5]
    assert not [l for l in ins if l.startswith("scratch_")]
    if quads:
        assert sum(l.startswith("global_load_dwordx2") for l in ins[:lo]) == quads


def test_pinned_weights_need_no_copies_in_the_time_loop():
    """The exact 7 x 7 instance keeps its widened weights at the registers its
    multiply-add blocks name (v8 .. v203): the time loop holds all 196
    multiply-adds, and nothing in it writes a weight register."""
    inst, name, _ = INSTANCES["dense_exact_7x7"]
    ins = kernel_asm(inst, name)
    lo, hi = time_loop(ins)
    body = ins[lo:hi + 1]
    fmas = [l for l in body if l.startswith(("v_fmac_f32", "v_fma_f32"))]
    assert len(fmas) == 196
    weights = {f"v{r}" for r in range(8, 204)}
    srcs = {l.replace(",", " ").split()[2] for l in fmas}
    assert srcs <= weights, sorted(srcs - weights)[:5]
    writes = [l for l in body if l.startswith("v_") and not l.startswith(("v_fmac_f32", "v_fma_f32"))
              and l.replace(",", " ").split()[1] in weights]
    assert not writes, writes[:5]
