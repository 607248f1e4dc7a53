"""Resource use of every compiled kernel, from the compiler's own report.

The build records the ``-Rpass-analysis=kernel-resource-usage`` remarks of
every device kernel in ``_build/kernel_resources.json``.  The persistent
design needs the weights in registers for the whole call: no kernel may use
scratch memory (private segment) or spill vector registers to it, and every
kernel must fit the waves its launch puts on a SIMD (team layout: 8 waves of
a 512-thread workgroup on 4 SIMDs = 2 per SIMD; spread layout: up to 4 waves
of a 256-thread workgroup = 1 per SIMD).
"""
import json
import os
import subprocess
import sys

import pytest

from persistent_rnn_fwd_amd import build as buildmod


@pytest.fixture(scope="module")
def resources():
    if not os.path.exists(buildmod.RESOURCES):
        pytest.skip("no build record; run persistent_rnn_fwd_amd.build first")
    with open(buildmod.RESOURCES) as fh:
        return json.load(fh)


def test_record_covers_every_kernel_family(resources):
    names = list(resources)
    for fam in ("dense_team_kernel", "sparse_team_kernel", "floor_team_kernel", "dense_kernel", "sparse_kernel",
                "floor_kernel", "fill_kernel", "placement_kernel"):
        assert any(fam in n for n in names), fam


def test_no_kernel_uses_scratch_or_spills(resources):
    bad = {n: r for n, r in resources.items()
           if r.get("ScratchSize", 0) != 0 or r.get("VGPRs Spill", 0) != 0 or r.get("Dynamic Stack") != "False"}
    assert not bad, sorted(bad)[:10]


def test_kernels_fit_their_launch(resources):
    for n, r in resources.items():
        need = 2 if "team_kernel" in n else 1
        assert r["Occupancy"] >= need, (n, r)


def test_remark_parser():
    text = ("x.h:1:1: remark: Function Name: _Zk [-Rpass-analysis=kernel-resource-usage]\n"
            "x.h:1:1: remark:     VGPRs: 82 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.h:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.h:1:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]\n")
    assert buildmod.parse_resource_remarks(text) == {"_Zk": {"VGPRs": 82, "ScratchSize": 0, "Dynamic Stack": "False"}}


def test_pinned_weight_blocks_match_their_generator():
    """team_pinned.h is the committed output of gen_team_pinned.py."""
    csrc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "persistent_rnn_fwd_amd", "csrc")
    out = subprocess.run([sys.executable, os.path.join(csrc, "gen_team_pinned.py")], capture_output=True, text=True,
                         check=True).stdout
    with open(os.path.join(csrc, "team_pinned.h")) as fh:
        assert fh.read() == out
