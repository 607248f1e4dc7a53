"""Races and determinism of the exchange protocol (through the C ABI).

Every output buffer is filled with NaN before a run, so a row that is never
written, or read before it was, shows up.  The recurrence is deterministic:
each output is one fixed sequence of fp32 operations on the same inputs, so
repeated runs must agree bit for bit, whatever the timing.  To vary the timing
on purpose, ``prnn_debug_jitter`` makes every wave sleep a pseudo-random number
of periods (drawn per workgroup, wave and step from a host seed) before it
publishes its rows: rows then arrive in another order and at other times, and
the results must still be bitwise those of the undisturbed run.
"""
import numpy as np
import pytest
import torch

import oracle
from persistent_rnn_fwd_amd import Handle, PrnnError, binding
from persistent_rnn_fwd_amd.inputs import WORKLOADS, generate, generate_stack

pytestmark = pytest.mark.gpu

JITTER_SPAN = 48          # up to ~48 x 64 shader clocks per wave and step
SEEDS = (1, 0xBEEF, 0x9E3779B9)


def to_dev(d):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in d.items()}


def nan_like(X):
    return torch.full(X.shape, float("nan"), dtype=torch.float32, device=X.device)


def forward(h, kind, g):
    out = nan_like(g["X"])
    if kind == "dense":
        h.forward_dense(g["W"], g["X"], g["h0"], out=out)
    else:
        h.forward_sparse(g["col"], g["val"], g["X"], g["h0"], out=out)
    h.synchronize()
    return out.cpu().numpy()


def reference(kind, d):
    if kind == "dense":
        return oracle.forward_dense(d["W"], d["X"], d["h0"])
    return oracle.forward_sparse(d["col"], d["val"], d["X"], d["h0"])


# (workload, layout, math, N: 0 = the workload's own[, XCDs per batch row: 0 = automatic])
PATHS = [
    ("dense_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_EXACT, 0),
    ("dense_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_SPLIT, 0),
    ("dense_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_HALF, 0),
    ("dense_f16_n1792", binding.LAYOUT_SPREAD, binding.MATH_EXACT, 0),
    ("dense_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_EXACT, 2048, 1),   # partly widened rows
    ("dense_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_EXACT, 2560, 1),   # 10 rows x 10 chunks
    ("dense_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_EXACT, 2560),      # split over 2 XCDs per row
    ("dense_f32_n256", binding.LAYOUT_TEAM, binding.MATH_AUTO, 0),
    ("sparse10_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_AUTO, 0),
    ("sparse10_f16_n1792", binding.LAYOUT_SPREAD, binding.MATH_AUTO, 0),
    ("sparse1_f16_n5760", binding.LAYOUT_TEAM, binding.MATH_AUTO, 0),    # 16-wave workgroups
    ("sparse5_f16_n5760", binding.LAYOUT_TEAM, binding.MATH_AUTO, 0),    # two XCDs per batch row, 12-wave workgroups
]


def path_id(p):
    n = f"-n{p[3]}" if p[3] else ""
    x = f"-xcd{p[4]}" if len(p) > 4 else ""
    return f"{p[0]}{n}-{'team' if p[1] == binding.LAYOUT_TEAM else 'spread'}-math{p[2]}{x}"


def setup(h, name, layout, math, T, seed, N=0, xcds=0):
    w = WORKLOADS[name].with_(T=T, **({"N": N} if N else {}))
    d = generate(w, seed=seed)
    h.set_layout(layout)
    h.set_math(math)
    h.set_xcds_per_row(xcds)
    return ("dense" if "W" in d else "sparse"), d, to_dev(d)


@pytest.mark.parametrize("path", PATHS, ids=path_id)
def test_twenty_repeats_bitwise_with_nan_poisoned_outputs(gpu, path):
    name, layout, math, N, xcds = (*path, 0)[:5]
    with Handle() as h:
        kind, d, g = setup(h, name, layout, math, T=40, seed=61, N=N, xcds=xcds)
        first = forward(h, kind, g)
        assert not np.isnan(first).any()
        tol = oracle.TOL_F32 if name.startswith("dense_f32") else oracle.TOL_F16
        assert oracle.tolerance_ratio(first, reference(kind, d), tol) <= 1.0
        for rep in range(19):
            again = forward(h, kind, g)
            assert np.array_equal(again.view(np.uint32), first.view(np.uint32)), f"repeat {rep + 2} differs"


@pytest.mark.parametrize("path", PATHS, ids=path_id)
def test_publish_jitter_leaves_results_bitwise_unchanged(gpu, path):
    name, layout, math, N, xcds = (*path, 0)[:5]
    with Handle() as h:
        kind, d, g = setup(h, name, layout, math, T=48, seed=62, N=N, xcds=xcds)
        base = forward(h, kind, g)
        assert not np.isnan(base).any()
        for seed in SEEDS:
            h.debug_jitter(seed, JITTER_SPAN)
            got = forward(h, kind, g)
            h.debug_jitter(0, 0)
            assert np.array_equal(got.view(np.uint32), base.view(np.uint32)), f"jitter seed {seed:#x} changed H"
        assert np.array_equal(forward(h, kind, g).view(np.uint32), base.view(np.uint32))


@pytest.mark.parametrize("mode", [binding.STACK_BLOCKED, binding.STACK_FUSED, binding.STACK_LAYERS])
def test_stack_jitter_leaves_results_bitwise_unchanged(gpu, mode):
    """The stack's hand-overs (between blocks, and per step in the fused mode,
    where a layer polls the layer below's outputs) under publish delays."""
    w = WORKLOADS["dense_f16_n1152"].with_(B=4, T=90, h0="randn", seed=63)
    st = generate_stack(w, 2)
    with Handle() as h:
        h.set_stack_mode(mode)
        layers = [{k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in ly.items()} for ly in st["layers"]]
        x = torch.from_numpy(st["x"]).cuda()
        h0s = [torch.from_numpy(v).cuda() for v in st["h0s"]]

        def run():
            outs = [nan_like(torch.empty(x.shape[:2] + (w.N,), device="cuda")) for _ in layers]
            h.forward_stack_dense(layers, x, h0s, outs=outs)
            h.synchronize()
            return [o.cpu().numpy() for o in outs]

        base = run()
        refs = oracle.forward_stack_dense(st["layers"], st["x"], st["h0s"])
        assert all(oracle.tolerance_ratio(b, r, oracle.TOL_F16) <= 1.0 for b, r in zip(base, refs))
        for seed in SEEDS:
            h.debug_jitter(seed, JITTER_SPAN)
            got = run()
            h.debug_jitter(0, 0)
            for l, (a, b) in enumerate(zip(got, base)):
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"layer {l}, jitter seed {seed:#x}"


def test_jitter_span_is_checked(gpu):
    with Handle() as h:
        with pytest.raises(PrnnError) as e:
            h.debug_jitter(1, -1)
        assert e.value.status == binding.BAD_PARAM
        with pytest.raises(PrnnError) as e:
            h.debug_jitter(1, 1025)
        assert e.value.status == binding.BAD_PARAM
        h.debug_jitter(1, 1024)
        h.debug_jitter(0, 0)
