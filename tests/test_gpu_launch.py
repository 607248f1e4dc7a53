"""Plain and cooperative dispatch of the persistent kernels (prnn_set_launch).

The kernels and their arithmetic do not depend on how they are dispatched, so
every path must give bitwise the same outputs either way: dense (team layout,
exact and half-h math, spread layout, split over 2 and 4 XCDs), sparse (team,
12- and 16-wave instances, split, rows of unequal length), whole layers, the
three stack modes and the floor.  Plain dispatch is the default where its
workgroups are dealt to the XCDs round-robin; a graph captured with
cooperative dispatch still replays correctly.
"""
import numpy as np
import pytest
import torch

import oracle
from persistent_rnn_fwd_amd import Handle, PrnnError, binding
from persistent_rnn_fwd_amd.inputs import WORKLOADS, Workload, generate, generate_layer, generate_stack

pytestmark = pytest.mark.gpu


def to_dev(d):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in d.items()}


def dense_case(name, T, **kw):
    w = WORKLOADS[name].with_(T=T, h0="randn", **kw)
    return w, to_dev(generate(w, seed=7))


def run_both(fn):
    """fn(handle) -> list of tensors, with cooperative then plain dispatch on one handle."""
    outs = {}
    with Handle() as h:
        for kind in (binding.LAUNCH_COOPERATIVE, binding.LAUNCH_PLAIN):
            h.set_launch(kind)
            r = fn(h)
            h.synchronize()
            outs[kind] = [t.clone() for t in r]
    return outs[binding.LAUNCH_COOPERATIVE], outs[binding.LAUNCH_PLAIN]


def assert_same(a, b, what):
    assert len(a) == len(b)
    for x, y in zip(a, b):
        assert torch.equal(x, y), what


def test_plain_is_the_default_and_kinds_are_checked(gpu, capfd, monkeypatch):
    monkeypatch.setenv("PRNN_LOG", "1")
    with Handle() as h:
        w, g = dense_case("dense_f16_n1152", 6)
        h.forward_dense(g["W"], g["X"], g["h0"])
        h.synchronize()
        with pytest.raises(PrnnError) as e:
            h.set_launch(2)
        assert e.value.status == binding.BAD_PARAM
    monkeypatch.delenv("PRNN_LOG")
    err = capfd.readouterr().err
    assert "team layout available, plain launches" in err, err
    lib = binding.load_library()
    assert lib.prnn_set_launch(None, binding.LAUNCH_PLAIN) == binding.BAD_PARAM


@pytest.mark.parametrize("name,layout,math,xcds", [
    ("dense_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_AUTO, 0),
    ("dense_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_HALF, 0),
    ("dense_f16_n1152", binding.LAYOUT_SPREAD, binding.MATH_AUTO, 0),
    ("dense_f32_n256", binding.LAYOUT_AUTO, binding.MATH_AUTO, 0),
    ("dense_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_AUTO, 2),
])
def test_dense_paths_agree_bitwise(gpu, name, layout, math, xcds):
    w, g = dense_case(name, 20)

    def fn(h):
        h.set_layout(layout)
        h.set_math(math)
        h.set_xcds_per_row(xcds)
        return [h.forward_dense(g["W"], g["X"], g["h0"])]
    a, b = run_both(fn)
    assert_same(a, b, name)
    ref = oracle.forward_dense(generate(w, seed=7)["W"], generate(w, seed=7)["X"], generate(w, seed=7)["h0"])
    tol = oracle.TOL_F16 if w.w_dtype == "f16" else oracle.TOL_F32
    assert oracle.tolerance_ratio(b[0].cpu().numpy(), ref, tol) <= 1.0


def test_split_over_four_xcds_agrees_bitwise(gpu):
    w = Workload("split_n4096_b2", "dense", 4096, 2, 9, "f16", seed=4096, h0="randn")
    g = to_dev(generate(w))
    a, b = run_both(lambda h: [h.forward_dense(g["W"], g["X"], g["h0"])])
    assert_same(a, b, "N=4096 over 4 XCDs")


@pytest.mark.parametrize("name,xcds", [("sparse10_f16_n1792", 0), ("sparse1_f16_n5760", 0), ("sparse10_f16_n2304", 0),
                                       ("sparse5_f16_n5760", 2)])
def test_sparse_paths_agree_bitwise(gpu, name, xcds):
    w = WORKLOADS[name].with_(T=12, h0="randn")
    g = to_dev(generate(w, seed=3))

    def fn(h):
        h.set_xcds_per_row(xcds)
        return [h.forward_sparse(g["col"], g["val"], g["X"], g["h0"])]
    a, b = run_both(fn)
    assert_same(a, b, name)


def test_rows_of_unequal_length_agree_bitwise(gpu):
    w = WORKLOADS["sparse10u_f16_n2304"].with_(T=10, h0="randn")
    g = to_dev(generate(w, seed=5))
    a, b = run_both(lambda h: [h.forward_sparse_rows(g["col"], g["val"], g["row_len"], g["X"], g["h0"])])
    assert_same(a, b, "rows")


def test_layers_and_stacks_agree_bitwise(gpu):
    w = WORKLOADS["dense_f16_n1152"].with_(N=640, B=2, T=70, h0="randn", seed=12)
    d = to_dev(generate_layer(w, 512))
    st = generate_stack(w, 3)
    layers = [to_dev(ly) for ly in st["layers"]]
    x = torch.from_numpy(st["x"]).cuda()
    h0s = [torch.from_numpy(v).cuda() for v in st["h0s"]]

    def fn(h):
        out = [h.forward_layer_dense(d["U"], d["bias"], d["W"], d["x"], d["h0"])]
        for mode in (binding.STACK_BLOCKED, binding.STACK_FUSED, binding.STACK_LAYERS):
            h.set_stack_mode(mode)
            out += h.forward_stack_dense(layers, x, h0s)
        h.set_stack_mode(binding.STACK_AUTO)
        return out
    a, b = run_both(fn)
    assert_same(a, b, "layer and stacks")
    refs = oracle.forward_stack_dense(st["layers"], st["x"], st["h0s"])
    for i in range(3):  # blocked, fused, layers
        for got, ref in zip(b[1 + 3 * i:4 + 3 * i], refs):
            assert oracle.tolerance_ratio(got.cpu().numpy(), ref, oracle.TOL_F16) <= 1.0


def test_floor_runs_either_way(gpu):
    with Handle() as h:
        out = torch.empty((64, 4, 1792), device="cuda")
        for kind in (binding.LAUNCH_COOPERATIVE, binding.LAUNCH_PLAIN):
            h.set_launch(kind)
            h.sync_floor(1792, 4, 64, out=out)
            h.synchronize()


def test_graph_captured_with_cooperative_dispatch(gpu):
    w, g = dense_case("dense_f16_n1152", 9)
    with Handle() as fresh:
        ref = fresh.forward_dense(g["W"], g["X"], g["h0"]).clone()
        fresh.synchronize()
    with Handle() as h:
        h.set_launch(binding.LAUNCH_COOPERATIVE)
        h.forward_dense(g["W"], g["X"], g["h0"])
        h.synchronize()
        out = torch.full_like(ref, float("nan"))
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            h.forward_dense(g["W"], g["X"], g["h0"], out=out)
        torch.cuda.synchronize()
        for rep in range(3):
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            h.synchronize()
            assert torch.equal(out, ref), f"replay {rep}"
