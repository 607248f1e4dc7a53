"""GPU parity of the half-h dense path (PRNN_MATH_HALF) through the C ABI.

In this mode the kernel rounds h_{t-1} to fp16 (nearest, ties to even) before
the product and adds two exact fp16 x fp16 products per instruction to fp32
sums.  Two bars are checked on the same seeded inputs:
  * against the plain fp64 definition (``oracle.forward_dense``), the
    fp16-weight bar |H - H_ref| <= 2e-2 (1 + |H_ref|);
  * one step at a time against the fp16-state model
    (``oracle.forward_dense_half_h``) started from the kernel's own previous
    output: the kernel stages exactly fp16(H[t-1]), so what remains is fp32
    summation error, checked at 2e-5 (1 + |h|).  Rounding the other way (toward
    zero, or not at all) misses this bar.
Closed forms with small integers are fp16-exact and must hold bitwise.
"""
import numpy as np
import pytest

import oracle
from persistent_rnn_fwd_amd import Handle, PrnnError, binding
from persistent_rnn_fwd_amd.inputs import WORKLOADS, Workload, generate

pytestmark = pytest.mark.gpu

STEP_TOL = 2e-5  # one-step agreement with the fp16-state model (fp32 sums of up to 2048 terms)


@pytest.fixture(scope="module")
def handle(gpu):
    h = Handle()
    yield h
    h.close()


def to_dev(d):
    import torch
    return {k: (torch.from_numpy(np.ascontiguousarray(v)).cuda() if isinstance(v, np.ndarray) else v)
            for k, v in d.items()}


def run(h, d, math=binding.MATH_HALF, grid=0, h0=True, layout=binding.LAYOUT_AUTO):
    g = to_dev(d)
    h.set_math(math)
    h.set_grid(grid)
    h.set_layout(layout)
    try:
        H = h.forward_dense(g["W"], g["X"], g["h0"] if h0 else None)
        h.synchronize()
    finally:
        h.set_math(binding.MATH_AUTO)
        h.set_grid(0)
        h.set_layout(binding.LAYOUT_AUTO)
    return H.cpu().numpy()


def one_step_ratio(H, d, h0=True):
    """max over t of the model's step from the kernel's own H[t-1] (h0 at t = 0)."""
    W, X = d["W"], d["X"]
    prev = d["h0"] if h0 else np.zeros(X.shape[1:], np.float32)
    worst = 0.0
    for t in range(X.shape[0]):
        ref = oracle.forward_dense_half_h(W, X[t:t + 1], prev)
        worst = max(worst, oracle.tolerance_ratio(H[t:t + 1], ref, STEP_TOL))
        prev = H[t]
    return worst


def check(H, d, what, h0=True):
    ref = oracle.forward_dense(d["W"], d["X"], d["h0"] if h0 else None)
    r = oracle.tolerance_ratio(H, ref, oracle.TOL_F16)
    assert r <= 1.0, f"{what}: error ratio {r:.3g} against the definition"
    s = one_step_ratio(H, d, h0)
    assert s <= 1.0, f"{what}: one-step ratio {s:.3g} against the fp16-state model"
    return r, s


@pytest.mark.parametrize("seed_off", [0, 2000])
@pytest.mark.parametrize("name", ["dense_f16_n1152", "dense_f16_n1792"])
def test_half_parity_workloads(handle, name, seed_off):
    w = WORKLOADS[name]
    d = generate(w, seed=w.seed + seed_off)
    H = run(handle, d)
    p = handle.last_plan()
    assert p["math"] == binding.MATH_HALF and p["layout"] == binding.LAYOUT_TEAM
    r, s = check(H, d, name)
    print(f"{name} seed+{seed_off}: ratio {r:.3g} of 2e-2, one-step ratio {s:.3g} of {STEP_TOL}")


@pytest.mark.parametrize("N,B,T,grid", [(1, 1, 3, 0), (3, 2, 4, 0), (7, 3, 5, 0), (100, 4, 6, 0), (257, 5, 4, 0),
                                        (511, 8, 3, 0), (1000, 8, 3, 0), (2048, 4, 3, 0), (1792, 4, 5, 240),
                                        (1152, 2, 6, 256), (777, 1, 7, 128)])
def test_half_shapes(handle, N, B, T, grid):
    w = Workload(f"dense_{N}", "dense", N, B, T, "f16", seed=N * 17 + B, h0="randn")
    d = generate(w)
    H = run(handle, d, grid=grid)
    assert handle.last_plan()["math"] == binding.MATH_HALF
    check(H, d, f"N={N} B={B} T={T} grid={grid}")


def test_half_without_h0(handle):
    w = WORKLOADS["dense_f16_n1792"].with_(T=12)
    d = generate(w, seed=77)
    H = run(handle, d, h0=False)
    check(H, d, "no h0", h0=False)


def test_half_closed_forms_bitwise(handle):
    """Integers below 2048 are fp16 values, so staging them is exact and the
    closed forms hold bit for bit."""
    rng = np.random.default_rng(51)
    T, B, N = 30, 4, 1792
    X = rng.integers(0, 50, size=(T, B, N)).astype(np.float32)
    h0 = rng.integers(0, 50, size=(B, N)).astype(np.float32)
    expect = h0[None].astype(np.float64) + np.cumsum(X.astype(np.float64), axis=0)
    assert expect.max() < 2048
    np.testing.assert_array_equal(run(handle, {"W": np.eye(N, dtype=np.float16), "X": X, "h0": h0}), expect)
    # W = 0: relu(X) exactly, whatever the staged state
    Xr = rng.standard_normal((T, B, N)).astype(np.float32)
    np.testing.assert_array_equal(run(handle, {"W": np.zeros((N, N), np.float16), "X": Xr, "h0": h0}),
                                  np.maximum(Xr, 0))
    # cyclic shift: h_t[i] = relu(x_t[i] + h_{t-1}[i + 1])
    N = 1152
    Xs = rng.integers(0, 9, size=(12, 2, N)).astype(np.float32)
    hs = rng.integers(0, 9, size=(2, N)).astype(np.float32)
    Wd = np.zeros((N, N), np.float16)
    Wd[np.arange(N), (np.arange(N) + 1) % N] = 1
    np.testing.assert_array_equal(run(handle, {"W": Wd, "X": Xs, "h0": hs}), oracle.forward_dense(Wd, Xs, hs))


def test_half_rounds_to_nearest_even(handle):
    """W = I with one state on and beside the fp16 grid: the next step adds
    exactly the rounded state (hand-worked: spacing 2^-10 on [1, 2))."""
    N, B = 256, 1
    u = 2.0 ** -10
    x0 = np.array([1 + 0.75 * u, 1 + 0.5 * u, 1 + 1.5 * u, 1 + 0.25 * u, 1 + 3 * u], np.float64)
    staged = np.array([1 + u, 1.0, 1 + 2 * u, 1.0, 1 + 3 * u])
    X = np.zeros((2, B, N), np.float32)
    X[0, 0, :5] = x0
    H = run(handle, {"W": np.eye(N, dtype=np.float16), "X": X, "h0": np.zeros((B, N), np.float32)})
    np.testing.assert_array_equal(H[0, 0, :5], x0)
    np.testing.assert_array_equal(H[1, 0, :5], staged)


def test_half_deterministic_chunkable_and_close_to_exact(handle):
    w = WORKLOADS["dense_f16_n1792"].with_(T=40, h0="randn")
    d = generate(w, seed=53)
    Hh = run(handle, d)
    np.testing.assert_array_equal(run(handle, d), Hh)
    Ha = run(handle, dict(d, X=d["X"][:17]))
    Hb = run(handle, dict(d, X=d["X"][17:], h0=Ha[-1]))
    np.testing.assert_array_equal(np.concatenate([Ha, Hb]), Hh)
    He = run(handle, d, math=binding.MATH_EXACT)
    assert oracle.tolerance_ratio(Hh, He, oracle.TOL_F16) < 0.2
    assert not np.array_equal(Hh, He)   # the state really is rounded


@pytest.mark.parametrize("where", ["x", "h0"])
def test_half_range_reported(gpu, where):
    """A state that rounds to an fp16 infinity is reported; the handle then
    runs again normally."""
    w = WORKLOADS["dense_f16_n1792"].with_(T=6, h0="randn")
    d = generate(w, seed=54)
    if where == "x":
        d["X"] = d["X"].copy()
        d["X"][2, 1, 7] = 1e6
    else:
        d["h0"] = d["h0"].copy()
        d["h0"][3, 100] = 7e4
    with Handle() as h:
        h.set_math(binding.MATH_HALF)
        g = to_dev(d)
        h.forward_dense(g["W"], g["X"], g["h0"])
        with pytest.raises(PrnnError) as e:
            h.synchronize()
        assert e.value.status == binding.EXECUTION_FAILED
        h.set_math(binding.MATH_EXACT)
        H = h.forward_dense(g["W"], g["X"], g["h0"])
        h.synchronize()
        assert oracle.tolerance_ratio(H.cpu().numpy(), oracle.forward_dense(d["W"], d["X"], d["h0"]),
                                      oracle.TOL_F16) <= 1.0


def test_half_scope(handle):
    """Half-h exists for fp16 W in the team layout only: beyond 2560 neurons
    or in the spread layout the call is NOT_SUPPORTED; fp32 W and sparse
    layers keep exact math."""
    w = Workload("dense_2561", "dense", 2561, 4, 2, "f16", seed=5)
    d = generate(w)
    with pytest.raises(PrnnError) as e:
        run(handle, d)
    assert e.value.status == binding.NOT_SUPPORTED
    w = WORKLOADS["dense_f16_n1152"].with_(T=3)
    with pytest.raises(PrnnError) as e:
        run(handle, generate(w), layout=binding.LAYOUT_SPREAD)
    assert e.value.status == binding.NOT_SUPPORTED
    w = WORKLOADS["dense_f32_n256"]
    d = generate(w)
    H = run(handle, d)
    assert handle.last_plan()["math"] == binding.MATH_EXACT
    assert oracle.tolerance_ratio(H, oracle.forward_dense(d["W"], d["X"], d["h0"]), oracle.TOL_F32) <= 1.0
    w = WORKLOADS["sparse10_f16_n1792"].with_(T=8)
    d = generate(w)
    g = to_dev(d)
    handle.set_math(binding.MATH_HALF)
    try:
        H = handle.forward_sparse(g["col"], g["val"], g["X"], g["h0"])
        handle.synchronize()
    finally:
        handle.set_math(binding.MATH_AUTO)
    assert handle.last_plan()["math"] == binding.MATH_EXACT
    assert oracle.tolerance_ratio(H.cpu().numpy(), oracle.forward_sparse(d["col"], d["val"], d["X"], d["h0"]),
                                  oracle.TOL_F16) <= 1.0


def test_half_trace_and_watchdog(gpu):
    w = WORKLOADS["dense_f16_n1792"].with_(T=24)
    d = generate(w, seed=55)
    with Handle() as h:
        h.set_math(binding.MATH_HALF)
        g = to_dev(d)
        H0 = h.forward_dense(g["W"], g["X"], g["h0"])
        h.synchronize()
        h.set_trace(True)
        H1 = h.forward_dense(g["W"], g["X"], g["h0"])
        h.synchronize()
        tr = h.get_trace()
        assert h.last_plan()["math"] == binding.MATH_HALF
        h.set_trace(False)
        np.testing.assert_array_equal(H0.cpu().numpy(), H1.cpu().numpy())
        live = tr[tr[:, 7] == w.T].astype(np.float64)
        assert live.shape[0] == w.B * (h.last_plan()["grid"] // 8) * 8
        assert np.all(live[:, :5].sum(1) <= live[:, 5])
        h.set_watchdog_us(2000)
        h.debug_skip_publish(3, 5)
        h.forward_dense(g["W"], g["X"], g["h0"])
        with pytest.raises(PrnnError) as e:
            h.synchronize()
        assert e.value.status == binding.EXECUTION_FAILED
        H2 = h.forward_dense(g["W"], g["X"], g["h0"])
        h.synchronize()
        np.testing.assert_array_equal(H2.cpu().numpy(), H0.cpu().numpy())


def test_half_layer_and_stack(gpu):
    """A whole dense layer follows the math setting (projection, then the
    half-h recurrence); a layer-by-layer stack does too; the blocked and fused
    stacks keep exact math (bitwise equal to the same stack with the default
    setting)."""
    from persistent_rnn_fwd_amd.inputs import generate_layer, generate_stack
    import torch
    w = WORKLOADS["dense_f16_n1792"].with_(T=48, h0="randn")
    d = generate_layer(w, 1792)
    g = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in d.items()}
    ref = oracle.forward_layer_dense(d["U"], d["bias"], d["W"], d["x"], d["h0"])
    with Handle() as h:
        h.set_math(binding.MATH_HALF)
        H = h.forward_layer_dense(g["U"], g["bias"], g["W"], g["x"], g["h0"])
        h.synchronize()
        assert h.last_plan()["math"] == binding.MATH_HALF
        assert oracle.tolerance_ratio(H.cpu().numpy(), ref, oracle.TOL_F16) <= 1.0
        h.set_math(binding.MATH_EXACT)
        He = h.forward_layer_dense(g["U"], g["bias"], g["W"], g["x"], g["h0"])
        h.synchronize()
        assert not torch.equal(H, He)

        sw = WORKLOADS["dense_f16_n1152"].with_(N=640, B=2, T=40, h0="randn", seed=31)
        st = generate_stack(sw, 2)
        layers = [{k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in ly.items()} for ly in st["layers"]]
        x = torch.from_numpy(st["x"]).cuda()
        h0s = [torch.from_numpy(v).cuda() for v in st["h0s"]]
        refs = oracle.forward_stack_dense(st["layers"], st["x"], st["h0s"])

        def stack(mode, math):
            h.set_stack_mode(mode)
            h.set_math(math)
            outs = h.forward_stack_dense(layers, x, h0s)
            h.synchronize()
            h.set_stack_mode(binding.STACK_AUTO)
            h.set_math(binding.MATH_AUTO)
            return [o.cpu().numpy() for o in outs]

        half_layers = stack(binding.STACK_LAYERS, binding.MATH_HALF)
        exact_layers = stack(binding.STACK_LAYERS, binding.MATH_EXACT)
        assert all(oracle.tolerance_ratio(a, r, oracle.TOL_F16) <= 1.0 for a, r in zip(half_layers, refs))
        assert not all(np.array_equal(a, b) for a, b in zip(half_layers, exact_layers))
        for mode in (binding.STACK_BLOCKED, binding.STACK_FUSED):
            a = stack(mode, binding.MATH_HALF)
            b = stack(mode, binding.MATH_AUTO)
            assert all(np.array_equal(p, q) for p, q in zip(a, b)), mode
