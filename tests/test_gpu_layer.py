"""GPU parity of the input projection and of whole layers (through the C ABI).

The projection X = x U^T + bias runs on the matrix cores (fp16 U; fp32 x as
fp16 hi + lo, or fp16 x) and is compared with ``oracle.project`` element by
element.  Its tolerance comes from the arithmetic: the products are exact
(hi and lo with fp16 U), the split sees x to 2^-22 of |x| and fp32 sums of I
terms add rounding of a few units of 2^-24 times the partial sums, so

    |X - X_ref| <= 1e-6 (1 + S),   S = |bias| + sum_i |U[n, i]| |x[m, i]|,

which is ~60x above the fp32 rounding seen here and ~10x below what dropping
the lo half would cost at I = 1792.  Inputs built from small integers times
(1 + 2^-13) are exact in every step and must match bitwise (a dropped lo
half fails that).  Layers (projection + recurrence) are compared with
``oracle.forward_layer_*`` at the recurrence's bar (2e-2 for fp16 W, 1e-4 for
fp32 W) and with the two calls run one after the other (bitwise).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from persistent_rnn_fwd_amd import Handle, PrnnError, binding
from persistent_rnn_fwd_amd.inputs import LAYER_WORKLOADS, WORKLOADS, generate_layer

pytestmark = pytest.mark.gpu

PROJ_TOL = 1e-6


@pytest.fixture(scope="module")
def handle(gpu):
    h = Handle()
    yield h
    h.close()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def proj_ratio(X, U, x, bias):
    ref = oracle.project(U, x, bias)
    S = np.abs(x.astype(np.float64)) @ np.abs(U.astype(np.float64)).T
    if bias is not None:
        S = S + np.abs(bias.astype(np.float64))
    return float(np.max(np.abs(X.astype(np.float64) - ref) / (PROJ_TOL * (1.0 + S))))


def draw(rng, M, N, I, x_dtype=np.float32, bias=True):
    U = (rng.standard_normal((N, I)) / np.sqrt(I)).astype(np.float16)
    x = rng.standard_normal((M, I)).astype(x_dtype)
    b = (0.1 * rng.standard_normal(N)).astype(np.float32) if bias else None
    return U, x, b


# (M, N, I): one 64 x 64 tile; ragged M and N; I not a multiple of 8 (the
# element-wise path) and of 32 (a partial last k-step); several XCD slices;
# the full layer size (T * B = 1024 rows, N = I = 1792).
SHAPES = [(64, 64, 64), (37, 45, 29), (100, 130, 200), (5, 300, 7), (1, 1, 1), (256, 192, 96),
          (1024, 1792, 1792)]


@pytest.mark.parametrize("M,N,I", SHAPES)
@pytest.mark.parametrize("xdt", [np.float32, np.float16])
def test_project_parity(handle, M, N, I, xdt):
    rng = np.random.default_rng(M * 1000 + N + I)
    U, x, b = draw(rng, M, N, I, xdt)
    X = handle.project(dev(U), dev(x), dev(b))
    handle.synchronize()
    r = proj_ratio(X.cpu().numpy(), U, x, b)
    print(f"project M={M} N={N} I={I} x={np.dtype(xdt).name}: ratio {r:.3g}")
    assert r <= 1.0


def test_project_no_bias_and_leading_dims(handle):
    rng = np.random.default_rng(3)
    U, x, _ = draw(rng, 24, 80, 48, bias=False)
    x3 = x.reshape(4, 6, 48)
    X = handle.project(dev(U), dev(x3))
    handle.synchronize()
    assert X.shape == (4, 6, 80)
    assert proj_ratio(X.cpu().numpy().reshape(24, 80), U, x, None) <= 1.0


@pytest.mark.parametrize("M,N,I", [(32, 48, 64), (45, 33, 37)])
def test_project_exact_inputs_bitwise(handle, M, N, I):
    """x = s (1 + 2^-13) with |s| <= 3 splits into hi = s and lo = s 2^-13 exactly;
    with integer U and bias every product and partial sum is exact in fp32."""
    rng = np.random.default_rng(11)
    s = rng.integers(-3, 4, size=(M, I)).astype(np.float64)
    x = (s * (1.0 + 2.0 ** -13)).astype(np.float32)
    U = rng.integers(-3, 4, size=(N, I)).astype(np.float16)
    b = rng.integers(-5, 6, size=N).astype(np.float32)
    X = handle.project(dev(U), dev(x), dev(b))
    handle.synchronize()
    ref = oracle.project(U, x, b)
    np.testing.assert_array_equal(X.cpu().numpy().astype(np.float64), ref)
    # and the lo half matters here: the hi part alone is off by sum(U s) 2^-13
    assert not np.array_equal(oracle.project(U, s.astype(np.float32), b), ref)


def test_project_identity_rows(handle):
    """U = I (N = I): X = x + bias exactly for fp16-representable x."""
    rng = np.random.default_rng(4)
    I = 96
    x = rng.standard_normal((50, I)).astype(np.float16).astype(np.float32)
    b = rng.standard_normal(I).astype(np.float16).astype(np.float32)
    X = handle.project(dev(np.eye(I, dtype=np.float16)), dev(x), dev(b))
    handle.synchronize()
    np.testing.assert_array_equal(X.cpu().numpy(), (x + b).astype(np.float32))


@pytest.mark.parametrize("bad", [70000.0, -65536.0, np.inf, -np.inf])
def test_project_range_reported(handle, bad):
    """|x| >= 2^16 or an infinite x does not fit the fp16 split: EXECUTION_FAILED
    at synchronize; the handle works again afterwards.  Just below 2^16 (hi =
    65504, lo = 31) the split is exact."""
    rng = np.random.default_rng(5)
    U, x, b = draw(rng, 16, 32, 64)
    x[3, 7] = bad
    handle.project(dev(U), dev(x), dev(b))
    with pytest.raises(PrnnError) as e:
        handle.synchronize()
    assert e.value.status == binding.EXECUTION_FAILED
    x[3, 7] = 65535.0
    X = handle.project(dev(U), dev(x), dev(b))
    handle.synchronize()
    assert proj_ratio(X.cpu().numpy(), U, x, b) <= 1.0


def test_project_argument_errors(handle):
    lib, h = handle._lib, handle._h
    U = torch.zeros((8, 8), dtype=torch.float16, device="cuda")
    x = torch.zeros((4, 8), dtype=torch.float32, device="cuda")
    X = torch.full((4, 8), 7.0, dtype=torch.float32, device="cuda")
    F, Hf = binding.DATA_FLOAT, binding.DATA_HALF
    assert lib.prnn_project(h, -1, 8, 8, F, x.data_ptr(), Hf, U.data_ptr(), None, X.data_ptr(), None) == \
        binding.BAD_PARAM
    assert lib.prnn_project(h, 4, 0, 8, F, x.data_ptr(), Hf, U.data_ptr(), None, X.data_ptr(), None) == \
        binding.BAD_PARAM
    assert lib.prnn_project(h, 4, 8, 8, 7, x.data_ptr(), Hf, U.data_ptr(), None, X.data_ptr(), None) == \
        binding.BAD_PARAM
    assert lib.prnn_project(h, 4, 8, 8, F, x.data_ptr(), F, U.data_ptr(), None, X.data_ptr(), None) == \
        binding.NOT_SUPPORTED
    assert lib.prnn_project(h, 4, 8, 8, F, x.data_ptr(), Hf, U.data_ptr(), None, x.data_ptr(), None) == \
        binding.BAD_PARAM                                   # X overlaps x
    assert lib.prnn_project(h, 4, 8, 8, F, x.data_ptr() + 2, Hf, U.data_ptr(), None, X.data_ptr(), None) == \
        binding.BAD_PARAM                                   # misaligned fp32 x
    assert lib.prnn_project(h, 0, 8, 8, F, None, Hf, None, None, None, None) == binding.SUCCESS
    handle.synchronize()
    assert bool((X == 7.0).all())                                  # nothing was written


# ---------------------------------------------------------------------------
# whole layers
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(LAYER_WORKLOADS))
def test_layer_parity_full_size(handle, name):
    base, I = LAYER_WORKLOADS[name]
    w = WORKLOADS[base]
    d = generate_layer(w, I)
    g = {k: dev(v) for k, v in d.items()}
    handle.set_grid(0)
    handle.set_layout(binding.LAYOUT_AUTO)
    if w.kind == "dense":
        H = handle.forward_layer_dense(g["U"], g["bias"], g["W"], g["x"], g["h0"])
        ref = oracle.forward_layer_dense(d["U"], d["bias"], d["W"], d["x"], d["h0"])
    else:
        H = handle.forward_layer_sparse(g["U"], g["bias"], g["col"], g["val"], g["x"], g["h0"])
        ref = oracle.forward_layer_sparse(d["U"], d["bias"], d["col"], d["val"], d["x"], d["h0"])
    handle.synchronize()
    r = oracle.tolerance_ratio(H.cpu().numpy(), ref, oracle.TOL_F16)
    print(f"{name}: error ratio {r:.3g}")
    assert r <= 1.0


@pytest.mark.parametrize("wdt,N,I,T", [("f32", 256, 100, 6), ("f16", 192, 64, 5), ("f16", 1152, 300, 4)])
@pytest.mark.parametrize("xdt", ["f32", "f16"])
def test_layer_parity_small(handle, wdt, N, I, T, xdt):
    w = WORKLOADS["dense_f32_n256"].with_(N=N, T=T, w_dtype=wdt, seed=17, h0="randn")
    d = generate_layer(w, I, x_dtype=xdt)
    g = {k: dev(v) for k, v in d.items()}
    H = handle.forward_layer_dense(g["U"], g["bias"], g["W"], g["x"], g["h0"])
    handle.synchronize()
    ref = oracle.forward_layer_dense(d["U"], d["bias"], d["W"], d["x"], d["h0"])
    tol = oracle.TOL_F32 if wdt == "f32" else oracle.TOL_F16
    assert oracle.tolerance_ratio(H.cpu().numpy(), ref, tol) <= 1.0


def test_layer_equals_projection_then_recurrence(handle):
    w = WORKLOADS["sparse10_f16_n1152"].with_(T=8, h0="randn")
    d = generate_layer(w, 512)
    g = {k: dev(v) for k, v in d.items()}
    H1 = handle.forward_layer_sparse(g["U"], g["bias"], g["col"], g["val"], g["x"], g["h0"])
    X = handle.project(g["U"], g["x"], g["bias"])
    H2 = handle.forward_sparse(g["col"], g["val"], X, g["h0"])
    handle.synchronize()
    assert torch.equal(H1, H2)


def test_layer_rejects_workspace_over_h0_and_enqueues_nothing(handle):
    N, I, B, T = 64, 32, 2, 3
    U = torch.zeros((N, I), dtype=torch.float16, device="cuda")
    W = torch.zeros((N, N), dtype=torch.float16, device="cuda")
    x = torch.zeros((T, B, I), dtype=torch.float32, device="cuda")
    ws = torch.zeros((T, B, N), dtype=torch.float32, device="cuda")
    H = torch.full((T, B, N), 9.0, dtype=torch.float32, device="cuda")
    h0 = ws[0]                                                     # inside the workspace
    lib = handle._lib
    F, Hf = binding.DATA_FLOAT, binding.DATA_HALF
    st = lib.prnn_forward_layer_dense(handle._h, N, I, B, T, F, x.data_ptr(), Hf, U.data_ptr(), None, Hf,
                                      W.data_ptr(), h0.data_ptr(), ws.data_ptr(), H.data_ptr(), None)
    assert st == binding.BAD_PARAM
    st = lib.prnn_forward_layer_dense(handle._h, N, I, B, T, F, x.data_ptr(), Hf, U.data_ptr(), None, Hf,
                                      W.data_ptr(), None, H.data_ptr(), H.data_ptr(), None)
    assert st == binding.BAD_PARAM                          # workspace is H
    handle.synchronize()
    assert bool((H == 9.0).all())


def test_project_long_ragged_reduction(handle):
    """I = 2050 (not a multiple of 8: the element-wise path over 65 k-steps)."""
    rng = np.random.default_rng(12)
    U, x, b = draw(rng, 70, 90, 2050)
    X = handle.project(dev(U), dev(x), dev(b))
    handle.synchronize()
    assert proj_ratio(X.cpu().numpy(), U, x, b) <= 1.0


@pytest.mark.parametrize("kind", ["dense", "sparse"])
def test_layer_chunked_in_time(handle, kind):
    """One layer call over T steps equals two calls over T1 and T - T1 steps with
    h0 = the first call's last state (within 1e-6; bitwise expected)."""
    base = "dense_f16_n1152" if kind == "dense" else "sparse10_f16_n1152"
    w = WORKLOADS[base].with_(N=640 if kind == "dense" else 1152, T=16, h0="randn", seed=41)
    d = generate_layer(w, 200)
    g = {k: dev(v) for k, v in d.items()}

    def layer(x, h0):
        if kind == "dense":
            return handle.forward_layer_dense(g["U"], g["bias"], g["W"], x, h0)
        return handle.forward_layer_sparse(g["U"], g["bias"], g["col"], g["val"], x, h0)
    full = layer(g["x"], g["h0"])
    a = layer(g["x"][:7].contiguous(), g["h0"])
    b = layer(g["x"][7:].contiguous(), a[-1].contiguous())
    handle.synchronize()
    both = torch.cat([a, b]).cpu().numpy()
    print(f"layer {kind} chunked: bitwise {np.array_equal(both, full.cpu().numpy())}")
    np.testing.assert_allclose(both, full.cpu().numpy(), rtol=1e-6, atol=1e-6)


def test_layer_sparse_fp32_values(handle):
    w = WORKLOADS["sparse10_f16_n1152"].with_(N=512, K=40, T=6, w_dtype="f32", h0="randn", seed=44)
    d = generate_layer(w, 128, x_dtype="f16")
    g = {k: dev(v) for k, v in d.items()}
    H = handle.forward_layer_sparse(g["U"], g["bias"], g["col"], g["val"], g["x"], g["h0"])
    handle.synchronize()
    ref = oracle.forward_layer_sparse(d["U"], d["bias"], d["col"], d["val"], d["x"], d["h0"])
    assert oracle.tolerance_ratio(H.cpu().numpy(), ref, oracle.TOL_F32) <= 1.0
