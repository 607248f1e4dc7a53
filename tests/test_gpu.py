"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Every test here runs the persistent kernels on an MI355X and compares with
``oracle`` element by element on the same seeded inputs:
  * the five workload families at their full sizes (N up to 5760, T = 256);
  * ragged and degenerate shapes: N not a multiple of 4, N = 1, several grid
    sizes (forcing uneven row splits), B = 1..8, T = 1..3 and T = 0, K = 1,
    K = N, K just above a 64-pair slot;
  * closed forms that must hold bitwise on the GPU (W = 0, W = I and cyclic
    shifts with small-integer inputs, positive homogeneity, identical batch
    rows, chunking in time, run-to-run determinism);
  * error paths: argument checks, oversize layers, and a forced watchdog expiry
    (a workgroup skips one publish; every wave still exits normally).
Tolerance per element: |H - H_ref| <= tol (1 + |H_ref|), tol = 1e-4 for fp32
weights and 2e-2 for fp16 weights with fp32 accumulation.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from persistent_rnn_fwd_amd import Handle, PrnnError, binding
from persistent_rnn_fwd_amd.inputs import WORKLOADS, Workload, generate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def handle(gpu):
    h = Handle()
    yield h
    h.close()


def to_dev(d):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in d.items()}


def run(handle, kind, d, grid=0, h0=True, layout=binding.LAYOUT_AUTO):
    g = to_dev(d)
    handle.set_grid(grid)
    handle.set_layout(layout)
    hh = g["h0"] if h0 else None
    if kind == "dense":
        H = handle.forward_dense(g["W"], g["X"], hh)
    else:
        H = handle.forward_sparse(g["col"], g["val"], g["X"], hh)
    handle.synchronize()
    return H.cpu().numpy()


def reference(kind, d, h0=True):
    hh = d["h0"] if h0 else None
    if kind == "dense":
        return oracle.forward_dense(d["W"], d["X"], hh)
    return oracle.forward_sparse(d["col"], d["val"], d["X"], hh)


def tol_of(d):
    w = d["W"] if "W" in d else d["val"]
    return oracle.TOL_F32 if w.dtype == np.float32 else oracle.TOL_F16


def assert_parity(H, ref, tol, what=""):
    r = oracle.tolerance_ratio(H, ref, tol)
    assert r <= 1.0, f"{what}: max error ratio {r:.3g} > 1 (tol {tol})"
    return r


# ---------------------------------------------------------------------------
# the workloads at full size
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed_off", [0, 1000])
@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_parity(handle, name, seed_off):
    w = WORKLOADS[name]
    d = generate(w, seed=w.seed + seed_off)
    H = run(handle, w.kind, d)
    assert np.isfinite(H).all()
    assert_parity(H, reference(w.kind, d), tol_of(d), name)


# the configured workloads (dense fp32 N=256; dense and 10 % sparse N=1152; dense, 10 % and 1 % sparse
# N=1792; 1 % sparse N=5760) with a third seed
CONFIGURED = ["dense_f32_n256", "dense_f16_n1152", "sparse10_f16_n1152", "dense_f16_n1792", "sparse10_f16_n1792",
              "sparse1_f16_n1792", "sparse1_f16_n5760"]


@pytest.mark.parametrize("name", CONFIGURED)
def test_configured_workload_parity_third_seed(handle, name):
    w = WORKLOADS[name]
    d = generate(w, seed=w.seed + 3000)
    H = run(handle, w.kind, d)
    assert np.isfinite(H).all()
    assert_parity(H, reference(w.kind, d), tol_of(d), name)


@pytest.mark.parametrize("name", ["dense_f16_n1792", "sparse10_f16_n1792"])
def test_workload_parity_random_h0(handle, name):
    w = WORKLOADS[name].with_(h0="randn", T=64)
    d = generate(w, seed=w.seed + 2000)
    assert_parity(run(handle, w.kind, d), reference(w.kind, d), tol_of(d), name)


# ---------------------------------------------------------------------------
# ragged and degenerate shapes, several grids
# ---------------------------------------------------------------------------
DENSE_SHAPES = [
    # N, B, T, wdtype, grid
    (1, 1, 3, "f32", 0),
    (3, 2, 5, "f32", 0),
    (7, 3, 4, "f16", 0),
    (100, 4, 9, "f32", 0),
    (100, 4, 9, "f16", 7),
    (257, 1, 6, "f32", 0),
    (257, 5, 6, "f16", 13),
    (256, 8, 8, "f32", 32),
    (511, 4, 3, "f16", 64),
    (1000, 2, 5, "f16", 0),
    (1152, 4, 2, "f16", 192),
    (1152, 4, 7, "f16", 128),
    (1792, 4, 5, "f16", 224),
    (2048, 4, 4, "f16", 0),
    (1024, 4, 4, "f32", 0),
]


LAYOUTS = [binding.LAYOUT_AUTO, binding.LAYOUT_SPREAD]


@pytest.mark.parametrize("N,B,T", [(2100, 2, 6), (2304, 4, 5), (2304, 1, 7), (2560, 3, 4), (2560, 8, 5)])
@pytest.mark.parametrize("math", [binding.MATH_EXACT, binding.MATH_HALF])
def test_dense_fp16_beyond_2048(handle, N, B, T, math):
    """Dense fp16 layers of 2049 to 2560 neurons in the team layout on one XCD
    per batch row (forced: automatically exact math splits them over several):
    9 or 10 rows x 9 or 10 chunks per wave (packed fp16 weights), exact or
    half-h."""
    w = Workload(f"dense_{N}", "dense", N, B, T, "f16", seed=N + 7, h0="randn")
    d = generate(w)
    handle.set_math(math)
    handle.set_xcds_per_row(1)
    try:
        H = run(handle, "dense", d)
        p = handle.last_plan()
    finally:
        handle.set_math(binding.MATH_AUTO)
        handle.set_xcds_per_row(0)
    assert p["layout"] == binding.LAYOUT_TEAM and p["math"] == math and p["rmax"] == p["chunks"] == -(-N // 256), p
    assert_parity(H, reference("dense", d), oracle.TOL_F16, f"N={N} math={math}")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("N,B,T,wdt,grid", DENSE_SHAPES)
def test_dense_shapes(handle, N, B, T, wdt, grid, layout):
    w = Workload(f"dense_{N}", "dense", N, B, T, wdt, seed=N * 7 + B, h0="randn")
    d = generate(w)
    H = run(handle, "dense", d, grid=grid, layout=layout)
    assert_parity(H, reference("dense", d), tol_of(d), f"N={N} B={B} T={T} {wdt} grid={grid} plan={handle.last_plan()}")


SPARSE_SHAPES = [
    # N, B, T, K, vdtype, grid
    (1, 1, 3, 1, "f32", 0),
    (5, 2, 4, 5, "f16", 0),
    (64, 4, 6, 64, "f32", 0),
    (100, 3, 5, 65, "f16", 0),
    (100, 4, 5, 1, "f16", 9),
    (257, 4, 7, 26, "f32", 0),
    (1000, 8, 4, 100, "f16", 0),
    (1152, 4, 5, 115, "f16", 192),
    (1792, 4, 5, 179, "f16", 200),
    (2051, 2, 3, 20, "f16", 0),
    (5760, 4, 3, 58, "f16", 240),
    (8000, 2, 3, 80, "f16", 0),
]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("N,B,T,K,vdt,grid", SPARSE_SHAPES)
def test_sparse_shapes(handle, N, B, T, K, vdt, grid, layout):
    w = Workload(f"sparse_{N}", "sparse", N, B, T, vdt, K=K, seed=N * 11 + K, h0="randn")
    d = generate(w)
    H = run(handle, "sparse", d, grid=grid, layout=layout)
    assert_parity(H, reference("sparse", d), tol_of(d),
                  f"N={N} B={B} T={T} K={K} {vdt} grid={grid} plan={handle.last_plan()}")


def test_zero_timesteps_leave_output_untouched(handle):
    W = torch.zeros(8, 8, device="cuda")
    X = torch.zeros(0, 2, 8, device="cuda")
    out = torch.empty(0, 2, 8, device="cuda")
    handle.forward_dense(W, X, out=out)
    handle.synchronize()


# ---------------------------------------------------------------------------
# closed forms, bitwise on the GPU
# ---------------------------------------------------------------------------
def test_zero_weights_give_relu_x_bitwise(handle):
    rng = np.random.default_rng(1)
    T, B, N = 6, 4, 300
    X = rng.standard_normal((T, B, N)).astype(np.float32)
    h0 = np.abs(rng.standard_normal((B, N))).astype(np.float32)
    for wdt in (np.float32, np.float16):
        H = run(handle, "dense", {"W": np.zeros((N, N), wdt), "X": X, "h0": h0})
        np.testing.assert_array_equal(H, np.maximum(X, 0))
    H = run(handle, "sparse", {"col": np.arange(N, dtype=np.int16).reshape(N, 1),
                               "val": np.zeros((N, 1), np.float16), "X": X, "h0": h0})
    np.testing.assert_array_equal(H, np.maximum(X, 0))


def test_identity_weights_give_prefix_sums_bitwise(handle):
    rng = np.random.default_rng(2)
    T, B, N = 40, 4, 1792
    X = rng.integers(0, 100, size=(T, B, N)).astype(np.float32)
    h0 = rng.integers(0, 100, size=(B, N)).astype(np.float32)
    expect = h0[None].astype(np.float64) + np.cumsum(X.astype(np.float64), axis=0)
    H = run(handle, "dense", {"W": np.eye(N, dtype=np.float16), "X": X, "h0": h0})
    np.testing.assert_array_equal(H, expect)
    H = run(handle, "sparse", {"col": np.arange(N, dtype=np.int16).reshape(N, 1),
                               "val": np.ones((N, 1), np.float16), "X": X, "h0": h0})
    np.testing.assert_array_equal(H, expect)


def test_cyclic_shift_bitwise(handle):
    """W[i, (i+1) % N] = 1: catches a transposed W or a misplaced row."""
    rng = np.random.default_rng(3)
    T, B, N = 12, 2, 1152
    X = rng.integers(0, 9, size=(T, B, N)).astype(np.float32)
    h0 = rng.integers(0, 9, size=(B, N)).astype(np.float32)
    Wd = np.zeros((N, N), np.float16)
    Wd[np.arange(N), (np.arange(N) + 1) % N] = 1
    ref = oracle.forward_dense(Wd, X, h0)
    np.testing.assert_array_equal(run(handle, "dense", {"W": Wd, "X": X, "h0": h0}), ref)
    col = ((np.arange(N) + 1) % N).astype(np.int16).reshape(N, 1)
    np.testing.assert_array_equal(
        run(handle, "sparse", {"col": col, "val": np.ones((N, 1), np.float32), "X": X, "h0": h0}), ref)


@pytest.mark.parametrize("N,wdt,xcds", [(1792, np.float16, 0), (2048, np.float16, 1), (2304, np.float16, 1),
                                        (2560, np.float16, 1), (2048, np.float16, 0), (2560, np.float16, 0),
                                        (1792, np.float32, 0), (1000, np.float32, 0)])
def test_small_integer_weights_bitwise(handle, N, wdt, xcds):
    """Three +-1 weights per row in random columns and small integer inputs keep
    every partial sum an exact fp32 integer (|h| < 2^13 over six steps), so
    any summation order gives the fp64 result bit for bit: every row of the
    widened, packed and partly widened team instances (one XCD per batch row,
    forced beyond N = 1792, or split automatically) is checked exactly."""
    rng = np.random.default_rng(N + 17)
    T, B = 6, 4
    W = np.zeros((N, N), wdt)
    for _ in range(3):
        W[np.arange(N), rng.integers(0, N, N)] += rng.choice([-1, 1], N).astype(wdt)
    X = rng.integers(-5, 6, size=(T, B, N)).astype(np.float32)
    h0 = rng.integers(0, 6, size=(B, N)).astype(np.float32)
    ref = oracle.forward_dense(W, X, h0)
    assert np.abs(ref).max() < 2 ** 13
    handle.set_xcds_per_row(xcds)
    try:
        H = run(handle, "dense", {"W": W, "X": X, "h0": h0})
        p = handle.last_plan()
    finally:
        handle.set_xcds_per_row(0)
    assert p["layout"] == binding.LAYOUT_TEAM, p
    assert p["xcds_per_row"] == (1 if xcds == 1 or N <= 1792 else 2), p
    np.testing.assert_array_equal(H, ref)


def test_sparse_matches_dense_copy(handle):
    w = WORKLOADS["sparse10_f16_n1152"].with_(T=32, h0="randn")
    d = generate(w, seed=5)
    Hs = run(handle, "sparse", d)
    Wd = oracle.sparse_to_dense(d["col"], d["val"], w.N).astype(np.float16)
    Hd = run(handle, "dense", {"W": Wd, "X": d["X"], "h0": d["h0"]})
    assert_parity(Hs, Hd.astype(np.float64), oracle.TOL_F16, "sparse vs dense copy")
    assert_parity(Hs, reference("sparse", d), oracle.TOL_F16)


def test_positive_homogeneity_bitwise(handle):
    w = WORKLOADS["dense_f16_n1792"].with_(T=20, h0="randn")
    d = generate(w, seed=9)
    H1 = run(handle, "dense", d)
    d2 = dict(d, X=d["X"] * 4, h0=d["h0"] * 4)
    np.testing.assert_array_equal(run(handle, "dense", d2), H1 * 4)


def test_identical_batch_rows_bitwise(handle):
    w = WORKLOADS["sparse10_f16_n1792"].with_(T=16, h0="randn")
    d = generate(w, seed=10)
    X = np.repeat(d["X"][:, :1], 4, axis=1)
    h0 = np.repeat(d["h0"][:1], 4, axis=0)
    H = run(handle, "sparse", dict(d, X=X, h0=h0))
    for b in range(1, 4):
        np.testing.assert_array_equal(H[:, b], H[:, 0])


@pytest.mark.parametrize("name", ["dense_f16_n1792", "sparse10_f16_n1792", "dense_f32_n256"])
def test_deterministic_and_chunkable(handle, name):
    w = WORKLOADS[name].with_(T=30, h0="randn")
    d = generate(w, seed=11)
    H1 = run(handle, w.kind, d)
    H2 = run(handle, w.kind, d)
    np.testing.assert_array_equal(H1, H2)
    T1 = 13
    Ha = run(handle, w.kind, dict(d, X=d["X"][:T1]))
    Hb = run(handle, w.kind, dict(d, X=d["X"][T1:], h0=Ha[-1]))
    np.testing.assert_array_equal(np.concatenate([Ha, Hb]), H1)


def test_nan_propagates_within_its_batch_row(handle):
    w = WORKLOADS["dense_f32_n256"].with_(T=6)
    d = generate(w, seed=12)
    d["X"] = d["X"].copy()
    d["X"][2, 1, 5] = np.nan
    H = run(handle, "dense", d)
    ref = reference("dense", d)
    np.testing.assert_array_equal(np.isnan(H), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert oracle.tolerance_ratio(H[ok], ref[ok], oracle.TOL_F32) <= 1.0


def test_plan_of_headline_layer(handle):
    d = generate(WORKLOADS["dense_f16_n1792"].with_(T=2))
    run(handle, "dense", d)
    p = handle.last_plan()
    assert p["layout"] == binding.LAYOUT_TEAM
    assert p["grid"] == 256 and p["rows_per_wave"] == 7 and p["waves_per_wg"] == 8
    run(handle, "dense", d, layout=binding.LAYOUT_SPREAD)
    p = handle.last_plan()
    assert p["layout"] == binding.LAYOUT_SPREAD
    assert p["grid"] == 256 and p["rows_per_wave"] == 7 and p["waves_per_wg"] == 4
    assert p["relay_slice"] == 1792 // 32   # auto picks the per-XCD relay at 256 workgroups


def test_dense_fp32_n1792_team_layout(handle):
    """fp32 W at N = 1792 runs in the team layout (7 rows x 7 chunks per wave,
    widened like fp16); the spread layout has no instance of that size."""
    w = WORKLOADS["dense_f16_n1792"].with_(w_dtype="f32", T=48, h0="randn")
    d = generate(w, seed=97)
    H = run(handle, "dense", d)
    p = handle.last_plan()
    assert p["layout"] == binding.LAYOUT_TEAM and p["rows_per_wave"] == 7 and p["rmax"] == 7, p
    assert_parity(H, reference("dense", d), oracle.TOL_F32, "fp32 N=1792")
    np.testing.assert_array_equal(run(handle, "dense", d), H)   # repeatable
    with pytest.raises(PrnnError) as e:
        run(handle, "dense", d, layout=binding.LAYOUT_SPREAD)
    assert e.value.status == binding.NOT_SUPPORTED
    handle.set_layout(binding.LAYOUT_AUTO)


def test_plan_of_large_sparse_layers(handle):
    """Sparse fp16 layers that would hold more than 8 rows per wave at 8 waves
    per workgroup run 12-wave workgroups, above 16 rows 16-wave ones first,
    where an instance fits (1 % at N = 5760: 16 waves of 12 rows; 5 % at
    N = 5760, whose 12 x 5 block does not fit 4 waves per SIMD: 12 waves of 15
    rows on one XCD, or, as it runs by default, 12 waves of 8 rows on two XCDs
    per batch row; N = 2304: 12 waves of 6 rows); N = 1792 keeps 8 waves of 7
    rows; the unbalanced 25 % layer, stored at its longest row's 1010 pairs (16
    slots), which no one-XCD instance holds: 8 waves of 5 rows on two XCDs per
    batch row)."""
    for name, waves, rows, xcds in [("sparse1_f16_n5760", 16, 12, 0), ("sparse5_f16_n5760", 12, 15, 1),
                                    ("sparse5_f16_n5760", 12, 8, 0), ("sparse10_f16_n2304", 12, 6, 0),
                                    ("sparse25_f16_n2304", 12, 6, 0), ("sparse10u_f16_n2304", 12, 6, 0),
                                    ("sparse25u_f16_n2304", 8, 5, 0), ("sparse10_f16_n1792", 8, 7, 0)]:
        w = WORKLOADS[name].with_(T=6)
        d = generate(w, seed=71)
        handle.set_xcds_per_row(xcds)
        try:
            H = run(handle, "sparse", d)
            p = handle.last_plan()
        finally:
            handle.set_xcds_per_row(0)
        assert p["layout"] == binding.LAYOUT_TEAM and p["waves_per_wg"] == waves and p["rows_per_wave"] == rows, p
        if name == "sparse25u_f16_n2304":
            assert p["xcds_per_row"] == 2, p
        assert_parity(H, reference("sparse", d), oracle.TOL_F16, name)
    # the 16-slot layer on one XCD: no instance (NOT_SUPPORTED in the TEAM layout)
    d = generate(WORKLOADS["sparse25u_f16_n2304"].with_(T=4), seed=73)
    handle.set_xcds_per_row(1)
    handle.set_layout(binding.LAYOUT_TEAM)
    try:
        with pytest.raises(PrnnError) as e:
            run(handle, "sparse", d)
        assert e.value.status == binding.NOT_SUPPORTED
    finally:
        handle.set_xcds_per_row(0)
        handle.set_layout(binding.LAYOUT_AUTO)
    # forced wave counts: 8 for the 1 % layer (23 rows per wave), 16 where no
    # instance or kernel has it (NOT_SUPPORTED in the TEAM layout), bad values
    w = WORKLOADS["sparse1_f16_n5760"].with_(T=6)
    d = generate(w, seed=72)
    handle.set_team_waves(8)
    try:
        H = run(handle, "sparse", d)
        p = handle.last_plan()
        assert p["waves_per_wg"] == 8 and p["rows_per_wave"] == 23
        assert_parity(H, reference("sparse", d), oracle.TOL_F16, "forced 8 waves")
        out = torch.empty((6, 4, 5760), device="cuda")
        handle.sync_floor(5760, 4, 6, out=out)
        assert handle.last_plan()["waves_per_wg"] == 8
        handle.set_team_waves(12)
        H = run(handle, "sparse", d)
        p = handle.last_plan()
        assert p["waves_per_wg"] == 12 and p["rows_per_wave"] == 15
        assert_parity(H, reference("sparse", d), oracle.TOL_F16, "forced 12 waves")
        handle.set_team_waves(16)
        for name, kind in [("sparse5_f16_n5760", "sparse"), ("dense_f16_n1152", "dense")]:
            w2 = WORKLOADS[name].with_(T=3)
            with pytest.raises(PrnnError) as e:
                run(handle, kind, generate(w2), layout=binding.LAYOUT_TEAM)
            assert e.value.status == binding.NOT_SUPPORTED
        with pytest.raises(PrnnError) as e:
            handle.set_team_waves(10)
        assert e.value.status == binding.BAD_PARAM
    finally:
        handle.set_team_waves(0)
        handle.set_layout(binding.LAYOUT_AUTO)
    # a ragged large layer, one slot per row, several forced grids
    for N, grid in [(6001, 0), (4500, 192), (8000, 256), (3001, 0), (2500, 256)]:
        w = Workload(f"sparse_{N}", "sparse", N, 3, 5, "f16", K=40, seed=N, h0="randn")
        d = generate(w)
        H = run(handle, "sparse", d, grid=grid)
        assert_parity(H, reference("sparse", d), oracle.TOL_F16, f"N={N} grid={grid} {handle.last_plan()}")


@pytest.mark.parametrize("name", ["dense_f16_n1792", "sparse10_f16_n1792", "sparse1_f16_n1792"])
def test_team_and_spread_agree_bitwise(handle, name):
    """At N = 1792 both layouts give every wave the same 7 rows, the same
    column-to-lane map and the same summation order: identical results."""
    w = WORKLOADS[name].with_(T=48, h0="randn")
    d = generate(w, seed=31)
    Ht = run(handle, w.kind, d, layout=binding.LAYOUT_TEAM)
    assert handle.last_plan()["layout"] == binding.LAYOUT_TEAM
    Hs = run(handle, w.kind, d, layout=binding.LAYOUT_SPREAD)
    np.testing.assert_array_equal(Ht, Hs)
    assert_parity(Ht, reference(w.kind, d), tol_of(d), name)


@pytest.mark.parametrize("B", [1, 3, 8])
def test_team_layout_batch_rows(handle, B):
    """B < 8 leaves XCDs that recompute a batch row without writing H; B = 8
    uses every XCD once."""
    for name in ("dense_f16_n1152", "sparse10_f16_n1792"):
        w = WORKLOADS[name].with_(T=20, B=B, h0="randn")
        d = generate(w, seed=40 + B)
        H = run(handle, w.kind, d, layout=binding.LAYOUT_TEAM)
        assert handle.last_plan()["layout"] == binding.LAYOUT_TEAM
        assert_parity(H, reference(w.kind, d), tol_of(d), f"{name} B={B}")


@pytest.mark.parametrize("name,grid", [("dense_f16_n1792", 0), ("sparse10_f16_n1792", 0),
                                       ("sparse1_f16_n5760", 0), ("dense_f16_n1152", 128),
                                       ("sparse10_f16_n1152", 192)])
def test_relay_and_direct_exchange_agree_bitwise(handle, name, grid):
    """Both exchanges deliver the same h_{t-1}, so the results are identical."""
    w = WORKLOADS[name].with_(T=40, h0="randn")
    d = generate(w, seed=21)
    out = {}
    for mode in (binding.EXCHANGE_DIRECT, binding.EXCHANGE_RELAY):
        handle.set_exchange(mode)
        out[mode] = run(handle, w.kind, d, grid=grid, layout=binding.LAYOUT_SPREAD)
        assert (handle.last_plan()["relay_slice"] > 0) == (mode == binding.EXCHANGE_RELAY)
    handle.set_exchange(binding.EXCHANGE_AUTO)
    np.testing.assert_array_equal(out[binding.EXCHANGE_DIRECT], out[binding.EXCHANGE_RELAY])
    assert_parity(out[binding.EXCHANGE_RELAY], reference(w.kind, d), tol_of(d), name)


def test_mixed_exchange_calls_on_one_handle(handle):
    """Calls that alternate exchanges, grids and lengths on one handle keep the
    ring and its XCD-local copies consistent (each call matches the oracle)."""
    w = WORKLOADS["dense_f32_n256"]
    S, T_ = binding.LAYOUT_SPREAD, binding.LAYOUT_TEAM
    seq = [(S, binding.EXCHANGE_RELAY, 0, 32), (S, binding.EXCHANGE_RELAY, 0, 1), (S, binding.EXCHANGE_RELAY, 0, 7),
           (S, binding.EXCHANGE_DIRECT, 0, 5), (S, binding.EXCHANGE_RELAY, 0, 6), (S, binding.EXCHANGE_RELAY, 128, 9),
           (S, binding.EXCHANGE_DIRECT, 64, 3), (T_, binding.EXCHANGE_AUTO, 0, 32), (T_, binding.EXCHANGE_AUTO, 0, 1),
           (T_, binding.EXCHANGE_AUTO, 64, 5), (S, binding.EXCHANGE_AUTO, 0, 4), (T_, binding.EXCHANGE_AUTO, 0, 9),
           (binding.LAYOUT_AUTO, binding.EXCHANGE_AUTO, 0, 32)]
    for i, (layout, mode, grid, T) in enumerate(seq):
        d = generate(w.with_(T=T, h0="randn", B=1 + i % 4), seed=300 + i)
        handle.set_exchange(mode)
        H = run(handle, "dense", d, grid=grid, layout=layout)
        assert_parity(H, reference("dense", d), oracle.TOL_F32,
                      f"call {i} layout {layout} mode {mode} grid {grid} T {T} plan {handle.last_plan()}")
    handle.set_exchange(binding.EXCHANGE_AUTO)


def test_forced_relay_needs_an_even_grid(handle):
    d = generate(WORKLOADS["dense_f16_n1152"].with_(T=2))
    handle.set_exchange(binding.EXCHANGE_RELAY)
    with pytest.raises(PrnnError) as e:
        run(handle, "dense", d, grid=100, layout=binding.LAYOUT_SPREAD)
    assert e.value.status == binding.NOT_SUPPORTED
    handle.set_exchange(binding.EXCHANGE_AUTO)
    handle.set_grid(0)


@pytest.mark.parametrize("layout", [binding.LAYOUT_TEAM, binding.LAYOUT_SPREAD])
def test_sync_floor_protocol(handle, layout):
    T, B, N = 16, 4, 1792
    handle.set_grid(0)
    handle.set_layout(layout)
    H = handle.sync_floor(N, B, T)
    handle.synchronize()
    assert handle.last_plan()["layout"] == layout
    expect = np.broadcast_to(np.arange(1, T + 1, dtype=np.float32)[:, None, None], (T, B, N))
    np.testing.assert_array_equal(H.cpu().numpy(), expect)
    handle.set_layout(binding.LAYOUT_AUTO)


# ---------------------------------------------------------------------------
# errors
# ---------------------------------------------------------------------------
def test_bad_params(handle):
    lib = binding.load_library()
    h = handle._h
    X = torch.zeros(4, 2, 64, device="cuda")
    H = torch.zeros(4, 2, 64, device="cuda")
    W = torch.zeros(64, 64, device="cuda")
    col = torch.zeros(64, 4, dtype=torch.int16, device="cuda")
    val = torch.zeros(64, 4, dtype=torch.float16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    bp = binding.BAD_PARAM
    dense = lambda N, B, T, wt, w, x, h0, out: lib.prnn_forward_dense(h, N, B, T, wt, w, x, h0, out, s)
    assert dense(64, 2, 4, 0, W.data_ptr(), X.data_ptr(), None, H.data_ptr()) == binding.SUCCESS
    assert dense(0, 2, 4, 0, W.data_ptr(), X.data_ptr(), None, H.data_ptr()) == bp
    assert dense(64, 9, 4, 0, W.data_ptr(), X.data_ptr(), None, H.data_ptr()) == bp
    assert dense(64, 2, -1, 0, W.data_ptr(), X.data_ptr(), None, H.data_ptr()) == bp
    assert dense(64, 2, 4, 7, W.data_ptr(), X.data_ptr(), None, H.data_ptr()) == bp
    assert dense(64, 2, 4, 0, None, X.data_ptr(), None, H.data_ptr()) == bp
    assert dense(64, 2, 4, 0, W.data_ptr(), X.data_ptr() + 2, None, H.data_ptr()) == bp
    assert dense(64, 2, 4, 0, W.data_ptr(), X.data_ptr(), None, X.data_ptr() + 256) == bp   # X and H overlap
    sparse = lambda N, K: lib.prnn_forward_sparse(h, N, 2, 4, K, col.data_ptr(), 1, val.data_ptr(),
                                                  X.data_ptr(), None, H.data_ptr(), s)
    assert sparse(64, 4) == binding.SUCCESS
    assert sparse(64, 0) == bp
    assert sparse(64, 65) == bp
    assert sparse(40000, 4) == bp
    handle.synchronize()


def test_not_supported(handle):
    N = 6000
    W = torch.zeros(N, N, dtype=torch.float16, device="cuda")
    X = torch.zeros(2, 4, N, device="cuda")
    with pytest.raises(PrnnError) as e:
        handle.forward_dense(W, X)
    assert e.value.status == binding.NOT_SUPPORTED
    handle.set_grid(1)
    W = torch.zeros(1792, 1792, dtype=torch.float16, device="cuda")
    with pytest.raises(PrnnError) as e:
        handle.forward_dense(W, torch.zeros(2, 4, 1792, device="cuda"))
    assert e.value.status == binding.NOT_SUPPORTED
    handle.set_grid(0)


# ---------------------------------------------------------------------------
# phase tracing
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["dense_f16_n1792", "sparse10_f16_n1792", "dense_f32_n256", "sparse1_f16_n5760",
                                  "dense_f16_n1152", "sparse10_f16_n1152"])
def test_trace_records_phases(gpu, name):
    """A traced run gives the untraced result bitwise; every wave of a team
    that serves a batch row records T steps whose phase cycles add up to its
    time loop; the other records stay zero."""
    w = WORKLOADS[name].with_(T=48)
    d = generate(w, seed=w.seed + 21)
    with Handle() as h:
        H0 = run(h, w.kind, d)
        h.set_trace(True)
        H1 = run(h, w.kind, d)
        tr = h.get_trace()
        plan = h.last_plan()
        h.set_trace(False)
        H2 = run(h, w.kind, d)
    assert np.array_equal(H0, H1) and np.array_equal(H0, H2)
    assert plan["layout"] == binding.LAYOUT_TEAM
    grid = plan["grid"]
    waves = plan["waves_per_wg"]
    assert waves == (16 if name == "sparse1_f16_n5760" else 8)   # the N = 5760 layer runs 16-wave workgroups
    assert tr.shape == (grid * waves, binding.TRACE_WORDS)
    rec = tr.reshape(grid, waves, binding.TRACE_WORDS).astype(np.float64)
    serving = (np.arange(grid) % 8) < w.B
    live = rec[serving]
    assert np.all(live[..., 7] == w.T)
    phases, loop = live[..., :5].sum(-1), live[..., 5]
    assert np.all(phases <= loop) and np.all(phases >= 0.9 * loop)
    assert np.all(rec[~serving] == 0)
    cycles_per_tick = loop / live[..., 6]
    assert np.all((cycles_per_tick > 5) & (cycles_per_tick < 40)), cycles_per_tick.min()


def test_trace_floor_and_errors(gpu):
    N, B, T = 1792, 4, 16
    with Handle() as h:
        with pytest.raises(PrnnError) as e:
            h.get_trace()                       # no traced call yet
        assert e.value.status == binding.BAD_PARAM
        h.set_trace(True)
        out = torch.empty((T, B, N), device="cuda")
        h.sync_floor(N, B, T, out=out)
        tr = h.get_trace()
        assert int((tr[:, 7] == T).sum()) == B * (h.last_plan()["grid"] // 8) * 8
        # a layer too large for 16 rows per wave at 8 waves: 16-wave workgroups, 16 records each
        h.sync_floor(5760, B, T, out=torch.empty((T, B, 5760), device="cuda"))
        tr = h.get_trace()
        p = h.last_plan()
        assert p["waves_per_wg"] == 16 and tr.shape[0] == p["grid"] * 16
        assert int((tr[:, 7] == T).sum()) == B * (p["grid"] // 8) * 16
        h.set_layout(binding.LAYOUT_SPREAD)     # trace instances are team-layout only
        w = WORKLOADS["dense_f16_n1792"].with_(T=4)
        g = to_dev(generate(w))
        with pytest.raises(PrnnError) as e:
            h.forward_dense(g["W"], g["X"], g["h0"])
        assert e.value.status == binding.NOT_SUPPORTED
        h.set_layout(binding.LAYOUT_AUTO)
        h.set_trace(False)
        h.forward_dense(g["W"], g["X"], g["h0"])
        h.synchronize()


@pytest.mark.parametrize("layout", [binding.LAYOUT_TEAM, binding.LAYOUT_SPREAD])
@pytest.mark.parametrize("kind", ["dense", "sparse"])
def test_watchdog_reports_and_recovers(gpu, kind, layout):
    """A workgroup that never publishes step 5 makes the consumers' bounded
    waits expire: the run reports EXECUTION_FAILED and the handle recovers."""
    name = "dense_f16_n1792" if kind == "dense" else "sparse10_f16_n1792"
    w = WORKLOADS[name].with_(T=12)
    d = generate(w, seed=13)
    with Handle() as h:
        h.set_layout(layout)
        h.set_watchdog_us(2000)
        h.debug_skip_publish(3, 5)
        g = to_dev(d)
        fwd = (lambda: h.forward_dense(g["W"], g["X"], g["h0"])) if kind == "dense" else \
              (lambda: h.forward_sparse(g["col"], g["val"], g["X"], g["h0"]))
        fwd()
        with pytest.raises(PrnnError) as e:
            h.synchronize()
        assert e.value.status == binding.EXECUTION_FAILED
        h.synchronize()           # reported once
        H = fwd()                 # the ring was reset: a clean run works again
        h.synchronize()
        assert_parity(H.cpu().numpy(), reference(kind, d), oracle.TOL_F16)


# ---------------------------------------------------------------------------
# dense fp16 on the matrix cores (MATH_SPLIT: h as fp16 hi + lo)
# ---------------------------------------------------------------------------
def run_split(handle, d, grid=0, h0=True):
    handle.set_math(binding.MATH_SPLIT)
    try:
        H = run(handle, "dense", d, grid=grid, h0=h0)
        assert handle.last_plan()["math"] == binding.MATH_SPLIT
    finally:
        handle.set_math(binding.MATH_AUTO)
    return H


@pytest.mark.parametrize("name", ["dense_f16_n1152", "dense_f16_n1792"])
def test_split_parity_workloads(handle, name):
    w = WORKLOADS[name]
    d = generate(w, seed=w.seed + 3000)
    H = run_split(handle, d)
    assert_parity(H, reference("dense", d), oracle.TOL_F16, name)
    p = handle.last_plan()
    assert p["layout"] == binding.LAYOUT_TEAM and p["waves_per_wg"] == 8


@pytest.mark.parametrize("N,B,T,grid", [(1, 1, 3, 0), (3, 2, 4, 0), (7, 3, 5, 0), (100, 4, 6, 0), (257, 5, 4, 0),
                                        (1000, 8, 3, 0), (2048, 4, 3, 0), (1792, 4, 5, 240), (1152, 2, 6, 256)])
def test_split_shapes(handle, N, B, T, grid):
    w = Workload(f"dense_{N}", "dense", N, B, T, "f16", seed=N * 13 + B, h0="randn")
    d = generate(w)
    H = run_split(handle, d, grid=grid)
    assert_parity(H, reference("dense", d), oracle.TOL_F16, f"N={N} B={B} grid={grid} {handle.last_plan()}")


def test_split_closed_forms_bitwise(handle):
    """hi + lo holds small integers exactly, so the closed forms stay exact."""
    rng = np.random.default_rng(41)
    T, B, N = 30, 4, 1792
    X = rng.integers(0, 100, size=(T, B, N)).astype(np.float32)
    h0 = rng.integers(0, 100, size=(B, N)).astype(np.float32)
    expect = h0[None].astype(np.float64) + np.cumsum(X.astype(np.float64), axis=0)
    np.testing.assert_array_equal(run_split(handle, {"W": np.eye(N, dtype=np.float16), "X": X, "h0": h0}), expect)
    Xr = rng.standard_normal((T, B, N)).astype(np.float32)
    np.testing.assert_array_equal(run_split(handle, {"W": np.zeros((N, N), np.float16), "X": Xr, "h0": h0}),
                                  np.maximum(Xr, 0))
    N = 1152
    Xs = rng.integers(0, 9, size=(12, 2, N)).astype(np.float32)
    hs = rng.integers(0, 9, size=(2, N)).astype(np.float32)
    Wd = np.zeros((N, N), np.float16)
    Wd[np.arange(N), (np.arange(N) + 1) % N] = 1
    np.testing.assert_array_equal(run_split(handle, {"W": Wd, "X": Xs, "h0": hs}), oracle.forward_dense(Wd, Xs, hs))


def test_split_close_to_exact_deterministic_and_chunkable(handle):
    w = WORKLOADS["dense_f16_n1792"].with_(T=40, h0="randn")
    d = generate(w, seed=43)
    He = run(handle, "dense", d)
    Hs = run_split(handle, d)
    assert np.all(np.abs(Hs - He) <= 2e-5 * (1 + np.abs(He)))
    np.testing.assert_array_equal(run_split(handle, d), Hs)
    Ha = run_split(handle, dict(d, X=d["X"][:17]))
    Hb = run_split(handle, dict(d, X=d["X"][17:], h0=Ha[-1]))
    np.testing.assert_array_equal(np.concatenate([Ha, Hb]), Hs)


def test_split_range_reported(gpu):
    """|h| beyond the fp16 range of the split is reported, then the handle recovers."""
    w = WORKLOADS["dense_f16_n1792"].with_(T=6)
    d = generate(w, seed=44)
    d["X"] = d["X"].copy()
    d["X"][2, 1, 7] = 1e6
    with Handle() as h:
        h.set_math(binding.MATH_SPLIT)
        g = to_dev(d)
        h.forward_dense(g["W"], g["X"], g["h0"])
        with pytest.raises(PrnnError) as e:
            h.synchronize()
        assert e.value.status == binding.EXECUTION_FAILED
        h.set_math(binding.MATH_EXACT)
        H = h.forward_dense(g["W"], g["X"], g["h0"])
        h.synchronize()
        assert_parity(H.cpu().numpy(), reference("dense", d), oracle.TOL_F16)


def test_split_scope(handle):
    """The matrix-core form exists for fp16 W in the team layout up to 2048
    neurons: beyond that (where exact and half-h math still run) or in the
    spread layout the call is NOT_SUPPORTED; fp32 W keeps exact math."""
    handle.set_math(binding.MATH_SPLIT)
    try:
        d = generate(Workload("dense_2304", "dense", 2304, 4, 2, "f16", seed=6))
        with pytest.raises(PrnnError) as e:
            run(handle, "dense", d)
        assert e.value.status == binding.NOT_SUPPORTED
        d = generate(WORKLOADS["dense_f16_n1152"].with_(T=3))
        with pytest.raises(PrnnError) as e:
            run(handle, "dense", d, layout=binding.LAYOUT_SPREAD)
        assert e.value.status == binding.NOT_SUPPORTED
        d = generate(WORKLOADS["dense_f32_n256"])
        H = run(handle, "dense", d)
        assert handle.last_plan()["math"] == binding.MATH_EXACT
        assert_parity(H, reference("dense", d), oracle.TOL_F32, "fp32 W under SPLIT")
    finally:
        handle.set_math(binding.MATH_AUTO)


def test_split_trace_and_watchdog(gpu):
    w = WORKLOADS["dense_f16_n1792"].with_(T=24)
    d = generate(w, seed=45)
    with Handle() as h:
        h.set_math(binding.MATH_SPLIT)
        H0 = run(h, "dense", d)
        h.set_trace(True)
        H1 = run(h, "dense", d)
        tr = h.get_trace()
        h.set_trace(False)
        np.testing.assert_array_equal(H0, H1)
        live = tr[tr[:, 7] == w.T].astype(np.float64)
        assert live.shape[0] == 4 * (h.last_plan()["grid"] // 8) * 8
        assert np.all(live[:, :5].sum(1) <= live[:, 5])
        h.set_watchdog_us(2000)
        h.debug_skip_publish(3, 5)
        g = to_dev(d)
        h.forward_dense(g["W"], g["X"], g["h0"])
        with pytest.raises(PrnnError) as e:
            h.synchronize()
        assert e.value.status == binding.EXECUTION_FAILED
        H2 = h.forward_dense(g["W"], g["X"], g["h0"])
        h.synchronize()
        np.testing.assert_array_equal(H2.cpu().numpy(), H0)


def test_log_lines_on_stderr(gpu, capfd, monkeypatch):
    """PRNN_LOG=1 when a handle is created: one stderr line per launch with its
    plan and one per failed run that prnn_synchronize reports; without it the
    library prints nothing."""
    w = WORKLOADS["sparse1_f16_n5760"].with_(T=4)
    d = generate(w, seed=81)
    g = to_dev(d)
    monkeypatch.setenv("PRNN_LOG", "1")
    with Handle() as h:
        h.forward_sparse(g["col"], g["val"], g["X"], g["h0"])
        h.synchronize()
        h.sync_floor(w.N, w.B, w.T, out=torch.empty((w.T, w.B, w.N), device="cuda"))
        h.synchronize()
        h.set_watchdog_us(2000)
        h.debug_skip_publish(2, 1)
        h.forward_sparse(g["col"], g["val"], g["X"], g["h0"])
        with pytest.raises(PrnnError):
            h.synchronize()
    err = capfd.readouterr().err
    assert "prnn: handle on device" in err
    assert ("prnn: recurrence N=5760 B=4 T=4 layout=team xcds/row=1 grid=256 waves/wg=16 rows/wave=12 "
            "instance=(12,1)") in err
    assert "prnn: floor N=5760 B=4 T=4 layout=team xcds/row=1 grid=256 waves/wg=16" in err
    assert "prnn: run failed: a wait for h_{t-1} expired (watchdog)" in err
    monkeypatch.delenv("PRNN_LOG")
    with Handle() as h:
        h.forward_sparse(g["col"], g["val"], g["X"], g["h0"])
        h.synchronize()
    assert "prnn:" not in capfd.readouterr().err


@pytest.mark.parametrize("kind,name,T", [("dense", "dense_f16_n1152", 15), ("sparse", "sparse10_f16_n1792", 13),
                                         ("dense", "dense_f32_n256", 7), ("dense", "split_n3072_b4", 9),
                                         ("dense", "split_n4096_b2", 6), ("rows", "sparse10u_f16_n2304", 11)])
def test_graph_capture_and_replay(gpu, kind, name, T):
    """A call captured into a HIP graph replays correctly any number of times,
    with eager calls of another length on the same handle between the replays:
    every replay and every eager call equals, bitwise, a fresh handle's result.
    Also for dense layers split over 2 and 4 XCDs per batch row (the shared
    ring's fill is captured too) and for sparse rows of unequal length (the
    ordering kernel is captured)."""
    if name.startswith("split_"):
        N, B = int(name.split("_n")[1].split("_")[0]), int(name.split("_b")[1])
        w = Workload(name, "dense", N, B, T, "f16", seed=N, h0="randn")
    else:
        w = WORKLOADS[name].with_(T=T, h0="randn")
    d, d2 = generate(w, seed=91), generate(w.with_(T=T + 2), seed=92)
    g, g2 = to_dev(d), to_dev(d2)

    def call(h, gg, out=None):
        if kind == "dense":
            return h.forward_dense(gg["W"], gg["X"], gg["h0"], out=out)
        if kind == "rows":
            return h.forward_sparse_rows(gg["col"], gg["val"], gg["row_len"], gg["X"], gg["h0"], out=out)
        return h.forward_sparse(gg["col"], gg["val"], gg["X"], gg["h0"], out=out)

    with Handle() as fresh:
        ref = call(fresh, g).clone()
        ref2 = call(fresh, g2).clone()
        fresh.synchronize()
    with Handle() as h:
        call(h, g2)                      # warm-up: the exchange buffer exists before capture
        h.synchronize()
        out = torch.full_like(ref, float("nan"))
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            call(h, g, out=out)
        torch.cuda.synchronize()
        for rep in range(4):
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            h.synchronize()
            assert torch.equal(out, ref), f"replay {rep}"
            e = call(h, g2)
            h.synchronize()
            assert torch.equal(e, ref2), f"eager call after replay {rep}"
        if name.startswith("split_"):
            assert h.last_plan()["xcds_per_row"] > 1
    if kind == "rows":
        ref_np = oracle.forward_sparse_rows(d["col"], d["val"], d["row_len"], d["X"], d["h0"])
    else:
        ref_np = reference(kind, d)
    assert oracle.tolerance_ratio(ref.cpu().numpy(), ref_np, tol_of(d)) <= 1.0
