"""Edges of the boundary's contract, on the GPU, through the C ABI.

* Signed initial states.  An initial state is any fp32 vector, while every
  word the kernels exchange carries its step tag in the sign bit (the state
  after a ReLU is never negative).  h0 must therefore enter every path as a
  plain value, never through the exchange: each path runs here with
  h0 ~ N(0, 1), about half of it negative, against the fp64 oracle.
* The sparse format's documented edges ("persistent-rnn", section "Important
  Constraints": the data must be laid out in the library's format, so the
  format's corners are part of the contract): a column repeated within a row
  adds its values, like the dense matrix with those values summed; a column
  outside [0, N) (negative ones included) reads zero.
* W aligned only to its element size (a view at an offset inside a larger
  buffer) gives bitwise the result of an aligned copy.
* A failed run is returned by the next call on the handle, without a
  synchronisation through the library, then the handle works again.
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


def ref_of(kind, d):
    if kind == "dense":
        return oracle.forward_dense(d["W"], d["X"], d["h0"])
    return oracle.forward_sparse(d["col"], d["val"], d["X"], d["h0"])


def tol_of(d):
    w = d["W"] if "W" in d else d["val"]
    return oracle.TOL_F32 if w.dtype == np.float32 else oracle.TOL_F16


def check(H, ref, tol, what):
    r = oracle.tolerance_ratio(H, ref, tol)
    assert r <= 1.0, f"{what}: max error ratio {r:.3g} > 1"


# (workload, layout, math, N: 0 = the workload's own) -- every kernel family
PATHS = [
    ("dense_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_EXACT, 0),
    ("dense_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_SPLIT, 0),
    ("dense_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_HALF, 0),
    ("dense_f16_n1792", binding.LAYOUT_SPREAD, binding.MATH_EXACT, 0),
    ("dense_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_EXACT, 2560),        # split over 2 XCDs per row
    ("dense_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_EXACT, 2560, 1),     # one XCD, 10 rows x 10 chunks
    ("dense_f32_n256", binding.LAYOUT_TEAM, binding.MATH_AUTO, 0),
    ("dense_f32_n256", binding.LAYOUT_SPREAD, binding.MATH_AUTO, 0),
    ("sparse10_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_AUTO, 0),
    ("sparse10_f16_n1792", binding.LAYOUT_SPREAD, binding.MATH_AUTO, 0),
    ("sparse1_f16_n5760", binding.LAYOUT_TEAM, binding.MATH_AUTO, 0),    # 16-wave workgroups
    ("sparse5_f16_n5760", binding.LAYOUT_TEAM, binding.MATH_AUTO, 0),    # two XCDs per batch row, 12-wave workgroups
]


def path_id(p):
    n = f"-n{p[3]}" if p[3] else ""
    x = f"-xcd{p[4]}" if len(p) > 4 else ""
    return f"{p[0]}{n}-{'team' if p[1] == binding.LAYOUT_TEAM else 'spread'}-math{p[2]}{x}"


@pytest.mark.parametrize("path", PATHS, ids=path_id)
def test_signed_h0_every_path(gpu, path):
    name, layout, math, N, xcds = (*path, 0)[:5]
    w = WORKLOADS[name].with_(T=24, h0="randn", **({"N": N} if N else {}))
    d = generate(w, seed=w.seed + 4000)
    assert (d["h0"] < 0).mean() > 0.4
    g = to_dev(d)
    with Handle() as h:
        h.set_layout(layout)
        h.set_math(math)
        h.set_xcds_per_row(xcds)
        if "W" in d:
            H = h.forward_dense(g["W"], g["X"], g["h0"])
        else:
            H = h.forward_sparse(g["col"], g["val"], g["X"], g["h0"])
        h.synchronize()
        plan = h.last_plan()
    assert plan["layout"] == layout
    if math in (binding.MATH_SPLIT, binding.MATH_HALF):
        assert plan["math"] == math
    kind = "dense" if "W" in d else "sparse"
    check(H.cpu().numpy(), ref_of(kind, d), tol_of(d), path_id(path))


def test_signed_h0_first_step_exact(gpu):
    """With W = I and integer values the first step is h0 + X exactly, so a
    negative h0 word that lost or kept its sign bit by mistake shows bitwise."""
    N, B, T = 1024, 4, 3
    rng = np.random.default_rng(5)
    h0 = rng.integers(-8, 9, size=(B, N)).astype(np.float32)
    X = rng.integers(-4, 5, size=(T, B, N)).astype(np.float32)
    for wdt in (np.float16, np.float32):
        W = np.eye(N, dtype=wdt)
        ref = oracle.forward_dense(W, X, h0)
        with Handle() as h:
            for layout in (binding.LAYOUT_TEAM, binding.LAYOUT_SPREAD):
                h.set_layout(layout)
                H = h.forward_dense(torch.from_numpy(W).cuda(), torch.from_numpy(X).cuda(),
                                    torch.from_numpy(h0).cuda())
                h.synchronize()
                np.testing.assert_array_equal(H.cpu().numpy(), ref.astype(np.float32))


@pytest.mark.parametrize("kind", ["dense", "sparse"])
def test_signed_h0_layer(gpu, kind):
    base = "dense_f16_n1792" if kind == "dense" else "sparse10_f16_n1792"
    w = WORKLOADS[base].with_(T=16, h0="randn")
    d = generate_layer(w, 640, seed=81)
    assert (d["h0"] < 0).any()
    g = to_dev(d)
    with Handle() as h:
        if kind == "dense":
            H = h.forward_layer_dense(g["U"], g["bias"], g["W"], g["x"], g["h0"])
            ref = oracle.forward_layer_dense(d["U"], d["bias"], d["W"], d["x"], d["h0"])
        else:
            H = h.forward_layer_sparse(g["U"], g["bias"], g["col"], g["val"], g["x"], g["h0"])
            ref = oracle.forward_layer_sparse(d["U"], d["bias"], d["col"], d["val"], d["x"], d["h0"])
        h.synchronize()
    check(H.cpu().numpy(), ref, oracle.TOL_F16, f"layer {kind}")


@pytest.mark.parametrize("mode", [binding.STACK_BLOCKED, binding.STACK_FUSED, binding.STACK_LAYERS])
def test_signed_h0_stack(gpu, mode):
    w = WORKLOADS["dense_f16_n1152"].with_(N=640, B=2, T=80, h0="randn", seed=91)
    st = generate_stack(w, 3)
    assert all((h0 < 0).any() for h0 in st["h0s"])
    layers = [{k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in ly.items()} for ly in st["layers"]]
    with Handle() as h:
        h.set_stack_mode(mode)
        outs = h.forward_stack_dense(layers, torch.from_numpy(st["x"]).cuda(),
                                     [torch.from_numpy(v).cuda() for v in st["h0s"]])
        h.synchronize()
    refs = oracle.forward_stack_dense(st["layers"], st["x"], st["h0s"])
    for l, (o, r) in enumerate(zip(outs, refs)):
        check(o.cpu().numpy(), r, oracle.TOL_F16, f"stack mode {mode} layer {l}")


# ---------------------------------------------------------------------------
# the sparse format's edges
# ---------------------------------------------------------------------------
def repeated_columns(N, K, seed, vdt):
    """Rows whose K columns repeat: each row draws K // 3 + 1 distinct columns
    and fills its K slots from them, so every row repeats some."""
    rng = np.random.default_rng(seed)
    col = np.empty((N, K), dtype=np.int16)
    for i in range(N):
        pool = rng.choice(N, size=K // 3 + 1, replace=False)
        col[i] = np.sort(rng.choice(pool, size=K, replace=True))
    val = (rng.standard_normal((N, K)) * (0.8 / np.sqrt(K))).astype(vdt)
    return col, val


SPARSE_EDGE_CASES = [
    # N, K, B, T, values, layout
    (1792, 179, 4, 20, np.float16, binding.LAYOUT_TEAM),
    (1792, 179, 4, 20, np.float16, binding.LAYOUT_SPREAD),
    (1152, 115, 3, 12, np.float32, binding.LAYOUT_TEAM),
    (1152, 115, 3, 12, np.float32, binding.LAYOUT_SPREAD),
    (5760, 58, 2, 8, np.float16, binding.LAYOUT_TEAM),     # 16-wave workgroups
    (333, 70, 5, 9, np.float16, binding.LAYOUT_AUTO),      # ragged N, two 64-pair slots
]


def sparse_case_id(c):
    return f"N{c[0]}-K{c[1]}-B{c[2]}-{np.dtype(c[4]).name}-layout{c[5]}"


@pytest.mark.parametrize("case", SPARSE_EDGE_CASES, ids=sparse_case_id)
def test_sparse_repeated_columns_add_up(gpu, case):
    N, K, B, T, vdt, layout = case
    col, val = repeated_columns(N, K, N + K, vdt)
    assert any(len(np.unique(r)) < K for r in col)
    rng = np.random.default_rng(N * 3 + K)
    X = rng.standard_normal((T, B, N)).astype(np.float32)
    h0 = rng.standard_normal((B, N)).astype(np.float32)
    ref = oracle.forward_sparse(col, val, X, h0)
    # the same sums through the dense matrix the pairs stand for
    np.testing.assert_allclose(oracle.forward_dense(oracle.sparse_to_dense(col, val), X, h0), ref,
                               rtol=1e-12, atol=1e-12)
    with Handle() as h:
        h.set_layout(layout)
        H = h.forward_sparse(torch.from_numpy(col).cuda(), torch.from_numpy(val).cuda(),
                             torch.from_numpy(X).cuda(), torch.from_numpy(h0).cuda())
        h.synchronize()
    check(H.cpu().numpy(), ref, oracle.TOL_F32 if vdt == np.float32 else oracle.TOL_F16, sparse_case_id(case))


@pytest.mark.parametrize("case", SPARSE_EDGE_CASES, ids=sparse_case_id)
def test_sparse_out_of_range_columns_read_zero(gpu, case):
    """Columns in [N, 32767] and negative ones (as int16) read zero: the run
    equals the oracle's on the same pairs with those pairs' values set to 0
    (their column moved into range, where a zero value adds nothing)."""
    N, K, B, T, vdt, layout = case
    rng = np.random.default_rng(7 * N + K)
    col = np.empty((N, K), dtype=np.int16)
    for i in range(N):
        col[i] = np.sort(rng.choice(N, size=K, replace=False))
    val = (rng.standard_normal((N, K)) * (0.8 / np.sqrt(K))).astype(vdt)
    bad = rng.random((N, K)) < 0.2
    choices = np.array([N, N + 1, 32767, -1, -2, -32768], dtype=np.int64)
    col[bad] = choices[rng.integers(0, len(choices), size=int(bad.sum()))].astype(np.int16)
    assert (col < 0).any() and (col >= N).any()
    X = rng.standard_normal((T, B, N)).astype(np.float32)
    h0 = rng.standard_normal((B, N)).astype(np.float32)
    col_model = np.where(bad, 0, col).astype(np.int16)
    val_model = np.where(bad, 0, val).astype(vdt)
    ref = oracle.forward_sparse(col_model, val_model, X, h0)
    with Handle() as h:
        h.set_layout(layout)
        H = h.forward_sparse(torch.from_numpy(col).cuda(), torch.from_numpy(val).cuda(),
                             torch.from_numpy(X).cuda(), torch.from_numpy(h0).cuda())
        h.synchronize()
    check(H.cpu().numpy(), ref, oracle.TOL_F32 if vdt == np.float32 else oracle.TOL_F16, sparse_case_id(case))


# ---------------------------------------------------------------------------
# W aligned only to its element
# ---------------------------------------------------------------------------
W_ALIGN_CASES = [
    # N, weights, byte offset of W, layout, math
    (1792, np.float16, 2, binding.LAYOUT_TEAM, binding.MATH_EXACT),
    (1792, np.float16, 4, binding.LAYOUT_TEAM, binding.MATH_EXACT),
    (1792, np.float16, 8, binding.LAYOUT_TEAM, binding.MATH_HALF),
    (1792, np.float16, 4, binding.LAYOUT_TEAM, binding.MATH_SPLIT),
    (1792, np.float16, 4, binding.LAYOUT_SPREAD, binding.MATH_EXACT),
    (1024, np.float32, 4, binding.LAYOUT_TEAM, binding.MATH_AUTO),
    (1024, np.float32, 8, binding.LAYOUT_SPREAD, binding.MATH_AUTO),
]


@pytest.mark.parametrize("case", W_ALIGN_CASES, ids=lambda c: f"N{c[0]}-{np.dtype(c[1]).name}-off{c[2]}-l{c[3]}-m{c[4]}")
def test_dense_w_at_an_element_offset(gpu, case):
    N, wdt, off, layout, math = case
    w = Workload("align", "dense", N, 4, 12, "f16" if wdt == np.float16 else "f32", seed=N + off, h0="randn")
    d = generate(w)
    g = to_dev(d)
    esz = np.dtype(wdt).itemsize
    big = torch.zeros(N * N + 64, dtype=g["W"].dtype, device="cuda")
    assert big.data_ptr() % 256 == 0 and off % esz == 0
    Woff = big[off // esz: off // esz + N * N].view(N, N)
    Woff.copy_(g["W"])
    assert Woff.data_ptr() % 16 == off % 16
    with Handle() as h:
        h.set_layout(layout)
        h.set_math(math)
        H_al = h.forward_dense(g["W"], g["X"], g["h0"])
        H_off = h.forward_dense(Woff, g["X"], g["h0"])
        h.synchronize()
    assert torch.equal(H_al, H_off)
    check(H_off.cpu().numpy(), ref_of("dense", d), tol_of(d), "offset W")


def test_dense_w_below_element_alignment_rejected(gpu):
    lib = binding.load_library()
    X = torch.zeros(2, 1, 64, device="cuda")
    H = torch.zeros(2, 1, 64, device="cuda")
    W = torch.zeros(64 * 64 + 8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    with Handle() as h:
        assert lib.prnn_forward_dense(h._h, 64, 1, 2, binding.DATA_FLOAT, W.data_ptr() + 2, X.data_ptr(), None,
                                      H.data_ptr(), s) == binding.BAD_PARAM
        assert lib.prnn_forward_dense(h._h, 64, 1, 2, binding.DATA_HALF, W.data_ptr() + 1, X.data_ptr(), None,
                                      H.data_ptr(), s) == binding.BAD_PARAM
        assert lib.prnn_forward_dense(h._h, 64, 1, 2, binding.DATA_HALF, W.data_ptr() + 2, X.data_ptr(), None,
                                      H.data_ptr(), s) == binding.SUCCESS
        h.synchronize()


# ---------------------------------------------------------------------------
# a failed run is returned by the next call
# ---------------------------------------------------------------------------
FAIL_CASES = [
    ("dense_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_EXACT),
    ("dense_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_SPLIT),
    ("dense_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_HALF),
    ("dense_f16_n1792", binding.LAYOUT_SPREAD, binding.MATH_EXACT),
    ("sparse10_f16_n1792", binding.LAYOUT_TEAM, binding.MATH_AUTO),
    ("sparse10_f16_n1792", binding.LAYOUT_SPREAD, binding.MATH_AUTO),
    ("sparse1_f16_n5760", binding.LAYOUT_TEAM, binding.MATH_AUTO),
]


@pytest.mark.parametrize("case", FAIL_CASES, ids=lambda c: f"{c[0]}-l{c[1]}-m{c[2]}")
def test_watchdog_failure_returned_by_the_next_call(gpu, case):
    """A workgroup that never publishes step 5 makes the consumers' bounded
    waits expire.  After the device has finished (torch's synchronisation,
    not the library's), the next forward call returns EXECUTION_FAILED and
    enqueues nothing; the call after it runs cleanly."""
    name, layout, math = case
    w = WORKLOADS[name].with_(T=12, h0="randn")
    d = generate(w, seed=23)
    g = to_dev(d)
    kind = "dense" if "W" in d else "sparse"
    with Handle() as h:
        h.set_layout(layout)
        h.set_math(math)
        h.set_watchdog_us(2000)

        def fwd(out):
            if kind == "dense":
                return h.forward_dense(g["W"], g["X"], g["h0"], out=out)
            return h.forward_sparse(g["col"], g["val"], g["X"], g["h0"], out=out)

        h.debug_skip_publish(3, 5)
        fwd(torch.empty_like(g["X"]))
        torch.cuda.synchronize()
        sentinel = torch.full_like(g["X"], 7.0)
        with pytest.raises(PrnnError) as e:
            fwd(sentinel)
        assert e.value.status == binding.EXECUTION_FAILED
        torch.cuda.synchronize()
        assert bool((sentinel == 7.0).all()), "the reporting call must enqueue nothing"
        H = fwd(torch.empty_like(g["X"]))
        h.synchronize()          # nothing left to report
        check(H.cpu().numpy(), ref_of(kind, d), tol_of(d), "after recovery")


def test_range_failure_of_projection_returned_by_the_next_call(gpu):
    """An fp32 x beyond the fp16 range of the hi + lo split fails the
    projection; the next call returns it, then calls work again."""
    w = WORKLOADS["dense_f16_n1152"].with_(N=256, T=4, B=2)
    d = generate_layer(w, 128, seed=3)
    d["x"][1, 0, 5] = 1e6
    g = to_dev(d)
    with Handle() as h:
        h.project(g["U"], g["x"])
        torch.cuda.synchronize()
        with pytest.raises(PrnnError) as e:
            h.forward_dense(g["W"], g["X"], g["h0"])
        assert e.value.status == binding.EXECUTION_FAILED
        H = h.forward_dense(g["W"], g["X"], g["h0"])
        h.synchronize()
    check(H.cpu().numpy(), oracle.forward_dense(d["W"], d["X"], d["h0"]), oracle.TOL_F16, "after recovery")


def test_pending_failure_returned_by_destroy(gpu):
    w = WORKLOADS["sparse10_f16_n1152"].with_(T=10)
    d = generate(w, seed=29)
    g = to_dev(d)
    h = Handle()
    h.set_watchdog_us(2000)
    h.debug_skip_publish(1, 4)
    h.forward_sparse(g["col"], g["val"], g["X"], g["h0"])
    with pytest.raises(PrnnError) as e:
        h.close()
    assert e.value.status == binding.EXECUTION_FAILED


def test_failure_reported_once(gpu):
    """Reported by the next call, the failure is not reported again: neither
    prnn_synchronize nor prnn_destroy returns it a second time."""
    w = WORKLOADS["dense_f16_n1152"].with_(T=10, h0="randn")
    d = generate(w, seed=31)
    g = to_dev(d)
    h = Handle()
    h.set_watchdog_us(2000)
    h.debug_skip_publish(2, 3)
    h.forward_dense(g["W"], g["X"], g["h0"])
    torch.cuda.synchronize()
    with pytest.raises(PrnnError):
        h.forward_dense(g["W"], g["X"], g["h0"])
    h.synchronize()
    h.close()
