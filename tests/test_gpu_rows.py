"""Sparse layers whose rows hold different numbers of nonzeros
(prnn_forward_sparse_rows) against oracle.forward_sparse_rows.

The unbalanced workload at its full size; random lengths from 0 to K with
pairs past each row's length holding values and columns that must not count;
small-integer inputs that make every sum exact (bitwise); full-length rows
against the row-balanced call; lengths outside [0, K] (clamped); empty rows;
NaN-poisoned repeats and publish jitter; a forced watchdog expiry; argument
errors; rows on two XCDs per batch row (the unbalanced 25 % layer, whose rows
no one-XCD instance holds, and forced widths).
"""
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


def run_rows(h, d, out=None):
    g = to_dev(d)
    H = h.forward_sparse_rows(g["col"], g["val"], g["row_len"], g["X"], g.get("h0"), out=out)
    h.synchronize()
    return H.cpu().numpy()


def ragged_case(N, B, T, K, seed, h0=True):
    """Random lengths in [0, K] (some 0, some K), real pairs on distinct columns,
    and past each row's length values and columns (out of range too) that the
    call must not use."""
    rng = np.random.default_rng(seed)
    row_len = rng.integers(0, K + 1, size=N).astype(np.int32)
    row_len[rng.choice(N, min(N, 3), replace=False)] = 0
    row_len[rng.choice(N, min(N, 3), replace=False)] = K
    col = np.empty((N, K), np.int16)
    val = np.empty((N, K), np.float16)
    for i in range(N):
        L = int(row_len[i])
        col[i, :L] = np.sort(rng.choice(N, L, replace=False))
        col[i, L:] = rng.integers(-N, 2 * N, size=K - L)
        val[i, :L] = rng.standard_normal(L) * (0.8 / np.sqrt(max(L, 1)))
        val[i, L:] = rng.standard_normal(K - L) * 100.0
    d = {"col": col, "val": val, "row_len": row_len,
         "X": rng.standard_normal((T, B, N)).astype(np.float32)}
    if h0:
        d["h0"] = rng.standard_normal((B, N)).astype(np.float32)
    return d


def ref_of(d):
    col = d["col"].astype(np.int64)
    return oracle.forward_sparse_rows(col, d["val"], d["row_len"], d["X"], d.get("h0"))


def test_unbalanced_workload_full_size(handle):
    w = WORKLOADS["sparse10u_f16_n2304"].with_(h0="randn")
    d = generate(w, seed=w.seed + 7)
    H = run_rows(handle, d)
    p = handle.last_plan()
    assert p["layout"] == binding.LAYOUT_TEAM and p["waves_per_wg"] == 12, p
    r = oracle.tolerance_ratio(H, ref_of(d), oracle.TOL_F16)
    assert r <= 1.0, f"error ratio {r:.3g} plan={p}"


@pytest.mark.parametrize("N,B,T,K", [(300, 2, 5, 40), (1000, 3, 6, 100), (1000, 8, 3, 256), (1792, 4, 5, 300),
                                     (2304, 4, 4, 250), (2304, 1, 3, 640), (77, 5, 4, 64), (1, 1, 3, 1)])
def test_ragged_rows_parity(handle, N, B, T, K):
    d = ragged_case(N, B, T, K, seed=N + K)
    H = run_rows(handle, d)
    r = oracle.tolerance_ratio(H, ref_of(d), oracle.TOL_F16)
    assert r <= 1.0, f"N={N} B={B} K={K}: error ratio {r:.3g} plan={handle.last_plan()}"


@pytest.mark.parametrize("N,K", [(1000, 100), (2304, 617)])
def test_ragged_rows_small_integers_bitwise(handle, N, K):
    """Values +-1 on up to K columns and small integer inputs keep every sum an
    exact fp32 integer: each row, whatever its length and its wave, must equal
    the fp64 oracle bit for bit."""
    rng = np.random.default_rng(N)
    T, B = 5, 4
    row_len = rng.integers(0, K + 1, size=N).astype(np.int32)
    col = np.empty((N, K), np.int16)
    val = np.zeros((N, K), np.float16)
    for i in range(N):
        L = int(row_len[i])
        col[i] = rng.choice(N, K, replace=False)
        val[i, :L] = rng.choice([-1.0, 1.0], L) * (rng.random(L) < 0.02)
        val[i, L:] = 7.0                            # past the row: must not count
    X = rng.integers(-5, 6, size=(T, B, N)).astype(np.float32)
    h0 = rng.integers(-5, 6, size=(B, N)).astype(np.float32)
    d = {"col": col, "val": val, "row_len": row_len, "X": X, "h0": h0}
    ref = ref_of(d)
    assert np.abs(ref).max() < 2 ** 20
    np.testing.assert_array_equal(run_rows(handle, d), ref)


@pytest.mark.parametrize("name", ["sparse10_f16_n1792", "sparse10_f16_n2304"])
def test_full_length_rows_match_the_row_balanced_call(handle, name):
    w = WORKLOADS[name].with_(T=24, h0="randn")
    d = generate(w, seed=11)
    d["row_len"] = np.full(w.N, w.K, np.int32)
    H = run_rows(handle, d)
    g = to_dev(d)
    Hb = handle.forward_sparse(g["col"], g["val"], g["X"], g["h0"])
    handle.synchronize()
    ref = oracle.forward_sparse(d["col"], d["val"], d["X"], d["h0"])
    assert oracle.tolerance_ratio(H, ref, oracle.TOL_F16) <= 1.0
    assert oracle.tolerance_ratio(Hb.cpu().numpy(), ref, oracle.TOL_F16) <= 1.0


def test_lengths_outside_the_row_are_clamped(handle):
    """Lengths below 0 read as 0 and above K as K (those rows then use all K
    pairs, so they get real columns and values throughout)."""
    d = ragged_case(500, 2, 4, 80, seed=3)
    rng = np.random.default_rng(30)
    d["row_len"][:10] = -7
    d["row_len"][10:20] = 80 + 13
    for i in range(10, 20):
        d["col"][i] = np.sort(rng.choice(500, 80, replace=False))
        d["val"][i] = rng.standard_normal(80) * 0.09
    H = run_rows(handle, d)
    clamped = dict(d, row_len=np.clip(d["row_len"], 0, 80))
    assert oracle.tolerance_ratio(H, ref_of(clamped), oracle.TOL_F16) <= 1.0


def test_all_rows_empty_give_relu_x_bitwise(handle):
    d = ragged_case(700, 3, 5, 50, seed=4)
    d["row_len"][:] = 0
    np.testing.assert_array_equal(run_rows(handle, d), np.maximum(d["X"], 0))


def test_ragged_rows_without_h0(handle):
    d = ragged_case(1000, 2, 5, 120, seed=5, h0=False)
    assert oracle.tolerance_ratio(run_rows(handle, d), ref_of(d), oracle.TOL_F16) <= 1.0


def test_ragged_rows_repeats_and_jitter_bitwise(gpu):
    w = WORKLOADS["sparse10u_f16_n2304"].with_(T=32, h0="randn")
    d = generate(w, seed=21)
    g = to_dev(d)
    out = torch.empty_like(g["X"])
    with Handle() as h:
        out.fill_(float("nan"))
        first = h.forward_sparse_rows(g["col"], g["val"], g["row_len"], g["X"], g["h0"], out=out).clone()
        h.synchronize()
        assert not torch.isnan(first).any()
        for _ in range(6):
            out.fill_(float("nan"))
            h.forward_sparse_rows(g["col"], g["val"], g["row_len"], g["X"], g["h0"], out=out)
            h.synchronize()
            assert torch.equal(out, first)
        for seed in (1, 2, 3):
            h.debug_jitter(seed, 48)
            out.fill_(float("nan"))
            h.forward_sparse_rows(g["col"], g["val"], g["row_len"], g["X"], g["h0"], out=out)
            h.synchronize()
            assert torch.equal(out, first)
        h.debug_jitter(0, 0)
    assert oracle.tolerance_ratio(first.cpu().numpy(), ref_of(d), oracle.TOL_F16) <= 1.0


def test_ragged_rows_watchdog(gpu):
    w = WORKLOADS["sparse10u_f16_n2304"].with_(T=12, h0="randn")
    d = generate(w, seed=23)
    g = to_dev(d)
    with Handle() as h:
        h.set_watchdog_us(2000)
        h.debug_skip_publish(4, 5)
        h.forward_sparse_rows(g["col"], g["val"], g["row_len"], g["X"], g["h0"])
        with pytest.raises(PrnnError) as e:
            h.forward_sparse_rows(g["col"], g["val"], g["row_len"], g["X"], g["h0"])   # the next call reports it
            h.synchronize()
        assert e.value.status == binding.EXECUTION_FAILED
        H = h.forward_sparse_rows(g["col"], g["val"], g["row_len"], g["X"], g["h0"])
        h.synchronize()
        assert oracle.tolerance_ratio(H.cpu().numpy(), ref_of(d), oracle.TOL_F16) <= 1.0


@pytest.mark.parametrize("seed_off", [0, 1000])
def test_unbalanced_25_percent_layer_on_two_xcds(handle, seed_off):
    """The unbalanced 25 % layer's rows reach 1010 pairs (16 slots), more than
    a one-XCD instance holds: it runs on two XCDs per batch row, each XCD's
    part ordered by length on its own and dealt to its waves (8 waves of 5
    rows); full size against the oracle.  Forced onto one XCD: NOT_SUPPORTED,
    nothing enqueued."""
    w = WORKLOADS["sparse25u_f16_n2304"].with_(h0="randn")
    d = generate(w, seed=w.seed + seed_off)
    H = run_rows(handle, d)
    p = handle.last_plan()
    assert p["xcds_per_row"] == 2 and p["waves_per_wg"] == 8 and p["rows_per_wave"] == 5, p
    assert oracle.tolerance_ratio(H, ref_of(d), oracle.TOL_F16) <= 1.0
    if seed_off == 0:
        g = to_dev(generate(w.with_(T=3), seed=5))
        out = torch.full_like(g["X"], 7.0)
        handle.set_xcds_per_row(1)
        try:
            with pytest.raises(PrnnError) as e:
                handle.forward_sparse_rows(g["col"], g["val"], g["row_len"], g["X"], g["h0"], out=out)
            assert e.value.status == binding.NOT_SUPPORTED
        finally:
            handle.set_xcds_per_row(0)
        handle.synchronize()
        assert bool((out == 7.0).all())


@pytest.mark.parametrize("N,K", [(2304, 1000), (1500, 700), (300, 200)])
def test_rows_on_two_xcds_forced(handle, N, K):
    """prnn_set_xcds_per_row(2) puts rows of unequal length on two XCDs per
    batch row at any size an instance holds: random lengths 0 .. K with
    garbage past each row, against the oracle; with +-1 values and small
    integer inputs every sum is exact, so the result equals the oracle bit for
    bit."""
    d = ragged_case(N, 4, 5, K, seed=N + 7)
    handle.set_xcds_per_row(2)
    try:
        H = run_rows(handle, d)
        assert handle.last_plan()["xcds_per_row"] == 2
        assert oracle.tolerance_ratio(H, ref_of(d), oracle.TOL_F16) <= 1.0
        rng = np.random.default_rng(N)
        T, B = 4, 4
        row_len = rng.integers(0, K + 1, size=N).astype(np.int32)
        col = np.empty((N, K), np.int16)
        val = np.zeros((N, K), np.float16)
        for i in range(N):
            L = int(row_len[i])
            col[i] = rng.choice(N, K, replace=False)
            val[i, :L] = rng.choice([-1.0, 1.0], L) * (rng.random(L) < 0.02)
            val[i, L:] = 7.0
        e = {"col": col, "val": val, "row_len": row_len,
             "X": rng.integers(-5, 6, size=(T, B, N)).astype(np.float32),
             "h0": rng.integers(-5, 6, size=(B, N)).astype(np.float32)}
        np.testing.assert_array_equal(run_rows(handle, e), ref_of(e))
    finally:
        handle.set_xcds_per_row(0)


def test_rows_on_two_xcds_repeats_and_jitter_bitwise(gpu):
    w = WORKLOADS["sparse25u_f16_n2304"].with_(T=24, h0="randn")
    d = generate(w, seed=31)
    g = to_dev(d)
    out = torch.empty_like(g["X"])
    with Handle() as h:
        out.fill_(float("nan"))
        first = h.forward_sparse_rows(g["col"], g["val"], g["row_len"], g["X"], g["h0"], out=out).clone()
        h.synchronize()
        assert h.last_plan()["xcds_per_row"] == 2
        for seed in (0, 1, 2):
            h.debug_jitter(seed, 48 if seed else 0)
            out.fill_(float("nan"))
            h.forward_sparse_rows(g["col"], g["val"], g["row_len"], g["X"], g["h0"], out=out)
            h.synchronize()
            assert torch.equal(out, first)
        h.debug_jitter(0, 0)
    assert oracle.tolerance_ratio(first.cpu().numpy(), ref_of(d), oracle.TOL_F16) <= 1.0


def test_ragged_rows_argument_errors(handle):
    lib = binding.load_library()
    s = torch.cuda.current_stream().cuda_stream
    N, K, T, B = 64, 8, 2, 1
    col = torch.zeros(N, K, dtype=torch.int16, device="cuda")
    val = torch.zeros(N, K, dtype=torch.float16, device="cuda")
    rl = torch.zeros(N, dtype=torch.int32, device="cuda")
    X = torch.zeros(T, B, N, device="cuda")
    H = torch.empty(T, B, N, device="cuda")
    call = lambda **kw: lib.prnn_forward_sparse_rows(
        handle._h, kw.get("N", N), B, T, kw.get("K", K), col.data_ptr(), kw.get("vt", binding.DATA_HALF),
        val.data_ptr(), kw.get("rl", rl.data_ptr()), X.data_ptr(), None, H.data_ptr(), s)
    assert call() == binding.SUCCESS
    assert call(rl=None) == binding.BAD_PARAM
    assert call(rl=rl.data_ptr() + 2) == binding.BAD_PARAM
    assert call(K=0) == binding.BAD_PARAM and call(K=N + 1) == binding.BAD_PARAM
    assert call(vt=binding.DATA_FLOAT) == binding.NOT_SUPPORTED
    handle.synchronize()
    big = 1100
    with pytest.raises(PrnnError) as e:
        handle.forward_sparse_rows(torch.zeros(big, 1025, dtype=torch.int16, device="cuda"),
                                   torch.zeros(big, 1025, dtype=torch.float16, device="cuda"),
                                   torch.zeros(big, dtype=torch.int32, device="cuda"), torch.zeros(2, 1, big, device="cuda"))
    assert e.value.status == binding.NOT_SUPPORTED
    handle.set_layout(binding.LAYOUT_SPREAD)
    try:
        with pytest.raises(PrnnError) as e:
            handle.forward_sparse_rows(col, val, rl, X)
        assert e.value.status == binding.NOT_SUPPORTED
    finally:
        handle.set_layout(binding.LAYOUT_AUTO)
