"""Dense fp16 layers split over several XCDs per batch row: 2 XCDs (B <= 4,
N <= 3584) or 4 XCDs (B <= 2, N <= 5120), the parts exchanging their rows of
h_{t-1} through device-coherent memory.  Automatic beyond N = 1792 (4 XCDs
where B <= 2 and N > 2048), and the only form beyond N = 2560; forced with
prnn_set_xcds_per_row at any size.

Parity against the fp64 oracle at the fp16-weight bar, bitwise closed forms
that catch a row or a part in the wrong place, chunked calls with changing
batch sizes (the tail stamps of teams without a batch row), the watchdog,
NaN-poisoned repeats and seeded publish jitter, and a whole layer.
"""
import numpy as np
import pytest
import torch

import oracle
from persistent_rnn_fwd_amd import Handle, PrnnError, binding
from persistent_rnn_fwd_amd.inputs import Workload, generate, generate_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def handle(gpu):
    h = Handle()
    yield h
    h.close()


def to_dev(d):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in d.items()}


def run(handle, d, h0=True):
    g = to_dev(d)
    H = handle.forward_dense(g["W"], g["X"], g["h0"] if h0 else None)
    handle.synchronize()
    return H.cpu().numpy()


def expect_xp(N, B):
    """XCDs per batch row the planner takes beyond N = 1792: 4 where B <= 2 and
    N > 2048 or where only a 4-way instance holds the rows (N > 3584), else 2."""
    chunks = -(-N // 256)
    return 4 if (B <= 2 and N > 2048) or chunks > 14 else 2


# (N, B, T): ragged N (parts of unequal length), both split widths, every
# batch size a width allows
SHAPES = [(2600, 3, 5), (3072, 4, 6), (3072, 1, 4), (3500, 2, 4), (3584, 4, 3),
          (3600, 2, 3), (4096, 2, 4), (4000, 1, 5), (5120, 2, 3)]


@pytest.mark.parametrize("N,B,T", SHAPES)
def test_split_parity(handle, N, B, T):
    w = Workload(f"dense_{N}", "dense", N, B, T, "f16", seed=N + 11, h0="randn")
    d = generate(w)
    H = run(handle, d)
    p = handle.last_plan()
    assert p["layout"] == binding.LAYOUT_TEAM and p["xcds_per_row"] == expect_xp(N, B), p
    r = oracle.tolerance_ratio(H, oracle.forward_dense(d["W"], d["X"], d["h0"]), oracle.TOL_F16)
    assert r <= 1.0, f"N={N} B={B}: error ratio {r:.3g} plan={p}"


@pytest.mark.parametrize("N,B", [(2600, 4), (3072, 4), (4096, 2), (5120, 1)])
def test_split_small_integer_weights_bitwise(handle, N, B):
    """Three +-1 weights per row in random columns and small integer inputs:
    every partial sum is an exact fp32 integer, so every row, widened or
    packed, in every part, must equal the fp64 oracle bit for bit."""
    rng = np.random.default_rng(N + 5)
    T = 6
    W = np.zeros((N, N), np.float16)
    for _ in range(3):
        W[np.arange(N), rng.integers(0, N, N)] += rng.choice([-1, 1], N).astype(np.float16)
    X = rng.integers(-5, 6, size=(T, B, N)).astype(np.float32)
    h0 = rng.integers(-5, 6, size=(B, N)).astype(np.float32)
    ref = oracle.forward_dense(W, X, h0)
    assert np.abs(ref).max() < 2 ** 13
    H = run(handle, {"W": W, "X": X, "h0": h0})
    assert handle.last_plan()["xcds_per_row"] > 1
    np.testing.assert_array_equal(H, ref)


@pytest.mark.parametrize("N,B,shift", [(3072, 4, 1), (3072, 2, 1536), (4096, 2, 1), (4096, 1, 3000)])
def test_split_cyclic_shift_bitwise(handle, N, B, shift):
    """W[i, (i + shift) % N] = 1: each row takes a value produced by another
    row, across a part boundary for the rows near it (shift 1) or for most
    rows (a shift of half the layer and more)."""
    rng = np.random.default_rng(N + shift)
    T = 10
    X = rng.integers(0, 9, size=(T, B, N)).astype(np.float32)
    h0 = rng.integers(0, 9, size=(B, N)).astype(np.float32)
    W = np.zeros((N, N), np.float16)
    W[np.arange(N), (np.arange(N) + shift) % N] = 1
    np.testing.assert_array_equal(run(handle, {"W": W, "X": X, "h0": h0}), oracle.forward_dense(W, X, h0))


@pytest.mark.parametrize("N,B,Bs", [(3072, 4, 3), (4096, 2, 1)])
def test_split_chunked_calls_and_batch_changes(handle, N, B, Bs):
    """Calls that continue the ring's step counter: a sequence cut in three
    (h0 = the last output) equals one call bitwise, and calls with fewer batch
    rows in between (the same split width; teams without a batch row stamp
    their rows) leave the next full call correct."""
    T = 9
    w = Workload(f"dense_{N}", "dense", N, B, T, "f16", seed=77, h0="randn")
    d = generate(w)
    g = to_dev(d)
    whole = handle.forward_dense(g["W"], g["X"], g["h0"])
    xp = handle.last_plan()["xcds_per_row"]
    h, parts = g["h0"], []
    for t0, t1 in ((0, 2), (2, 7), (7, 9)):
        Hp = handle.forward_dense(g["W"], g["X"][t0:t1].contiguous(), h)
        h = Hp[-1].contiguous()
        parts.append(Hp)
        small = handle.forward_dense(g["W"], g["X"][t0:t1, :Bs].contiguous(), g["h0"][:Bs].contiguous())
        assert handle.last_plan()["xcds_per_row"] == xp
    handle.synchronize()
    assert torch.equal(torch.cat(parts), whole)
    ref1 = oracle.forward_dense(d["W"], d["X"][7:9, :Bs], d["h0"][:Bs])
    assert oracle.tolerance_ratio(small.cpu().numpy(), ref1, oracle.TOL_F16) <= 1.0
    assert oracle.tolerance_ratio(whole.cpu().numpy(), oracle.forward_dense(d["W"], d["X"], d["h0"]),
                                  oracle.TOL_F16) <= 1.0


def test_split_then_single_xcd_layers_on_one_handle(handle):
    """Switching between a split layer and a single-XCD layer resets the ring
    (its layout changes): both stay correct, in either order."""
    big = generate(Workload("dense_3072", "dense", 3072, 2, 5, "f16", seed=81, h0="randn"))
    small = generate(Workload("dense_1792", "dense", 1792, 2, 5, "f16", seed=82, h0="randn"))
    for d in (big, small, big, small):
        H = run(handle, d)
        assert oracle.tolerance_ratio(H, oracle.forward_dense(d["W"], d["X"], d["h0"]), oracle.TOL_F16) <= 1.0


@pytest.mark.parametrize("N,B", [(3072, 5), (2600, 8), (4096, 3), (5376, 1)])
def test_split_limits(handle, N, B):
    """Beyond the split widths' batch or size limits: NOT_SUPPORTED, nothing run."""
    W = torch.zeros(N, N, dtype=torch.float16, device="cuda")
    X = torch.zeros(2, B, N, device="cuda")
    with pytest.raises(PrnnError) as e:
        handle.forward_dense(W, X)
    assert e.value.status == binding.NOT_SUPPORTED


@pytest.mark.parametrize("math", [binding.MATH_SPLIT, binding.MATH_HALF])
def test_split_layout_exact_math_only(handle, math):
    W = torch.zeros(3072, 3072, dtype=torch.float16, device="cuda")
    X = torch.zeros(2, 2, 3072, device="cuda")
    handle.set_math(math)
    try:
        with pytest.raises(PrnnError) as e:
            handle.forward_dense(W, X)
        assert e.value.status == binding.NOT_SUPPORTED
    finally:
        handle.set_math(binding.MATH_AUTO)


@pytest.mark.parametrize("N,B", [(3072, 4), (4096, 2)])
def test_split_watchdog_reports_and_recovers(gpu, N, B):
    """A workgroup that skips one publish makes the other parts' bounded waits
    expire: the next call reports EXECUTION_FAILED and a clean run works."""
    d = generate(Workload(f"dense_{N}", "dense", N, B, 10, "f16", seed=91, h0="randn"))
    g = to_dev(d)
    with Handle() as h:
        h.set_watchdog_us(2000)
        h.debug_skip_publish(5, 4)
        h.forward_dense(g["W"], g["X"], g["h0"])
        with pytest.raises(PrnnError) as e:
            h.synchronize()
        assert e.value.status == binding.EXECUTION_FAILED
        H = h.forward_dense(g["W"], g["X"], g["h0"])
        h.synchronize()
        assert oracle.tolerance_ratio(H.cpu().numpy(), oracle.forward_dense(d["W"], d["X"], d["h0"]),
                                      oracle.TOL_F16) <= 1.0


@pytest.mark.parametrize("N,B", [(3072, 4), (4096, 2)])
def test_split_repeats_and_jitter_bitwise(gpu, N, B):
    """Outputs filled with NaN before each run; 8 repeats and three seeds of
    publish jitter (span 48) all give bitwise the first result."""
    d = generate(Workload(f"dense_{N}", "dense", N, B, 16, "f16", seed=93, h0="randn"))
    g = to_dev(d)
    out = torch.empty_like(g["X"])
    with Handle() as h:
        out.fill_(float("nan"))
        first = h.forward_dense(g["W"], g["X"], g["h0"], out=out).clone()
        h.synchronize()
        assert not torch.isnan(first).any()
        for _ in range(8):
            out.fill_(float("nan"))
            h.forward_dense(g["W"], g["X"], g["h0"], out=out)
            h.synchronize()
            assert torch.equal(out, first)
        for seed in (1, 2, 3):
            h.debug_jitter(seed, 48)
            out.fill_(float("nan"))
            h.forward_dense(g["W"], g["X"], g["h0"], out=out)
            h.synchronize()
            assert torch.equal(out, first)
        h.debug_jitter(0, 0)
    assert oracle.tolerance_ratio(first.cpu().numpy(), oracle.forward_dense(d["W"], d["X"], d["h0"]),
                                  oracle.TOL_F16) <= 1.0


def test_split_layer(handle):
    """A whole layer at N = I = 3072 (projection, then the split recurrence)."""
    w = Workload("layer_3072", "dense", 3072, 4, 8, "f16", seed=95, h0="randn")
    d = generate_layer(w, 3072)
    g = to_dev(d)
    H = handle.forward_layer_dense(g["U"], g["bias"], g["W"], g["x"], g["h0"])
    handle.synchronize()
    assert handle.last_plan()["xcds_per_row"] == 2
    ref = oracle.forward_layer_dense(d["U"], d["bias"], d["W"], d["x"], d["h0"])
    assert oracle.tolerance_ratio(H.cpu().numpy(), ref, oracle.TOL_F16) <= 1.0


@pytest.mark.parametrize("N,B,xcds", [(1152, 4, 2), (1000, 3, 2), (1100, 2, 4), (1792, 2, 4), (300, 1, 4),
                                      (2048, 4, 2), (2304, 2, 2), (2560, 1, 4)])
def test_split_forced_at_any_size(handle, N, B, xcds):
    """prnn_set_xcds_per_row forces a split width on layers that fit one XCD:
    ragged N, a last part shorter than the others or empty (N = 1100 and 300
    on 4 XCDs), against the oracle."""
    w = Workload(f"dense_{N}", "dense", N, B, 5, "f16", seed=N + xcds, h0="randn")
    d = generate(w)
    handle.set_xcds_per_row(xcds)
    try:
        H = run(handle, d)
        p = handle.last_plan()
    finally:
        handle.set_xcds_per_row(0)
    assert p["layout"] == binding.LAYOUT_TEAM and p["xcds_per_row"] == xcds, p
    r = oracle.tolerance_ratio(H, oracle.forward_dense(d["W"], d["X"], d["h0"]), oracle.TOL_F16)
    assert r <= 1.0, f"N={N} B={B} xcds={xcds}: error ratio {r:.3g} plan={p}"


def test_split_width_setting(handle):
    """0, 1, 2 and 4 are accepted, anything else is BAD_PARAM; a width the
    call cannot use (one XCD beyond N = 2560, four with B = 3) is
    NOT_SUPPORTED in the team layout; fp32 W ignores the setting."""
    for bad in (-1, 3, 8):
        with pytest.raises(PrnnError) as e:
            handle.set_xcds_per_row(bad)
        assert e.value.status == binding.BAD_PARAM
    handle.set_layout(binding.LAYOUT_TEAM)
    try:
        for N, B, xcds in ((3072, 2, 1), (2048, 3, 4)):
            handle.set_xcds_per_row(xcds)
            with pytest.raises(PrnnError) as e:
                handle.forward_dense(torch.zeros(N, N, dtype=torch.float16, device="cuda"),
                                     torch.zeros(2, B, N, device="cuda"))
            assert e.value.status == binding.NOT_SUPPORTED
        handle.set_xcds_per_row(2)
        d = generate(Workload("dense_f32", "dense", 1000, 2, 4, "f32", seed=3, h0="randn"))
        H = run(handle, d)
        assert handle.last_plan()["xcds_per_row"] == 1
        assert oracle.tolerance_ratio(H, oracle.forward_dense(d["W"], d["X"], d["h0"]), oracle.TOL_F32) <= 1.0
    finally:
        handle.set_xcds_per_row(0)
        handle.set_layout(binding.LAYOUT_AUTO)


@pytest.mark.parametrize("N,B", [(3072, 4), (4096, 2), (2304, 4)])
def test_split_floor_follows_the_layer(handle, N, B):
    """prnn_sync_floor runs the split protocol where the dense fp16 layer of
    the same N and B is split: every row of every step holds t + 1."""
    T = 7
    out = torch.full((T, B, N), float("nan"), device="cuda")
    handle.sync_floor(N, B, T, out=out)
    handle.synchronize()
    assert handle.last_plan()["xcds_per_row"] == expect_xp(N, B)
    expect = torch.arange(1, T + 1, dtype=torch.float32, device="cuda").view(T, 1, 1).expand(T, B, N)
    assert torch.equal(out, expect)


# ---------------------------------------------------------------------------
# row-balanced sparse fp16 layers on two XCDs per batch row: automatic for
# blocks of more than 60 slots per wave (5 % at N = 5760), forced at any size
# ---------------------------------------------------------------------------
def run_sparse(handle, d):
    g = to_dev(d)
    H = handle.forward_sparse(g["col"], g["val"], g["X"], g["h0"])
    handle.synchronize()
    return H.cpu().numpy()


def sparse_ref(d):
    return oracle.forward_sparse(d["col"], d["val"], d["X"], d["h0"])


def test_sparse_split_automatic_for_the_5_percent_layer(handle):
    from persistent_rnn_fwd_amd.inputs import WORKLOADS
    w = WORKLOADS["sparse5_f16_n5760"].with_(T=40, h0="randn")
    d = generate(w, seed=71)
    H = run_sparse(handle, d)
    p = handle.last_plan()
    assert p["xcds_per_row"] == 2 and p["waves_per_wg"] == 12, p
    assert oracle.tolerance_ratio(H, sparse_ref(d), oracle.TOL_F16) <= 1.0
    for name in ("sparse1_f16_n5760", "sparse10_f16_n1792", "sparse25_f16_n2304"):   # lighter blocks stay on one XCD
        run_sparse(handle, generate(WORKLOADS[name].with_(T=2)))
        assert handle.last_plan()["xcds_per_row"] == 1, name


@pytest.mark.parametrize("N,B,T,K", [(1000, 3, 6, 100), (2304, 4, 5, 576), (777, 4, 5, 50), (5760, 2, 4, 288),
                                     (300, 1, 5, 17), (2304, 4, 4, 230)])
def test_sparse_split_forced_parity(handle, N, B, T, K):
    w = Workload(f"sparse_{N}", "sparse", N, B, T, "f16", K=K, seed=N + K, h0="randn")
    d = generate(w)
    handle.set_xcds_per_row(2)
    try:
        H = run_sparse(handle, d)
        p = handle.last_plan()
    finally:
        handle.set_xcds_per_row(0)
    assert p["layout"] == binding.LAYOUT_TEAM and p["xcds_per_row"] == 2, p
    r = oracle.tolerance_ratio(H, sparse_ref(d), oracle.TOL_F16)
    assert r <= 1.0, f"N={N} B={B} K={K}: error ratio {r:.3g} plan={p}"


@pytest.mark.parametrize("N,K", [(1792, 179), (5760, 288)])
def test_sparse_split_small_integers_bitwise(handle, N, K):
    rng = np.random.default_rng(N + K)
    T, B = 5, 4
    col = np.stack([np.sort(rng.choice(N, K, replace=False)) for _ in range(N)]).astype(np.int16)
    val = (rng.choice([-1.0, 1.0], (N, K)) * (rng.random((N, K)) < 0.03)).astype(np.float16)
    X = rng.integers(-5, 6, size=(T, B, N)).astype(np.float32)
    h0 = rng.integers(-5, 6, size=(B, N)).astype(np.float32)
    d = {"col": col, "val": val, "X": X, "h0": h0}
    ref = sparse_ref(d)
    assert np.abs(ref).max() < 2 ** 20
    handle.set_xcds_per_row(2)
    try:
        H = run_sparse(handle, d)
        assert handle.last_plan()["xcds_per_row"] == 2
    finally:
        handle.set_xcds_per_row(0)
    np.testing.assert_array_equal(H, ref)


def test_sparse_split_limits(handle):
    """Two XCDs need B <= 4; four are not offered to sparse layers; fp32
    values keep one XCD per batch row."""
    col = torch.zeros(1000, 10, dtype=torch.int16, device="cuda")
    val = torch.zeros(1000, 10, dtype=torch.float16, device="cuda")
    handle.set_layout(binding.LAYOUT_TEAM)
    try:
        for xcds, B in ((2, 5), (4, 2)):
            handle.set_xcds_per_row(xcds)
            with pytest.raises(PrnnError) as e:
                handle.forward_sparse(col, val, torch.zeros(2, B, 1000, device="cuda"))
            assert e.value.status == binding.NOT_SUPPORTED
        handle.set_xcds_per_row(2)
        handle.forward_sparse(col, val.float(), torch.zeros(2, 2, 1000, device="cuda"))
        handle.synchronize()
        assert handle.last_plan()["xcds_per_row"] == 1
    finally:
        handle.set_xcds_per_row(0)
        handle.set_layout(binding.LAYOUT_AUTO)


@pytest.mark.parametrize("waves", [8, 12])
def test_sparse_split_floor_in_the_layer_plan(handle, waves):
    """The floor with a forced width and wave count runs the split protocol in
    that shape (the bench measures each layer's floor in its own plan)."""
    N, B, T = 5760, 4, 6
    out = torch.full((T, B, N), float("nan"), device="cuda")
    handle.set_xcds_per_row(2)
    handle.set_team_waves(waves)
    try:
        handle.sync_floor(N, B, T, out=out)
        handle.synchronize()
        p = handle.last_plan()
    finally:
        handle.set_xcds_per_row(0)
        handle.set_team_waves(0)
    assert p["xcds_per_row"] == 2 and p["waves_per_wg"] == waves, p
    expect = torch.arange(1, T + 1, dtype=torch.float32, device="cuda").view(T, 1, 1).expand(T, B, N)
    assert torch.equal(out, expect)


def test_sparse_split_repeats_jitter_and_chunks_bitwise(gpu):
    from persistent_rnn_fwd_amd.inputs import WORKLOADS
    w = WORKLOADS["sparse5_f16_n5760"].with_(T=18, h0="randn")
    d = generate(w, seed=73)
    g = to_dev(d)
    out = torch.empty_like(g["X"])
    with Handle() as h:
        out.fill_(float("nan"))
        first = h.forward_sparse(g["col"], g["val"], g["X"], g["h0"], out=out).clone()
        h.synchronize()
        assert h.last_plan()["xcds_per_row"] == 2 and not torch.isnan(first).any()
        for seed in (0, 1, 2):
            h.debug_jitter(seed, 48 if seed else 0)
            out.fill_(float("nan"))
            h.forward_sparse(g["col"], g["val"], g["X"], g["h0"], out=out)
            h.synchronize()
            assert torch.equal(out, first)
        h.debug_jitter(0, 0)
        # the sequence in two calls, with a call of 3 batch rows between them
        a = h.forward_sparse(g["col"], g["val"], g["X"][:7].contiguous(), g["h0"])
        h.forward_sparse(g["col"], g["val"], g["X"][:4, :3].contiguous(), g["h0"][:3].contiguous())
        b = h.forward_sparse(g["col"], g["val"], g["X"][7:].contiguous(), a[-1].contiguous())
        h.synchronize()
        assert torch.equal(torch.cat([a, b]), first)
    assert oracle.tolerance_ratio(first.cpu().numpy(), sparse_ref(d), oracle.TOL_F16) <= 1.0


def test_sparse_split_watchdog(gpu):
    from persistent_rnn_fwd_amd.inputs import WORKLOADS
    w = WORKLOADS["sparse5_f16_n5760"].with_(T=10, h0="randn")
    d = generate(w, seed=75)
    g = to_dev(d)
    with Handle() as h:
        h.set_watchdog_us(2000)
        h.debug_skip_publish(3, 4)
        h.forward_sparse(g["col"], g["val"], g["X"], g["h0"])
        with pytest.raises(PrnnError) as e:
            h.synchronize()
        assert e.value.status == binding.EXECUTION_FAILED
        H = h.forward_sparse(g["col"], g["val"], g["X"], g["h0"])
        h.synchronize()
        assert oracle.tolerance_ratio(H.cpu().numpy(), sparse_ref(d), oracle.TOL_F16) <= 1.0
