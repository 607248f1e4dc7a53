"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: a hand-worked
example, brute force in exact rational arithmetic, closed forms (W = 0,
W = I, cyclic shifts, the linear regime as one block-triangular linear solve,
diagonal W) and invariants (batch independence, chunking in time, positive
homogeneity, sparse == its dense copy).  Together they fail on a dropped term,
a wrong sign, a transposed W, an off-by-one in time, an ignored h0, a wrong
activation and a swapped sparse index.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from persistent_rnn_fwd_amd.inputs import WORKLOADS, generate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# hand-worked example
# ---------------------------------------------------------------------------
def _golden():
    with open(os.path.join(GOLDEN, "hand_worked_n2_b2_t3.json")) as f:
        return json.load(f)


def test_golden_dense():
    g = _golden()
    H = oracle.forward_dense(np.array(g["W"]), np.array(g["X"]), np.array(g["h0"]))
    np.testing.assert_array_equal(H, np.array(g["H"]))


def test_golden_sparse():
    g = _golden()
    H = oracle.forward_sparse(np.array(g["col"]), np.array(g["val"]), np.array(g["X"]), np.array(g["h0"]))
    np.testing.assert_array_equal(H, np.array(g["H"]))


def test_golden_catches_transpose():
    g = _golden()
    H = oracle.forward_dense(np.array(g["W"]).T, np.array(g["X"]), np.array(g["h0"]))
    assert not np.array_equal(H, np.array(g["H"]))


# ---------------------------------------------------------------------------
# brute force in exact rationals
# ---------------------------------------------------------------------------
def _brute_dense(W, X, h0):
    """Element-by-element loops over Fractions: exact, no floating point."""
    T, B, N = len(X), len(X[0]), len(W)
    h = [[Fraction(v) for v in row] for row in h0]
    out = []
    for t in range(T):
        new = []
        for b in range(B):
            row = []
            for i in range(N):
                s = Fraction(X[t][b][i])
                for j in range(N):
                    s += Fraction(W[i][j]) * h[b][j]
                row.append(s if s > 0 else Fraction(0))
            new.append(row)
        out.append(new)
        h = new
    return out


def _brute_sparse(col, val, X, h0):
    T, B, N, K = len(X), len(X[0]), len(col), len(col[0])
    h = [[Fraction(v) for v in row] for row in h0]
    out = []
    for t in range(T):
        new = []
        for b in range(B):
            row = []
            for i in range(N):
                s = Fraction(X[t][b][i])
                for k in range(K):
                    s += Fraction(val[i][k]) * h[b][col[i][k]]
                row.append(s if s > 0 else Fraction(0))
            new.append(row)
        out.append(new)
        h = new
    return out


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_dense_exact(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 5))
    B = int(rng.integers(1, 3))
    T = int(rng.integers(1, 4))
    # dyadic values: every partial sum is exact in fp64
    W = rng.integers(-3, 4, size=(N, N)) / 2.0
    X = rng.integers(-3, 4, size=(T, B, N)) / 4.0
    h0 = rng.integers(0, 4, size=(B, N)) / 2.0
    ref = _brute_dense(W.tolist(), X.tolist(), h0.tolist())
    H = oracle.forward_dense(W, X, h0)
    np.testing.assert_array_equal(H, np.array(ref, dtype=np.float64))


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_sparse_exact(seed):
    rng = np.random.default_rng(100 + seed)
    N = int(rng.integers(1, 5))
    K = int(rng.integers(1, N + 1))
    B = int(rng.integers(1, 3))
    T = int(rng.integers(1, 4))
    col = np.stack([np.sort(rng.choice(N, K, replace=False)) for _ in range(N)])
    val = rng.integers(-3, 4, size=(N, K)) / 2.0
    X = rng.integers(-3, 4, size=(T, B, N)) / 4.0
    h0 = rng.integers(0, 4, size=(B, N)) / 2.0
    ref = _brute_sparse(col.tolist(), val.tolist(), X.tolist(), h0.tolist())
    H = oracle.forward_sparse(col, val, X, h0)
    np.testing.assert_array_equal(H, np.array(ref, dtype=np.float64))


def _brute_sparse_rows(col, val, row_len, X, h0):
    """Rows of unequal length in exact rationals: row i sums its first
    row_len[i] pairs and nothing else."""
    T, B, N = len(X), len(X[0]), len(col)
    h = [[Fraction(v) for v in row] for row in h0]
    out = []
    for t in range(T):
        new = []
        for b in range(B):
            row = []
            for i in range(N):
                s = Fraction(X[t][b][i])
                for k in range(row_len[i]):
                    s += Fraction(val[i][k]) * h[b][col[i][k]]
                row.append(s if s > 0 else Fraction(0))
            new.append(row)
        out.append(new)
        h = new
    return out


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_sparse_rows_exact(seed):
    """Lengths 0..K per row, and pairs past each row's length holding values
    and columns (some out of range) that must not count."""
    rng = np.random.default_rng(300 + seed)
    N = int(rng.integers(1, 6))
    K = int(rng.integers(1, N + 1))
    B = int(rng.integers(1, 3))
    T = int(rng.integers(1, 4))
    col = np.stack([rng.choice(N, K, replace=False) for _ in range(N)])
    val = rng.integers(-3, 4, size=(N, K)) / 2.0
    row_len = rng.integers(0, K + 1, size=N)
    for i in range(N):                                       # garbage past the row
        col[i, row_len[i]:] = rng.integers(-3, N + 4, size=K - row_len[i])
        val[i, row_len[i]:] = rng.integers(5, 9, size=K - row_len[i])
    X = rng.integers(-3, 4, size=(T, B, N)) / 4.0
    h0 = rng.integers(-2, 4, size=(B, N)) / 2.0
    ref = _brute_sparse_rows(col.tolist(), val.tolist(), row_len.tolist(), X.tolist(), h0.tolist())
    H = oracle.forward_sparse_rows(col, val, row_len, X, h0)
    np.testing.assert_array_equal(H, np.array(ref, dtype=np.float64))


def test_sparse_rows_full_length_is_row_balanced():
    rng = np.random.default_rng(5)
    N, K, T, B = 40, 7, 6, 3
    col = np.stack([rng.choice(N, K, replace=False) for _ in range(N)])
    val = rng.standard_normal((N, K))
    X = rng.standard_normal((T, B, N))
    h0 = rng.standard_normal((B, N))
    np.testing.assert_array_equal(oracle.forward_sparse_rows(col, val, np.full(N, K), X, h0),
                                  oracle.forward_sparse(col, val, X, h0))


def test_sparse_rows_empty_rows_and_the_dense_copy():
    """Empty rows give relu(x) whatever h is; the rest equals the dense matrix
    of the pairs inside each row; NaN and infinities past a row's length never
    reach H."""
    rng = np.random.default_rng(6)
    N, K, T, B = 30, 9, 5, 2
    col = np.stack([rng.choice(N, K, replace=False) for _ in range(N)])
    val = rng.standard_normal((N, K)) * 0.3
    row_len = rng.integers(0, K + 1, size=N)
    row_len[:4] = 0
    X = rng.standard_normal((T, B, N))
    h0 = rng.standard_normal((B, N))
    Wd = np.zeros((N, N))
    for i in range(N):
        for k in range(row_len[i]):
            Wd[i, col[i, k]] += val[i, k]
        val[i, row_len[i]:] = np.nan if i % 2 else np.inf
    H = oracle.forward_sparse_rows(col, val, row_len, X, h0)
    assert np.isfinite(H).all()
    np.testing.assert_array_equal(H[:, :, :4], np.maximum(X[:, :, :4], 0.0))
    np.testing.assert_allclose(H, oracle.forward_dense(Wd, X, h0), rtol=1e-12, atol=1e-12)


def test_sparse_rows_rejects_bad_lengths():
    col = np.zeros((3, 2), np.int64)
    val = np.zeros((3, 2))
    X = np.zeros((1, 1, 3))
    for bad in ([0, 3, 1], [-1, 0, 0], [0, 0]):
        with pytest.raises(ValueError):
            oracle.forward_sparse_rows(col, val, np.array(bad), X)


def test_generator_unbalanced_rows_in_both_forms():
    """The unbalanced workload read as rows of unequal length (row_len) and as
    the padded row-balanced matrix is the same W."""
    w = WORKLOADS["sparse10u_f16_n2304"].with_(T=3)
    d = generate(w)
    np.testing.assert_allclose(oracle.forward_sparse_rows(d["col"], d["val"], d["row_len"], d["X"], d["h0"]),
                               oracle.forward_sparse(d["col"], d["val"], d["X"], d["h0"]), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
def test_zero_weights_give_relu_of_x():
    rng = np.random.default_rng(1)
    T, B, N = 5, 3, 17
    X = rng.standard_normal((T, B, N))
    h0 = np.abs(rng.standard_normal((B, N)))
    H = oracle.forward_dense(np.zeros((N, N)), X, h0)
    np.testing.assert_array_equal(H, np.where(X > 0, X, 0.0))
    col = np.arange(N).reshape(N, 1)
    Hs = oracle.forward_sparse(col, np.zeros((N, 1)), X, h0)
    np.testing.assert_array_equal(Hs, np.where(X > 0, X, 0.0))


def test_identity_weights_give_prefix_sums():
    rng = np.random.default_rng(2)
    T, B, N = 9, 2, 13
    X = rng.integers(0, 50, size=(T, B, N)).astype(np.float64)
    h0 = rng.integers(0, 50, size=(B, N)).astype(np.float64)
    expect = h0[None] + np.cumsum(X, axis=0)
    np.testing.assert_array_equal(oracle.forward_dense(np.eye(N), X, h0), expect)
    col = np.arange(N).reshape(N, 1)
    np.testing.assert_array_equal(oracle.forward_sparse(col, np.ones((N, 1)), X, h0), expect)


def test_cyclic_shift_closed_form():
    """W[i, (i+1) % N] = 1 shifts the state by one place per step.

    With X >= 0 nothing is clipped, so H[t] = sum_{s<=t} roll(X[s], -(t-s))
    + roll(h0, -(t+1)); using W^T instead would roll the other way."""
    rng = np.random.default_rng(3)
    T, B, N = 7, 2, 11
    X = rng.integers(0, 9, size=(T, B, N)).astype(np.float64)
    h0 = rng.integers(0, 9, size=(B, N)).astype(np.float64)
    W = np.zeros((N, N))
    W[np.arange(N), (np.arange(N) + 1) % N] = 1.0
    expect = np.empty((T, B, N))
    for t in range(T):
        acc = np.roll(h0, -(t + 1), axis=1)
        for s in range(t + 1):
            acc = acc + np.roll(X[s], -(t - s), axis=1)
        expect[t] = acc
    np.testing.assert_array_equal(oracle.forward_dense(W, X, h0), expect)
    col = ((np.arange(N) + 1) % N).reshape(N, 1)
    np.testing.assert_array_equal(oracle.forward_sparse(col, np.ones((N, 1)), X, h0), expect)


def test_linear_regime_block_triangular_solve():
    """With W >= 0, X > 0, h0 >= 0 no ReLU clips, so the T steps are one linear
    system: h_0 - 0 = x_0 + W h0, h_t - W h_{t-1} = x_t, solved by LU."""
    rng = np.random.default_rng(4)
    T, B, N = 6, 3, 8
    W = rng.uniform(0, 0.2, size=(N, N))
    X = rng.uniform(0.1, 1.0, size=(T, B, N))
    h0 = rng.uniform(0, 1.0, size=(B, N))
    M = np.eye(T * N)
    for t in range(1, T):
        M[t * N:(t + 1) * N, (t - 1) * N:t * N] = -W
    expect = np.empty((T, B, N))
    for b in range(B):
        rhs = X[:, b, :].copy()
        rhs[0] += W @ h0[b]
        expect[:, b, :] = np.linalg.solve(M, rhs.reshape(-1)).reshape(T, N)
    H = oracle.forward_dense(W, X, h0)
    np.testing.assert_allclose(H, expect, rtol=1e-12, atol=1e-12)
    # the same system through the sparse route (K = N, every column listed)
    col = np.tile(np.arange(N), (N, 1))
    np.testing.assert_allclose(oracle.forward_sparse(col, W, X, h0), expect, rtol=1e-12, atol=1e-12)


def test_diagonal_weights_scalar_recurrences():
    rng = np.random.default_rng(5)
    T, B, N = 10, 2, 6
    a = rng.uniform(-1.5, 1.5, size=N)
    X = rng.standard_normal((T, B, N))
    h0 = np.abs(rng.standard_normal((B, N)))
    H = oracle.forward_dense(np.diag(a), X, h0)
    for b in range(B):
        for i in range(N):
            h = h0[b, i]
            for t in range(T):
                h = max(a[i] * h + X[t, b, i], 0.0)
                assert H[t, b, i] == pytest.approx(h, rel=1e-14, abs=1e-14)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def _small_problem(seed, T=12, B=4, N=24):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, N)) * 0.8 / np.sqrt(N)
    X = rng.standard_normal((T, B, N))
    h0 = np.abs(rng.standard_normal((B, N)))
    return W, X, h0


def test_batch_rows_are_independent():
    W, X, h0 = _small_problem(6)
    H = oracle.forward_dense(W, X, h0)
    for b in range(X.shape[1]):
        Hb = oracle.forward_dense(W, X[:, b:b + 1], h0[b:b + 1])
        np.testing.assert_allclose(H[:, b:b + 1], Hb, rtol=1e-13, atol=1e-13)
    # identical batch rows give identical outputs
    X2 = np.repeat(X[:, :1], 3, axis=1)
    H2 = oracle.forward_dense(W, X2, np.repeat(h0[:1], 3, axis=0))
    assert np.array_equal(H2[:, 0], H2[:, 1]) and np.array_equal(H2[:, 0], H2[:, 2])


def test_chunking_in_time_is_exact():
    W, X, h0 = _small_problem(7)
    H = oracle.forward_dense(W, X, h0)
    for T1 in (1, 5, 11):
        Ha = oracle.forward_dense(W, X[:T1], h0)
        Hb = oracle.forward_dense(W, X[T1:], Ha[-1])
        np.testing.assert_array_equal(np.concatenate([Ha, Hb]), H)


def test_positive_homogeneity_is_exact():
    W, X, h0 = _small_problem(8)
    H = oracle.forward_dense(W, X, h0)
    for k in (-3, 1, 7):
        np.testing.assert_array_equal(oracle.forward_dense(W, X * 2.0 ** k, h0 * 2.0 ** k), H * 2.0 ** k)


def test_sparse_equals_dense_copy():
    rng = np.random.default_rng(9)
    T, B, N, K = 10, 4, 40, 7
    col = np.stack([np.sort(rng.choice(N, K, replace=False)) for _ in range(N)])
    val = rng.standard_normal((N, K)) * 0.8 / np.sqrt(K)
    X = rng.standard_normal((T, B, N))
    h0 = np.abs(rng.standard_normal((B, N)))
    Wd = oracle.sparse_to_dense(col, val, N)
    # the dense copy has exactly the listed entries
    assert np.count_nonzero(Wd) == np.count_nonzero(val)
    for i in range(N):
        for k in range(K):
            assert Wd[i, col[i, k]] == val[i, k]
    np.testing.assert_allclose(oracle.forward_sparse(col, val, X, h0),
                               oracle.forward_dense(Wd, X, h0), rtol=1e-13, atol=1e-13)
    # the order of the (col, val) pairs inside a row does not matter
    perm = np.stack([rng.permutation(K) for _ in range(N)])
    col_p = np.take_along_axis(col, perm, axis=1)
    val_p = np.take_along_axis(val, perm, axis=1)
    np.testing.assert_allclose(oracle.forward_sparse(col_p, val_p, X, h0),
                               oracle.forward_sparse(col, val, X, h0), rtol=1e-13, atol=1e-13)


def test_nan_propagates_and_empty_sequence():
    W, X, h0 = _small_problem(10, T=4, B=2, N=5)
    X = X.copy()
    X[1, 0, 2] = np.nan
    H = oracle.forward_dense(W, X, h0)
    assert np.isnan(H[1, 0, 2]) and np.isnan(H[2, 0]).all()   # spreads through W
    assert not np.isnan(H[:, 1]).any()                          # not across batch rows
    assert oracle.forward_dense(W, X[:0], h0).shape == (0, 2, 5)


def test_tolerance_ratio():
    ref = np.array([0.0, 1.0, 10.0])
    assert oracle.tolerance_ratio(ref, ref, 1e-4) == 0.0
    assert oracle.tolerance_ratio(ref + np.array([1e-4, 0, 0]), ref, 1e-4) == pytest.approx(1.0)
    assert oracle.tolerance_ratio(ref + np.array([0, 0, 11e-4]), ref, 1e-4) == pytest.approx(1.0)
    assert oracle.tolerance_ratio(np.array([np.nan, 1, 10]), ref, 1e-4) == float("inf")
    both = np.array([np.nan, 1.0])
    assert oracle.tolerance_ratio(both, both, 1e-4) == 0.0


# ---------------------------------------------------------------------------
# generators and tolerance sanity
# ---------------------------------------------------------------------------
def test_generator_sparse_pattern_and_values():
    w = WORKLOADS["sparse10_f16_n1152"]
    d = generate(w)
    col, val = d["col"], d["val"]
    assert col.dtype == np.int16 and col.shape == (1152, 115)
    assert val.dtype == np.float16 and val.shape == (1152, 115)
    assert (np.diff(col.astype(np.int64), axis=1) > 0).all()      # sorted, distinct
    assert col.min() >= 0 and col.max() < 1152
    std = float(np.std(val.astype(np.float64)))
    assert abs(std - 0.8 / np.sqrt(115)) < 0.02 * 0.8 / np.sqrt(115) * 5
    assert d["X"].dtype == np.float32 and d["X"].shape == (256, 4, 1152)
    assert not d["h0"].any()
    # deterministic per seed, different across seeds
    d2 = generate(w)
    assert np.array_equal(d2["col"], col) and np.array_equal(d2["X"], d["X"])
    d3 = generate(w, seed=w.seed + 1000)
    assert not np.array_equal(d3["col"], col)


def test_generator_magnitude_pruned_rows():
    """Unbalanced rows: K kept entries per row on average, stored at the longest
    row's width, kept entries first (sorted by column) then zero-valued padding
    on distinct unused columns; row_len counts the kept entries; kept values
    have row norm 0.8."""
    w = WORKLOADS["sparse10u_f16_n2304"]
    d = generate(w)
    col, val, row_len = d["col"].astype(np.int64), d["val"].astype(np.float64), d["row_len"]
    N = w.N
    assert col.shape == val.shape and col.shape[0] == N and col.shape[1] > w.K
    assert row_len.dtype == np.int32 and row_len.shape == (N,) and row_len.max() == col.shape[1]
    assert col.min() >= 0 and col.max() < N
    for i in range(0, N, 97):
        L = row_len[i]
        assert len(set(col[i].tolist())) == col.shape[1]                 # distinct
        assert (np.diff(col[i, :L]) > 0).all() and (np.diff(col[i, L:]) > 0).all()
        assert not val[i, L:].any()
    kept = (val != 0).sum(axis=1)
    assert (kept <= row_len).all() and (row_len - kept).max() <= 2     # fp16 zeros of tiny values aside
    assert abs(kept.mean() - w.K) < 0.01 * w.K          # fp16 zeros of tiny values aside
    assert kept.max() == col.shape[1] or kept.max() >= 0.98 * col.shape[1]
    assert kept.max() > 1.3 * w.K                        # rows really are unbalanced
    norms = np.sqrt((val * val).sum(axis=1))
    assert np.allclose(norms, 0.8, rtol=2e-3)
    # the padded form is the same matrix as the unpadded one: sparse == dense copy
    X = generate(w.with_(T=3))["X"]
    Wd = oracle.sparse_to_dense(d["col"], d["val"], N)
    np.testing.assert_allclose(oracle.forward_sparse(d["col"], d["val"], X, None),
                               oracle.forward_dense(Wd, X, None), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("name", ["dense_f32_n256", "sparse10_f16_n1152"])
def test_generator_spectral_radius_near_0p8(name):
    w = WORKLOADS[name]
    d = generate(w)
    if w.kind == "dense":
        Wd = d["W"].astype(np.float64)
    else:
        Wd = oracle.sparse_to_dense(d["col"], d["val"], w.N)
    rho = np.max(np.abs(np.linalg.eigvals(Wd)))
    assert 0.65 < rho < 0.95


def test_fp32_arithmetic_meets_fp32_bar():
    """An fp32 evaluation of the recurrence passes 1e-4 (1 + |h|) with margin,
    so the bar is reachable by any fp32 summation order."""
    w = WORKLOADS["dense_f32_n256"]
    d = generate(w, seed=w.seed + 1000)
    H = oracle.forward_dense(d["W"], d["X"], d["h0"])
    W32 = d["W"].astype(np.float32)
    h = d["h0"].astype(np.float32)
    H32 = np.empty_like(d["X"])
    for t in range(w.T):
        h = np.maximum(d["X"][t] + h @ W32.T, np.float32(0))
        H32[t] = h
    assert oracle.tolerance_ratio(H32, H, oracle.TOL_F32) < 0.2


# ---------------------------------------------------------------------------
# The half-h model (state rounded to fp16 before the product)
# ---------------------------------------------------------------------------
def test_half_h_model_rounding_by_hand():
    """One neuron, W = [[1]]: H[t] = X[t] + r(H[t-1]).  Each expected value is
    worked by hand from the binary16 grid (spacing 2^-10 on [1, 2)): 3/4 of a
    step rounds up, exactly 1/2 of a step goes to the even neighbour, below 1/2
    rounds down.  Only the product's copy is rounded, so H[0] keeps every bit."""
    u = 2.0 ** -10
    W = np.ones((1, 1))
    cases = [  # (X[0], the value r(X[0]) that H[1] = 0 + r(H[0]) must equal)
        (1 + 0.75 * u, 1 + u),        # rounds up
        (1 + 0.5 * u, 1.0),           # tie: 1.0 has the even last bit
        (1 + 1.5 * u, 1 + 2 * u),     # tie: 1 + 2u has the even last bit
        (1 + 0.25 * u, 1.0),          # rounds down
        (1 + 3 * u, 1 + 3 * u),       # on the grid: unchanged
    ]
    for x0, staged in cases:
        X = np.array([x0, 0.0, 0.5]).reshape(3, 1, 1)
        H = oracle.forward_dense_half_h(W, X)
        assert H[0, 0, 0] == x0
        assert H[1, 0, 0] == staged
        assert H[2, 0, 0] == 0.5 + staged   # staged is on the grid, so r() keeps it
    # h0 is staged like any other state: r(h0) enters step 0
    H = oracle.forward_dense_half_h(W, np.zeros((1, 1, 1)), np.array([[1 + 0.75 * u]]))
    assert H[0, 0, 0] == 1 + u
    # beyond the fp16 range the staged state is infinite
    H = oracle.forward_dense_half_h(W, np.array([70000.0, 0.0]).reshape(2, 1, 1))
    assert H[0, 0, 0] == 70000.0 and np.isinf(H[1, 0, 0])
    # a negative weight with a rounded state: -1 * r(1 + 0.75u) + 3
    H = oracle.forward_dense_half_h(-W, np.array([1 + 0.75 * u, 3.0]).reshape(2, 1, 1))
    assert H[1, 0, 0] == 3.0 - (1 + u)


def test_half_h_model_equals_definition_on_fp16_grid():
    """When every state is an fp16 value (integers below 2048) the rounding is
    the identity, so the model equals the plain definition exactly."""
    rng = np.random.default_rng(7)
    N, B, T = 9, 3, 12
    W = rng.choice([-1.0, 0.0, 0.0, 0.0, 0.0, 1.0], size=(N, N))
    X = rng.integers(-3, 4, size=(T, B, N)).astype(np.float64)
    h0 = rng.integers(0, 3, size=(B, N)).astype(np.float64)
    H = oracle.forward_dense(W, X, h0)
    assert np.abs(H).max() < 2048 and np.all(H == np.round(H))
    np.testing.assert_array_equal(oracle.forward_dense_half_h(W, X, h0), H)
    # identity weights: prefix sums, also exact
    Xp = rng.integers(0, 40, size=(T, B, N)).astype(np.float64)
    np.testing.assert_array_equal(oracle.forward_dense_half_h(np.eye(N), Xp, h0),
                                  h0[None] + np.cumsum(Xp, axis=0))


def test_half_h_model_differs_from_definition_off_grid():
    """Off the fp16 grid the model must not collapse into the definition (a
    model that forgot to round would pass the grid test above)."""
    w = WORKLOADS["dense_f16_n1152"].with_(T=8)
    d = generate(w)
    Hq = oracle.forward_dense_half_h(d["W"], d["X"], d["h0"])
    H = oracle.forward_dense(d["W"], d["X"], d["h0"])
    assert np.array_equal(Hq[0], H[0])          # h0 = 0 stages exactly
    assert not np.array_equal(Hq[1:], H[1:])
    assert oracle.tolerance_ratio(Hq, H, oracle.TOL_F16) > 0


@pytest.mark.parametrize("name", ["dense_f16_n1152", "dense_f16_n1792"])
def test_fp16_hidden_state_model_meets_fp16_bar(name):
    """Rounding the state to fp16 at every step stays well inside the fp16-weight
    bar 2e-2 (1 + |h|) over the whole configured sequence (T = 256)."""
    w = WORKLOADS[name]
    d = generate(w)
    H = oracle.forward_dense(d["W"], d["X"], d["h0"])
    Hq = oracle.forward_dense_half_h(d["W"], d["X"], d["h0"])
    assert oracle.tolerance_ratio(Hq, H, oracle.TOL_F16) < 0.2
