"""Pins for the projection, layer and stack oracle (CPU only).

Each test checks ``oracle.layer`` against something other than itself: brute
force in exact rational arithmetic (projection, a whole layer, a two-layer
stack), closed forms (identity and scaled-permutation projections, a stack
whose layers pass their input through) and the input generator's scale.  A
dropped bias, a transposed U, an off-by-one between layers or a layer fed
the wrong input fails one of them.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from persistent_rnn_fwd_amd.inputs import LAYER_WORKLOADS, WORKLOADS, generate_layer, generate_stack


def _brute_project(U, x, bias):
    """X[m][n] = bias[n] + sum_i U[n][i] x[m][i], element by element in Fractions."""
    N, I = len(U), len(U[0])
    return [[Fraction(bias[n]) + sum(Fraction(U[n][i]) * Fraction(row[i]) for i in range(I)) for n in range(N)]
            for row in x]


def _brute_recurrence(W, X, h0):
    T, B, N = len(X), len(X[0]), len(W)
    h = [[Fraction(v) for v in r] for r in h0]
    out = []
    for t in range(T):
        new = []
        for b in range(B):
            new.append([max(Fraction(X[t][b][i]) + sum(Fraction(W[i][j]) * h[b][j] for j in range(N)), Fraction(0))
                        for i in range(N)])
        h = new
        out.append(new)
    return out


def _ints(rng, shape, lo=-3, hi=3):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float64)


@pytest.mark.parametrize("seed", range(4))
def test_project_matches_rational_brute_force(seed):
    rng = np.random.default_rng(seed)
    N, I, M = 3, 5, 4
    U, x, bias = _ints(rng, (N, I)), _ints(rng, (M, I)), _ints(rng, (N,))
    ref = _brute_project(U.tolist(), x.tolist(), bias.tolist())
    np.testing.assert_array_equal(oracle.project(U, x, bias), np.array(ref, dtype=np.float64))


def test_project_identity_and_scaled_permutation():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, 2, 6))
    bias = rng.standard_normal(6)
    np.testing.assert_array_equal(oracle.project(np.eye(6), x, bias), x + bias)
    perm = rng.permutation(6)
    P = np.zeros((6, 6))
    P[np.arange(6), perm] = 2.0                       # row n picks input perm[n], times 2
    np.testing.assert_array_equal(oracle.project(P, x), 2.0 * x[..., perm])


def test_project_orientation_and_bias_matter():
    rng = np.random.default_rng(8)
    U = _ints(rng, (4, 4))
    while np.array_equal(U, U.T):
        U = _ints(rng, (4, 4))
    x = _ints(rng, (2, 4))
    bias = np.ones(4)
    ref = np.array(_brute_project(U.tolist(), x.tolist(), bias.tolist()), dtype=np.float64)
    assert not np.array_equal(oracle.project(U.T, x, bias), ref)
    assert not np.array_equal(oracle.project(U, x, None), ref)


@pytest.mark.parametrize("seed", range(3))
def test_layer_matches_rational_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    N, I, B, T = 3, 4, 2, 3
    U, W, bias = _ints(rng, (N, I)), _ints(rng, (N, N), -1, 1), _ints(rng, (N,))
    x, h0 = _ints(rng, (T, B, I)), _ints(rng, (B, N), 0, 2)
    X = [_brute_project(U.tolist(), x[t].tolist(), bias.tolist()) for t in range(T)]
    ref = _brute_recurrence(W.tolist(), X, h0.tolist())
    np.testing.assert_array_equal(oracle.forward_layer_dense(U, bias, W, x, h0), np.array(ref, dtype=np.float64))
    # the sparse layer over a row-balanced form of the same W
    col = np.tile(np.arange(N), (N, 1))
    np.testing.assert_array_equal(oracle.forward_layer_sparse(U, bias, col, W, x, h0),
                                  np.array(ref, dtype=np.float64))


def test_stack_matches_rational_brute_force():
    rng = np.random.default_rng(5)
    N, B, T = 3, 2, 3
    layers = [{"U": _ints(rng, (N, N), -2, 2), "bias": _ints(rng, (N,)), "W": _ints(rng, (N, N), -1, 1)}
              for _ in range(2)]
    x = _ints(rng, (T, B, N))
    h0s = [_ints(rng, (B, N), 0, 2) for _ in range(2)]
    inp = x.tolist()
    refs = []
    for l, L in enumerate(layers):
        X = [_brute_project(L["U"].tolist(), inp[t], L["bias"].tolist()) for t in range(T)]
        H = _brute_recurrence(L["W"].tolist(), X, h0s[l].tolist())
        refs.append(np.array(H, dtype=np.float64))
        inp = H
    got = oracle.forward_stack_dense(layers, x, h0s)
    assert len(got) == 2
    for g, r in zip(got, refs):
        np.testing.assert_array_equal(g, r)


def test_stack_of_pass_through_layers():
    """U = I, bias = 0, W = 0: every layer is relu of its input, so each layer's
    output is relu(x) (relu is idempotent)."""
    rng = np.random.default_rng(9)
    N = 5
    x = rng.standard_normal((4, 2, N))
    layers = [{"U": np.eye(N), "bias": np.zeros(N), "W": np.zeros((N, N))} for _ in range(3)]
    for H in oracle.forward_stack_dense(layers, x):
        np.testing.assert_array_equal(H, np.maximum(x, 0.0))


def test_sparse_stack_matches_rational_brute_force():
    """Two sparse layers (K pairs per row, a repeated column in one row) in
    exact rationals, each through its dense equivalent."""
    rng = np.random.default_rng(15)
    N, K, B, T = 4, 2, 2, 3
    layers = []
    for _ in range(2):
        col = np.stack([rng.choice(N, K, replace=False) for _ in range(N)])
        col[1] = [2, 2]
        layers.append({"U": _ints(rng, (N, N), -2, 2), "bias": _ints(rng, (N,)), "col": col,
                       "val": _ints(rng, (N, K), -1, 1)})
    x = _ints(rng, (T, B, N))
    h0s = [_ints(rng, (B, N), -1, 2) for _ in range(2)]
    inp = x.tolist()
    refs = []
    for l, L in enumerate(layers):
        Wd = [[Fraction(0)] * N for _ in range(N)]
        for i in range(N):
            for k in range(K):
                Wd[i][int(L["col"][i][k])] += Fraction(L["val"][i][k])
        X = [_brute_project(L["U"].tolist(), inp[t], L["bias"].tolist()) for t in range(T)]
        H = _brute_recurrence(Wd, X, h0s[l].tolist())
        refs.append(np.array(H, dtype=np.float64))
        inp = H
    got = oracle.forward_stack_sparse(layers, x, h0s)
    assert len(got) == 2
    for g, r in zip(got, refs):
        np.testing.assert_array_equal(g, r)


def test_sparse_stack_generator_and_dense_copy():
    """The sparse stack generator gives each layer its own pattern and values;
    the sparse stack equals the dense stack of the layers' dense copies."""
    w = WORKLOADS["sparse10_f16_n1152"].with_(T=3, h0="randn")
    st = generate_stack(w, 2)
    L0, L1 = st["layers"]
    assert L0["col"].shape == (w.N, w.K) and L0["val"].dtype == np.float16 and "W" not in L0
    assert not np.array_equal(L0["col"], L1["col"])
    dense = [{"U": L["U"], "bias": L["bias"], "W": oracle.sparse_to_dense(L["col"], L["val"], w.N)}
             for L in st["layers"]]
    for a, b in zip(oracle.forward_stack_sparse(st["layers"], st["x"], st["h0s"]),
                    oracle.forward_stack_dense(dense, st["x"], st["h0s"])):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_layer_generator_shapes_and_scale():
    name, I = next(iter(LAYER_WORKLOADS.values()))
    w = WORKLOADS[name].with_(T=16)
    d = generate_layer(w, I)
    assert d["U"].dtype == np.float16 and d["U"].shape == (w.N, I)
    assert d["bias"].dtype == np.float32 and d["bias"].shape == (w.N,)
    assert d["x"].dtype == np.float32 and d["x"].shape == (w.T, w.B, I)
    X = oracle.project(d["U"], d["x"], None)
    assert 0.9 < X.std() < 1.1                          # U x ~ N(0, 1), like the recurrence workloads' X
    d2 = generate_layer(w, I)
    assert all(np.array_equal(d[k], d2[k]) for k in ("U", "bias", "x"))
    assert generate_layer(w, I, x_dtype="f16")["x"].dtype == np.float16


def test_stack_generator():
    w = WORKLOADS["dense_f16_n1152"].with_(T=2)
    st = generate_stack(w, 3)
    assert len(st["layers"]) == 3 and len(st["h0s"]) == 3
    assert not np.array_equal(st["layers"][0]["W"], st["layers"][1]["W"])
    assert st["x"].shape == (w.T, w.B, w.N)
