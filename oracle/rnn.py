"""Plain fp64 CPU oracle for the basic-RNN forward recurrence.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import this module.  It shares no code with the HIP library and
imports nothing from it; it takes plain numpy arrays and returns plain numpy
arrays.

What it computes (for every timestep t = 0 .. T-1, batch row b, neuron i):

    a[t, b, i] = X[t, b, i] + sum_j W[i, j] * h[t-1, b, j]
    H[t, b, i] = max(a[t, b, i], 0)           with h[-1] = h0 (zeros if absent)

* A basic (vanilla) RNN layer, the only layer kind the persistent library
  supports ("persistent-rnn", section "Important Constraints").
* X holds the input projection of every timestep, computed ahead of the
  recurrence: the "single layer" stage of "Optimizing Performance of Recurrent
  Neural Networks on GPUs" (Abstract) takes the input-side product out of the
  sequential loop, so only W.h_{t-1} stays inside it.
* The activation is ReLU.  The pages name none; ReLU is the plain reading for
  a basic RNN layer whose state is a rectified sum.
* Row i of W belongs to output neuron i.  Sparse W is row-balanced: every row
  holds the same number K of nonzeros ("Sparse Persistent RNNs: Squeezing
  Large Recurrent Networks On-Chip", table "Measured effects reported in the
  paper", load-balanced pruning row), stored as col[i, k], val[i, k].
* Inputs are widened exactly to fp64 (fp16 and fp32 values are exact in
  fp64); all arithmetic is fp64.  The sign of a zero is not significant; NaN
  propagates through the ReLU (numpy.maximum keeps NaN).

The loop over t is explicit; the product W.h uses numpy's matmul and the
sparse product a gather and a sum, with no blocking or reordering beyond that.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _check_xh(X: np.ndarray, h0: Optional[np.ndarray], N: int):
    if X.ndim != 3 or X.shape[2] != N:
        raise ValueError(f"X must be [T, B, {N}], got {X.shape}")
    T, B, _ = X.shape
    if h0 is None:
        h = np.zeros((B, N), dtype=np.float64)
    else:
        h = _f64(h0)
        if h.shape != (B, N):
            raise ValueError(f"h0 must be [{B}, {N}], got {h.shape}")
    return T, B, h


def forward_dense(W, X, h0=None) -> np.ndarray:
    """H[t] = relu(X[t] + H[t-1] @ W^T), H[-1] = h0.  Returns fp64 [T, B, N]."""
    W = _f64(W)
    X = _f64(X)
    if W.ndim != 2 or W.shape[0] != W.shape[1]:
        raise ValueError(f"W must be square, got {W.shape}")
    N = W.shape[0]
    T, B, h = _check_xh(X, h0, N)
    H = np.empty((T, B, N), dtype=np.float64)
    for t in range(T):
        # a[b, i] = X[t, b, i] + sum_j h[b, j] * W[i, j]
        a = X[t] + h @ W.T
        h = np.maximum(a, 0.0)
        H[t] = h
    return H


def forward_dense_half_h(W, X, h0=None) -> np.ndarray:
    """The dense recurrence with the state rounded to fp16 before the product.

        a[t, b, i] = X[t, b, i] + sum_j W[i, j] * r(h[t-1, b, j]),  H[t] = max(a, 0)

    where r() rounds to IEEE binary16, to nearest with ties to even (numpy's
    float16 conversion; a value beyond the fp16 range becomes infinite).  Only
    the copy of the state that enters the product is rounded: H itself, X, h0
    and every sum stay fp64.  This is a model of a kernel that stages the state
    in fp16 beside fp16 weights with fp32 sums (the "fp16 weights, fp32
    accumulation" precision), used to show what such staging costs against
    forward_dense, which remains the definition."""
    W = _f64(W)
    X = _f64(X)
    if W.ndim != 2 or W.shape[0] != W.shape[1]:
        raise ValueError(f"W must be square, got {W.shape}")
    N = W.shape[0]
    T, B, h = _check_xh(X, h0, N)
    H = np.empty((T, B, N), dtype=np.float64)
    for t in range(T):
        staged = h.astype(np.float16).astype(np.float64)   # r(h[t-1])
        a = X[t] + staged @ W.T
        h = np.maximum(a, 0.0)
        H[t] = h
    return H


def forward_sparse(col, val, X, h0=None) -> np.ndarray:
    """Row-balanced sparse W: a[b, i] = X[t, b, i] + sum_k val[i, k] * h[b, col[i, k]]."""
    col = np.asarray(col).astype(np.int64)
    val = _f64(val)
    X = _f64(X)
    if col.ndim != 2 or col.shape != val.shape:
        raise ValueError("col and val must both be [N, K]")
    N, K = col.shape
    if col.size and (col.min() < 0 or col.max() >= N):
        raise ValueError("column index out of range")
    T, B, h = _check_xh(X, h0, N)
    H = np.empty((T, B, N), dtype=np.float64)
    for t in range(T):
        gathered = h[:, col]                     # [B, N, K]: h[b, col[i, k]]
        a = X[t] + (gathered * val[None, :, :]).sum(axis=2)
        h = np.maximum(a, 0.0)
        H[t] = h
    return H


def forward_sparse_rows(col, val, row_len, X, h0=None) -> np.ndarray:
    """Sparse W whose rows hold different numbers of nonzeros: row i is its
    first row_len[i] pairs, a[b, i] = X[t, b, i] + sum_{k < row_len[i]}
    val[i, k] * h[b, col[i, k]].  Pairs at k >= row_len[i] are not part of W
    and contribute nothing, whatever they hold (values, NaN, columns out of
    range).  This is the unbalanced sparsity that the pages set against
    load-balanced pruning ("Sparse Persistent RNNs: Squeezing Large Recurrent
    Networks On-Chip", table "Measured effects reported in the paper",
    load-balanced pruning row), stored at the width K of the longest row."""
    col = np.asarray(col).astype(np.int64)
    val = _f64(val)
    X = _f64(X)
    if col.ndim != 2 or col.shape != val.shape:
        raise ValueError("col and val must both be [N, K]")
    N, K = col.shape
    row_len = np.asarray(row_len).astype(np.int64)
    if row_len.shape != (N,) or (row_len.size and (row_len.min() < 0 or row_len.max() > K)):
        raise ValueError("row_len must be [N] with entries in [0, K]")
    live = np.arange(K)[None, :] < row_len[:, None]            # [N, K]: pair k belongs to row i
    if live.any() and (col[live].min() < 0 or col[live].max() >= N):
        raise ValueError("column index out of range")
    safe_col = np.where(live, col, 0)                           # never index with a pair outside its row
    T, B, h = _check_xh(X, h0, N)
    H = np.empty((T, B, N), dtype=np.float64)
    for t in range(T):
        with np.errstate(invalid="ignore", over="ignore"):    # products outside the rows are discarded
            terms = h[:, safe_col] * val[None, :, :]            # [B, N, K]
        a = X[t] + np.where(live[None, :, :], terms, 0.0).sum(axis=2)
        h = np.maximum(a, 0.0)
        H[t] = h
    return H


def sparse_to_dense(col, val, N: Optional[int] = None) -> np.ndarray:
    """The dense fp64 matrix a row-balanced (col, val) pair stands for.

    W[i, col[i, k]] += val[i, k]; a repeated column would add up, which is what
    the sparse sum above does too."""
    col = np.asarray(col).astype(np.int64)
    val = _f64(val)
    n = col.shape[0] if N is None else N
    W = np.zeros((n, n), dtype=np.float64)
    rows = np.repeat(np.arange(col.shape[0]), col.shape[1])
    np.add.at(W, (rows, col.ravel()), val.ravel())
    return W


def tolerance_ratio(H_test, H_ref, tol: float) -> float:
    """max over elements of |H_test - H_ref| / (tol * (1 + |H_ref|)).

    A value <= 1 passes the per-element bar |d| <= tol * (1 + |h|)."""
    H_test = _f64(H_test)
    H_ref = _f64(H_ref)
    if H_test.shape != H_ref.shape:
        raise ValueError(f"shape mismatch {H_test.shape} vs {H_ref.shape}")
    if H_ref.size == 0:
        return 0.0
    d = np.abs(H_test - H_ref)
    bad = np.isnan(d)
    if bad.any():
        # NaN in one and not the other is a failure; NaN in both is agreement.
        both = np.isnan(H_test) & np.isnan(H_ref)
        if (bad & ~both).any():
            return float("inf")
        d = np.where(both, 0.0, d)
    return float(np.max(d / (tol * (1.0 + np.abs(np.nan_to_num(H_ref))))))


# Per-element tolerances: fp32 weights, and fp16 weights with fp32 accumulation.
TOL_F32 = 1e-4
TOL_F16 = 2e-2
