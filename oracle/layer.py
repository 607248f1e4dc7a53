"""fp64 CPU oracle of the input projection, a full RNN layer and a stack of layers.

TEST INFRASTRUCTURE, like ``oracle.rnn``: only the tests, the smoke check and
the benchmark's CPU baseline may import it; it shares no code with the HIP
library.

* Input projection ("Optimizing Performance of Recurrent Neural Networks on
  GPUs", Abstract: the single-layer stage).  The input-side product of a
  layer does not depend on the previous state, so for a whole sequence it is
  one matrix product computed ahead of the recurrence:

      X[t, b, n] = bias[n] + sum_i U[n, i] * x[t, b, i]

  with U [N, I] (row n belongs to output neuron n, like W) and x [T, B, I].
* A layer is that projection followed by the recurrence of ``oracle.rnn``:
  H = forward_*(W, X = project(U, x, bias), h0).
* A stack of layers (the same page, the entire-network stage) feeds layer l's
  output sequence H_l to layer l + 1 as its input x; every layer keeps its own
  U, bias, W and h0.  Layer l + 1's step t depends only on layer l's step t,
  which is what lets the layers run as a wavefront; the definition itself is
  the plain layer-by-layer composition.

All inputs are widened exactly to fp64 and all arithmetic is fp64; the
projection uses numpy's matmul, with no blocking or reordering beyond that.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .rnn import forward_dense, forward_sparse


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def project(U, x, bias=None) -> np.ndarray:
    """X[..., n] = bias[n] + sum_i U[n, i] * x[..., i].  Returns fp64 with x's leading shape."""
    U = _f64(U)
    x = _f64(x)
    if U.ndim != 2:
        raise ValueError(f"U must be [N, I], got {U.shape}")
    N, I = U.shape
    if x.shape[-1] != I:
        raise ValueError(f"x must end in I={I}, got {x.shape}")
    X = x @ U.T
    if bias is not None:
        b = _f64(bias)
        if b.shape != (N,):
            raise ValueError(f"bias must be [{N}], got {b.shape}")
        X = X + b
    return X


def forward_layer_dense(U, bias, W, x, h0=None) -> np.ndarray:
    """One dense layer: the recurrence over the projected input sequence."""
    return forward_dense(W, project(U, x, bias), h0)


def forward_layer_sparse(U, bias, col, val, x, h0=None) -> np.ndarray:
    """One row-balanced sparse layer: the recurrence over the projected input sequence."""
    return forward_sparse(col, val, project(U, x, bias), h0)


def forward_stack_dense(layers: Sequence[dict], x, h0s: Optional[Sequence] = None) -> list:
    """Layers given as dicts with keys U, bias, W.  Returns every layer's H, fp64 [T, B, N_l]."""
    outs = []
    inp = _f64(x)
    for l, layer in enumerate(layers):
        h0 = None if h0s is None else h0s[l]
        H = forward_layer_dense(layer["U"], layer.get("bias"), layer["W"], inp, h0)
        outs.append(H)
        inp = H
    return outs


def forward_stack_sparse(layers: Sequence[dict], x, h0s: Optional[Sequence] = None) -> list:
    """A stack of row-balanced sparse layers, given as dicts with keys U, bias,
    col, val (the entire-network stage over the sparse layers of "Sparse
    Persistent RNNs: Squeezing Large Recurrent Networks On-Chip").  Returns
    every layer's H, fp64 [T, B, N_l]."""
    outs = []
    inp = _f64(x)
    for l, layer in enumerate(layers):
        h0 = None if h0s is None else h0s[l]
        H = forward_layer_sparse(layer["U"], layer.get("bias"), layer["col"], layer["val"], inp, h0)
        outs.append(H)
        inp = H
    return outs
