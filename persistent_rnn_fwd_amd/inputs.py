"""Seeded synthetic inputs for the basic-RNN forward recurrence.

This module only draws random numbers and lays them out.  It holds none of the
recurrence's arithmetic, so both the fp64 CPU oracle (through the tests) and the
HIP path (through the tests and the benchmark) can be fed from it.

Workloads follow the layer sizes, batch size, densities and sequence length on
the pages:
  * "Sparse Persistent RNNs: Squeezing Large Recurrent Networks On-Chip",
    table "Measured effects reported in the paper": layer sizes 1152, 1792 and
    5760, batch size 4, densities 10 % and 1 %, 256 timesteps, and
    load-balanced (row-balanced) pruning, i.e. the same number of nonzeros in
    every row;
  * "persistent-rnn" (Fast Recurrent Networks Library), "What This Project
    Does": small batches, "like 4".

Value distributions (the pages state none):
  dense W   ~ N(0, 0.8^2 / N)   (circular law: spectral radius ~0.8)
  sparse W  ~ N(0, 0.8^2 / K)   on K distinct columns per row, drawn uniformly
                                without replacement and stored sorted
  X         ~ N(0, 1)           fp32, the pre-activations W_x x_t + b
  h0        = 0                 (or N(0,1), signed, when asked for: an initial
                                state is any fp32 vector, not only a ReLU output;
                                |N(0,1)| with "absrandn")

Unbalanced rows ("magnitude" pruning), for the pages' load-balanced vs
unbalanced pruning comparison: a dense Gaussian matrix whose rows carry
log-normal scales exp(N(0, 0.1^2)) is pruned by keeping the N K largest
magnitudes of the whole matrix, so rows keep different numbers of entries
(K on average); each row's kept values are rescaled to L2 norm 0.8 and the
rows are stored in the row-balanced format at the width of the longest row:
each row's kept entries first (sorted by column), then padding on distinct
unused columns (sorted) with value 0, and ``row_len`` [N] int32 gives the
number of kept entries of each row.

Layers (input projection + recurrence, "Optimizing Performance of Recurrent
Neural Networks on GPUs", Abstract): on top of a recurrence workload, the
layer input x ~ N(0, 1) fp32 [T, B, I], U ~ N(0, 1 / I) rounded to fp16 [N, I]
and bias ~ N(0, 0.1^2) fp32 [N], so that U x has the N(0, 1) scale of the
recurrence workloads' X.  The pages give no input width; I = N (a layer of a
stack, whose input is the layer below's output) is the plain reading.  These
arrays come from their own streams, ``SeedSequence([seed, 1, I]).spawn(3)``.
A stack of L layers draws layer l's U, bias and W from
``SeedSequence([seed, 2, l]).spawn(3)``.

Random streams: ``numpy.random.SeedSequence(seed).spawn(3)`` gives independent
generators for W, X and h0, in that order.  fp16 weights are produced by
rounding the fp64 draw to the nearest fp16 (numpy's round-to-nearest-even);
the oracle and the GPU consume the same stored array, so the rounding is part
of the input, never part of the error.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One synthetic recurrence problem (sizes, weight format, seed)."""

    name: str
    kind: str            # "dense" or "sparse"
    N: int               # hidden size (rows = columns of W)
    B: int               # batch
    T: int               # timesteps
    w_dtype: str         # "f32" or "f16" (dense W, or sparse values)
    K: int = 0           # nonzeros per row (sparse only)
    seed: int = 0
    h0: str = "zeros"    # "zeros", "randn" (N(0,1), signed) or "absrandn" (|N(0,1)|)
    rows: str = "balanced"  # sparse: "balanced" (K per row) or "magnitude" (K on average, padded)

    @property
    def nnz(self) -> int:
        return self.N * (self.K if self.kind == "sparse" else self.N)

    @property
    def flop_per_step(self) -> int:
        """Multiply-adds of W.h_{t-1} counted as 2 flops each, all batch rows."""
        return 2 * self.B * self.nnz

    @property
    def weight_bytes(self) -> int:
        if self.kind == "dense":
            return self.N * self.N * (4 if self.w_dtype == "f32" else 2)
        return self.N * self.K * ((4 if self.w_dtype == "f32" else 2) + 2)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workload families.  K is the nonzero count per row at the stated
# density (1152*10% -> 115, 1792*10% -> 179, 1792*1% -> 18, 5760*1% -> 58).
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("dense_f32_n256", "dense", 256, 4, 32, "f32", seed=101),
        Workload("dense_f16_n1152", "dense", 1152, 4, 256, "f16", seed=102),
        Workload("sparse10_f16_n1152", "sparse", 1152, 4, 256, "f16", K=115, seed=103),
        Workload("dense_f16_n1792", "dense", 1792, 4, 256, "f16", seed=104),
        Workload("sparse10_f16_n1792", "sparse", 1792, 4, 256, "f16", K=179, seed=104),
        Workload("sparse1_f16_n1792", "sparse", 1792, 4, 256, "f16", K=18, seed=104),
        Workload("sparse1_f16_n5760", "sparse", 5760, 4, 256, "f16", K=58, seed=105),
        Workload("sparse10_f16_n2304", "sparse", 2304, 4, 256, "f16", K=230, seed=106),
        Workload("sparse25_f16_n2304", "sparse", 2304, 4, 256, "f16", K=576, seed=107),
        Workload("sparse10u_f16_n2304", "sparse", 2304, 4, 256, "f16", K=230, seed=106, rows="magnitude"),
        Workload("sparse25u_f16_n2304", "sparse", 2304, 4, 256, "f16", K=576, seed=107, rows="magnitude"),
        Workload("sparse5_f16_n5760", "sparse", 5760, 4, 256, "f16", K=288, seed=108),
    ]
}


def _np_dtype(w_dtype: str):
    if w_dtype == "f32":
        return np.float32
    if w_dtype == "f16":
        return np.float16
    raise ValueError(f"unknown weight dtype {w_dtype!r}")


def draw_sparse_pattern(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """K distinct column indices per row, uniform without replacement, sorted.

    Returns int16 [N, K] (so N must be at most 32767)."""
    if not (1 <= K <= N):
        raise ValueError("need 1 <= K <= N")
    if N > 32767:
        raise ValueError("int16 column indices need N <= 32767")
    col = np.empty((N, K), dtype=np.int16)
    for i in range(N):
        col[i] = np.sort(rng.choice(N, size=K, replace=False))
    return col


def draw_magnitude_pruned(rng: np.random.Generator, N: int, K: int, wdt, sigma: float = 0.1):
    """Unbalanced sparse W (see the module docstring), stored row-balanced at
    the width of the longest row: returns (col int16 [N, Kmax], val [N, Kmax],
    row_len int32 [N]), each row's kept entries first."""
    if not 1 <= K <= N or N > 32767:
        raise ValueError("need 1 <= K <= N <= 32767")
    scale = np.exp(rng.normal(0.0, sigma, size=N))
    g = rng.standard_normal((N, N)) * scale[:, None]
    mag = np.abs(g)
    thr = np.partition(mag.ravel(), mag.size - N * K)[mag.size - N * K]
    keep = mag >= thr
    empty = ~keep.any(axis=1)                    # every row keeps at least its largest entry
    keep[empty, np.argmax(mag[empty], axis=1)] = True
    kmax = int(keep.sum(axis=1).max())
    col = np.empty((N, kmax), dtype=np.int16)
    val = np.zeros((N, kmax), dtype=np.float64)
    row_len = keep.sum(axis=1).astype(np.int32)
    for i in range(N):
        real = np.flatnonzero(keep[i])                       # sorted
        v = g[i, real]
        v = v * (0.8 / np.sqrt(np.sum(v * v)))
        pad = np.flatnonzero(~keep[i])[: kmax - real.size]   # distinct unused columns, value 0, sorted
        col[i] = np.concatenate([real, pad])
        val[i, : real.size] = v
    return col, val.astype(wdt), row_len


def generate(w: Workload, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw one problem.

    Returns a dict with host numpy arrays:
      dense : ``W`` [N, N] (float32 or float16), row i = output neuron i
      sparse: ``col`` int16 [N, K], ``val`` [N, K] (float32 or float16);
              unbalanced rows also ``row_len`` int32 [N] (entries per row)
      both  : ``X`` float32 [T, B, N], ``h0`` float32 [B, N]
    """
    seed = w.seed if seed is None else seed
    s_w, s_x, s_h = np.random.SeedSequence(seed).spawn(3)
    rng_w, rng_x, rng_h = (np.random.default_rng(s) for s in (s_w, s_x, s_h))
    out: Dict[str, np.ndarray] = {}
    wdt = _np_dtype(w.w_dtype)
    if w.kind == "dense":
        out["W"] = (rng_w.standard_normal((w.N, w.N)) * (0.8 / np.sqrt(w.N))).astype(wdt)
    elif w.kind == "sparse" and w.rows == "magnitude":
        out["col"], out["val"], out["row_len"] = draw_magnitude_pruned(rng_w, w.N, w.K, wdt)
    elif w.kind == "sparse":
        out["col"] = draw_sparse_pattern(rng_w, w.N, w.K)
        out["val"] = (rng_w.standard_normal((w.N, w.K)) * (0.8 / np.sqrt(w.K))).astype(wdt)
    else:
        raise ValueError(f"unknown kind {w.kind!r}")
    out["X"] = rng_x.standard_normal((w.T, w.B, w.N)).astype(np.float32)
    if w.h0 == "zeros":
        out["h0"] = np.zeros((w.B, w.N), dtype=np.float32)
    elif w.h0 == "randn":
        out["h0"] = rng_h.standard_normal((w.B, w.N)).astype(np.float32)
    elif w.h0 == "absrandn":
        out["h0"] = np.abs(rng_h.standard_normal((w.B, w.N))).astype(np.float32)
    else:
        raise ValueError(f"unknown h0 mode {w.h0!r}")
    return out


# Layers: a recurrence workload plus its input width I.
LAYER_WORKLOADS: Dict[str, tuple] = {
    "layer_dense_f16_n1792": ("dense_f16_n1792", 1792),
    "layer_sparse10_f16_n1792": ("sparse10_f16_n1792", 1792),
}


def generate_layer(w: Workload, I: int, seed: Optional[int] = None, x_dtype: str = "f32") -> Dict[str, np.ndarray]:
    """``generate(w)`` (W or col/val, h0; its X is not used by a layer) plus
    ``U`` float16 [N, I], ``bias`` float32 [N] and the layer input ``x``
    [T, B, I] (float32, or float16 with x_dtype="f16")."""
    seed = w.seed if seed is None else seed
    out = generate(w, seed)
    s_u, s_b, s_x = np.random.SeedSequence([seed, 1, I]).spawn(3)
    rng_u, rng_b, rng_x = (np.random.default_rng(t) for t in (s_u, s_b, s_x))
    out["U"] = (rng_u.standard_normal((w.N, I)) / np.sqrt(I)).astype(np.float16)
    out["bias"] = (0.1 * rng_b.standard_normal(w.N)).astype(np.float32)
    out["x"] = rng_x.standard_normal((w.T, w.B, I)).astype(_np_dtype(x_dtype))
    return out


def generate_stack(w: Workload, L: int, seed: Optional[int] = None) -> Dict[str, object]:
    """L layers of width N = I = w.N: ``layers`` = [{U, bias, W}] for a dense
    workload, [{U, bias, col, val}] (row-balanced, K per row) for a sparse one
    (fp16 U, and W or val, as in ``generate_layer`` and ``generate``), the input
    ``x`` fp32 [T, B, N] and per-layer ``h0s`` (zeros, N(0,1) with w.h0 ==
    "randn", |N(0,1)| with "absrandn")."""
    if w.kind == "sparse" and w.rows != "balanced":
        raise ValueError("sparse stacks are row-balanced")
    seed = w.seed if seed is None else seed
    base = generate_layer(w, w.N, seed)
    layers, h0s = [], []
    for l in range(L):
        s_u, s_b, s_w = np.random.SeedSequence([seed, 2, l]).spawn(3)
        rng_u, rng_b, rng_w = (np.random.default_rng(t) for t in (s_u, s_b, s_w))
        layer = {
            "U": (rng_u.standard_normal((w.N, w.N)) / np.sqrt(w.N)).astype(np.float16),
            "bias": (0.1 * rng_b.standard_normal(w.N)).astype(np.float32),
        }
        if w.kind == "dense":
            layer["W"] = (rng_w.standard_normal((w.N, w.N)) * (0.8 / np.sqrt(w.N))).astype(_np_dtype(w.w_dtype))
        else:
            layer["col"] = draw_sparse_pattern(rng_w, w.N, w.K)
            layer["val"] = (rng_w.standard_normal((w.N, w.K)) * (0.8 / np.sqrt(w.K))).astype(_np_dtype(w.w_dtype))
        layers.append(layer)
        if l == 0:
            h0 = base["h0"]
        elif w.h0 in ("randn", "absrandn"):
            h0 = rng_b.standard_normal((w.B, w.N)).astype(np.float32)
            h0 = np.abs(h0) if w.h0 == "absrandn" else h0
        else:
            h0 = np.zeros((w.B, w.N), dtype=np.float32)
        h0s.append(h0)
    return {"layers": layers, "x": base["x"], "h0s": h0s}
