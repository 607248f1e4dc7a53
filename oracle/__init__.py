"""fp64 CPU oracle of the basic-RNN forward recurrence.

TEST INFRASTRUCTURE: imported only by ``tests/``, by ``__graft_entry__.smoke()``
and by the benchmark's CPU-baseline leg.  The product library never imports it
and never falls back to it.

Pins: every function here is checked in ``tests/test_oracle.py`` against
brute force in exact rational arithmetic, closed forms (W = 0, W = I, cyclic
permutations, the linear regime's block-triangular solve, diagonal W),
invariants (batch independence, chunking in time, positive homogeneity) and a
hand-worked example under ``tests/golden/``.  The projection, layer and stack
functions (``oracle.layer``) are pinned in ``tests/test_oracle_layer.py``.
"""
from .rnn import (  # noqa: F401
    TOL_F16,
    TOL_F32,
    forward_dense,
    forward_dense_half_h,
    forward_sparse,
    forward_sparse_rows,
    sparse_to_dense,
    tolerance_ratio,
)
from .layer import (  # noqa: F401
    forward_layer_dense,
    forward_layer_sparse,
    forward_stack_dense,
    forward_stack_sparse,
    project,
)
