"""Persistent basic-RNN forward recurrence for AMD Instinct MI355X (gfx950).

    H[t] = relu(X[t] + W H[t-1]),  H[-1] = h0

with W dense (fp32 / fp16) or row-balanced sparse (int16 columns, fp16 / fp32
values), run as one persistent HIP kernel per call with W resident on chip.
The kernels and the C ABI live in ``libprnn.so`` (``include/prnn.h``); this
package holds its ctypes binding (``binding``), the build script (``build``)
and seeded synthetic inputs (``inputs``).
"""
from .binding import (  # noqa: F401
    Handle,
    PrnnError,
    default_handle,
    forward_dense,
    forward_sparse,
    load_library,
)
