"""ctypes binding of libprnn.so (the C ABI declared in include/prnn.h).

Argument marshalling only: torch tensors supply device memory and the current
stream; every step of the recurrence runs in the library's HIP kernels.  If the
library has not been built, every entry point raises; nothing falls back to
another implementation.
"""
from __future__ import annotations

import atexit
import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libprnn.so")

STATUS_NAMES = {
    0: "PRNN_STATUS_SUCCESS",
    1: "PRNN_STATUS_BAD_PARAM",
    2: "PRNN_STATUS_NOT_SUPPORTED",
    3: "PRNN_STATUS_ALLOC_FAILED",
    4: "PRNN_STATUS_EXECUTION_FAILED",
    5: "PRNN_STATUS_INTERNAL_ERROR",
}
SUCCESS, BAD_PARAM, NOT_SUPPORTED, ALLOC_FAILED, EXECUTION_FAILED, INTERNAL_ERROR = range(6)
DATA_FLOAT, DATA_HALF = 0, 1
EXCHANGE_AUTO, EXCHANGE_DIRECT, EXCHANGE_RELAY = 0, 1, 2
LAYOUT_AUTO, LAYOUT_SPREAD, LAYOUT_TEAM = 0, 1, 2
MATH_AUTO, MATH_EXACT, MATH_SPLIT, MATH_HALF = 0, 1, 2, 3
STACK_AUTO, STACK_BLOCKED, STACK_FUSED, STACK_LAYERS = 0, 1, 2, 3
LAUNCH_COOPERATIVE, LAUNCH_PLAIN = 0, 1
TRACE_WORDS = 8  # per-wave trace record: see Handle.get_trace

# Every function include/prnn.h declares, with its ctypes signature.
_H = ctypes.c_void_p
_P = ctypes.c_void_p
_I = ctypes.c_int
SIGNATURES = {
    "prnn_create": (_I, [ctypes.POINTER(_H)]),
    "prnn_destroy": (_I, [_H]),
    "prnn_forward_dense": (_I, [_H, _I, _I, _I, _I, _P, _P, _P, _P, _P]),
    "prnn_forward_sparse": (_I, [_H, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P, _P]),
    "prnn_forward_sparse_rows": (_I, [_H, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P, _P, _P]),
    "prnn_sync_floor": (_I, [_H, _I, _I, _I, _P, _P]),
    "prnn_synchronize": (_I, [_H, _P]),
    "prnn_set_grid": (_I, [_H, _I]),
    "prnn_set_team_waves": (_I, [_H, _I]),
    "prnn_set_xcds_per_row": (_I, [_H, _I]),
    "prnn_set_watchdog_us": (_I, [_H, ctypes.c_uint32]),
    "prnn_set_exchange": (_I, [_H, _I]),
    "prnn_set_layout": (_I, [_H, _I]),
    "prnn_set_math": (_I, [_H, _I]),
    "prnn_get_last_plan": (_I, [_H, _P]),
    "prnn_debug_skip_publish": (_I, [_H, _I, _I]),
    "prnn_debug_jitter": (_I, [_H, ctypes.c_uint32, _I]),
    "prnn_set_trace": (_I, [_H, _I]),
    "prnn_get_trace": (_I, [_H, _P, ctypes.c_size_t, ctypes.POINTER(_I), _P]),
    "prnn_status_string": (ctypes.c_char_p, [_I]),
    "prnn_project": (_I, [_H, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P]),
    "prnn_forward_layer_dense": (_I, [_H, _I, _I, _I, _I, _I, _P, _I, _P, _P, _I, _P, _P, _P, _P, _P]),
    "prnn_forward_layer_sparse": (_I, [_H, _I, _I, _I, _I, _I, _I, _P, _I, _P, _P, _P, _I, _P, _P, _P, _P, _P]),
    "prnn_forward_stack_dense": (_I, [_H, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
    "prnn_forward_stack_sparse": (_I, [_H, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P]),
    "prnn_set_stack_mode": (_I, [_H, _I]),
    "prnn_set_launch": (_I, [_H, _I]),
    "prnn_forward_dense_noalloc": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
}


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("layout", ctypes.c_int),
        ("grid", ctypes.c_int),
        ("waves_per_wg", ctypes.c_int),
        ("rows_per_wave", ctypes.c_int),
        ("rmax", ctypes.c_int),
        ("chunks", ctypes.c_int),
        ("lds_bytes", ctypes.c_int),
        ("relay_slice", ctypes.c_int),
        ("first_step", ctypes.c_uint64),
        ("math", ctypes.c_int),
        ("xcds_per_row", ctypes.c_int),
    ]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class PrnnError(RuntimeError):
    def __init__(self, where: str, status: int):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}")


_lib = None


def load_library() -> ctypes.CDLL:
    """Loads libprnn.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m persistent_rnn_fwd_amd.build` "
                "(the HIP library is required; there is no fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(where: str, status: int):
    if status != SUCCESS:
        raise PrnnError(where, status)


def _stream_ptr(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _need(t: torch.Tensor, name: str, dtypes, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class Handle:
    """A library handle (prnn_create) bound to the current GPU."""

    def __init__(self):
        self._lib = load_library()
        h = _H()
        _check("prnn_create", self._lib.prnn_create(ctypes.byref(h)))
        self._h = h
        self.device = torch.device("cuda", torch.cuda.current_device())

    # -- lifetime ---------------------------------------------------------
    def close(self):
        if getattr(self, "_h", None):
            st = self._lib.prnn_destroy(self._h)
            self._h = None
            _check("prnn_destroy", st)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            if getattr(self, "_h", None):
                self._lib.prnn_destroy(self._h)
                self._h = None
        except Exception:
            pass

    # -- options ------------------------------------------------------------
    def set_grid(self, workgroups: int):
        _check("prnn_set_grid", self._lib.prnn_set_grid(self._h, int(workgroups)))

    def set_team_waves(self, waves: int):
        """Waves per team-layout workgroup for later calls: 0 (automatic), 8, 12 or 16."""
        _check("prnn_set_team_waves", self._lib.prnn_set_team_waves(self._h, int(waves)))

    def set_exchange(self, mode: int):
        """EXCHANGE_AUTO, EXCHANGE_DIRECT or EXCHANGE_RELAY for later calls."""
        _check("prnn_set_exchange", self._lib.prnn_set_exchange(self._h, int(mode)))

    def set_layout(self, layout: int):
        """LAYOUT_AUTO, LAYOUT_SPREAD or LAYOUT_TEAM for later calls."""
        _check("prnn_set_layout", self._lib.prnn_set_layout(self._h, int(layout)))

    def set_stack_mode(self, mode: int):
        """STACK_AUTO, STACK_BLOCKED, STACK_FUSED or STACK_LAYERS for later stack calls."""
        _check("prnn_set_stack_mode", self._lib.prnn_set_stack_mode(self._h, mode))

    def set_math(self, mode: int):
        """MATH_AUTO, MATH_EXACT, MATH_SPLIT or MATH_HALF (dense fp16) for later calls."""
        _check("prnn_set_math", self._lib.prnn_set_math(self._h, int(mode)))

    def set_xcds_per_row(self, xcds: int):
        """XCDs per batch row of dense fp16 layers for later calls: 0 (automatic), 1, 2 or 4."""
        _check("prnn_set_xcds_per_row", self._lib.prnn_set_xcds_per_row(self._h, int(xcds)))

    def set_launch(self, kind: int):
        """LAUNCH_COOPERATIVE or LAUNCH_PLAIN dispatch of the persistent kernels for later calls."""
        _check("prnn_set_launch", self._lib.prnn_set_launch(self._h, int(kind)))

    def set_watchdog_us(self, us: int):
        _check("prnn_set_watchdog_us", self._lib.prnn_set_watchdog_us(self._h, int(us)))

    def debug_skip_publish(self, wg: int, step: int):
        _check("prnn_debug_skip_publish", self._lib.prnn_debug_skip_publish(self._h, int(wg), int(step)))

    def debug_jitter(self, seed: int, span: int):
        """Test only: random publish delays of up to ``span`` sleep periods (0: off)."""
        _check("prnn_debug_jitter", self._lib.prnn_debug_jitter(self._h, int(seed) & 0xFFFFFFFF, int(span)))

    def last_plan(self) -> dict:
        info = PlanInfo()
        _check("prnn_get_last_plan", self._lib.prnn_get_last_plan(self._h, ctypes.byref(info)))
        return info.as_dict()

    def synchronize(self, stream: Optional[torch.cuda.Stream] = None):
        _check("prnn_synchronize", self._lib.prnn_synchronize(self._h, _stream_ptr(stream)))

    def set_trace(self, enable: bool):
        _check("prnn_set_trace", self._lib.prnn_set_trace(self._h, 1 if enable else 0))

    def get_trace(self, stream: Optional[torch.cuda.Stream] = None):
        """Phase records of the last traced call: uint64 array [grid * waves_per_wg, 8]
        (stage, barrier, compute, reduce, epilogue cycles; loop cycles; loop
        ticks of the 100 MHz clock; steps), one row per wave."""
        import numpy as np
        records = ctypes.c_int(0)
        st = self._lib.prnn_get_trace(self._h, None, 0, ctypes.byref(records), _stream_ptr(stream))
        if records.value <= 0:
            _check("prnn_get_trace", st)
        buf = np.zeros((records.value, TRACE_WORDS), dtype=np.uint64)
        _check("prnn_get_trace", self._lib.prnn_get_trace(self._h, buf.ctypes.data, buf.size, ctypes.byref(records),
                                                          _stream_ptr(stream)))
        return buf

    # -- the recurrence -----------------------------------------------------
    def forward_dense(self, W: torch.Tensor, X: torch.Tensor, h0: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """H[t] = relu(X[t] + H[t-1] W^T); W [N, N] fp32/fp16, X [T, B, N] fp32."""
        T, B, N = X.shape
        _need(W, "W", (torch.float32, torch.float16), (N, N))
        _need(X, "X", (torch.float32,), (T, B, N))
        if h0 is not None:
            _need(h0, "h0", (torch.float32,), (B, N))
        if out is None:
            out = torch.empty((T, B, N), dtype=torch.float32, device=X.device)
        _need(out, "out", (torch.float32,), (T, B, N))
        wt = DATA_FLOAT if W.dtype == torch.float32 else DATA_HALF
        st = self._lib.prnn_forward_dense(self._h, N, B, T, wt, W.data_ptr(), X.data_ptr(),
                                          h0.data_ptr() if h0 is not None else None, out.data_ptr(),
                                          _stream_ptr(stream))
        _check("prnn_forward_dense", st)
        return out

    def forward_sparse(self, col: torch.Tensor, val: torch.Tensor, X: torch.Tensor,
                       h0: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
        """Row-balanced sparse W: col int16 [N, K], val fp16/fp32 [N, K]."""
        T, B, N = X.shape
        K = col.shape[1] if col.dim() == 2 else -1
        _need(col, "col", (torch.int16,), (N, K))
        _need(val, "val", (torch.float32, torch.float16), (N, K))
        _need(X, "X", (torch.float32,), (T, B, N))
        if h0 is not None:
            _need(h0, "h0", (torch.float32,), (B, N))
        if out is None:
            out = torch.empty((T, B, N), dtype=torch.float32, device=X.device)
        _need(out, "out", (torch.float32,), (T, B, N))
        vt = DATA_FLOAT if val.dtype == torch.float32 else DATA_HALF
        st = self._lib.prnn_forward_sparse(self._h, N, B, T, K, col.data_ptr(), vt, val.data_ptr(),
                                           X.data_ptr(), h0.data_ptr() if h0 is not None else None,
                                           out.data_ptr(), _stream_ptr(stream))
        _check("prnn_forward_sparse", st)
        return out

    def forward_sparse_rows(self, col: torch.Tensor, val: torch.Tensor, row_len: torch.Tensor, X: torch.Tensor,
                            h0: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
        """Sparse W with rows of unequal length: col int16 [N, K], val fp16 [N, K],
        row_len int32 [N] (row i is its first row_len[i] pairs)."""
        T, B, N = X.shape
        K = col.shape[1] if col.dim() == 2 else -1
        _need(col, "col", (torch.int16,), (N, K))
        _need(val, "val", (torch.float32, torch.float16), (N, K))
        _need(row_len, "row_len", (torch.int32,), (N,))
        _need(X, "X", (torch.float32,), (T, B, N))
        if h0 is not None:
            _need(h0, "h0", (torch.float32,), (B, N))
        if out is None:
            out = torch.empty((T, B, N), dtype=torch.float32, device=X.device)
        _need(out, "out", (torch.float32,), (T, B, N))
        vt = DATA_FLOAT if val.dtype == torch.float32 else DATA_HALF
        st = self._lib.prnn_forward_sparse_rows(self._h, N, B, T, K, col.data_ptr(), vt, val.data_ptr(),
                                                row_len.data_ptr(), X.data_ptr(),
                                                h0.data_ptr() if h0 is not None else None, out.data_ptr(),
                                                _stream_ptr(stream))
        _check("prnn_forward_sparse_rows", st)
        return out

    # -- the input projection and whole layers ------------------------------
    def project(self, U: torch.Tensor, x: torch.Tensor, bias: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """X[..., n] = bias[n] + sum_i U[n, i] x[..., i]; U fp16 [N, I], x fp32/fp16 [..., I]."""
        N, I = U.shape
        lead = tuple(x.shape[:-1])
        M = 1
        for d in lead:
            M *= int(d)
        _need(U, "U", (torch.float16,), (N, I))
        _need(x, "x", (torch.float32, torch.float16), lead + (I,))
        if bias is not None:
            _need(bias, "bias", (torch.float32,), (N,))
        if out is None:
            out = torch.empty(lead + (N,), dtype=torch.float32, device=x.device)
        _need(out, "out", (torch.float32,), lead + (N,))
        xt = DATA_FLOAT if x.dtype == torch.float32 else DATA_HALF
        st = self._lib.prnn_project(self._h, M, N, I, xt, x.data_ptr(), DATA_HALF, U.data_ptr(),
                                    bias.data_ptr() if bias is not None else None, out.data_ptr(),
                                    _stream_ptr(stream))
        _check("prnn_project", st)
        return out

    def _layer_buffers(self, x, U, bias, h0, N, workspace, out):
        T, B, I = x.shape
        _need(U, "U", (torch.float16,), (N, I))
        _need(x, "x", (torch.float32, torch.float16), (T, B, I))
        if bias is not None:
            _need(bias, "bias", (torch.float32,), (N,))
        if h0 is not None:
            _need(h0, "h0", (torch.float32,), (B, N))
        if workspace is None:
            workspace = torch.empty((T, B, N), dtype=torch.float32, device=x.device)
        _need(workspace, "workspace", (torch.float32,), (T, B, N))
        if out is None:
            out = torch.empty((T, B, N), dtype=torch.float32, device=x.device)
        _need(out, "out", (torch.float32,), (T, B, N))
        return T, B, I, workspace, out

    def forward_layer_dense(self, U: torch.Tensor, bias: Optional[torch.Tensor], W: torch.Tensor, x: torch.Tensor,
                            h0: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """One dense layer: X = x U^T + bias into `workspace` [T, B, N], then the recurrence."""
        N = W.shape[0]
        _need(W, "W", (torch.float32, torch.float16), (N, N))
        T, B, I, workspace, out = self._layer_buffers(x, U, bias, h0, N, workspace, out)
        xt = DATA_FLOAT if x.dtype == torch.float32 else DATA_HALF
        wt = DATA_FLOAT if W.dtype == torch.float32 else DATA_HALF
        st = self._lib.prnn_forward_layer_dense(
            self._h, N, I, B, T, xt, x.data_ptr(), DATA_HALF, U.data_ptr(),
            bias.data_ptr() if bias is not None else None, wt, W.data_ptr(),
            h0.data_ptr() if h0 is not None else None, workspace.data_ptr(), out.data_ptr(), _stream_ptr(stream))
        _check("prnn_forward_layer_dense", st)
        return out

    def forward_layer_sparse(self, U: torch.Tensor, bias: Optional[torch.Tensor], col: torch.Tensor,
                             val: torch.Tensor, x: torch.Tensor, h0: Optional[torch.Tensor] = None,
                             out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                             stream=None) -> torch.Tensor:
        """One row-balanced sparse layer: the projection, then the sparse recurrence."""
        N = col.shape[0]
        K = col.shape[1] if col.dim() == 2 else -1
        _need(col, "col", (torch.int16,), (N, K))
        _need(val, "val", (torch.float32, torch.float16), (N, K))
        T, B, I, workspace, out = self._layer_buffers(x, U, bias, h0, N, workspace, out)
        xt = DATA_FLOAT if x.dtype == torch.float32 else DATA_HALF
        vt = DATA_FLOAT if val.dtype == torch.float32 else DATA_HALF
        st = self._lib.prnn_forward_layer_sparse(
            self._h, N, I, B, T, K, xt, x.data_ptr(), DATA_HALF, U.data_ptr(),
            bias.data_ptr() if bias is not None else None, col.data_ptr(), vt, val.data_ptr(),
            h0.data_ptr() if h0 is not None else None, workspace.data_ptr(), out.data_ptr(), _stream_ptr(stream))
        _check("prnn_forward_layer_sparse", st)
        return out

    def forward_stack_dense(self, layers, x: torch.Tensor, h0s=None, outs=None,
                            workspace: Optional[torch.Tensor] = None, stream=None):
        """A stack of dense fp16 layers as one wavefront.  layers: list of dicts
        with U (fp16 [N, I] for the first, [N, N] after), bias (fp32 [N] or
        None) and W (fp16 [N, N]); x [T, B, I]; h0s: None or one [B, N] (or
        None) per layer.  Returns the list of every layer's H [T, B, N]."""
        L = len(layers)
        T, B, I = x.shape
        N = layers[0]["W"].shape[0]
        _need(x, "x", (torch.float32, torch.float16), (T, B, I))
        for l, ly in enumerate(layers):
            _need(ly["U"], f"layers[{l}].U", (torch.float16,), (N, I if l == 0 else N))
            _need(ly["W"], f"layers[{l}].W", (torch.float16,), (N, N))
            if ly.get("bias") is not None:
                _need(ly["bias"], f"layers[{l}].bias", (torch.float32,), (N,))
            if h0s is not None and h0s[l] is not None:
                _need(h0s[l], f"h0s[{l}]", (torch.float32,), (B, N))
        if workspace is None:
            workspace = torch.empty((T, B, N), dtype=torch.float32, device=x.device)
        _need(workspace, "workspace", (torch.float32,), (T, B, N))
        if outs is None:
            outs = [torch.empty((T, B, N), dtype=torch.float32, device=x.device) for _ in range(L)]
        for l, o in enumerate(outs):
            _need(o, f"outs[{l}]", (torch.float32,), (T, B, N))
        ptrs = lambda ts: (ctypes.c_void_p * L)(*[(t.data_ptr() if t is not None else None) for t in ts])
        Up, Wp, Hp = ptrs([ly["U"] for ly in layers]), ptrs([ly["W"] for ly in layers]), ptrs(outs)
        bp = ptrs([ly.get("bias") for ly in layers])
        hp = ptrs(h0s) if h0s is not None else None
        xt = DATA_FLOAT if x.dtype == torch.float32 else DATA_HALF
        st = self._lib.prnn_forward_stack_dense(self._h, L, N, I, B, T, xt, x.data_ptr(), Up, bp, Wp, hp,
                                                workspace.data_ptr(), Hp, _stream_ptr(stream))
        _check("prnn_forward_stack_dense", st)
        return outs

    def forward_stack_sparse(self, layers, x: torch.Tensor, h0s=None, outs=None,
                             workspace: Optional[torch.Tensor] = None, stream=None):
        """A stack of row-balanced sparse layers, one after another.  layers: list
        of dicts with U (fp16 [N, I] for the first, [N, N] after), bias (fp32
        [N] or None), col (int16 [N, K]) and val (fp16 or fp32 [N, K], one dtype
        for all layers); x [T, B, I]; h0s: None or one [B, N] (or None) per
        layer.  Returns the list of every layer's H [T, B, N]."""
        L = len(layers)
        T, B, I = x.shape
        N, K = layers[0]["col"].shape
        vdt = layers[0]["val"].dtype
        _need(x, "x", (torch.float32, torch.float16), (T, B, I))
        for l, ly in enumerate(layers):
            _need(ly["U"], f"layers[{l}].U", (torch.float16,), (N, I if l == 0 else N))
            _need(ly["col"], f"layers[{l}].col", (torch.int16,), (N, K))
            _need(ly["val"], f"layers[{l}].val", (vdt,), (N, K))
            if ly.get("bias") is not None:
                _need(ly["bias"], f"layers[{l}].bias", (torch.float32,), (N,))
            if h0s is not None and h0s[l] is not None:
                _need(h0s[l], f"h0s[{l}]", (torch.float32,), (B, N))
        if workspace is None:
            workspace = torch.empty((T, B, N), dtype=torch.float32, device=x.device)
        _need(workspace, "workspace", (torch.float32,), (T, B, N))
        if outs is None:
            outs = [torch.empty((T, B, N), dtype=torch.float32, device=x.device) for _ in range(L)]
        for l, o in enumerate(outs):
            _need(o, f"outs[{l}]", (torch.float32,), (T, B, N))
        ptrs = lambda ts: (ctypes.c_void_p * L)(*[(t.data_ptr() if t is not None else None) for t in ts])
        Up, Cp, Vp, Hp = (ptrs([ly["U"] for ly in layers]), ptrs([ly["col"] for ly in layers]),
                          ptrs([ly["val"] for ly in layers]), ptrs(outs))
        bp = ptrs([ly.get("bias") for ly in layers])
        hp = ptrs(h0s) if h0s is not None else None
        xt = DATA_FLOAT if x.dtype == torch.float32 else DATA_HALF
        vt = DATA_FLOAT if vdt == torch.float32 else DATA_HALF
        st = self._lib.prnn_forward_stack_sparse(self._h, L, N, I, B, T, K, xt, x.data_ptr(), Up, bp, Cp, vt, Vp, hp,
                                                 workspace.data_ptr(), Hp, _stream_ptr(stream))
        _check("prnn_forward_stack_sparse", st)
        return outs

    def sync_floor(self, N: int, B: int, T: int, out: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
        """The exchange/step protocol of a dense call without arithmetic."""
        if out is None:
            out = torch.empty((T, B, N), dtype=torch.float32, device=self.device)
        _need(out, "out", (torch.float32,), (T, B, N))
        _check("prnn_sync_floor", self._lib.prnn_sync_floor(self._h, N, B, T, out.data_ptr(), _stream_ptr(stream)))
        return out


_default_handles = {}


@atexit.register
def _close_default_handles():
    """Destroys the module's default handles at interpreter exit, before the
    HIP runtime and torch tear down (handlers run in reverse order of
    registration, and torch registers its own when it is imported, before
    this module's)."""
    while _default_handles:
        _, h = _default_handles.popitem()
        try:
            h.close()
        except Exception:
            pass


def default_handle() -> Handle:
    dev = torch.cuda.current_device()
    h = _default_handles.get(dev)
    if h is None:
        h = _default_handles[dev] = Handle()
    return h


def forward_dense(W, X, h0=None, out=None, stream=None):
    return default_handle().forward_dense(W, X, h0, out, stream)


def forward_sparse(col, val, X, h0=None, out=None, stream=None):
    return default_handle().forward_sparse(col, val, X, h0, out, stream)


NOALLOC_MAX_N = 2560  # PRNN_NOALLOC_MAX_N


def forward_dense_noalloc(W: torch.Tensor, X: torch.Tensor, h0: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """prnn_forward_dense_noalloc: the dense recurrence without a handle, on the
    library's fixed device array (nothing allocated by the library).  status:
    None or a one-element int32/uint32 device tensor, 0 after a good run."""
    lib = load_library()
    T, B, N = X.shape
    _need(W, "W", (torch.float32, torch.float16), (N, N))
    _need(X, "X", (torch.float32,), (T, B, N))
    if h0 is not None:
        _need(h0, "h0", (torch.float32,), (B, N))
    if out is None:
        out = torch.empty((T, B, N), dtype=torch.float32, device=X.device)
    _need(out, "out", (torch.float32,), (T, B, N))
    if status is not None:
        _need(status, "status", (torch.int32, torch.uint32), (1,))
    wt = DATA_FLOAT if W.dtype == torch.float32 else DATA_HALF
    st = lib.prnn_forward_dense_noalloc(N, B, T, wt, W.data_ptr(), X.data_ptr(),
                                        h0.data_ptr() if h0 is not None else None, out.data_ptr(),
                                        status.data_ptr() if status is not None else None, _stream_ptr(stream))
    _check("prnn_forward_dense_noalloc", st)
    return out
