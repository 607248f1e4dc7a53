#!/usr/bin/env python3
"""Benchmark of the persistent basic-RNN forward on one MI355X.

Workload (one bench step = one pass of the whole recurrence for each weight
format of the headline layer): N = 1792 neurons, batch B = 4, T = 256
timesteps,
  * one call with dense fp16 W        (nnz = N^2),
  * one call with 10 % row-balanced sparse fp16 W (K = 179 nonzeros per row),
both with fp32 X / H and fp32 accumulation, inputs resident in HBM.

Prints ONE JSON line:
  value        RNN timesteps/s over the step (2 * T timesteps per step)
  roofline     the dominant kernel's algorithmic flops per launch over its
               mean launch time (HIP events on the launch stream) against the
               fp32 vector peak; traffic from a committed counter run if it
               still matches the kernel sources, else null
  cpu_baseline the fp64 oracle on the host, on a bounded sample of the same
               workload (timesteps/s, threads it used)
  detail       per-format timesteps/s, GFLOP/s, per-step time by the slope
               between T = 256 and T = 128, the measured sync floor per step,
               equivalent weight bytes/s, the max error ratio vs the oracle,
               p10/p50/p90 of the timed launches and the dense/sparse ratio
  baselines    the same recurrence as a per-step library loop on the GPU
               (hipBLAS fp32 GEMM + add + ReLU per step, eager and captured in
               a HIP graph; a per-step CSR SpMM for the sparse layer) and as a
               torch-CPU fp32 loop on the host's threads, with the speedups of
               the persistent kernels over them (context, not the target)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP32_VECTOR_PEAK = 157.3e12   # MI355X published fp32 vector peak, FLOP/s
HBM_PEAK = 8.0e12             # MI355X HBM3E, bytes/s
COUNTER_FILE = os.path.join(ROOT, "profiles", "counters_rnn_fwd_n1792.json")
KERNEL_SOURCES = ["device_common.h", "kernels.h", "dense_kernel.h", "sparse_kernel.h", "team_kernel.h", "team_mfma.h",
                  "dense_f16.hip", "dense_f32.hip", "sparse_f16.hip", "sparse_f32.hip", "team_f16.hip", "team_f32.hip",
                  "team_half.hip", "team_split.hip", "team_rows.hip", "team_pinned.h", "project_tile.h", "project.hip",
                  "stack.hip", "noalloc.hip", "host_internal.h"]


def code_only(text: str) -> str:
    """The source without its comments and with whitespace collapsed: what
    the compiler sees, so that a comment edit keeps the counters valid."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "persistent_rnn_fwd_amd", "csrc", f)) as fh:
            h.update(code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the host oracle leg (profiling runs)")
    ap.add_argument("--no-check", action="store_true", help="skip the oracle check of the GPU output")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the host oracle sample")
    ap.add_argument("--only-timed", action="store_true",
                    help="run only warmup + the timed region (every launch is a T=256 call; for profiles)")
    ap.add_argument("--no-baselines", action="store_true", help="skip the library and torch-CPU loop baselines")
    ap.add_argument("--no-layers", action="store_true", help="skip the whole-layer (projection + recurrence) table")
    ap.add_argument("--profile-layers", action="store_true",
                    help="with --only-timed: also run 5 half-h dense calls, 3 calls of each N=5760 sparse layer, 5 input "
                         "projections and one layer call (N=1792) and one "
                         "2-layer stack wavefront (N=1152), T=256, after the timed loop, for profilers")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-config table (every workload, not timed "
                    "in the headline step)")
    ap.add_argument("--no-config-loops", action="store_true", help="skip the per-config library loop baselines")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one plain copy kernel of this many MiB first (counter calibration)")
    return ap.parse_args()


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return " ".join(line.split(":", 1)[1].split())
    except OSError:
        pass
    return "unknown CPU"


def percentiles(xs):
    import numpy as np
    p10, p50, p90 = np.percentile(np.asarray(xs, dtype=np.float64), [10, 50, 90])
    return {"p10": round(float(p10), 4), "p50": round(float(p50), 4), "p90": round(float(p90), 4)}


def gpu_clock_report():
    """Shader clock as amd-smi reports it after the run (a child process; text kept short)."""
    import subprocess
    for cmd in (["amd-smi", "metric", "--clock", "--json"], ["rocm-smi", "--showclocks", "--json"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
        except (OSError, subprocess.SubprocessError) as e:
            last = f"{cmd[0]}: {type(e).__name__}"
            continue
        text = (r.stdout or "") + (r.stderr or "")
        try:
            data = json.loads(r.stdout)
        except ValueError:
            last = f"{cmd[0]}: " + " ".join(text.split())[:200]
            continue
        found = {}

        def walk(o, path):
            if isinstance(o, dict):
                for k, v in o.items():
                    walk(v, path + [str(k)])
            elif isinstance(o, list):
                for i, v in enumerate(o):
                    walk(v, path + [str(i)])
            else:
                key = "/".join(path).lower()
                if ("gfx" in key or "sclk" in key) and len(found) < 12:
                    found["/".join(path)] = o
        walk(data, [])
        return {"tool": cmd[0], "values": found}
    return {"tool": None, "error": last}


def library_baselines(torch, dev, host, wd, ws, T, persistent_ms):
    """The recurrence as a per-step library loop on the GPU, and as a torch-CPU
    loop: h = relu(X[t] + h W^T) one step at a time (the plain formulation the
    persistent kernels replace).  fp32 throughout (the fp16 weights widened
    exactly), inputs already on the device.  Returns timesteps/s per variant and
    the persistent kernels' speedups over them."""
    import warnings
    import numpy as np
    warnings.filterwarnings("ignore", message="Sparse CSR tensor support")
    stream = torch.cuda.current_stream()
    N, B = wd.N, wd.B
    W32 = torch.from_numpy(host[wd.name]["W"].astype(np.float32)).to(dev)
    Wt = W32.t().contiguous()
    X = torch.from_numpy(host[wd.name]["X"]).to(dev)
    h0 = torch.zeros((B, N), dtype=torch.float32, device=dev)
    Hb = torch.empty((T, B, N), dtype=torch.float32, device=dev)

    def gemm_loop(Wt_, X_, H_):
        h = h0
        for t in range(T):
            torch.addmm(X_[t], h, Wt_, out=H_[t])
            H_[t].relu_()
            h = H_[t]

    def time_ms(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in es:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in es]))

    out = {}
    eager_ms = time_ms(lambda: gemm_loop(Wt, X, Hb))
    out["hipblas_eager"] = {"timesteps_per_s": round(T / (eager_ms * 1e-3), 1), "ms_per_call": round(eager_ms, 4),
                            "what": "per step: torch.addmm (hipBLAS fp32 GEMM, [4,1792]x[1792,1792]) + relu_, eager"}
    ref = Hb.clone()

    # the same loop captured once in a HIP graph; every replay is checked
    # against the eager result, with eager work and syncs between replays
    try:
        Hg = torch.empty_like(Hb)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            gemm_loop(Wt, X, Hg)  # warm the library outside the capture
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            gemm_loop(Wt, X, Hg)
        bad = 0
        for _ in range(3):
            Hg.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            bad += int(not torch.equal(Hg, ref))
            gemm_loop(Wt, X, Hb)   # eager work between the replays
            torch.cuda.synchronize()
        if bad:
            out["hipblas_graph"] = {"timesteps_per_s": None, "error": f"{bad} of 3 replays differ from eager"}
        else:
            g_ms = time_ms(graph.replay)
            out["hipblas_graph"] = {"timesteps_per_s": round(T / (g_ms * 1e-3), 1), "ms_per_call": round(g_ms, 4),
                                    "what": "the eager loop captured in one HIP graph, replayed"}
        del graph
    except Exception as e:  # the baseline is context: report, do not fail the bench
        out["hipblas_graph"] = {"timesteps_per_s": None, "error": f"{type(e).__name__}: {str(e)[:160]}"}

    # sparse layer as a per-step CSR SpMM (fp32 values)
    try:
        d = host[ws.name]
        K = ws.K
        crow = torch.arange(0, (N + 1) * K, K, dtype=torch.int64, device=dev)[: N + 1]
        col = torch.from_numpy(d["col"].astype(np.int64).reshape(-1)).to(dev)
        val = torch.from_numpy(d["val"].astype(np.float32).reshape(-1)).to(dev)
        Wcsr = torch.sparse_csr_tensor(crow, col, val, size=(N, N))
        Xs = torch.from_numpy(d["X"]).to(dev)
        Hs = torch.empty((T, B, N), dtype=torch.float32, device=dev)

        def spmm_loop():
            h = h0
            for t in range(T):
                y = torch.sparse.mm(Wcsr, h.t().contiguous())   # [N, B]
                torch.add(Xs[t], y.t(), out=Hs[t])
                Hs[t].relu_()
                h = Hs[t]
        s_ms = time_ms(spmm_loop, reps=5)
        out["hipsparse_eager"] = {"timesteps_per_s": round(T / (s_ms * 1e-3), 1), "ms_per_call": round(s_ms, 4),
                                  "what": "per step: torch.sparse.mm (CSR fp32, K=179 per row) + add + relu_, eager"}
    except Exception as e:
        out["hipsparse_eager"] = {"timesteps_per_s": None, "error": f"{type(e).__name__}: {str(e)[:160]}"}

    # torch-CPU fp32 loop on the host threads, bounded sample
    Wc = torch.from_numpy(host[wd.name]["W"].astype(np.float32)).t().contiguous()
    Xc = torch.from_numpy(host[wd.name]["X"])
    h = torch.zeros((B, N), dtype=torch.float32)
    steps, a = 0, time.perf_counter()
    while time.perf_counter() - a < 3.0 and steps < 100 * T:
        for t in range(T):
            h = torch.relu(torch.addmm(Xc[t], h, Wc))
        steps += T
    spent = time.perf_counter() - a
    out["cpu_torch_loop"] = {"timesteps_per_s": round(steps / spent, 1), "threads": torch.get_num_threads(),
                             "what": f"torch CPU fp32 addmm + relu per step, dense N=1792 B=4, {steps} steps"}

    def speedup(persistent, base):
        v = out[base].get("timesteps_per_s")
        return round(T / (persistent * 1e-3) / v, 2) if v else None
    # persistent_ms: {"dense": ms per call, "sparse10": ms per call}
    out["speedups"] = {
        "dense_persistent_vs_hipblas_eager": speedup(persistent_ms["dense"], "hipblas_eager"),
        "dense_persistent_vs_hipblas_graph": speedup(persistent_ms["dense"], "hipblas_graph"),
        "sparse10_persistent_vs_hipblas_eager": speedup(persistent_ms["sparse10"], "hipblas_eager"),
        "sparse10_persistent_vs_hipblas_graph": speedup(persistent_ms["sparse10"], "hipblas_graph"),
        "sparse10_persistent_vs_hipsparse_eager": speedup(persistent_ms["sparse10"], "hipsparse_eager"),
    }
    return out


def config_library_loops(torch, dev, w, d, persistent_ms, reps=5):
    """The workload as per-step library loops on the GPU, fp32 throughout:
    dense GEMM (hipBLAS through torch.addmm, with the sparse matrix's dense
    equivalent for sparse layers), eager and captured in one HIP graph, and
    for sparse layers a CSR SpMM (torch.sparse.mm) loop.  Returns timesteps/s
    per loop and the persistent kernel's speedup over each (the pages compare
    the sparse persistent kernel with dense and sparse GEMM loops)."""
    import warnings
    import numpy as np
    warnings.filterwarnings("ignore", message="Sparse CSR tensor support")
    stream = torch.cuda.current_stream()
    T, B, N = w.T, w.B, w.N
    if w.kind == "dense":
        W32 = d["W"].astype(np.float32)
    else:
        W32 = np.zeros((N, N), np.float32)
        np.add.at(W32, (np.repeat(np.arange(N), d["col"].shape[1]), d["col"].astype(np.int64).ravel()),
                  d["val"].astype(np.float32).ravel())
    Wt = torch.from_numpy(W32.T.copy()).to(dev)
    X = torch.from_numpy(d["X"]).to(dev)
    h0 = torch.from_numpy(d["h0"]).to(dev)
    Hb = torch.empty((T, B, N), dtype=torch.float32, device=dev)

    def gemm_loop(H_):
        h = h0
        for t in range(T):
            torch.addmm(X[t], h, Wt, out=H_[t])
            H_[t].relu_()
            h = H_[t]

    def time_ms(fn):
        fn()
        torch.cuda.synchronize()
        es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in es:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in es]))

    out = {}
    per_s = lambda ms: round(T / (ms * 1e-3), 1)
    mine = per_s(persistent_ms)
    g_ms = time_ms(lambda: gemm_loop(Hb))
    out["dense_gemm_eager"] = per_s(g_ms)
    ref = Hb.clone()
    try:
        Hg = torch.empty_like(Hb)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            gemm_loop(Hg)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            gemm_loop(Hg)
        bad = 0
        for _ in range(2):
            Hg.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            bad += int(not torch.equal(Hg, ref))
            gemm_loop(Hb)
            torch.cuda.synchronize()
        out["dense_gemm_graph"] = None if bad else per_s(time_ms(graph.replay))
        del graph
    except Exception as e:  # context only: report, do not fail the bench
        out["dense_gemm_graph"] = None
        out["dense_gemm_graph_error"] = f"{type(e).__name__}: {str(e)[:120]}"
    if w.kind == "sparse":
        try:
            K = d["col"].shape[1]
            crow = torch.arange(0, (N + 1) * K, K, dtype=torch.int64, device=dev)[: N + 1]
            colt = torch.from_numpy(d["col"].astype(np.int64).reshape(-1)).to(dev)
            valt = torch.from_numpy(d["val"].astype(np.float32).reshape(-1)).to(dev)
            Wcsr = torch.sparse_csr_tensor(crow, colt, valt, size=(N, N))

            def spmm_loop():
                h = h0
                for t in range(T):
                    y = torch.sparse.mm(Wcsr, h.t().contiguous())
                    torch.add(X[t], y.t(), out=Hb[t])
                    Hb[t].relu_()
                    h = Hb[t]
            out["sparse_gemm_eager"] = per_s(time_ms(spmm_loop))
        except Exception as e:
            out["sparse_gemm_eager"] = None
            out["sparse_gemm_error"] = f"{type(e).__name__}: {str(e)[:120]}"
    out["speedup"] = {k: (round(mine / v, 2) if v else None) for k, v in list(out.items())
                      if k in ("dense_gemm_eager", "dense_gemm_graph", "sparse_gemm_eager")}
    del Wt, X, h0, Hb, ref
    return out


def per_config_table(torch, dev, Handle, WORKLOADS, generate, timed, no_check=False, loops=True):
    """Per workload: timesteps/s of a full call, per-step time by the slope
    between T and T/2, the sync floor at the same N, B, T, and the error ratio
    of the timed output against the oracle."""
    import numpy as np
    from persistent_rnn_fwd_amd import PrnnError, binding as _b
    rows = {}
    h = Handle()
    # every workload in the default math, then the dense fp16 layers again with
    # h_{t-1} staged as fp16 (the opt-in half-h math), and the layers of
    # unbalanced rows again as rows of unequal length (prnn_forward_sparse_rows)
    cases = [(name, w, _b.MATH_AUTO, False) for name, w in WORKLOADS.items()]
    cases += [(name + "_half_h", w, _b.MATH_HALF, False) for name, w in WORKLOADS.items()
              if w.kind == "dense" and w.w_dtype == "f16"]
    cases += [(name + "_rows", w, _b.MATH_AUTO, True) for name, w in WORKLOADS.items() if w.rows == "magnitude"]
    for name, w, math, ragged in cases:
        h.set_math(math)
        d = generate(w)
        g = {k: torch.from_numpy(v).to(dev) for k, v in d.items()}
        T, B, N = w.T, w.B, w.N
        o = torch.empty((T, B, N), dtype=torch.float32, device=dev)

        def call(t=T):
            if w.kind == "dense":
                h.forward_dense(g["W"], g["X"][:t], g["h0"], out=o[:t])
            elif ragged:
                h.forward_sparse_rows(g["col"], g["val"], g["row_len"], g["X"][:t], g["h0"], out=o[:t])
            else:
                h.forward_sparse(g["col"], g["val"], g["X"][:t], g["h0"], out=o[:t])
        try:
            full, half = timed(call, other=lambda: call(T // 2))
        except PrnnError as e:
            if e.status != _b.NOT_SUPPORTED:
                raise
            # the unbalanced 25 % layer's rows (up to 1010 pairs) do not fit
            # the rows-of-unequal-length instances
            rows[name] = {"N": N, "K": w.K, "T": T, "w": w.w_dtype, "not_supported": True}
            del g, o
            continue
        step_us = (full - half) * 1e3 / (T - T // 2)
        h.synchronize()
        plan = {k: v for k, v in h.last_plan().items() if k != "first_step"}
        fo = torch.empty((T, B, N), dtype=torch.float32, device=dev)
        # the floor in the layer's own plan: same layout, waves per workgroup
        # and XCDs per batch row
        if plan["layout"] == _b.LAYOUT_TEAM:
            h.set_team_waves(plan["waves_per_wg"])
            h.set_xcds_per_row(plan["xcds_per_row"])
        f_full, f_half = timed(lambda: h.sync_floor(N, B, T, out=fo),
                               other=lambda: h.sync_floor(N, B, T // 2, out=fo[: T // 2]))
        h.set_team_waves(0)
        h.set_xcds_per_row(0)
        floor_us = (f_full - f_half) * 1e3 / (T - T // 2)
        err = None
        if not no_check:
            import oracle
            call()
            h.synchronize()
            ref = (oracle.forward_dense(d["W"], d["X"], d["h0"]) if w.kind == "dense"
                   else oracle.forward_sparse_rows(d["col"], d["val"], d["row_len"], d["X"], d["h0"]) if ragged
                   else oracle.forward_sparse(d["col"], d["val"], d["X"], d["h0"]))
            tol = oracle.TOL_F32 if w.w_dtype == "f32" else oracle.TOL_F16
            err = round(float(oracle.tolerance_ratio(o.cpu().numpy(), ref, tol)), 5)
        rows[name] = {
            "N": N, "K": w.K if w.kind == "sparse" else N, "T": T, "w": w.w_dtype,
            "timesteps_per_s": round(T / (full * 1e-3), 1),
            "us_per_step_slope": round(step_us, 3),
            "floor_us_per_step": round(floor_us, 3),
            "vs_floor": round(step_us / floor_us, 3) if floor_us > 0 else None,
            "gflop_per_s": round(w.flop_per_step * T / (full * 1e-3) / 1e9, 2),
            "pct_fp32_vector_peak": round(100 * w.flop_per_step * T / (full * 1e-3) / FP32_VECTOR_PEAK, 3),
            # the bytes a per-step re-read of W would move, per second, against 8 TB/s of HBM
            "equiv_weight_tb_per_s": round(w.weight_bytes * T / (full * 1e-3) / 1e12, 3),
            "equiv_weight_frac_of_hbm": round(w.weight_bytes * T / (full * 1e-3) / 8e12, 3),
            "max_err_ratio": err,
            "plan": plan,
        }
        del g, o, fo
    h.set_math(_b.MATH_AUTO)
    h.close()
    # the library loops after every persistent measurement: they draw more
    # power, and a layer timed right after one ran measurably slower
    if loops:
        for name, w, math, ragged in cases:
            row = rows[name]
            if name.endswith(("_half_h", "_rows")) or row.get("not_supported"):
                continue
            full_ms = w.T / row["timesteps_per_s"] * 1e3
            row["library_loops_timesteps_per_s"] = config_library_loops(torch, dev, w, generate(w), full_ms)
    return rows


MFMA_F16_PEAK = 2.5e15  # MI355X dense fp16 matrix peak, flop/s


def layer_table(torch, dev, Handle, timed, no_check=False):
    """Whole layers (input projection + recurrence) at the layer sizes: the
    projection's time and its throughput against the fp16 matrix peak
    (algorithmic flops 2 M N I; fp32 x issues twice the products, hi and lo),
    the layer's timesteps/s, and the error ratios against the oracle."""
    import numpy as np
    from persistent_rnn_fwd_amd.inputs import LAYER_WORKLOADS, WORKLOADS, generate_layer
    rows = {}
    h = Handle()
    for name, (base, I) in LAYER_WORKLOADS.items():
        w = WORKLOADS[base]
        d = generate_layer(w, I)
        g = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in d.items()}
        T, B, N = w.T, w.B, w.N
        Xw = torch.empty((T, B, N), dtype=torch.float32, device=dev)
        H = torch.empty((T, B, N), dtype=torch.float32, device=dev)
        proj_ms = timed(lambda: h.project(g["U"], g["x"], g["bias"], out=Xw))
        if w.kind == "dense":
            run = lambda: h.forward_layer_dense(g["U"], g["bias"], g["W"], g["x"], g["h0"], out=H, workspace=Xw)
        else:
            run = lambda: h.forward_layer_sparse(g["U"], g["bias"], g["col"], g["val"], g["x"], g["h0"], out=H,
                                                 workspace=Xw)
        layer_ms = timed(run)
        flop = 2.0 * T * B * N * I
        row = {
            "N": N, "I": I, "T": T, "B": B, "kind": w.kind,
            "projection_us": round(proj_ms * 1e3, 2),
            "projection_tflops": round(flop / (proj_ms * 1e-3) / 1e12, 1),
            "projection_frac_of_fp16_mfma_peak": round(flop / (proj_ms * 1e-3) / MFMA_F16_PEAK, 4),
            "layer_us": round(layer_ms * 1e3, 1),
            "layer_timesteps_per_s": round(T / (layer_ms * 1e-3), 1),
            "projection_share_of_layer": round(proj_ms / layer_ms, 3),
        }
        if not no_check:
            import oracle
            run()
            h.synchronize()
            ref = (oracle.forward_layer_dense(d["U"], d["bias"], d["W"], d["x"], d["h0"]) if w.kind == "dense"
                   else oracle.forward_layer_sparse(d["U"], d["bias"], d["col"], d["val"], d["x"], d["h0"]))
            row["layer_max_err_ratio"] = round(float(oracle.tolerance_ratio(H.cpu().numpy(), ref, oracle.TOL_F16)), 6)
            Xref = oracle.project(d["U"], d["x"], d["bias"])
            S = np.abs(d["x"].astype(np.float64)) @ np.abs(d["U"].astype(np.float64)).T + np.abs(d["bias"])
            row["projection_max_err_ratio"] = round(float(np.max(np.abs(Xw.cpu().numpy() - Xref) / (1e-6 * (1 + S)))), 4)
        rows[name] = row
        del g, Xw, H
    h.close()
    return rows


def stack_table(torch, dev, Handle, timed, no_check=False):
    """Two-layer stacks (B = 4, T = 256) through prnn_forward_stack_dense (its
    default, the blocked wavefront) against the same two layers run as two
    layer calls, at N = 1152 and 1792."""
    import numpy as np
    from persistent_rnn_fwd_amd.inputs import WORKLOADS, generate_stack
    rows = {}
    h = Handle()
    for base in ("dense_f16_n1152", "dense_f16_n1792"):
        w = WORKLOADS[base]
        st = generate_stack(w, 2)
        layers = [{k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in ly.items()} for ly in st["layers"]]
        x = torch.from_numpy(st["x"]).to(dev)
        h0s = [torch.from_numpy(v).to(dev) for v in st["h0s"]]
        T, B, N = w.T, w.B, w.N
        outs = [torch.empty((T, B, N), dtype=torch.float32, device=dev) for _ in range(2)]
        ws = torch.empty((T, B, N), dtype=torch.float32, device=dev)
        seq = [torch.empty((T, B, N), dtype=torch.float32, device=dev) for _ in range(2)]
        wave = lambda: h.forward_stack_dense(layers, x, h0s, outs=outs, workspace=ws)

        def sequential():
            h.forward_layer_dense(layers[0]["U"], layers[0]["bias"], layers[0]["W"], x, h0s[0], out=seq[0], workspace=ws)
            h.forward_layer_dense(layers[1]["U"], layers[1]["bias"], layers[1]["W"], seq[0], h0s[1], out=seq[1],
                                  workspace=ws)
        t_wave = timed(wave)
        t_seq = timed(sequential)
        row = {
            "layers": 2, "N": N, "B": B, "T": T,
            "stack_runs_as": "blocked wavefront (blocks of about 64 steps)",
            "wavefront_us": round(t_wave * 1e3, 1),
            "wavefront_timesteps_per_s": round(T / (t_wave * 1e-3), 1),
            "sequential_layers_us": round(t_seq * 1e3, 1),
            "speedup_over_sequential": round(t_seq / t_wave, 3),
        }
        if not no_check:
            import oracle
            wave()
            h.synchronize()
            refs = oracle.forward_stack_dense(st["layers"], st["x"], st["h0s"])
            row["max_err_ratio"] = round(max(float(oracle.tolerance_ratio(o.cpu().numpy(), r, oracle.TOL_F16))
                                             for o, r in zip(outs, refs)), 6)
        rows[f"stack2_{base}"] = row
    h.close()
    return rows


def large_dense_table(torch, dev, Handle, timed, no_check=False):
    """Dense fp16 layers beyond the headline size (T = 256, synthetic W ~
    N(0, 0.8^2/N), X ~ N(0, 1)): per-step slope between T and T/2, the floor of
    the same form, the XCDs per batch row the plan takes (split team layout
    beyond N = 1792), and the error ratio of an 8-step call against the oracle."""
    from persistent_rnn_fwd_amd.inputs import Workload, generate
    rows = {}
    h = Handle()
    T = 256
    for N, B in ((2048, 4), (2560, 4), (3072, 4), (3584, 4), (4096, 2), (5120, 2)):
        w = Workload(f"dense_f16_n{N}_b{B}", "dense", N, B, T, "f16", seed=N + B)
        d = generate(w)
        W = torch.from_numpy(d["W"]).to(dev)
        X = torch.from_numpy(d["X"]).to(dev)
        o = torch.empty_like(X)
        full, half = timed(lambda: h.forward_dense(W, X, out=o), other=lambda: h.forward_dense(W, X[:T // 2], out=o[:T // 2]))
        plan = h.last_plan()
        f_full, f_half = timed(lambda: h.sync_floor(N, B, T, out=o),
                               other=lambda: h.sync_floor(N, B, T // 2, out=o[:T // 2]))
        step = (full - half) / (T // 2) * 1e3
        floor = (f_full - f_half) / (T // 2) * 1e3
        row = {"N": N, "B": B, "T": T, "xcds_per_row": plan["xcds_per_row"], "rows_per_wave": plan["rows_per_wave"],
               "timesteps_per_s": round(T / (full * 1e-3), 1), "us_per_step_slope": round(step, 3),
               "floor_us_per_step": round(floor, 3), "vs_floor": round(step / floor, 3),
               "gflop_per_s": round(2 * B * N * N / (step * 1e-6) / 1e9, 1)}
        if not no_check:
            import oracle
            Hs = h.forward_dense(W, X[:8].contiguous())
            h.synchronize()
            row["max_err_ratio"] = round(float(oracle.tolerance_ratio(
                Hs.cpu().numpy(), oracle.forward_dense(d["W"], d["X"][:8]), oracle.TOL_F16)), 6)
        rows[w.name] = row
        del W, X, o
    h.close()
    return rows


def trace_breakdown(torch, dev, Handle, g, wd, ws, T):
    """Per-phase time per step from one traced call of each headline kernel
    and of the floor (team layout): mean over the waves that serve a batch
    row, and the largest wave mean.  Traced calls run a little slower than
    untraced ones (every phase mark reads the clock)."""
    import numpy as np
    names = ["stage", "barrier", "compute", "reduce", "epilogue"]
    out = {}
    h = Handle()
    h.set_trace(True)
    N, B = wd.N, wd.B
    o = torch.empty((T, B, N), dtype=torch.float32, device=dev)
    runs = {
        wd.name: lambda: h.forward_dense(g[wd.name]["W"], g[wd.name]["X"], g[wd.name]["h0"], out=o),
        ws.name: lambda: h.forward_sparse(g[ws.name]["col"], g[ws.name]["val"], g[ws.name]["X"], g[ws.name]["h0"], out=o),
        "sync_floor": lambda: h.sync_floor(N, B, T, out=o),
        wd.name + "_half_h": lambda: h.forward_dense(g[wd.name]["W"], g[wd.name]["X"], g[wd.name]["h0"], out=o),
    }
    from persistent_rnn_fwd_amd import binding as _b
    for name, fn in runs.items():
        h.set_math(_b.MATH_HALF if name.endswith("_half_h") else _b.MATH_AUTO)
        fn()
        fn()
        rec = h.get_trace().astype(np.float64)
        live = rec[rec[:, 7] == T]
        ghz = float(np.mean(live[:, 5] / (live[:, 6] * 10.0)))
        us = live[:, :6] / (ghz * 1e3) / T
        out[name] = {"clock_ghz": round(ghz, 3), "waves": int(live.shape[0]),
                     "loop_us_per_step": round(float(us[:, 5].mean()), 3)}
        for i, n in enumerate(names):
            out[name][n] = {"mean_us": round(float(us[:, i].mean()), 3), "max_wave_us": round(float(us[:, i].max()), 3)}
    h.set_math(_b.MATH_AUTO)
    h.set_trace(False)
    h.close()
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from persistent_rnn_fwd_amd import Handle
    from persistent_rnn_fwd_amd.inputs import WORKLOADS, generate

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    wd = WORKLOADS["dense_f16_n1792"]
    ws = WORKLOADS["sparse10_f16_n1792"]
    w1 = WORKLOADS["sparse1_f16_n1792"]
    N, B, T = wd.N, wd.B, wd.T
    host = {w.name: generate(w) for w in (wd, ws, w1)}
    g = {name: {k: torch.from_numpy(v).to(dev) for k, v in d.items()} for name, d in host.items()}
    out = {name: torch.empty((T, B, N), dtype=torch.float32, device=dev) for name in host}

    if args.copy_mib > 0:
        # a plain elementwise copy of known size: reads and writes copy_mib MiB
        src = torch.ones(args.copy_mib * 2**18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    h = Handle()
    stream = torch.cuda.current_stream()

    def call(name, t=T):
        d, o = g[name], out[name]
        if "W" in d:
            h.forward_dense(d["W"], d["X"][:t], d["h0"], out=o[:t])
        else:
            h.forward_sparse(d["col"], d["val"], d["X"][:t], d["h0"], out=o[:t])

    # correctness of the timed configuration (not timed)
    err = {}
    if not args.no_check:
        import oracle
        for w in (wd, ws, w1):
            call(w.name)
            h.synchronize()
            d = host[w.name]
            ref = (oracle.forward_dense(d["W"], d["X"], d["h0"]) if w.kind == "dense"
                   else oracle.forward_sparse(d["col"], d["val"], d["X"], d["h0"]))
            err[w.name] = oracle.tolerance_ratio(out[w.name].cpu().numpy(), ref, oracle.TOL_F16)
            if err[w.name] > 1.0:
                print(f"bench.py: {w.name} fails the oracle tolerance (ratio {err[w.name]:.3g})", file=sys.stderr)
                sys.exit(1)

    # warmup
    for _ in range(args.warmup):
        call(wd.name)
        call(ws.name)
    h.synchronize()

    # timed region: K steps, each one dense call and one sparse call, with an
    # event pair around every launch on the launch stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev[k][0].record(stream)
        call(wd.name)
        ev[k][1].record(stream)
        ev[k][2].record(stream)
        call(ws.name)
        ev[k][3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    h.synchronize()
    dense_list = [e[0].elapsed_time(e[1]) for e in ev]
    sparse_list = [e[2].elapsed_time(e[3]) for e in ev]
    dense_ms = float(np.mean(dense_list))
    sparse_ms = float(np.mean(sparse_list))
    ms_per_step = wall * 1e3 / args.steps

    def timed(fn, reps=20, other=None):
        """Median ms of fn over reps calls; with `other`, the two alternate
        call by call and both medians are returned (a slope between them
        then sees no drift of the clock between two blocks of calls)."""
        fns = [fn] if other is None else [fn, other]
        for f in fns:
            f()
        torch.cuda.synchronize()
        es = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
              for _ in fns]
        for r in range(reps):
            for f, ev in zip(fns, es):
                ev[r][0].record(stream)
                f()
                ev[r][1].record(stream)
        torch.cuda.synchronize()
        med = [float(np.median([a.elapsed_time(b) for a, b in ev])) for ev in es]
        return med[0] if other is None else tuple(med)

    detail = {}
    if args.only_timed and args.profile_layers:
        from persistent_rnn_fwd_amd.inputs import generate_layer, generate_stack
        dl = generate_layer(wd, wd.N)
        gl = {k: torch.from_numpy(v).to(dev) for k, v in dl.items()}
        Xw = torch.empty((T, B, N), dtype=torch.float32, device=dev)
        for _ in range(5):
            h.project(gl["U"], gl["x"], gl["bias"], out=Xw)
        h.forward_layer_dense(gl["U"], gl["bias"], gl["W"], gl["x"], gl["h0"], out=out[wd.name], workspace=Xw)
        from persistent_rnn_fwd_amd import binding as _b
        h.set_math(_b.MATH_HALF)     # the dense layer with h staged as fp16
        for _ in range(5):
            call(wd.name)
        h.set_math(_b.MATH_AUTO)
        for big in ("sparse1_f16_n5760", "sparse5_f16_n5760"):   # 16- and 12-wave workgroups
            wb = WORKLOADS[big]
            gb = {k: torch.from_numpy(v).to(dev) for k, v in generate(wb).items()}
            ob = torch.empty((wb.T, wb.B, wb.N), dtype=torch.float32, device=dev)
            for _ in range(3):
                h.forward_sparse(gb["col"], gb["val"], gb["X"], gb["h0"], out=ob)
            h.synchronize()
            del gb, ob
        st = generate_stack(WORKLOADS["dense_f16_n1152"], 2)  # the largest wavefront size
        layers = [{k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in ly.items()} for ly in st["layers"]]
        h.forward_stack_dense(layers, torch.from_numpy(st["x"]).to(dev))
        h.synchronize()
    if args.only_timed:
        h.close()
        print(json.dumps({"metric": "RNN timesteps/s & eff. GFLOP/s, N=1792 B=4 dense+10% sparse; % roofline",
                          "value": round(2 * T / (ms_per_step * 1e-3), 1), "unit": "timesteps/s",
                          "ms_per_step": round(ms_per_step, 4), "steps": args.steps, "warmup": args.warmup,
                          "dense_mean_launch_ms": round(dense_ms, 4),
                          "sparse_mean_launch_ms": round(sparse_ms, 4), "profile_mode": True}), flush=True)
        return

    # per-step time by the slope between T and T/2, and the sync floor
    floor_out = torch.empty((T, B, N), dtype=torch.float32, device=dev)
    f_full, f_half = timed(lambda: h.sync_floor(N, B, T, out=floor_out),
                           other=lambda: h.sync_floor(N, B, T // 2, out=floor_out[: T // 2]))
    floor_us = (f_full - f_half) * 1e3 / (T - T // 2)
    h.synchronize()
    for w in (wd, ws, w1):
        full, half = timed(lambda: call(w.name), other=lambda: call(w.name, T // 2))
        step_us = (full - half) * 1e3 / (T - T // 2)
        flop = w.flop_per_step
        detail[w.name] = {
            "ms_per_call": round(full, 4),
            "timesteps_per_s": round(T / (full * 1e-3), 1),
            "us_per_step_slope": round(step_us, 3),
            "vs_sync_floor": round(step_us / floor_us, 3) if floor_us > 0 else None,
            "gflop_per_s": round(flop * T / (full * 1e-3) / 1e9, 2),
            "pct_fp32_vector_peak": round(100 * flop * T / (full * 1e-3) / FP32_VECTOR_PEAK, 3),
            "weight_bytes": w.weight_bytes,
            "equiv_weight_TB_per_s": round(w.weight_bytes * T / (full * 1e-3) / 1e12, 3),
            "max_err_ratio": round(err[w.name], 5) if w.name in err else None,
            "plan": None,
        }
        h.synchronize()
        detail[w.name]["plan"] = {k: v for k, v in h.last_plan().items() if k != "first_step"}
    detail["sync_floor_us_per_step"] = round(floor_us, 3)
    detail["sync_floor_ms_per_call"] = round(f_full, 4)

    # the dense layers in the other math modes, not in the headline step:
    # SPLIT (matrix cores, h as fp16 hi + lo) and HALF (h rounded to fp16,
    # two products per v_dot2_f32_f16)
    from persistent_rnn_fwd_amd import binding as _b
    w2 = WORKLOADS["dense_f16_n1152"]
    host[w2.name] = generate(w2)
    g[w2.name] = {k: torch.from_numpy(v).to(dev) for k, v in host[w2.name].items()}
    out[w2.name] = torch.empty((w2.T, w2.B, w2.N), dtype=torch.float32, device=dev)
    for mode, label, w in ((_b.MATH_SPLIT, "split_math", wd), (_b.MATH_HALF, "half_h", wd), (_b.MATH_HALF, "half_h", w2)):
        h.set_math(mode)
        fl = floor_us
        if w is not wd:
            f_a, f_b = timed(lambda: h.sync_floor(w.N, w.B, w.T, out=out[w.name]),
                             other=lambda: h.sync_floor(w.N, w.B, w.T // 2, out=out[w.name][: w.T // 2]))
            fl = (f_a - f_b) * 1e3 / (w.T - w.T // 2)
        full, half = timed(lambda: call(w.name, w.T), other=lambda: call(w.name, w.T // 2))
        step_us = (full - half) * 1e3 / (w.T - w.T // 2)
        h.synchronize()
        alt = {"ms_per_call": round(full, 4), "timesteps_per_s": round(w.T / (full * 1e-3), 1),
               "us_per_step_slope": round(step_us, 3), "sync_floor_us_per_step": round(fl, 3),
               "vs_sync_floor": round(step_us / fl, 3) if fl > 0 else None,
               "gflop_per_s": round(w.flop_per_step * w.T / (full * 1e-3) / 1e9, 2),
               "plan": {k: v for k, v in h.last_plan().items() if k != "first_step"}}
        if not args.no_check:
            import oracle
            call(w.name, w.T)
            h.synchronize()
            d = host[w.name]
            alt["max_err_ratio"] = round(float(oracle.tolerance_ratio(out[w.name].cpu().numpy(),
                                                                      oracle.forward_dense(d["W"], d["X"], d["h0"]),
                                                                      oracle.TOL_F16)), 5)
        h.set_math(_b.MATH_AUTO)
        detail[f"{w.name}_{label}"] = alt
    detail["timed_launch_ms"] = {"dense_f16_n1792": percentiles(dense_list), "sparse10_f16_n1792": percentiles(sparse_list)}
    sd, ss = detail[wd.name]["us_per_step_slope"], detail[ws.name]["us_per_step_slope"]
    detail["dense_over_sparse10_step_time"] = round(sd / ss, 3) if ss > 0 else None

    # every workload at its own size: per-step slope, floor at the same
    # size, error ratio against the oracle (not part of the headline step)
    configs = None
    if not args.no_configs:
        configs = per_config_table(torch, dev, Handle, WORKLOADS, generate, timed, no_check=args.no_check,
                                   loops=not args.no_config_loops)

    detail["trace_us_per_step"] = trace_breakdown(torch, dev, Handle, g, wd, ws, T)
    if not args.no_layers:
        detail["layers"] = layer_table(torch, dev, Handle, timed, no_check=args.no_check)
        detail["stacks"] = stack_table(torch, dev, Handle, timed, no_check=args.no_check)
        detail["large_dense"] = large_dense_table(torch, dev, Handle, timed, no_check=args.no_check)

    baselines = None
    if not args.no_baselines:
        baselines = library_baselines(torch, dev, host, wd, ws, T,
                                      {"dense": detail[wd.name]["ms_per_call"], "sparse10": detail[ws.name]["ms_per_call"]})
    detail["gpu_clock_after_run"] = gpu_clock_report()

    # roofline of the dominant kernel (larger mean launch time)
    dom, dom_ms = (wd, dense_ms) if dense_ms >= sparse_ms else (ws, sparse_ms)
    flop_per_launch = dom.flop_per_step * T
    achieved = flop_per_launch / (dom_ms * 1e-3)
    traffic = None
    if os.path.exists(COUNTER_FILE):
        try:
            c = json.load(open(COUNTER_FILE))
            if c.get("kernel_source_hash") == kernel_source_hash():
                traffic = c.get("kernels", {}).get(dom.name, {}).get("hbm_bytes_per_launch")
        except (OSError, ValueError):
            traffic = None
    roofline = {
        "bound": "alu",
        "kernel": f"dense persistent kernel ({dom.name})" if dom is wd else f"sparse persistent kernel ({dom.name})",
        "achieved": round(achieved / 1e12, 4),
        "peak": FP32_VECTOR_PEAK / 1e12,
        "unit": "TFLOP/s",
        "frac": round(achieved / FP32_VECTOR_PEAK, 5),
        # one XCD per batch row: at B < 8 only B of the 8 XCDs do arithmetic
        "serving_xcds": min(dom.B, 8),
        "peak_of_serving_xcds": FP32_VECTOR_PEAK * min(dom.B, 8) / 8 / 1e12,
        "frac_of_serving_xcds_peak": round(achieved / (FP32_VECTOR_PEAK * min(dom.B, 8) / 8), 5),
        "traffic": traffic,
        "mean_launch_ms": round(dom_ms, 4),
        "flop_per_launch": flop_per_launch,
    }

    # host baseline: the oracle as it stands, on a bounded sample
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_limits
        Ts, spent, steps_done = 8, 0.0, 0
        # one thread: the BLAS pools the oracle's numpy products use are
        # limited to 1 for the whole sample (numpy itself runs on one)
        with threadpool_limits(limits=1):
            while spent < args.cpu_seconds and Ts <= T:
                for w in (wd, ws):
                    d = host[w.name]
                    a = time.perf_counter()
                    if w.kind == "dense":
                        oracle.forward_dense(d["W"], d["X"][:Ts], d["h0"])
                    else:
                        oracle.forward_sparse(d["col"], d["val"], d["X"][:Ts], d["h0"])
                    spent += time.perf_counter() - a
                    steps_done += Ts
                Ts = min(2 * Ts, T) if Ts < T else Ts
        cpu = {
            "value": round(steps_done / spent, 1),
            "unit": "timesteps/s",
            "cores": 1,
            "kind": "oracle",
            "sample": f"fp64 numpy oracle on one thread, dense + 10% sparse N=1792 B=4, {steps_done} timesteps "
                      f"in {spent:.1f} s (host: {os.cpu_count()} CPUs visible, {_cpu_model()})",
        }

    h.close()
    line = {
        "metric": "RNN timesteps/s & eff. GFLOP/s, N=1792 B=4 dense+10% sparse; % roofline",
        "value": round(2 * T / (ms_per_step * 1e-3), 1),
        "unit": "timesteps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "basic-RNN forward N=1792 B=4 T=256: one dense fp16-W call + one 10% "
                        "row-balanced sparse fp16-W call (K=179) per step, fp32 X/H/accumulate",
            "N": N, "B": B, "T": T, "K_sparse": ws.K, "weights": "f16",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "baselines": baselines,
        "configs": configs,
        "detail": detail,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
