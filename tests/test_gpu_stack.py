"""GPU parity of stacks of layers (through the C ABI): dense layers run as a
wavefront, and row-balanced sparse layers one after another.

``prnn_forward_stack_dense`` runs layer 0's input projection, then the layers
at the same time (layer l, batch row b on its own XCD): in blocks of steps,
layer l + 1 one block behind layer l (BLOCKED, the default), or fused per
step (FUSED); or one layer after another (LAYERS, and for N > 1792).  It is compared with
``oracle.forward_stack_dense`` element by element on every layer's output, at
the recurrence's fp16 bar (|H - H_ref| <= 2e-2 (1 + |H_ref|)), for stacks of
2 to 8 layers, full and ragged sizes, with and without initial states.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from persistent_rnn_fwd_amd import Handle, PrnnError, binding
from persistent_rnn_fwd_amd.inputs import WORKLOADS, generate_stack

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def handle(gpu):
    h = Handle()
    yield h
    h.close()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_stack(handle, st, h0=True, mode=binding.STACK_AUTO):
    handle.set_stack_mode(mode)
    layers = [{k: dev(v) for k, v in ly.items()} for ly in st["layers"]]
    h0s = [dev(h) for h in st["h0s"]] if h0 else None
    outs = handle.forward_stack_dense(layers, dev(st["x"]), h0s)
    handle.synchronize()
    handle.set_stack_mode(binding.STACK_AUTO)
    return [o.cpu().numpy() for o in outs]


def check(st, got, h0=True):
    refs = oracle.forward_stack_dense(st["layers"], st["x"], st["h0s"] if h0 else None)
    ratios = [oracle.tolerance_ratio(g, r, oracle.TOL_F16) for g, r in zip(got, refs)]
    return ratios


# (L, B, N, T, h0 mode): full size at N=1152 (the largest wavefront, 5 rows x
# 5 chunks per wave and part); N=1792 and N=2048 (layers one after another:
# widened weights would not fit); deeper stacks at smaller B; ragged N (not a
# multiple of 4, of 256, or of the 256 waves of a team).
CASES = [
    (2, 1, 2048, 6, "randn"),
    (3, 2, 640, 150, "randn"),   # two blocks of 75 steps
    (2, 4, 1792, 97, "zeros"),   # blocks of 49 and 48 steps
    (2, 4, 1152, 256, "zeros"),
    (2, 4, 1792, 64, "randn"),
    (4, 2, 256, 32, "randn"),
    (8, 1, 200, 16, "randn"),
    (3, 2, 1000, 20, "zeros"),
    (2, 3, 777, 12, "randn"),
]


@pytest.mark.parametrize("L,B,N,T,h0", CASES)
def test_stack_parity(handle, L, B, N, T, h0):
    w = WORKLOADS["dense_f16_n1152"].with_(N=N, B=B, T=T, h0=h0, seed=300 + L * 10 + B)
    st = generate_stack(w, L)
    handle.set_grid(0)
    got = run_stack(handle, st)
    ratios = check(st, got)
    print(f"stack L={L} B={B} N={N} T={T}: error ratios {[f'{r:.3g}' for r in ratios]}")
    assert max(ratios) <= 1.0


@pytest.mark.parametrize("mode", [binding.STACK_BLOCKED, binding.STACK_FUSED, binding.STACK_LAYERS])
@pytest.mark.parametrize("L,B,N,T", [(2, 4, 1152, 200), (4, 2, 256, 70), (3, 2, 777, 33)])
def test_stack_modes_agree_with_the_oracle(handle, mode, L, B, N, T):
    w = WORKLOADS["dense_f16_n1152"].with_(N=N, B=B, T=T, h0="randn", seed=500 + L + B)
    st = generate_stack(w, L)
    got = run_stack(handle, st, mode=mode)
    ratios = check(st, got)
    print(f"stack mode {mode} L={L} B={B} N={N} T={T}: error ratios {[f'{r:.3g}' for r in ratios]}")
    assert max(ratios) <= 1.0


def test_stack_forced_mode_that_does_not_fit(handle):
    w = WORKLOADS["dense_f16_n1152"].with_(N=1792, B=2, T=4, seed=6)
    st = generate_stack(w, 2)
    with pytest.raises(PrnnError) as e:                       # fused needs N <= 1280
        run_stack(handle, st, mode=binding.STACK_FUSED)
    assert e.value.status == binding.NOT_SUPPORTED
    handle.set_stack_mode(binding.STACK_AUTO)
    with pytest.raises(PrnnError) as e:
        handle.set_stack_mode(9)
    assert e.value.status == binding.BAD_PARAM


def test_stack_deterministic_and_grid_independent_parity(handle):
    w = WORKLOADS["dense_f16_n1152"].with_(N=512, B=2, T=24, h0="randn", seed=9)
    st = generate_stack(w, 3)
    a = run_stack(handle, st)
    b = run_stack(handle, st)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    handle.set_grid(128)                 # 16 workgroups per team: more rows per wave
    c = run_stack(handle, st)
    handle.set_grid(0)
    assert max(check(st, c)) <= 1.0


def test_single_layer_stack_matches_layer_call(handle):
    """L = 1 is one layer: the same arithmetic as prnn_forward_layer_dense up to
    the order of the sums."""
    w = WORKLOADS["dense_f16_n1152"].with_(T=32, h0="randn", seed=21)
    st = generate_stack(w, 1)
    got = run_stack(handle, st)[0]
    ly = {k: dev(v) for k, v in st["layers"][0].items()}
    H = handle.forward_layer_dense(ly["U"], ly["bias"], ly["W"], dev(st["x"]), dev(st["h0s"][0]))
    handle.synchronize()
    ref = oracle.forward_stack_dense(st["layers"], st["x"], st["h0s"])[0]
    assert oracle.tolerance_ratio(got, ref, oracle.TOL_F16) <= 1.0
    np.testing.assert_allclose(got, H.cpu().numpy(), rtol=1e-5, atol=1e-5)


def test_stack_errors(handle):
    w = WORKLOADS["dense_f16_n1152"].with_(N=256, B=4, T=4, seed=5)
    st = generate_stack(w, 3)
    layers = [{k: dev(v) for k, v in ly.items()} for ly in st["layers"]]
    with pytest.raises(PrnnError) as e:                       # L B = 12 > 8 XCDs
        handle.forward_stack_dense(layers, dev(st["x"]))
    assert e.value.status == binding.NOT_SUPPORTED
    two = layers[:2]
    x = dev(st["x"])
    outs = [torch.full((4, 4, 256), 3.0, device="cuda") for _ in range(2)]
    with pytest.raises(PrnnError) as e:                       # an output doubles as the workspace
        handle.forward_stack_dense(two, x, outs=outs, workspace=outs[1])
    assert e.value.status == binding.BAD_PARAM
    with pytest.raises(PrnnError) as e:                       # two layers share one output
        handle.forward_stack_dense(two, x, outs=[outs[0], outs[0]])
    assert e.value.status == binding.BAD_PARAM
    handle.synchronize()
    assert all(bool((o == 3.0).all()) for o in outs)           # nothing ran
    empty = handle.forward_stack_dense(two, x[:0], outs=[o[:0] for o in outs])
    assert all(o.numel() == 0 for o in empty)


@pytest.mark.parametrize("N", [384, 1792])
def test_stack_chunked_in_time(handle, N):
    """A stack over T steps equals two stack calls over T1 and T - T1 steps, the
    second starting from every layer's last state (within 1e-6)."""
    w = WORKLOADS["dense_f16_n1152"].with_(N=N, B=2, T=140, h0="randn", seed=77)
    st = generate_stack(w, 3)
    layers = [{k: dev(v) for k, v in ly.items()} for ly in st["layers"]]
    x = dev(st["x"])
    h0s = [dev(v) for v in st["h0s"]]
    full = handle.forward_stack_dense(layers, x, h0s)
    a = handle.forward_stack_dense(layers, x[:65].contiguous(), h0s)
    b = handle.forward_stack_dense(layers, x[65:].contiguous(), [o[-1].contiguous() for o in a])
    handle.synchronize()
    for l in range(3):
        both = torch.cat([a[l], b[l]]).cpu().numpy()
        np.testing.assert_allclose(both, full[l].cpu().numpy(), rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("mode", [binding.STACK_BLOCKED, binding.STACK_FUSED, binding.STACK_LAYERS])
def test_stack_without_biases_or_states_and_fp16_input(handle, mode):
    """bias None for every layer, no initial states (zeros), fp16 network input."""
    w = WORKLOADS["dense_f16_n1152"].with_(N=320, B=2, T=70, seed=88)
    st = generate_stack(w, 3)
    for ly in st["layers"]:
        ly["bias"] = None
    x16 = st["x"].astype(np.float16)
    handle.set_stack_mode(mode)
    layers = [{"U": dev(ly["U"]), "W": dev(ly["W"]), "bias": None} for ly in st["layers"]]
    outs = handle.forward_stack_dense(layers, dev(x16))
    handle.synchronize()
    handle.set_stack_mode(binding.STACK_AUTO)
    refs = oracle.forward_stack_dense(st["layers"], x16, None)
    for o, r in zip(outs, refs):
        assert oracle.tolerance_ratio(o.cpu().numpy(), r, oracle.TOL_F16) <= 1.0


# ---------------------------------------------------------------------------
# stacks of row-balanced sparse layers (prnn_forward_stack_sparse: one layer
# after another) against oracle.forward_stack_sparse
# ---------------------------------------------------------------------------
def run_sparse_stack(handle, st, h0=True, x_dtype=np.float32):
    layers = [{k: dev(v) for k, v in ly.items()} for ly in st["layers"]]
    h0s = [dev(h) for h in st["h0s"]] if h0 else None
    outs = handle.forward_stack_sparse(layers, dev(st["x"].astype(x_dtype)), h0s)
    handle.synchronize()
    return [o.cpu().numpy() for o in outs]


@pytest.mark.parametrize("name,L,B,T", [("sparse10_f16_n1152", 2, 4, 256), ("sparse10_f16_n1792", 3, 4, 40),
                                        ("sparse1_f16_n5760", 2, 4, 16), ("sparse10_f16_n2304", 2, 2, 20)])
def test_sparse_stack_parity(handle, name, L, B, T):
    w = WORKLOADS[name].with_(T=T, B=B, h0="randn")
    st = generate_stack(w, L)
    got = run_sparse_stack(handle, st)
    refs = oracle.forward_stack_sparse(st["layers"], st["x"], st["h0s"])
    for l, (g, r) in enumerate(zip(got, refs)):
        assert oracle.tolerance_ratio(g, r, oracle.TOL_F16) <= 1.0, f"{name} layer {l}"


def test_sparse_stack_ragged_fp32_values_and_fp16_input(handle):
    from persistent_rnn_fwd_amd.inputs import Workload
    w = Workload("sparse_1000", "sparse", 1000, 3, 12, "f32", K=77, seed=41, h0="randn")
    st = generate_stack(w, 3)
    got = run_sparse_stack(handle, st, x_dtype=np.float16)
    x16 = st["x"].astype(np.float16)
    refs = oracle.forward_stack_sparse(st["layers"], x16, st["h0s"])
    for g, r in zip(got, refs):
        assert oracle.tolerance_ratio(g, r, oracle.TOL_F32) <= 1.0


def test_sparse_stack_equals_layer_calls_bitwise(handle):
    w = WORKLOADS["sparse10_f16_n1792"].with_(T=20, h0="randn")
    st = generate_stack(w, 2)
    got = run_sparse_stack(handle, st, h0=False)
    layers = [{k: dev(v) for k, v in ly.items()} for ly in st["layers"]]
    inp = dev(st["x"])
    for l, ly in enumerate(layers):
        H = handle.forward_layer_sparse(ly["U"], ly["bias"], ly["col"], ly["val"], inp)
        handle.synchronize()
        np.testing.assert_array_equal(H.cpu().numpy(), got[l])
        inp = H


def test_sparse_stack_errors(handle):
    w = WORKLOADS["sparse10_f16_n1152"].with_(T=4)
    st = generate_stack(w, 2)
    layers = [{k: dev(v) for k, v in ly.items()} for ly in st["layers"]]
    x = dev(st["x"])
    outs = [torch.empty((w.T, w.B, w.N), device="cuda") for _ in range(2)]
    with pytest.raises(PrnnError) as e:                      # two layers writing one output
        handle.forward_stack_sparse(layers, x, outs=[outs[0], outs[0]])
    assert e.value.status == binding.BAD_PARAM
    with pytest.raises(PrnnError) as e:                      # the workspace is an output
        handle.forward_stack_sparse(layers, x, outs=outs, workspace=outs[1])
    assert e.value.status == binding.BAD_PARAM
    lib = binding.load_library()
    s = torch.cuda.current_stream().cuda_stream
    arr = lambda ts: (ctypes.c_void_p * 2)(*[t.data_ptr() for t in ts])
    U, C, V, H = (arr([ly["U"] for ly in layers]), arr([ly["col"] for ly in layers]),
                  arr([ly["val"] for ly in layers]), arr(outs))
    ws = torch.empty((w.T, w.B, w.N), device="cuda")
    call = lambda L=2, K=w.K, vt=binding.DATA_HALF, T=w.T: lib.prnn_forward_stack_sparse(
        handle._h, L, w.N, w.N, w.B, T, K, binding.DATA_FLOAT, x.data_ptr(), U, None, C, vt, V, None,
        ws.data_ptr(), H, s)
    assert call(L=0) == binding.BAD_PARAM
    assert call(K=0) == binding.BAD_PARAM and call(K=w.N + 1) == binding.BAD_PARAM
    assert call(vt=7) == binding.BAD_PARAM
    assert call(T=0) == binding.SUCCESS
    assert call() == binding.SUCCESS
    handle.synchronize()
    refs = oracle.forward_stack_sparse([dict(ly, bias=None) for ly in st["layers"]], st["x"], None)
    for o, r in zip(outs, refs):
        assert oracle.tolerance_ratio(o.cpu().numpy(), r, oracle.TOL_F16) <= 1.0
