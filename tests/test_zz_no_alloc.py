"""prnn_forward_dense_noalloc (the entry point that allocates nothing) against
prnn_forward_dense on the same inputs, through the C ABI.

Both run the same team-layout kernels with the same plan, so their outputs
must agree bit for bit; both are also checked against the fp64 oracle.  Two
calls in a row, the second smaller, show that the fixed exchange array is
reset between calls (the second call's rows and steps differ from what the
first left in it).
"""
import numpy as np
import pytest
import torch

import oracle
from persistent_rnn_fwd_amd import Handle, PrnnError, binding
from persistent_rnn_fwd_amd.inputs import WORKLOADS, Workload, generate

pytestmark = pytest.mark.gpu


def to_dev(d):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in d.items()}


def tol_of(d):
    return oracle.TOL_F32 if d["W"].dtype == np.float32 else oracle.TOL_F16


def one_call(w, seed, status):
    d = generate(w, seed=seed)
    g = to_dev(d)
    H_na = torch.full(g["X"].shape, float("nan"), device="cuda")
    binding.forward_dense_noalloc(g["W"], g["X"], g["h0"], out=H_na, status=status)
    with Handle() as h:
        H_ref = h.forward_dense(g["W"], g["X"], g["h0"])
        h.synchronize()
    torch.cuda.synchronize()
    return d, H_na.cpu().numpy(), H_ref.cpu().numpy()


def test_noalloc_matches_prnn_forward_dense_two_calls(gpu):
    status = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    cases = [
        WORKLOADS["dense_f16_n1792"].with_(T=64, h0="randn"),                  # the headline layer
        Workload("smaller", "dense", 1000, 2, 17, "f32", seed=5, h0="randn"),  # smaller, ragged, fp32 W
    ]
    for i, w in enumerate(cases):
        d, H_na, H_ref = one_call(w, w.seed + 77, status)
        assert int(status.item()) == 0, f"call {i}: status {int(status.item())}"
        np.testing.assert_array_equal(H_na, H_ref)
        r = oracle.tolerance_ratio(H_na, oracle.forward_dense(d["W"], d["X"], d["h0"]), tol_of(d))
        assert r <= 1.0, f"call {i}: error ratio {r:.3g}"


@pytest.mark.parametrize("N,B", [(binding.NOALLOC_MAX_N, 3), (2304, 2)])
def test_noalloc_without_status_and_at_its_capacity(gpu, N, B):
    """The largest layer the array holds (split over 2 XCDs per batch row by
    default, like prnn_forward_dense), and a layer split over 4 (B <= 2)."""
    w = Workload("cap", "dense", N, B, 6, "f16", seed=9, h0="randn")
    d, H_na, H_ref = one_call(w, 9, None)
    np.testing.assert_array_equal(H_na, H_ref)
    assert oracle.tolerance_ratio(H_na, oracle.forward_dense(d["W"], d["X"], d["h0"]), oracle.TOL_F16) <= 1.0


def test_noalloc_rejects_sizes_beyond_its_array(gpu):
    N = binding.NOALLOC_MAX_N + 1
    W = torch.zeros(N, N, dtype=torch.float16, device="cuda")
    X = torch.zeros(2, 1, N, device="cuda")
    with pytest.raises(PrnnError) as e:
        binding.forward_dense_noalloc(W, X)
    assert e.value.status == binding.NOT_SUPPORTED
    lib = binding.load_library()
    s = torch.cuda.current_stream().cuda_stream
    assert lib.prnn_forward_dense_noalloc(64, 9, 2, binding.DATA_HALF, W.data_ptr(), X.data_ptr(), None,
                                          X.data_ptr(), None, s) == binding.BAD_PARAM
    assert lib.prnn_forward_dense_noalloc(64, 1, 0, binding.DATA_HALF, None, None, None, None, None,
                                          s) == binding.SUCCESS
