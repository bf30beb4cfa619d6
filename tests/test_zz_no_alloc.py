"""GPU check of bnn_weight_scale_tensor_noalloc, the entry point that
allocates nothing (for callers that cannot allocate device memory): its
per-tensor scale ("Extreme Quantization", eq. (8)) must equal the one of
bnn_weight_scale_tensor, which takes a caller-owned workspace, on two calls
in a row (the second with fewer rows, so a stale scratch would show), and at
the largest row count it accepts.  Calls go through the C ABI."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import require_gpu, banner, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bnn():
    require_gpu()
    import xnor_popcount_gemm_amd as m
    m.lib()
    return m


def _bits(t):
    return host(t).view(np.uint32)


def test_noalloc_scale_matches_workspace_entry_point(bnn):
    outs = []
    for seed, (N, K) in ((7001, (11008, 4096)), (7002, (300, 1000)), (7003, (1, 33))):
        W = workloads.normal_f32(seed, (N, K))
        Wd = dev(W)
        banner(f"weight_scale_tensor_noalloc N={N} K={K}")
        ref = bnn.weight_scale_tensor(Wd)
        out = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
        bnn.weight_scale_tensor_noalloc(Wd, out=out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(out), _bits(ref))
        np.testing.assert_array_equal(_bits(out), np.atleast_1d(oracle.alpha_tensor(W)).view(np.uint32))
        outs.append(float(host(out)[0]))
    assert len(set(outs)) == 3


def test_noalloc_scale_at_the_row_limit(bnn):
    N, K = bnn.NOALLOC_MAX_ROWS, 40
    W = workloads.normal_f32(7010, (N, K))
    Wd = dev(W)
    banner(f"weight_scale_tensor_noalloc N={N} K={K}")
    out = torch.empty(1, dtype=torch.float32, device="cuda")
    bnn.weight_scale_tensor_noalloc(Wd, out=out)
    ref = bnn.weight_scale_tensor(Wd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(out), _bits(ref))
    # one row more is refused before anything is launched
    Wb = torch.zeros((N + 1, 4), dtype=torch.float32, device="cuda")
    with pytest.raises(bnn.BnnError) as e:
        bnn.weight_scale_tensor_noalloc(Wb, out=out)
    assert e.value.status == 2
    # the same stream order on a non-default stream
    s = torch.cuda.Stream()
    W2 = workloads.normal_f32(7011, (5000, 300))
    with torch.cuda.stream(s):
        W2d = dev(W2)
        o2 = torch.empty(1, dtype=torch.float32, device="cuda")
        bnn.weight_scale_tensor_noalloc(W2d, out=o2)
    s.synchronize()
    np.testing.assert_array_equal(_bits(o2), np.atleast_1d(oracle.alpha_tensor(W2)).view(np.uint32))
