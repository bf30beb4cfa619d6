"""GPU parity of the XNOR GEMM on the fp4 matrix cores (bnn_xnor_gemm_mfma).

Sources: page "First Principles: Why Binary Ops Can Be Exponentially
Faster", section "1. Arithmetic: MAC -> XNOR + popcount", and "Extreme
Quantization: Binary, Ternary & 1-bit LLMs", eq. (6) (the integer D) and
eq. (1) (Y = alpha D).

Bar: D bit-exact and Y = fl32(alpha * D) bit-exact against the oracle, the
oracle's packed operands and alpha feeding the GPU.  All calls go through
the C ABI."""
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


def _ld(K, extra=0):
    kw = -(-K // 32)
    return -(-kw // 4) * 4 + extra


def _case(seed, M, N, K, ldx_extra=0, ldw_extra=0):
    X = workloads.normal_f32(seed, (M, K))
    W = workloads.normal_f32(seed + 1, (N, K))
    xs, ws = oracle.sign(X), oracle.sign(W)
    Xp = dev(oracle.pack_signs(xs, ld=_ld(K, ldx_extra)).view(np.int32))
    Wp = dev(oracle.pack_signs(ws, ld=_ld(K, ldw_extra)).view(np.int32))
    return xs, ws, Xp, Wp, oracle.alpha(W)


SHAPES = [(64, 256, 1000), (300, 100, 777), (257, 129, 1100), (1, 1, 1), (1, 7, 33), (5, 70, 4096),
          (129, 33, 31), (128, 128, 512), (130, 130, 513), (512, 64, 576), (70, 1, 32), (65, 96, 16),
          (256, 512, 8192), (3, 300, 11008), (200, 300, 2304), (1000, 257, 16385)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_xnor_gemm_mfma_matches_oracle(bnn, M, N, K):
    xs, ws, Xp, Wp, a = _case(8000 + K + M, M, N, K)
    banner(f"xnor_gemm_mfma M={M} N={N} K={K}")
    D, Y = bnn.xnor_gemm_mfma(Xp, Wp, K, alpha=dev(a), want_dot=True, want_scaled=True)
    torch.cuda.synchronize()
    D_ref = oracle.dot(xs, ws)
    np.testing.assert_array_equal(host(D), D_ref)
    np.testing.assert_array_equal(host(Y).view(np.uint32), oracle.scale(D_ref, a).view(np.uint32))


@pytest.mark.parametrize("tile", ["8x4", "4x8", "8x8"])
@pytest.mark.parametrize("M,N,K", [(300, 100, 777), (257, 129, 1100), (130, 513, 16385), (1, 7, 33)])
def test_xnor_gemm_mfma_every_tile(bnn, tile, M, N, K, monkeypatch):
    """The tuning override BNN_MFMA_TILE (MFMA blocks per wave) changes no result."""
    monkeypatch.setenv("BNN_MFMA_TILE", tile)
    xs, ws, Xp, Wp, a = _case(8200 + K + M, M, N, K)
    banner(f"xnor_gemm_mfma tile={tile} M={M} N={N} K={K}")
    D, Y = bnn.xnor_gemm_mfma(Xp, Wp, K, alpha=dev(a), want_dot=True, want_scaled=True)
    torch.cuda.synchronize()
    D_ref = oracle.dot(xs, ws)
    np.testing.assert_array_equal(host(D), D_ref)
    np.testing.assert_array_equal(host(Y).view(np.uint32), oracle.scale(D_ref, a).view(np.uint32))


def test_xnor_gemm_mfma_wide_ld_and_strided_outputs(bnn):
    """Leading dimensions past the data words (their pad words are the
    packed layout's zeros), outputs with ld > N, D alone and Y alone."""
    M, N, K = 150, 90, 700
    xs, ws, Xp, Wp, a = _case(8100, M, N, K, ldx_extra=12, ldw_extra=4)
    Db = torch.full((M, N + 7), -5, dtype=torch.int32, device="cuda")
    Yb = torch.full((M, N + 3), 7.0, dtype=torch.float32, device="cuda")
    banner("xnor_gemm_mfma strided")
    bnn.xnor_gemm_mfma(Xp, Wp, K, alpha=dev(a), want_dot=True, want_scaled=False, D=Db[:, :N])
    bnn.xnor_gemm_mfma(Xp, Wp, K, alpha=dev(a), want_dot=False, want_scaled=True, Y=Yb[:, :N])
    torch.cuda.synchronize()
    D_ref = oracle.dot(xs, ws)
    np.testing.assert_array_equal(host(Db)[:, :N], D_ref)
    assert np.all(host(Db)[:, N:] == -5)
    np.testing.assert_array_equal(host(Yb)[:, :N].view(np.uint32), oracle.scale(D_ref, a).view(np.uint32))
    assert np.all(host(Yb)[:, N:] == 7.0)


def test_xnor_gemm_mfma_largest_k(bnn):
    """K = 2^24, the largest K the ABI accepts: rows of all +1 and all -1
    reach D = +K and -K, where the fp32 accumulator holds 2^24 exactly."""
    K = 1 << 24
    M = N = 3
    xs = np.ones((M, K), np.int8)
    xs[1] = -1
    xs[2, ::3] = -1
    ws = np.ones((N, K), np.int8)
    ws[2, 1::2] = -1
    Xp = dev(oracle.pack_signs(xs, ld=_ld(K)).view(np.int32))
    Wp = dev(oracle.pack_signs(ws, ld=_ld(K)).view(np.int32))
    banner("xnor_gemm_mfma K=2^24")
    D, _ = bnn.xnor_gemm_mfma(Xp, Wp, K)
    torch.cuda.synchronize()
    D_ref = oracle.dot(xs, ws)
    assert D_ref[0, 0] == K and D_ref[1, 0] == -K
    np.testing.assert_array_equal(host(D), D_ref)


def test_xnor_gemm_mfma_full_8192(bnn):
    """The 8192^3 GEMM of the large-GEMM workload, every element of D and Y
    against the oracle."""
    n = 8192
    xs, ws, Xp, Wp, a = _case(workloads.seed_for(4, 0) + 7, n, n, n)
    banner("xnor_gemm_mfma 8192^3")
    D, Y = bnn.xnor_gemm_mfma(Xp, Wp, n, alpha=dev(a), want_dot=True, want_scaled=True)
    torch.cuda.synchronize()
    D_ref = oracle.dot(xs, ws)
    np.testing.assert_array_equal(host(D), D_ref)
    np.testing.assert_array_equal(host(Y).view(np.uint32), oracle.scale(D_ref, a).view(np.uint32))
