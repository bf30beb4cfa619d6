"""GPU parity of binary weights x fp16 activations (bnn_bwn_f16_gemv).

Source: page "Extreme Quantization: Binary, Ternary & 1-bit LLMs", "Binary
Neural Networks" eq. (1)-(2) (BinaryConnect / BWN: real activations, +1/-1
weights that add or subtract them, one scale per output row).

Bar.  The oracle sums exactly (integer units of 2^-24).  The kernel sums in
fp32, so:
  * integer-valued activations (every partial sum an integer below 2^24, so
    exact in fp32): Y bit-equal to fl32(alpha * S);
  * other fp16 activations: |Y - alpha S| <= |alpha| gamma_n sum_k |x_k| (1 +
    2u) + 2u |alpha S|, with u = 2^-24, gamma_n = n u / (1 - n u) and n the
    rounded-addition depth the header states for the kernel's sum order.
All calls go through the C ABI; the weights are the oracle's signs packed by
the oracle, or random packed words read by both sides."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import require_gpu, banner, dev, host

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module")
def bnn():
    require_gpu()
    import xnor_popcount_gemm_amd as m
    m.lib()
    return m


def _depth(K):
    kw4 = -(-K // 128)
    G = 1
    while G < kw4 and G < 64:
        G *= 2
    return 128 * (-(-kw4 // G)) + 6


def _ld(K):
    """Packed words per weight row: ceil(K/32) rounded up to a multiple of 4."""
    kw = -(-K // 32)
    return -(-kw // 4) * 4


def _packed(W):
    return dev(oracle.pack_signs(oracle.sign(W), ld=_ld(W.shape[1])).view(np.int32))


def _x16(M, K, ld=None):
    ld = K if ld is None else ld
    return torch.zeros((M, ld), dtype=torch.float16, device="cuda")


def _run(bnn, Wp, K, x16_host, a, alpha_tensor=False):
    M = x16_host.shape[0]
    ld = -(-K // 8) * 8
    Xd = _x16(M, K, ld)
    Xd[:, :K] = torch.from_numpy(x16_host).cuda()
    Y = bnn.bwn_f16_gemv(Wp, K, Xd, dev(np.atleast_1d(a).astype(np.float32)), alpha_tensor=alpha_tensor)
    torch.cuda.synchronize()
    return host(Y)


def _within_bound(Y, x16, S, a, K, what):
    a64 = np.asarray(a, np.float64)[None, :]
    n = _depth(K)
    gam = n * U / (1 - n * U)
    sabs = np.abs(x16.astype(np.float64)).sum(axis=1)[:, None]
    tol = np.abs(a64) * gam * sabs * (1 + 2 * U) + 2 * U * np.abs(a64 * S)
    err = np.abs(Y.astype(np.float64) - a64 * S)
    bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs beyond the bound; worst ratio "
                           f"{float((err / np.maximum(tol, 1e-300)).max()):.3g}")
    return float((err / np.maximum(tol, 1e-300)).max())


SHAPES = [(1, 11008, 4096), (1, 4096, 11008), (2, 300, 1000), (1, 7, 1), (1, 130, 33), (1, 64, 16384),
          (2, 257, 16383), (1, 1, 128), (3, 65, 129), (1, 33, 8200),
          # the table kernel's size classes and K pieces: 64 KiB / 128 KiB tables,
          # one pass up to K = 8192, a second pass of one element after it
          (1, 70, 4097), (2, 129, 8192), (1, 65, 8193), (1, 3, 2049)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_f16_gemv_integer_activations_bit_exact(bnn, M, N, K):
    rng = np.random.default_rng(9000 + K)
    x = rng.integers(-8, 9, size=(M, K)).astype(np.float16)
    W = workloads.normal_f32(9001 + N, (N, K))
    a = oracle.alpha(W)
    Wp = _packed(W)
    banner(f"bwn f16 gemv integer x M={M} N={N} K={K}")
    Y = _run(bnn, Wp, K, x, a)
    Sx = oracle.bwn_f16_units(x, oracle.sign(W))
    assert np.all(Sx % (1 << 24) == 0)
    S32 = (Sx >> 24).astype(np.float32)                     # exact: |S| <= 8 K < 2^24
    want = (a[None, :] * S32).astype(np.float32)
    np.testing.assert_array_equal(Y.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("alpha_tensor", [False, True])
def test_f16_gemv_random_within_bound(bnn, M, N, K, alpha_tensor):
    rng = np.random.default_rng(9100 + K)
    x = rng.standard_normal((M, K)).astype(np.float16)
    # fp16 subnormals, zeros of both signs and large values among them
    idx = rng.integers(0, K, size=(M, max(1, K // 50)))
    for m in range(M):
        x[m, idx[m]] = rng.choice(np.array([2.0 ** -24, -2.0 ** -20, 0.0, -0.0, 3e-5, 1000.0, -2048.0],
                                           np.float16), size=idx.shape[1])
    W = workloads.normal_f32(9101 + N, (N, K))
    a = np.atleast_1d(oracle.alpha_tensor(W)) if alpha_tensor else oracle.alpha(W)
    Wp = _packed(W)
    banner(f"bwn f16 gemv random x M={M} N={N} K={K} alpha_tensor={alpha_tensor}")
    Y = _run(bnn, Wp, K, x, a, alpha_tensor)
    S, _ = oracle.bwn_f16(x, W, np.ones(N, np.float32))
    aa = np.full(N, a[0], np.float32) if alpha_tensor else a
    _within_bound(Y, x, S, aa, K, "Y")


@pytest.mark.parametrize("N,K", [(262144 + 37, 1000), (2100000, 100)])
def test_f16_gemv_many_rows_random_words(bnn, N, K):
    """Enough rows for the unrolled row-steps (several weight rows' loads in
    flight per wave); random packed words, pad bits included (the
    activations past K are 0, so pad bits add nothing).  The oracle checks
    3000 sampled rows, the first and the last among them."""
    words = workloads.random_words(9200 + N, (N, _ld(K)))
    a = workloads.normal_f32(9201, (N,))
    rng = np.random.default_rng(9202)
    x = rng.standard_normal((1, K)).astype(np.float16)
    banner(f"bwn f16 gemv many rows N={N} K={K}")
    Y = _run(bnn, dev(words.view(np.int32)), K, x, a)
    rows = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, size=3000)]))
    ws = oracle.unpack_signs(words[rows], K)
    S = oracle.bwn_f16_units(x, ws).astype(np.float64) * U
    _within_bound(Y[:, rows], x, S, a[rows], K, "Y")


@pytest.mark.parametrize("variant", [{"BNN_F16_KERNEL": "regs"}, {"BNN_F16_PIECE": "4096"}])
@pytest.mark.parametrize("M,N,K", [(1, 300, 1000), (1, 257, 4096), (2, 129, 11008), (1, 65, 16384), (1, 9, 8193)])
def test_f16_gemv_variants(bnn, variant, M, N, K, monkeypatch):
    """The register-held-activation kernel (BNN_F16_KERNEL=regs) and the
    table kernel in 4096-wide K pieces (BNN_F16_PIECE=4096), both within the
    stated bound, and bit-exact for integer activations."""
    for k, v in variant.items():
        monkeypatch.setenv(k, v)
    rng = np.random.default_rng(9300 + K)
    W = workloads.normal_f32(9301 + N, (N, K))
    a = oracle.alpha(W)
    Wp = _packed(W)
    banner(f"bwn f16 gemv {variant} M={M} N={N} K={K}")
    xi = rng.integers(-8, 9, size=(M, K)).astype(np.float16)
    Y = _run(bnn, Wp, K, xi, a)
    S32 = (oracle.bwn_f16_units(xi, oracle.sign(W)) >> 24).astype(np.float32)
    np.testing.assert_array_equal(Y.view(np.uint32), (a[None, :] * S32).astype(np.float32).view(np.uint32))
    x = rng.standard_normal((M, K)).astype(np.float16)
    Y = _run(bnn, Wp, K, x, a)
    S, _ = oracle.bwn_f16(x, W, np.ones(N, np.float32))
    _within_bound(Y, x, S, a, K, "Y")
