"""GPU parity of ternary weights {-1, 0, +1} against the CPU oracle.

Sources: page "Extreme Quantization: Binary, Ternary & 1-bit LLMs",
"Ternary Quantization" eq. (7) (threshold Delta) and "BitNet b1.58" eq. (9)
(RoundClip(W / gamma, -1, 1), gamma = ||W||_1 / (nm)).

Bar: sign and nonzero planes (with pads), nonzero counts, int32 dot
products and packed threshold bits bit-exact; fp32 outputs computed from
identical inputs by the same rounded operations, bit-exact (NaN matches NaN).
All calls go through the C ABI."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import require_gpu, banner, dev, host, host_u32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bnn():
    require_gpu()
    import xnor_popcount_gemm_amd as m
    m.lib()
    return m


def _bits_equal(got, want, what):
    gf, wf = np.asarray(got, np.float32), np.asarray(want, np.float32)
    bad = (gf.view(np.uint32) != wf.view(np.uint32)) & ~(np.isnan(gf) & np.isnan(wf))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} differ; first {idx.tolist()} "
                             f"got {gf[tuple(idx.T)]} want {wf[tuple(idx.T)]}")


def _weights(seed, N, K, edges=True):
    W = workloads.normal_f32(seed, (N, K))
    if edges and N >= 2:
        W[1] = workloads.inject_edge_values(W[1:2], seed + 1, 0.05)[0]
    return W


# ---------------------------------------------------------------- pack
@pytest.mark.parametrize("N,K", [(1, 1), (7, 33), (64, 1000), (300, 4096), (3, 11008), (17, 257)])
@pytest.mark.parametrize("mode", ["roundclip", "threshold", "threshold_zero", "threshold_neg"])
def test_pack_weights_ternary(bnn, N, K, mode):
    W = _weights(9000 + K, N, K)
    banner(f"pack_weights_ternary {mode} N={N} K={K}")
    Wd = dev(W)
    if mode == "roundclip":
        Wf = W.copy()
        Wf[~np.isfinite(Wf)] = 0.0                  # a finite gamma
        gam = oracle.alpha_tensor(Wf)               # the oracle's gamma feeds the GPU pack
        Wd = dev(Wf)
        Sp, Zp, nnz = bnn.pack_weights_ternary(Wd, gamma=dev(np.array([gam], np.float32)))
        g_gpu = bnn.weight_scale_tensor(Wd)         # and the GPU's own gamma is checked apart
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(g_gpu).view(np.uint32), np.array([gam], np.float32).view(np.uint32))
        T = oracle.ternary_roundclip(Wf, gam)
    else:
        delta = {"threshold": 0.5, "threshold_zero": 0.0, "threshold_neg": -0.25}[mode]
        Sp, Zp, nnz = bnn.pack_weights_ternary(Wd, delta=delta)
        torch.cuda.synchronize()
        T = oracle.ternary_threshold(W, delta)
    S, Z, n = oracle.pack_ternary(T, ld=Sp.shape[1])
    np.testing.assert_array_equal(host_u32(Sp), S)
    np.testing.assert_array_equal(host_u32(Zp), Z)
    np.testing.assert_array_equal(host(nnz), n)


# ---------------------------------------------------------------- ternary x binary activations
def _ternary_case(bnn, seed, N, K):
    """Ternary weights from the oracle's gamma (eq. (9)): the GPU packs with
    that gamma; the GPU's own gamma is checked against it bit for bit."""
    W = _weights(seed, N, K, edges=False)
    gam = oracle.alpha_tensor(W)
    Wd = dev(W)
    g = dev(np.array([gam], np.float32))
    Sp, Zp, nnz = bnn.pack_weights_ternary(Wd, gamma=g)
    g_gpu = bnn.weight_scale_tensor(Wd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(g_gpu).view(np.uint32), np.array([gam], np.float32).view(np.uint32))
    T = oracle.ternary_roundclip(W, gam)
    return T, gam, Sp, Zp, nnz, g


@pytest.mark.parametrize("M,N,K", [(1, 300, 1000), (2, 4096, 4096), (4, 129, 333), (64, 256, 1000),
                                   (300, 100, 577), (1000, 64, 576), (257, 130, 4096), (129, 33, 31),
                                   # 3 and 5 full 8-word chunks (odd chunk after the two-chunk
                                   # K loop), the second with a tail
                                   (130, 70, 768), (257, 64, 1300),
                                   # GEMV rows of 8 granules per lane, up to the widest K
                                   # the GEMV takes; one word past it runs the GEMM
                                   (1, 130, 40000), (3, 130, 65536), (2, 40, 65537)])
@pytest.mark.parametrize("kernel", ["wlane", "rows"])
def test_ternary_binary_linear_fused(bnn, kernel, M, N, K, monkeypatch):
    """Both GEMM kernels (one weight row per lane, one activation row per
    lane); small M takes the GEMV either way."""
    monkeypatch.setenv("BNN_TERN_KERNEL", kernel)
    T, gam, Sp, Zp, nnz, g = _ternary_case(bnn, 9100 + K, N, K)
    X = workloads.normal_f32(9200 + K, (M, K))
    xs = oracle.sign(X)
    D_ref = oracle.dot_i8(xs, T)
    Xp = bnn.pack_activations(dev(X))
    R = workloads.normal_f32(9300 + N, (M, N))
    bias = workloads.normal_f32(9400 + N, (N,))
    gma, beta, mean, var, eps = workloads.bn_params(9500 + N, N)
    alpha_vec = np.full(N, gam, np.float32)
    tau, dirv = bnn.fold_bn_thresholds(gma, beta, mean, var, eps, alpha_vec)
    f = bnn.EPI_DOT_I32 | bnn.EPI_SCALE_F32 | bnn.EPI_ALPHA_TENSOR | bnn.W_TERNARY
    banner(f"ternary x binary fused kernel={kernel} M={M} N={N} K={K}")
    out = bnn.linear_fused(Xp, Sp, K, f | bnn.EPI_BIAS_F32 | bnn.EPI_RESIDUAL_F32, alpha=g, bias=dev(bias),
                           R=dev(R), Zp=Zp, nnz=nnz)
    th = bnn.linear_fused(Xp, Sp, K, bnn.EPI_THRESH_PACK | bnn.W_TERNARY, tau=dev(tau), dir=dev(dirv),
                          Zp=Zp, nnz=nnz)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out["D"]), D_ref)
    _bits_equal(host(out["Y"]), oracle.scale_bias_residual(D_ref, np.atleast_1d(gam), bias, R), "Y")
    ld = th["Op"].shape[1]
    s_ref, _ = oracle.bn_next_sign(D_ref, alpha_vec, gma, beta, mean, var, eps)
    np.testing.assert_array_equal(host_u32(th["Op"]), oracle.pack_signs(s_ref, ld=ld))


@pytest.mark.parametrize("M,N,K", [(33, 1, 100), (64, 63, 64), (31, 65, 1000), (97, 255, 2049),
                                   (40, 256, 4096), (70, 257, 300), (130, 300, 31)])
def test_ternary_gemm_weight_row_lanes(bnn, M, N, K):
    """The GEMM with one weight row per lane: ragged row tiles (M not a
    multiple of 32), waves past N and a partial last wave (N around 64 and
    256), K tails below one chunk and one word; per-row alpha, D, Y with bias
    and residual, and SIGN_PACK whose pad bits and pad words start non-zero."""
    T, gam, Sp, Zp, nnz, g = _ternary_case(bnn, 9800 + K + N, N, K)
    X = workloads.normal_f32(9801 + K, (M, K))
    D_ref = oracle.dot_i8(oracle.sign(X), T)
    a = np.abs(workloads.normal_f32(9802 + N, (N,))) + np.float32(0.1)
    bias = workloads.normal_f32(9803 + N, (N,))
    R = workloads.normal_f32(9804 + N, (M, N))
    b1 = workloads.normal_f32(9805 + N, (N,)) * np.float32(0.5)
    Xp = bnn.pack_activations(dev(X))
    ld = bnn.padded_ld(N)
    Op = torch.full((M, ld), -1, dtype=torch.int32, device="cuda")
    f = (bnn.EPI_DOT_I32 | bnn.EPI_SCALE_F32 | bnn.EPI_BIAS_F32 | bnn.EPI_RESIDUAL_F32 | bnn.EPI_SIGN_PACK
         | bnn.W_TERNARY)
    banner(f"ternary gemm weight-row lanes M={M} N={N} K={K}")
    out = bnn.linear_fused(Xp, Sp, K, f, alpha=dev(a), bias=dev(bias), R=dev(R), beta=dev(b1), Op=Op,
                           Zp=Zp, nnz=nnz)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out["D"]), D_ref)
    Y_ref = oracle.scale_bias_residual(D_ref, a, bias, R)
    _bits_equal(host(out["Y"]), Y_ref, "Y")
    np.testing.assert_array_equal(host_u32(Op), oracle.pack_signs(oracle.rsign(Y_ref, b1), ld=ld))


@pytest.mark.parametrize("tn", [8, 16, 32, 64])
def test_ternary_gemm_every_column_tile(bnn, tn, monkeypatch):
    monkeypatch.setenv("BNN_TERN_KERNEL", "rows")
    M, N, K = 300, 130, 1000
    T, gam, Sp, Zp, nnz, g = _ternary_case(bnn, 9600, N, K)
    X = workloads.normal_f32(9601, (M, K))
    D_ref = oracle.dot_i8(oracle.sign(X), T)
    Xp = bnn.pack_activations(dev(X))
    monkeypatch.setenv("BNN_GEMM_TN", str(tn))
    banner(f"ternary gemm TN={tn}")
    out = bnn.linear_fused(Xp, Sp, K, bnn.EPI_DOT_I32 | bnn.W_TERNARY, Zp=Zp, nnz=nnz)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out["D"]), D_ref)


# ---------------------------------------------------------------- ternary x INT8 activations (BitNet b1.58)
@pytest.mark.parametrize("M,N,K", [(1, 300, 1000), (2, 129, 4096), (1, 64, 11008), (1, 5, 32768),
                                   (2, 33, 16384)])
def test_ternary_i8_gemv(bnn, M, N, K):
    T, gam, Sp, Zp, nnz, g = _ternary_case(bnn, 9700 + K, N, K)
    X = workloads.normal_f32(9800 + K, (M, K))
    Q, xs = oracle.quantize_absmax_i8(X)
    q = bnn.quantize_act_i8(dev(X), want_int8=False)
    banner(f"ternary x int8 gemv M={M} N={N} K={K}")
    out = bnn.bwn_i8_linear(Sp, K, bnn.EPI_DOT_I32 | bnn.EPI_SCALE_F32 | bnn.EPI_ALPHA_TENSOR | bnn.W_TERNARY,
                            Xb=q["Xb"], xscale=q["xscale"], alpha=g, Zp=Zp)
    torch.cuda.synchronize()
    D_ref = oracle.dot_i8(Q, T)
    np.testing.assert_array_equal(host(out["D"]), D_ref)
    _bits_equal(host(out["Y"]), oracle.scale_i8(D_ref, np.atleast_1d(gam), xs), "Y")


@pytest.mark.parametrize("M,N,K", [(3, 5, 64), (64, 128, 1000), (130, 257, 100), (600, 200, 1000),
                                   (257, 385, 4096), (3, 1000, 11008)])
def test_ternary_i8_gemm(bnn, M, N, K):
    T, gam, Sp, Zp, nnz, g = _ternary_case(bnn, 9900 + K, N, K)
    rng = np.random.default_rng(9901 + K)
    Q = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    Qd = torch.zeros((M, bnn.i8_ld(K)), dtype=torch.int8, device="cuda")
    Qd[:, :K] = dev(Q)
    banner(f"ternary x int8 gemm M={M} N={N} K={K}")
    out = bnn.bwn_i8_linear(Sp, K, bnn.EPI_DOT_I32 | bnn.EPI_SCALE_F32 | bnn.EPI_ALPHA_TENSOR | bnn.W_TERNARY,
                            Xq=Qd[:, :K], alpha=g, Zp=Zp)
    torch.cuda.synchronize()
    D_ref = oracle.dot_i8(Q, T)
    np.testing.assert_array_equal(host(out["D"]), D_ref)
    _bits_equal(host(out["Y"]), oracle.scale(D_ref, np.full(N, gam, np.float32)), "Y")


def test_ternary_b158_decode_chain(bnn):
    """fp32 weights -> gamma -> RoundClip ternary planes; fp32 activation ->
    INT8 planes; one decode step on the decode shapes [11008, 4096] and
    [4096, 11008]."""
    for N, K in ((11008, 4096), (4096, 11008)):
        W = workloads.normal_f32(9950 + K, (N, K))
        X = workloads.normal_f32(9960 + K, (1, K))
        banner(f"b1.58 chain N={N} K={K}")
        Wd = dev(W)
        g = bnn.weight_scale_tensor(Wd)
        Sp, Zp, nnz = bnn.pack_weights_ternary(Wd, gamma=g)
        q = bnn.quantize_act_i8(dev(X), want_int8=False)
        out = bnn.bwn_i8_linear(Sp, K, bnn.EPI_DOT_I32 | bnn.EPI_SCALE_F32 | bnn.EPI_ALPHA_TENSOR | bnn.W_TERNARY,
                                Xb=q["Xb"], xscale=q["xscale"], alpha=g, Zp=Zp)
        torch.cuda.synchronize()
        gam = oracle.alpha_tensor(W)          # the oracle's own chain, end to end
        T = oracle.ternary_roundclip(W, gam)
        Q, xs = oracle.quantize_absmax_i8(X)
        D_ref = oracle.dot_i8(Q, T)
        np.testing.assert_array_equal(host(g).view(np.uint32), np.array([gam], np.float32).view(np.uint32))
        np.testing.assert_array_equal(host(out["D"]), D_ref)
        _bits_equal(host(out["Y"]), oracle.scale_i8(D_ref, np.atleast_1d(gam), xs), "Y")
