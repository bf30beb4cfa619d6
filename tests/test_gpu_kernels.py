"""GPU parity of each kernel family against the CPU oracle, at sizes the
oracle finishes in seconds that still span several tiles and ragged tails.

Bar: packed words (including pad bits and pad words) and int32 dot products
bit-exact; alpha and alpha-scaled fp32 within 1e-6 relative (the sum of |w|
may round differently in its last fp64 bits, at most one fp32 ulp in alpha);
the residual sum within 1e-6 of the operands' magnitude.  All calls go through
the C ABI (the ctypes binding)."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import (require_gpu, banner, dev, host, host_u32, assert_f32_close,
                      exact_fraction)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bnn():
    require_gpu()
    import xnor_popcount_gemm_amd as m
    m.lib()
    return m


def _signs_with_edges(seed, shape, frac=0.02):
    x = workloads.normal_f32(seed, shape)
    return workloads.inject_edge_values(x, seed + 7, frac)


# ---------------------------------------------------------------- pack
@pytest.mark.parametrize("N,K", [(256, 1000), (7, 1), (9, 31), (33, 32), (5, 33), (64, 65),
                                 (300, 4096), (3, 11008), (129, 2304), (17, 257)])
def test_pack_weights_bits_and_alpha(bnn, N, K):
    W = _signs_with_edges(100 + K, (N, K))
    W[0, :] = np.abs(W[0, :])                   # a row with no NaN, finite alpha
    W[0, :][~np.isfinite(W[0, :])] = 1.0
    banner(f"pack_weights N={N} K={K}")
    Wp, a = bnn.pack_weights(dev(W))
    torch.cuda.synchronize()
    ld = Wp.shape[1]
    np.testing.assert_array_equal(host_u32(Wp), oracle.pack_signs(oracle.sign(W), ld=ld))
    a_ref = oracle.alpha(W)
    assert_f32_close(host(a), a_ref, what="alpha")


def test_pack_weights_repeatable(bnn):
    """alpha's |w| sums are split over the waves of a workgroup and added in a
    fixed order: repeated calls give the same bits, also on fresh buffers."""
    N, K = 300, 16384
    W = workloads.normal_f32(150, (N, K))
    Wd = dev(W)
    banner(f"pack_weights repeatability N={N} K={K}")
    runs = [bnn.pack_weights(Wd) for _ in range(3)]
    torch.cuda.synchronize()
    a0, p0 = host(runs[0][1]).view(np.uint32), host_u32(runs[0][0])
    for Wp, a in runs[1:]:
        np.testing.assert_array_equal(host(a).view(np.uint32), a0)
        np.testing.assert_array_equal(host_u32(Wp), p0)
    assert_f32_close(host(runs[0][1]), oracle.alpha(W), what="alpha")


@pytest.mark.parametrize("M,K,extra_ld", [(64, 1000, 0), (3, 70, 12), (1, 4096, 0), (1, 11008, 0),
                                          (100, 129, 4), (2, 5, 0),
                                          # short rows (ld 4 or 8): several rows per wave step,
                                          # with and without pad words stored apart, ragged row counts
                                          (1000, 64, 0), (333, 33, 0), (5, 1, 0), (257, 100, 0),
                                          (130, 256, 0), (77, 200, 0), (65, 60, 4), (3, 128, 4)])
def test_pack_activations_dense(bnn, M, K, extra_ld):
    X = _signs_with_edges(200 + K, (M, K))
    ld = bnn.padded_ld(K) + extra_ld
    out = torch.full((M, ld), -1, dtype=torch.int32, device="cuda")   # pads must be overwritten
    banner(f"pack_activations dense M={M} K={K} ld={ld}")
    bnn.pack_activations(dev(X), out=out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_u32(out), oracle.pack_signs(oracle.sign(X), ld=ld))


@pytest.mark.parametrize("M,K", [(37, 301), (1000, 64), (129, 250)])
def test_pack_unaligned_source_rows(bnn, M, K):
    # ld of the fp32 source not a multiple of 4 -> the scalar-load path
    big = workloads.normal_f32(250 + K, (M, K + 3))
    Xt = dev(big)[:, :K]
    assert Xt.stride(0) == K + 3
    banner("pack_activations scalar path")
    Xp = bnn.pack_activations(Xt)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_u32(Xp), oracle.pack_signs(oracle.sign(big[:, :K]), ld=Xp.shape[1]))


@pytest.mark.parametrize("B,H,W,C", [(2, 5, 4, 8), (1, 3, 3, 64), (2, 6, 7, 64), (1, 4, 4, 256), (2, 3, 4, 128), (1, 2, 3, 512), (1, 1, 5, 64),
                                     (2, 3, 5, 3), (1, 2, 2, 36), (3, 1, 1, 32)])
def test_pack_im2col3x3(bnn, B, H, W, C):
    X = _signs_with_edges(300 + C, (B, H, W, C))
    banner(f"pack im2col B={B} H={H} W={W} C={C}")
    Xp = bnn.pack_activations(dev(X), conv3x3=True)
    torch.cuda.synchronize()
    want = oracle.pack_signs(oracle.im2col_signs(X), ld=Xp.shape[1])
    np.testing.assert_array_equal(host_u32(Xp), want)


# ---------------------------------------------------------------- GEMM / GEMV
def _packed_pair(M, N, K, seed):
    X = workloads.normal_f32(seed, (M, K))
    W = workloads.normal_f32(seed + 1, (N, K))
    return X, W


GEMM_SHAPES = [(64, 256, 1000), (300, 100, 777), (257, 129, 1100), (5, 70, 4096), (1, 7, 33),
               (2, 300, 11008), (4, 33, 64), (512, 64, 576), (70, 1, 32), (1, 1, 1), (65, 96, 16),
               (256, 512, 8192),
               # 3 and 5 full 16-word chunks (the K loop takes two chunks per
               # iteration and ends on an odd one), the second with a tail
               (257, 64, 1536), (130, 70, 2600)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_xnor_gemm_dot_and_scale(bnn, M, N, K):
    X, W = _packed_pair(M, N, K, 400 + M + N + K)
    banner(f"xnor_gemm M={M} N={N} K={K}")
    Wp, a = bnn.pack_weights(dev(W))
    Xp = bnn.pack_activations(dev(X))
    D, Y = bnn.xnor_gemm(Xp, Wp, K, alpha=a, want_dot=True, want_scaled=True)
    torch.cuda.synchronize()
    D_ref, Y_ref, a_ref = oracle.binary_linear(X, W)
    np.testing.assert_array_equal(host(D), D_ref)
    assert_f32_close(host(a), a_ref, what="alpha")
    assert_f32_close(host(Y), Y_ref, what="Y")
    # Y must be exactly alpha * D with the GPU's own alpha (one rounding)
    np.testing.assert_array_equal(host(Y), (host(a)[None, :] * host(D).astype(np.float32)).astype(np.float32))


@pytest.mark.parametrize("tn", ["16", "32", "64"])
@pytest.mark.parametrize("M,N,K", [(300, 100, 777), (257, 129, 1100), (600, 200, 2304)])
def test_xnor_gemm_every_column_tile(bnn, tn, M, N, K):
    X, W = _packed_pair(M, N, K, 500 + M)
    old = os.environ.get("BNN_GEMM_TN")
    os.environ["BNN_GEMM_TN"] = tn
    try:
        banner(f"xnor_gemm TN={tn} M={M} N={N} K={K}")
        Wp, a = bnn.pack_weights(dev(W))
        Xp = bnn.pack_activations(dev(X))
        D, _ = bnn.xnor_gemm(Xp, Wp, K)
        torch.cuda.synchronize()
    finally:
        if old is None:
            os.environ.pop("BNN_GEMM_TN", None)
        else:
            os.environ["BNN_GEMM_TN"] = old
    np.testing.assert_array_equal(host(D), oracle.dot(oracle.sign(X), oracle.sign(W)))


@pytest.mark.parametrize("waves", ["4", "8", "16"])
@pytest.mark.parametrize("M,N,K", [(1100, 100, 777), (700, 70, 5000)])
def test_xnor_gemm_every_wave_count(bnn, waves, M, N, K, monkeypatch):
    """Workgroups of 4, 8 and 16 waves (BNN_GEMM_WAVES) on the LDS epilogue
    (K <= 4096) and on the direct one, with ragged row tiles (M = 1100 is one
    full and one partial 1024-row tile at 16 waves)."""
    monkeypatch.setenv("BNN_GEMM_WAVES", waves)
    X, W = _packed_pair(M, N, K, 520 + M)
    banner(f"xnor_gemm waves={waves} M={M} N={N} K={K}")
    Wp, a = bnn.pack_weights(dev(W))
    Xp = bnn.pack_activations(dev(X))
    D, Y = bnn.xnor_gemm(Xp, Wp, K, alpha=a, want_dot=True, want_scaled=True)
    torch.cuda.synchronize()
    D_ref, Y_ref, _ = oracle.binary_linear(X, W)
    np.testing.assert_array_equal(host(D), D_ref)
    np.testing.assert_array_equal(host(Y), (host(a)[None, :] * host(D).astype(np.float32)).astype(np.float32))


@pytest.mark.parametrize("epi", ["direct", "staged"])
@pytest.mark.parametrize("tn", ["8", "16", "32", "64"])
@pytest.mark.parametrize("M,N,K", [(300, 128, 576), (257, 192, 2304), (130, 64, 4200), (70, 96, 100)])
def test_xnor_gemm_every_epilogue_mode(bnn, epi, tn, M, N, K, monkeypatch):
    """The two epilogue modes (BNN_GEMM_EPI: from registers, staged through
    LDS) on every column tile, with D, Y = fl32(fl32(alpha D) + bias) + R; K
    tails of an 8-word chunk (576: 16 + 2, 4200: 128 + 8 + 2 words) and of
    single granules.  The oracle's alpha drives the epilogue."""
    monkeypatch.setenv("BNN_GEMM_EPI", epi)
    monkeypatch.setenv("BNN_GEMM_TN", tn)
    X, W = _packed_pair(M, N, K, 560 + M + K)
    R = workloads.normal_f32(561 + K, (M, N))
    bias = workloads.normal_f32(562 + N, (N,))
    a_ref = oracle.alpha(W)
    Wp, _ = bnn.pack_weights(dev(W))
    Xp = bnn.pack_activations(dev(X))
    banner(f"xnor_gemm epilogue={epi} TN={tn} M={M} N={N} K={K}")
    out = bnn.linear_fused(Xp, Wp, K, bnn.EPI_DOT_I32 | bnn.EPI_SCALE_F32 | bnn.EPI_BIAS_F32 | bnn.EPI_RESIDUAL_F32,
                           alpha=dev(a_ref), bias=dev(bias), R=dev(R))
    plain = bnn.linear_fused(Xp, Wp, K, bnn.EPI_SCALE_F32, alpha=dev(a_ref))
    torch.cuda.synchronize()
    D_ref = oracle.dot(oracle.sign(X), oracle.sign(W))
    np.testing.assert_array_equal(host(out["D"]), D_ref)
    np.testing.assert_array_equal(host(out["Y"]).view(np.uint32),
                                  oracle.scale_bias_residual(D_ref, a_ref, bias, R).view(np.uint32))
    np.testing.assert_array_equal(host(plain["Y"]).view(np.uint32), oracle.scale(D_ref, a_ref).view(np.uint32))


@pytest.mark.parametrize("K", [32767, 32768, 40000])
def test_xnor_gemm_staged_long_rows(bnn, K):
    """The staged epilogue with rows past 2^15 bits; rows of all +1 or all -1
    reach |D| = K."""
    M, N = 130, 64
    X, W = _packed_pair(M, N, K, 590 + K)
    X[0, :] = 1.0
    X[1, :] = -1.0
    W[0, :] = 1.0
    a_ref = oracle.alpha(W)
    Wp, _ = bnn.pack_weights(dev(W))
    Xp = bnn.pack_activations(dev(X))
    banner(f"xnor_gemm staged K={K}")
    out = bnn.linear_fused(Xp, Wp, K, bnn.EPI_DOT_I32 | bnn.EPI_SCALE_F32, alpha=dev(a_ref))
    torch.cuda.synchronize()
    D_ref = oracle.dot(oracle.sign(X), oracle.sign(W))
    assert D_ref[0, 0] == K and D_ref[1, 0] == -K
    np.testing.assert_array_equal(host(out["D"]), D_ref)
    np.testing.assert_array_equal(host(out["Y"]).view(np.uint32), oracle.scale(D_ref, a_ref).view(np.uint32))


@pytest.mark.parametrize("prefetch", ["1", "0"])
@pytest.mark.parametrize("epi", ["direct", "staged"])
@pytest.mark.parametrize("C,B,H,Wd,Co", [(64, 2, 5, 7, 96), (128, 2, 5, 7, 96), (256, 2, 5, 7, 96),
                                         (512, 2, 5, 7, 96), (64, 3, 9, 11, 80), (256, 3, 9, 11, 64)])
def test_conv3x3_every_epilogue_mode(bnn, epi, prefetch, C, B, H, Wd, Co, monkeypatch):
    """The implicit-im2col conv with each epilogue mode, with and without the
    residual prefetch (C = 512: K = 4608, 144 words per row; 297 pixels: two
    row tiles, the second ragged)."""
    monkeypatch.setenv("BNN_GEMM_EPI", epi)
    monkeypatch.setenv("BNN_CONV_PREFETCH", prefetch)
    X = workloads.normal_f32(570 + C, (B, H, Wd, C))
    Wt = workloads.normal_f32(571 + C, (Co, 3, 3, C))
    R = workloads.normal_f32(572 + C, (B * H * Wd, Co))
    M, K = B * H * Wd, 9 * C
    Wf = np.ascontiguousarray(Wt.reshape(Co, K))
    a_ref = oracle.alpha(Wf)
    S = oracle.sign(X.reshape(M, C)).reshape(X.shape)
    D_ref = oracle.dot(oracle.im2col_pm1(S), oracle.sign(Wf))
    Ximg = bnn.pack_activations(dev(X.reshape(M, C)))
    Wp, _ = bnn.pack_weights(dev(Wf))
    banner(f"conv3x3 epilogue={epi} prefetch={prefetch} C={C} B={B} H={H} W={Wd} Co={Co}")
    out = bnn.conv3x3_fused(Ximg, Wp, (B, H, Wd, C), bnn.EPI_DOT_I32 | bnn.EPI_SCALE_F32 | bnn.EPI_RESIDUAL_F32,
                            alpha=dev(a_ref), R=dev(R))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out["D"]), D_ref)
    np.testing.assert_array_equal(host(out["Y"]).view(np.uint32), oracle.scale_residual(D_ref, a_ref, R).view(np.uint32))


@pytest.mark.parametrize("u", ["1", "2", "4"])
def test_gemv_every_row_step_count(bnn, u, monkeypatch):
    """The GEMV's row steps per wave (BNN_GEMV_U) on a matrix tall enough that
    the unrolled kernel runs (K = 16384: one row per lane group of 64; at
    N = 32773 a wave takes 4 rows at U = 4, with a ragged last wave).  Random
    packed words with no pad bits (K is a multiple of 32); the oracle checks
    400 sampled rows, the invariants hold on every row."""
    monkeypatch.setenv("BNN_GEMV_U", u)
    N, K = 32773, 16384
    kw = K // 32
    Wh = workloads.random_words(530, (N, kw))
    Xh = workloads.random_words(532, (1, kw))
    Wp, Xp = dev(Wh.view(np.int32)), dev(Xh.view(np.int32))
    banner(f"xnor_gemv U={u} N={N} K={K}")
    D, _ = bnn.xnor_gemm(Xp, Wp, K)
    torch.cuda.synchronize()
    d = host(D)[0]
    rows = np.unique(np.concatenate([np.arange(8), np.arange(N - 8, N),
                                     np.random.default_rng(531).integers(0, N, 384)]))
    want = oracle.dot(oracle.unpack_signs(Xh, K), oracle.unpack_signs(Wh[rows], K))[0]
    np.testing.assert_array_equal(d[rows], want)
    assert np.all(np.abs(d) <= K) and np.all((d - K) % 2 == 0)


@pytest.mark.parametrize("M", [1, 3, 4])
@pytest.mark.parametrize("K", [20000, 32768, 40000, 65504, 65536, 65537])
def test_gemv_granules_per_lane(bnn, M, K):
    """GEMV rows wider than 64 lanes x 2 granules: 4 granules per lane
    (K = 20000, 32768) and 8 (K = 40000 up to 65536, the widest row the GEMV
    takes); K = 65537 is one word past it and runs the GEMM instead."""
    N = 130
    X, W = _packed_pair(M, N, K, 560 + K + M)
    banner(f"xnor_gemv M={M} N={N} K={K}")
    Wp, a = bnn.pack_weights(dev(W))
    Xp = bnn.pack_activations(dev(X))
    D, Y = bnn.xnor_gemm(Xp, Wp, K, alpha=a, want_dot=True, want_scaled=True)
    torch.cuda.synchronize()
    D_ref, _, _ = oracle.binary_linear(X, W)
    np.testing.assert_array_equal(host(D), D_ref)
    np.testing.assert_array_equal(host(Y), (host(a)[None, :] * host(D).astype(np.float32)).astype(np.float32))


def test_xnor_gemm_largest_k(bnn):
    """K = 2^24, the largest K the C ABI accepts (BNN_MAX_K): |D| reaches K,
    which (float)D still holds exactly.  Weight rows: X's own signs (D = K),
    their negation with zeros made negative too (D = -K), and a random row."""
    K = 1 << 24
    X = workloads.normal_f32(540, (2, K))
    W = np.empty((3, K), np.float32)
    W[0] = X[0]
    W[1] = np.where(X[0] >= 0, np.float32(-1.0), np.float32(1.0))
    W[2] = workloads.normal_f32(541, (1, K))[0]
    banner(f"xnor_gemm M=2 N=3 K={K}")
    Wp, a = bnn.pack_weights(dev(W))
    Xp = bnn.pack_activations(dev(X))
    D, Y = bnn.xnor_gemm(Xp, Wp, K, alpha=a, want_dot=True, want_scaled=True)
    torch.cuda.synchronize()
    D_ref, Y_ref, a_ref = oracle.binary_linear(X, W)
    assert D_ref[0, 0] == K and D_ref[0, 1] == -K
    np.testing.assert_array_equal(host(D), D_ref)
    assert_f32_close(host(a), a_ref, what="alpha")
    np.testing.assert_array_equal(host(Y), (host(a)[None, :] * host(D).astype(np.float32)).astype(np.float32))


def test_xnor_gemm_strided_outputs(bnn):
    M, N, K = 130, 70, 500
    X, W = _packed_pair(M, N, K, 600)
    Wp, a = bnn.pack_weights(dev(W))
    Xp = bnn.pack_activations(dev(X))
    Dbig = torch.full((M, N + 5), 7, dtype=torch.int32, device="cuda")
    Ybig = torch.full((M, N + 3), 7.0, dtype=torch.float32, device="cuda")
    banner("xnor_gemm strided outputs")
    bnn.xnor_gemm(Xp, Wp, K, alpha=a, want_scaled=True, D=Dbig[:, :N], Y=Ybig[:, :N])
    torch.cuda.synchronize()
    D_ref, Y_ref, _ = oracle.binary_linear(X, W)
    np.testing.assert_array_equal(host(Dbig)[:, :N], D_ref)
    assert np.all(host(Dbig)[:, N:] == 7), "write outside the output columns"
    assert np.all(host(Ybig)[:, N:] == 7.0), "write outside the output columns"
    assert_f32_close(host(Ybig)[:, :N], Y_ref, what="Y")


def test_gemm_extreme_values(bnn):
    # all +1 against all -1 and identical rows: D = -K and +K exactly
    K = 1000
    X = np.ones((3, K), np.float32)
    W = np.stack([np.ones(K, np.float32), -np.ones(K, np.float32), np.zeros(K, np.float32)])
    Wp, a = bnn.pack_weights(dev(W))
    Xp = bnn.pack_activations(dev(X))
    D, Y = bnn.xnor_gemm(Xp, Wp, K, alpha=a, want_scaled=True)
    torch.cuda.synchronize()
    assert host(D).tolist() == [[K, -K, K]] * 3
    assert host(a).tolist() == [1.0, 1.0, 0.0]
    assert host(Y).tolist() == [[K, -K, 0.0]] * 3


# ---------------------------------------------------------------- fused epilogues
@pytest.mark.parametrize("M,N,K", [(64, 256, 1000), (300, 100, 777), (3, 40, 64), (1, 33, 4096),
                                   (257, 4096, 4096), (100, 31, 100)])
def test_fused_threshold_pack(bnn, M, N, K):
    X, W = _packed_pair(M, N, K, 700 + N)
    g, b, mu, var, eps = workloads.bn_params(701 + N, N)
    banner(f"fused thresh-pack M={M} N={N} K={K}")
    Wp, a = bnn.pack_weights(dev(W))
    Xp = bnn.pack_activations(dev(X))
    a_ref = oracle.alpha(W)
    tau, d = bnn.fold_bn_thresholds(g, b, mu, var, eps, a_ref)   # the library's fold of the oracle's alpha
    ldo = bnn.padded_ld(N) + 4
    Op = torch.full((M, ldo), -1, dtype=torch.int32, device="cuda")
    out = bnn.linear_fused(Xp, Wp, K, bnn.EPI_THRESH_PACK | bnn.EPI_DOT_I32,
                           tau=dev(tau), dir=dev(d), Op=Op)
    torch.cuda.synchronize()
    D_ref = oracle.dot(oracle.sign(X), oracle.sign(W))
    np.testing.assert_array_equal(host(out["D"]), D_ref)
    s_ref, _ = oracle.bn_next_sign(D_ref, a_ref, g, b, mu, var, eps)   # BatchNorm then sign, exactly
    np.testing.assert_array_equal(host_u32(Op), oracle.pack_signs(s_ref, ld=ldo))
    np.testing.assert_array_equal(host(a).view(np.uint32), a_ref.view(np.uint32))


@pytest.mark.parametrize("tn", ["8", "16", "32", "64"])
@pytest.mark.parametrize("M,N,K", [(300, 100, 777), (130, 20, 64), (70, 40, 4096), (257, 96, 200)])
def test_fused_threshold_pack_every_column_tile(bnn, tn, M, N, K):
    X, W = _packed_pair(M, N, K, 750 + N + int(tn))
    g, b, mu, var, eps = workloads.bn_params(751 + N, N)
    Wp, a = bnn.pack_weights(dev(W))
    Xp = bnn.pack_activations(dev(X))
    a_ref = oracle.alpha(W)
    tau, d = bnn.fold_bn_thresholds(g, b, mu, var, eps, a_ref)
    ldo = bnn.padded_ld(N) + 4
    Op = torch.full((M, ldo), -1, dtype=torch.int32, device="cuda")
    old = os.environ.get("BNN_GEMM_TN")
    os.environ["BNN_GEMM_TN"] = tn
    try:
        banner(f"fused thresh-pack TN={tn} M={M} N={N} K={K}")
        bnn.linear_fused(Xp, Wp, K, bnn.EPI_THRESH_PACK, tau=dev(tau), dir=dev(d), Op=Op)
        torch.cuda.synchronize()
    finally:
        if old is None:
            os.environ.pop("BNN_GEMM_TN", None)
        else:
            os.environ["BNN_GEMM_TN"] = old
    D_ref = oracle.dot(oracle.sign(X), oracle.sign(W))
    s_ref, _ = oracle.bn_next_sign(D_ref, a_ref, g, b, mu, var, eps)
    np.testing.assert_array_equal(host_u32(Op), oracle.pack_signs(s_ref, ld=ldo))


@pytest.mark.parametrize("tn", ["8", "16", "32", "64"])
@pytest.mark.parametrize("M,N,K", [(300, 64, 576), (257, 128, 2304), (65, 96, 100)])
def test_fused_epilogue_every_column_tile(bnn, tn, M, N, K):
    """DOT + SCALE + RESIDUAL through the staged (LDS) epilogue for small K."""
    X, W = _packed_pair(M, N, K, 850 + N + int(tn))
    R = workloads.normal_f32(852 + K, (M, N))
    Wp, a = bnn.pack_weights(dev(W))
    Xp = bnn.pack_activations(dev(X))
    old = os.environ.get("BNN_GEMM_TN")
    os.environ["BNN_GEMM_TN"] = tn
    try:
        banner(f"fused residual TN={tn} M={M} N={N} K={K}")
        out = bnn.linear_fused(Xp, Wp, K, bnn.EPI_SCALE_F32 | bnn.EPI_RESIDUAL_F32 | bnn.EPI_DOT_I32,
                               alpha=a, R=dev(R))
        torch.cuda.synchronize()
    finally:
        if old is None:
            os.environ.pop("BNN_GEMM_TN", None)
        else:
            os.environ["BNN_GEMM_TN"] = old
    D_ref = oracle.dot(oracle.sign(X), oracle.sign(W))
    a_ref = oracle.alpha(W)
    np.testing.assert_array_equal(host(out["D"]), D_ref)
    np.testing.assert_array_equal(host(a).view(np.uint32), a_ref.view(np.uint32))
    np.testing.assert_array_equal(host(out["Y"]), oracle.scale_residual(D_ref, a_ref, R))


@pytest.mark.parametrize("M,N,K", [(300, 64, 576), (50, 256, 2304), (2, 64, 576), (129, 70, 333)])
def test_fused_scale_residual(bnn, M, N, K):
    X, W = _packed_pair(M, N, K, 800 + K)
    R = workloads.normal_f32(802 + K, (M, N))
    banner(f"fused residual M={M} N={N} K={K}")
    Wp, a = bnn.pack_weights(dev(W))
    Xp = bnn.pack_activations(dev(X))
    out = bnn.linear_fused(Xp, Wp, K, bnn.EPI_SCALE_F32 | bnn.EPI_RESIDUAL_F32 | bnn.EPI_DOT_I32,
                           alpha=a, R=dev(R))
    torch.cuda.synchronize()
    D_ref = oracle.dot(oracle.sign(X), oracle.sign(W))
    np.testing.assert_array_equal(host(out["D"]), D_ref)
    a_ref = oracle.alpha(W)
    Y_ref = oracle.scale_residual(D_ref, a_ref, R)
    scale = np.abs(a_ref[None, :] * D_ref) + np.abs(R)
    assert_f32_close(host(out["Y"]), Y_ref, scale=scale, what="Y residual")
    # alpha and Y are in fact bit-exact
    np.testing.assert_array_equal(host(a).view(np.uint32), a_ref.view(np.uint32))
    np.testing.assert_array_equal(host(out["Y"]).view(np.uint32), Y_ref.view(np.uint32))


def test_fused_residual_in_place(bnn):
    M, N, K = 257, 64, 576
    X, W = _packed_pair(M, N, K, 900)
    R = workloads.normal_f32(901, (M, N))
    Wp, a = bnn.pack_weights(dev(W))
    Xp = bnn.pack_activations(dev(X))
    Rd = dev(R)
    banner("fused residual in place")
    bnn.linear_fused(Xp, Wp, K, bnn.EPI_SCALE_F32 | bnn.EPI_RESIDUAL_F32, alpha=a, R=Rd, Y=Rd)
    torch.cuda.synchronize()
    D_ref = oracle.dot(oracle.sign(X), oracle.sign(W))
    a_ref = oracle.alpha(W)
    np.testing.assert_array_equal(host(a).view(np.uint32), a_ref.view(np.uint32))
    np.testing.assert_array_equal(host(Rd), oracle.scale_residual(D_ref, a_ref, R))


# ---------------------------------------------------------------- FP first / last layers
@pytest.mark.parametrize("M,N,K", [(64, 128, 784), (100, 70, 33), (1, 32, 1), (130, 4096, 784),
                                   # 16-byte rows (matrix-core path) with a K tail inside the
                                   # last 16-wide chunk and partial row / column tiles
                                   (70, 100, 36), (33, 65, 20), (1, 17, 4), (40, 64, 1000)])
def test_dense_f32_sign_pack(bnn, M, N, K):
    X = workloads.uniform01_f32(1000 + K, (M, K))
    W = workloads.normal_f32(1001 + K, (N, K))
    banner(f"dense sign-pack M={M} N={N} K={K}")
    Op = bnn.dense_f32_sign_pack(dev(X), dev(W))
    torch.cuda.synchronize()
    H = oracle.dense_f64(X, W)
    # the kernel's double sum may run in another order: any order is within
    # K 2^-52 sum|x w| of the exact sum, so outside that bound the sign is unique
    bound = K * 2.0**-52 * (np.abs(X).astype(np.float64) @ np.abs(W).astype(np.float64).T)
    assert int((np.abs(H) <= bound).sum()) == 0, "near-ties in the test data"
    s = np.where(H >= 0.0, 1, -1).astype(np.int8)
    np.testing.assert_array_equal(host_u32(Op), oracle.pack_signs(s, ld=Op.shape[1]))


@pytest.mark.parametrize("tile", ["1,2", "1,4", "2,2", "2,4", "4,2", "4,4"])
def test_dense_f32_sign_pack_every_tile(bnn, tile, monkeypatch):
    """Every wave tile of the fp64 matrix-core first layer (BNN_DENSE_TILE
    "BM,BN" 16-row / 16-column blocks), with partial row and column tiles."""
    monkeypatch.setenv("BNN_DENSE_TILE", tile)
    M, N, K = 77, 150, 784
    X = workloads.uniform01_f32(1300, (M, K))
    W = workloads.normal_f32(1301, (N, K))
    banner(f"dense sign-pack tile {tile} M={M} N={N} K={K}")
    Op = bnn.dense_f32_sign_pack(dev(X), dev(W))
    torch.cuda.synchronize()
    H = oracle.dense_f64(X, W)
    bound = K * 2.0**-52 * (np.abs(X).astype(np.float64) @ np.abs(W).astype(np.float64).T)
    assert int((np.abs(H) <= bound).sum()) == 0, "near-ties in the test data"
    s = np.where(H >= 0.0, 1, -1).astype(np.int8)
    np.testing.assert_array_equal(host_u32(Op), oracle.pack_signs(s, ld=Op.shape[1]))


# 4 rows per workgroup (ragged M: 7, 130, 5, 1), 16 columns per pass (N = 17,
# 33: a second and third pass), K slices of 64 per wave (ragged K, K < 64)
@pytest.mark.parametrize("M,N,K", [(64, 10, 4096), (7, 3, 33), (130, 17, 1000), (1, 10, 4096), (5, 33, 257),
                                   (3, 1, 4), (1024, 10, 4096)])
def test_dense_binact_f32(bnn, M, N, K):
    rng = np.random.default_rng(1100 + K)
    s = np.where(rng.random((M, K)) < 0.5, 1, -1).astype(np.int8)
    W = workloads.normal_f32(1101 + K, (N, K))
    Xp = dev(oracle.pack_signs(s, ld=bnn.padded_ld(K)).view(np.int32))
    banner(f"dense binact M={M} N={N} K={K}")
    Y = bnn.dense_binact_f32(Xp, dev(W), K)
    torch.cuda.synchronize()
    Y_ref = oracle.dense_pm1_f32out(s, W)
    # double sums in another order differ by <= ~2K * 2^-53 * sum|W|; after the
    # fp32 rounding that is within 1e-6 relative, or 1e-9 * sum|W| absolute
    assert_f32_close(host(Y), Y_ref, scale=1e-3 * np.abs(W).sum(axis=1)[None, :], what="logits")


def test_deterministic_repeat(bnn):
    M, N, K = 300, 200, 1000
    X, W = _packed_pair(M, N, K, 1200)
    Wd, Xd = dev(W), dev(X)
    outs = []
    for _ in range(2):
        Wp, a = bnn.pack_weights(Wd)
        Xp = bnn.pack_activations(Xd)
        D, Y = bnn.xnor_gemm(Xp, Wp, K, alpha=a, want_scaled=True)
        torch.cuda.synchronize()
        outs.append((host_u32(Wp), host(a), host(D), host(Y)))
    for u, v in zip(outs[0], outs[1]):
        np.testing.assert_array_equal(u, v)
