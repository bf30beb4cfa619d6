"""GPU parity of the binary-weight x INT8-activation path, the per-tensor
weight scale and the bias epilogue against the CPU oracle.

Sources: page "Extreme Quantization: Binary, Ternary & 1-bit LLMs",
"Binary Neural Networks" eq. (1)-(2) (binary weights add or subtract the
activations), "BitNet: 1-bit Transformer" (INT8 activations; eq. (8), one
scale per matrix); page "First Principles", "y = Wx + b" (bias).

Bar: int8 codes, bit planes (with pads), row sums and int32 dot products
bit-exact; fp32 outputs computed from identical inputs by the same rounded
operations, so bit-exact as well (and never worse than 1e-6 relative); the
per-tensor scale (fp64 sums in a different order) within 1e-6 relative.
All calls go through the C ABI."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import require_gpu, banner, dev, host, host_u32, assert_f32_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bnn():
    require_gpu()
    import xnor_popcount_gemm_amd as m
    m.lib()
    return m


def _bits_equal(got, want, what):
    # bit patterns equal; any NaN matches any NaN (the host and the GPU
    # produce different default NaN payloads)
    gf, wf = np.asarray(got, np.float32), np.asarray(want, np.float32)
    g, w = gf.view(np.uint32), wf.view(np.uint32)
    bad = (g != w) & ~(np.isnan(gf) & np.isnan(wf))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} differ; first {idx.tolist()} "
                             f"got {np.asarray(got)[tuple(idx.T)]} want {np.asarray(want)[tuple(idx.T)]}")


def _act_rows(seed, M, K):
    """fp32 activation rows N(0,1) with edge rows: zeros, NaN/inf/denormal
    entries, and exact .5 ties (amax 254 gives the scale 0.5 exactly)."""
    X = workloads.normal_f32(seed, (M, K))
    if M >= 3:
        X[0, :] = 0.0
        X[1] = workloads.inject_edge_values(X[1:2], seed + 1, 0.05)[0]
        X[2, :] = np.float32(7.0) * np.sign(X[2, :])
        X[2, 0] = np.float32(254.0)
    if M >= 4:
        # only denormals and zeros: 127 / amax overflows to +inf
        X[3, :] = np.where(np.arange(K) % 3 == 0, 0.0, np.float32(1e-40) * np.sign(X[3, :]))
    return X


def _full_range_i8(seed, M, K):
    rng = np.random.default_rng(seed)
    Q = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    Q[:, 0] = -128
    return Q


# ---------------------------------------------------------------- quantize + planes
@pytest.mark.parametrize("M,K", [(3, 1), (4, 31), (5, 100), (3, 1000), (2, 4096), (3, 4097), (1, 11008),
                                 (64, 576), (7, 16385)])
def test_quantize_act_i8_matches_oracle(bnn, M, K):
    X = _act_rows(7000 + K, M, K)
    banner(f"quantize_act_i8 M={M} K={K}")
    out = bnn.quantize_act_i8(dev(X))
    torch.cuda.synchronize()
    Q_ref, s_ref = oracle.quantize_absmax_i8(X)
    np.testing.assert_array_equal(host(out["Xq"]), Q_ref)
    _bits_equal(host(out["xscale"]), s_ref, "xscale")
    ld = out["Xb"].shape[2]
    P_ref, xs_ref = oracle.pack_planes_i8(Q_ref, ld=ld)
    np.testing.assert_array_equal(host_u32(out["Xb"]), P_ref)
    np.testing.assert_array_equal(host(out["xsum"]), xs_ref)


def test_quantize_unaligned_source_and_single_outputs(bnn):
    M, K = 5, 301
    big = workloads.normal_f32(7101, (M, K + 3))
    Xt = dev(big)[:, :K]
    banner("quantize_act_i8 scalar path, int8 only / planes only")
    a = bnn.quantize_act_i8(Xt, want_planes=False)
    b = bnn.quantize_act_i8(Xt, want_int8=False)
    torch.cuda.synchronize()
    Q_ref, s_ref = oracle.quantize_absmax_i8(big[:, :K])
    np.testing.assert_array_equal(host(a["Xq"]), Q_ref)
    assert a["Xb"] is None and b["Xq"] is None
    P_ref, xs_ref = oracle.pack_planes_i8(Q_ref, ld=b["Xb"].shape[2])
    np.testing.assert_array_equal(host_u32(b["Xb"]), P_ref)
    np.testing.assert_array_equal(host(b["xsum"]), xs_ref)
    _bits_equal(host(b["xscale"]), s_ref, "xscale")
    banner("quantize_act_i8 int8 + row sums, no planes")
    c = bnn.quantize_act_i8(Xt, want_planes=False, want_xsum=True)
    torch.cuda.synchronize()
    assert c["Xb"] is None
    np.testing.assert_array_equal(host(c["Xq"]), Q_ref)
    np.testing.assert_array_equal(host(c["xsum"]), xs_ref)


@pytest.mark.parametrize("M,K,pad", [(1, 1, 0), (2, 33, 4), (3, 4096, 0), (5, 1000, 8), (1, 11008, 0),
                                     (4, 131072, 0)])
def test_pack_act_i8_matches_oracle(bnn, M, K, pad):
    Q = _full_range_i8(7200 + K, M, K)
    banner(f"pack_act_i8 M={M} K={K}")
    Qd = torch.zeros((M, bnn.i8_ld(K) + pad), dtype=torch.int8, device="cuda")
    Qd[:, :K] = dev(Q)
    Xb, xsum = bnn.pack_act_i8(Qd[:, :K])
    torch.cuda.synchronize()
    P_ref, xs_ref = oracle.pack_planes_i8(Q, ld=Xb.shape[2])
    np.testing.assert_array_equal(host_u32(Xb), P_ref)
    np.testing.assert_array_equal(host(xsum), xs_ref)


# ---------------------------------------------------------------- GEMV (bit planes) and GEMM (MFMA)
def _weights(seed, N, K):
    W = workloads.normal_f32(seed, (N, K))
    return W, oracle.sign(W), oracle.alpha(W)


def _check_linear(bnn, Q, xscale, W, ws, a, *, path, per_tensor=False):
    """Run D and Y through bnn_bwn_i8_linear on the given path and compare."""
    M, K = Q.shape
    N = W.shape[0]
    Wp, _ = bnn.pack_weights(dev(W), alpha=False)
    alpha = np.atleast_1d(oracle.alpha_tensor(W)) if per_tensor else a
    flags = bnn.EPI_DOT_I32 | bnn.EPI_SCALE_F32 | (bnn.EPI_ALPHA_TENSOR if per_tensor else 0)
    kw = {}
    if path == "gemv":
        Xb, xsum = bnn.pack_act_i8(dev(Q))
        kw = dict(Xb=Xb, xsum=xsum)
    else:
        Qd = torch.zeros((M, bnn.i8_ld(K)), dtype=torch.int8, device="cuda")
        Qd[:, :K] = dev(Q)
        kw = dict(Xq=Qd[:, :K])
        if path == "gemm_xsum":                     # row sums given: the 0/1 weight expansion
            kw["xsum"] = dev(Q.astype(np.int64).sum(axis=1).astype(np.int32))
    xs_d = dev(xscale) if xscale is not None else None
    out = bnn.bwn_i8_linear(Wp, K, flags, alpha=dev(alpha), xscale=xs_d, **kw)
    torch.cuda.synchronize()
    D_ref = oracle.dot_i8(Q, ws)
    np.testing.assert_array_equal(host(out["D"]), D_ref)
    if xscale is not None:
        Y_ref = oracle.scale_i8(D_ref, alpha, xscale)
    else:
        Y_ref = oracle.scale(D_ref, np.broadcast_to(alpha, (N,)).astype(np.float32))
    _bits_equal(host(out["Y"]), Y_ref, "Y")
    assert_f32_close(host(out["Y"]), Y_ref, what="Y")


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (1, 7, 33), (1, 300, 1000), (2, 129, 4096), (1, 64, 11008),
                                   (2, 33, 16384), (1, 5, 32768), (1, 2000, 100), (2, 1, 8192)])
def test_bwn_i8_gemv_matches_oracle(bnn, M, N, K):
    W, ws, a = _weights(7300 + K, N, K)
    X = _act_rows(7400 + K, M, K)
    Q, xs = oracle.quantize_absmax_i8(X)
    banner(f"bwn_i8 gemv quantized M={M} N={N} K={K}")
    _check_linear(bnn, Q, xs, W, ws, a, path="gemv")
    Qf = _full_range_i8(7500 + K, M, K)
    banner(f"bwn_i8 gemv full-range int8 M={M} N={N} K={K}")
    _check_linear(bnn, Qf, None, W, ws, a, path="gemv", per_tensor=True)


@pytest.mark.parametrize("shape", ["5,3", "5,4", "6,2", "6,4"])
def test_bwn_i8_gemv_every_lane_shape(bnn, shape, monkeypatch):
    """The GEMV's lane-group shapes (BNN_I8_SHAPE "glog2,cpl") on a row that
    each of them covers (K = 11008: 86 granules), including a ragged last row
    group (N = 301)."""
    monkeypatch.setenv("BNN_I8_SHAPE", shape)
    N, K = 301, 11008
    W, ws, a = _weights(7700, N, K)
    X = _act_rows(7701, 1, K)
    Q, xs = oracle.quantize_absmax_i8(X)
    banner(f"bwn_i8 gemv lane shape {shape} N={N} K={K}")
    _check_linear(bnn, Q, xs, W, ws, a, path="gemv")


@pytest.mark.parametrize("path", ["gemm", "gemm_xsum"])
def test_bwn_i8_gemm_largest_k(bnn, path):
    """K = 2^17, the largest K the INT8 path accepts (BNN_MAX_K_I8): an
    all -128 activation row against an all-negative weight row gives
    D = 128 * 2^17 = 2^24, the largest value (float)D still holds exactly."""
    M, N, K = 3, 40, 1 << 17
    W, _, _ = _weights(7950, N, K)
    W[0, :] = np.float32(-1.0)
    ws, a = oracle.sign(W), oracle.alpha(W)
    Q = _full_range_i8(7951, M, K)
    Q[0, :] = -128
    assert oracle.dot_i8(Q[:1], ws[:1])[0, 0] == 1 << 24
    banner(f"bwn_i8 {path} M={M} N={N} K={K}")
    _check_linear(bnn, Q, None, W, ws, a, path=path)


@pytest.mark.parametrize("u", ["1", "2"])
def test_bwn_i8_gemv_every_row_step_count(bnn, u, monkeypatch):
    """Row steps per wave (BNN_GEMV_U) on a matrix tall enough that the
    unrolled kernel runs (K = 4096: 4 rows per wave step; N = 65541 gives
    16386 steps, a ragged last wave at U = 2).  Random packed weight words
    with no pad bits (K is a multiple of 32); the oracle checks 400 sampled
    rows, the bound |D| <= sum |q| holds on every row."""
    monkeypatch.setenv("BNN_GEMV_U", u)
    N, K = 65541, 4096
    Wh = workloads.random_words(7900, (N, K // 32))
    Wp = dev(Wh.view(np.int32))
    X = _act_rows(7901, 1, K)
    Q, xs = oracle.quantize_absmax_i8(X)
    a = workloads.uniform01_f32(7902, (N,)) + np.float32(0.5)
    Xb, xsum = bnn.pack_act_i8(dev(Q))
    banner(f"bwn_i8 gemv U={u} N={N} K={K}")
    out = bnn.bwn_i8_linear(Wp, K, bnn.EPI_DOT_I32 | bnn.EPI_SCALE_F32, alpha=dev(a), xscale=dev(xs),
                            Xb=Xb, xsum=xsum)
    torch.cuda.synchronize()
    d, y = host(out["D"])[0], host(out["Y"])[0]
    rows = np.unique(np.concatenate([np.arange(8), np.arange(N - 8, N),
                                     np.random.default_rng(7903).integers(0, N, 384)]))
    D_ref = oracle.dot_i8(Q, oracle.unpack_signs(Wh[rows], K))
    np.testing.assert_array_equal(d[rows], D_ref[0])
    Y_ref = oracle.scale_i8(D_ref, a[rows], xs)
    _bits_equal(y[rows][None, :], Y_ref, "Y")
    assert np.all(np.abs(d) <= np.abs(Q.astype(np.int64)).sum())


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 64), (16, 16, 63), (64, 128, 1000), (130, 257, 100),
                                   (200, 300, 4096), (3, 1000, 11008), (129, 129, 129), (1, 64, 65),
                                   (600, 200, 1000), (513, 129, 130), (257, 385, 192)])
@pytest.mark.parametrize("path", ["gemm", "gemm_xsum"])
def test_bwn_i8_gemm_matches_oracle(bnn, M, N, K, path):
    W, ws, a = _weights(7600 + K, N, K)
    X = _act_rows(7700 + K, M, K)
    Q, xs = oracle.quantize_absmax_i8(X)
    banner(f"bwn_i8 {path} quantized M={M} N={N} K={K}")
    _check_linear(bnn, Q, xs, W, ws, a, path=path)
    Qf = _full_range_i8(7800 + K, M, K)
    banner(f"bwn_i8 {path} full-range int8 M={M} N={N} K={K}")
    _check_linear(bnn, Qf, None, W, ws, a, path=path, per_tensor=True)


@pytest.mark.parametrize("path", ["gemv", "gemm", "gemm_xsum"])
def test_bwn_i8_extreme_sums(bnn, path):
    # |D| reaches 128 K at the largest K: every activation -128, every weight -1
    M, N, K = (1 if path == "gemv" else 4), 8, 32768 if path == "gemv" else 131072
    # (with row sums: xsum = -2^24 and D = xsum - 2 sum q w reaches +2^24)
    Q = np.full((M, K), -128, np.int8)
    W = -np.ones((N, K), np.float32)
    W[1::2] *= -1.0                                  # odd rows +1
    ws = oracle.sign(W)
    banner(f"bwn_i8 {path} extremes K={K}")
    _check_linear(bnn, Q, None, W, ws, oracle.alpha(W), path=path)


def test_bwn_i8_strided_outputs_and_dot_only(bnn):
    M, N, K = 2, 100, 3000
    W, ws, a = _weights(7900, N, K)
    Q = _full_range_i8(7901, M, K)
    Wp, _ = bnn.pack_weights(dev(W), alpha=False)
    Xb, xsum = bnn.pack_act_i8(dev(Q))
    Qd = torch.zeros((M, bnn.i8_ld(K)), dtype=torch.int8, device="cuda")
    Qd[:, :K] = dev(Q)
    D_ref = oracle.dot_i8(Q, ws)
    for kw in (dict(Xb=Xb, xsum=xsum), dict(Xq=Qd[:, :K]), dict(Xq=Qd[:, :K], xsum=xsum, M=M)):
        Dbig = torch.full((M, N + 13), -7, dtype=torch.int32, device="cuda")
        banner(f"bwn_i8 strided D {list(kw)}")
        bnn.bwn_i8_linear(Wp, K, bnn.EPI_DOT_I32, D=Dbig[:, :N], **kw)
        torch.cuda.synchronize()
        h = host(Dbig)
        np.testing.assert_array_equal(h[:, :N], D_ref)
        assert (h[:, N:] == -7).all()


def test_bwn_i8_chain_from_fp32(bnn):
    """fp32 activations -> INT8 (quantize on the GPU) -> binary-weight linear,
    on the decode shape [11008, 4096] and its transpose."""
    for N, K in ((11008, 4096), (4096, 11008)):
        X = workloads.normal_f32(8000 + K, (1, K))
        W = workloads.normal_f32(8100 + K, (N, K))
        banner(f"bwn_i8 chain N={N} K={K}")
        Wp, a = bnn.pack_weights(dev(W))
        q = bnn.quantize_act_i8(dev(X))
        out = bnn.bwn_i8_linear(Wp, K, bnn.EPI_DOT_I32 | bnn.EPI_SCALE_F32, Xb=q["Xb"], xsum=q["xsum"],
                                xscale=q["xscale"], alpha=a)
        torch.cuda.synchronize()
        Qr, xsr, Dr, Yr, ar = oracle.binary_weight_linear_i8(X, W)
        np.testing.assert_array_equal(host(out["D"]), Dr)
        assert_f32_close(host(a), ar, what="alpha")
        assert_f32_close(host(out["Y"]), Yr, rtol=2e-6, what="Y")   # alpha may differ by one ulp


# ---------------------------------------------------------------- per-tensor scale, bias epilogue
@pytest.mark.parametrize("N,K", [(1, 1), (7, 33), (256, 1000), (11008, 4096), (3, 16385)])
def test_weight_scale_tensor(bnn, N, K):
    W = workloads.normal_f32(8200 + K, (N, K))
    banner(f"weight_scale_tensor N={N} K={K}")
    a = bnn.weight_scale_tensor(dev(W))
    torch.cuda.synchronize()
    assert_f32_close(host(a), np.atleast_1d(oracle.alpha_tensor(W)), what="alpha_tensor")


@pytest.mark.parametrize("M,N,K", [(1, 300, 1000), (2, 4096, 4096), (64, 256, 1000), (300, 100, 577),
                                   (1000, 64, 576)])
@pytest.mark.parametrize("flags", ["bias", "tensor", "tensor_bias_res"])
def test_fused_bias_and_tensor_scale(bnn, M, N, K, flags):
    X = workloads.normal_f32(8300 + K, (M, K))
    W = workloads.normal_f32(8400 + K, (N, K))
    bias = workloads.normal_f32(8500 + N, (N,))
    R = workloads.normal_f32(8600 + N, (M, N))
    xs, wsg = oracle.sign(X), oracle.sign(W)
    D_ref = oracle.dot(xs, wsg)
    a = oracle.alpha(W) if flags == "bias" else np.atleast_1d(oracle.alpha_tensor(W))
    f = bnn.EPI_SCALE_F32 | bnn.EPI_DOT_I32
    kw = {}
    if "bias" in flags:
        f |= bnn.EPI_BIAS_F32
        kw["bias"] = dev(bias)
    if "tensor" in flags:
        f |= bnn.EPI_ALPHA_TENSOR
    if "res" in flags:
        f |= bnn.EPI_RESIDUAL_F32
        kw["R"] = dev(R)
    banner(f"fused {flags} M={M} N={N} K={K}")
    Xp = bnn.pack_activations(dev(X))
    Wp, _ = bnn.pack_weights(dev(W), alpha=False)
    out = bnn.linear_fused(Xp, Wp, K, f, alpha=dev(a), **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out["D"]), D_ref)
    if "bias" in flags:
        Y_ref = oracle.scale_bias_residual(D_ref, a, bias, R if "res" in flags else None)
    else:
        Y_ref = oracle.scale(D_ref, np.broadcast_to(a, (N,)).astype(np.float32))
    _bits_equal(host(out["Y"]), Y_ref, "Y")
