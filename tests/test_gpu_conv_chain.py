"""GPU parity of chained binary conv blocks: RSign packing, the implicit-im2col
3x3 convolution and the fused sign-pack of the next block's input.

Sources: page "State of the Art Survey", ReActNet row (RSign: a shift before
the sign) and Bi-Real Net row (FP shortcut per block); page "First
Principles", section "1. Arithmetic" (pad bits encode +1).

Bar: packed images and packed sign outputs (with pads), int32 conv sums
bit-exact; fp32 outputs computed from identical inputs by the same rounded
operations, bit-exact.  All calls go through the C ABI."""
from __future__ import annotations

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
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} differ; first {idx.tolist()}")


def _beta(seed, C):
    return workloads.normal_f32(seed, (C,)) * np.float32(0.3)


@pytest.mark.parametrize("M,K", [(7, 64), (100, 256), (3, 1000), (64, 33),
                                 # 4-word rows with 1 or 2 data words (lane groups skip the pad)
                                 (50, 20), (1000, 64), (17, 128)])
def test_pack_activations_rsign(bnn, M, K):
    X = workloads.normal_f32(10000 + K, (M, K))
    X = workloads.inject_edge_values(X, 10001 + K, 0.03)
    beta = _beta(10002 + K, K)
    X[0, :] = beta                                   # exact ties: x == beta -> +1
    banner(f"pack_activations_rsign M={M} K={K}")
    Xp = bnn.pack_activations_rsign(dev(X), dev(beta))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_u32(Xp), oracle.pack_signs(oracle.rsign(X, beta), ld=Xp.shape[1]))


def _conv_ref(X, Wt, beta):
    B, H, W, C = X.shape
    S = oracle.rsign(X.reshape(-1, C), beta).reshape(X.shape)
    Wf = np.ascontiguousarray(Wt.reshape(Wt.shape[0], 9 * C))
    return oracle.dot(oracle.im2col_pm1(S), oracle.sign(Wf)), oracle.alpha(Wf)


@pytest.mark.parametrize("B,H,W,C,Cout", [(2, 5, 6, 64, 64), (1, 7, 3, 128, 100), (2, 4, 4, 256, 256),
                                          (1, 3, 5, 512, 64), (1, 1, 1, 64, 8), (3, 6, 7, 64, 33),
                                          # one-pixel-high and one-pixel-wide strips: the rows
                                          # or columns of taps outside are all padding
                                          (2, 1, 9, 64, 64), (2, 9, 1, 128, 40)])
def test_conv3x3_fused_matches_explicit(bnn, B, H, W, C, Cout):
    X = workloads.normal_f32(10100 + C, (B, H, W, C))
    Wt = workloads.normal_f32(10101 + C, (Cout, 3, 3, C))
    beta = _beta(10102 + C, C)
    D_ref, a = _conv_ref(X, Wt, beta)
    M = B * H * W
    banner(f"conv3x3 implicit B={B} H={H} W={W} C={C} Cout={Cout}")
    Ximg = bnn.pack_activations_rsign(dev(X.reshape(M, C)), dev(beta))
    Wp, ad = bnn.pack_weights(dev(np.ascontiguousarray(Wt.reshape(Cout, 9 * C))))
    # the oracle's alpha drives the GPU epilogue; the GPU's alpha is checked apart
    out = bnn.conv3x3_fused(Ximg, Wp, (B, H, W, C), bnn.EPI_DOT_I32 | bnn.EPI_SCALE_F32, alpha=dev(a))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(ad).view(np.uint32), a.view(np.uint32))
    np.testing.assert_array_equal(host(out["D"]), D_ref)
    _bits_equal(host(out["Y"]), oracle.scale(D_ref, a), "Y")
    # BatchNorm + sign on the implicit path too (the library's fold of the oracle's alpha)
    g, b, mu, var, eps = workloads.bn_params(10103 + C, Cout)
    tau, dirv = bnn.fold_bn_thresholds(g, b, mu, var, eps, a)
    th = bnn.conv3x3_fused(Ximg, Wp, (B, H, W, C), bnn.EPI_THRESH_PACK, tau=dev(tau), dir=dev(dirv))
    torch.cuda.synchronize()
    s_ref, _ = oracle.bn_next_sign(D_ref, a, g, b, mu, var, eps)
    np.testing.assert_array_equal(host_u32(th["Op"]), oracle.pack_signs(s_ref, ld=th["Op"].shape[1]))


@pytest.mark.parametrize("tn", [8, 16, 32, 64])
@pytest.mark.parametrize("C", [64, 256])
def test_conv_block_sign_pack_every_tile(bnn, tn, C, monkeypatch):
    B, H, W = 2, 6, 5
    X = workloads.normal_f32(10200 + C, (B, H, W, C))
    Wt = workloads.normal_f32(10201 + C, (C, 3, 3, C))
    b0, b1 = _beta(10202 + C, C), _beta(10203 + C, C)
    M = B * H * W
    D_ref, Y_ref, a = oracle.conv_block_rsign(X, Wt, b0)
    Y_ref = Y_ref.reshape(M, C)
    next_ref = oracle.pack_signs(oracle.rsign(Y_ref, b1), ld=bnn.padded_ld(C))
    monkeypatch.setenv("BNN_GEMM_TN", str(tn))
    banner(f"conv block sign-pack TN={tn} C={C}")
    Xd = dev(X.reshape(M, C))
    Ximg = bnn.pack_activations_rsign(Xd, dev(b0))
    Wp, ad = bnn.pack_weights(dev(np.ascontiguousarray(Wt.reshape(C, 9 * C))))
    Op = torch.full((M, bnn.padded_ld(C)), -1, dtype=torch.int32, device="cuda")   # pads must be rewritten
    out = bnn.conv3x3_fused(Ximg, Wp, (B, H, W, C),
                            bnn.EPI_DOT_I32 | bnn.EPI_SCALE_F32 | bnn.EPI_RESIDUAL_F32 | bnn.EPI_SIGN_PACK,
                            alpha=ad, R=Xd, beta=dev(b1), Op=Op)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out["D"]), D_ref)
    _bits_equal(host(out["Y"]), Y_ref, "Y")
    np.testing.assert_array_equal(host_u32(Op), next_ref)


def test_dense_sign_pack_epilogue(bnn):
    # the fused next-layer pack also serves dense layers (bnn_linear_fused)
    M, N, K = 300, 100, 577
    X = workloads.normal_f32(10300, (M, K))
    W = workloads.normal_f32(10301, (N, K))
    bt = _beta(10302, N)
    Xp = bnn.pack_activations(dev(X))
    Wp, ad = bnn.pack_weights(dev(W))
    a_ref = oracle.alpha(W)
    banner("dense sign-pack")
    out = bnn.linear_fused(Xp, Wp, K, bnn.EPI_SCALE_F32 | bnn.EPI_SIGN_PACK, alpha=dev(a_ref), beta=dev(bt))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(ad).view(np.uint32), a_ref.view(np.uint32))
    Y_ref = oracle.scale(oracle.dot(oracle.sign(X), oracle.sign(W)), a_ref)
    _bits_equal(host(out["Y"]), Y_ref, "Y")
    np.testing.assert_array_equal(host_u32(out["Op"]), oracle.pack_signs(oracle.rsign(Y_ref, bt), ld=out["Op"].shape[1]))


def _gpu_chain(bnn, X, Ws, betas):
    """Blocks l = 0..L-1: the packed image of block 0 from RSign(X, beta_0);
    block l writes Y_l and, fused, the packed RSign(Y_l, beta_{l+1})."""
    B, H, W, C = X.shape
    M = B * H * W
    Xd = dev(X.reshape(M, C))
    img = bnn.pack_activations_rsign(Xd, dev(betas[0]))
    R = Xd
    outs = []
    for l, Wt in enumerate(Ws):
        Wp, ad = bnn.pack_weights(dev(np.ascontiguousarray(Wt.reshape(C, 9 * C))))
        last = l + 1 == len(Ws)
        flags = bnn.EPI_DOT_I32 | bnn.EPI_SCALE_F32 | bnn.EPI_RESIDUAL_F32 | (0 if last else bnn.EPI_SIGN_PACK)
        o = bnn.conv3x3_fused(img, Wp, (B, H, W, C), flags, alpha=ad, R=R,
                              beta=None if last else dev(betas[l + 1]))
        outs.append((o["D"], o["Y"], o["Op"]))
        img, R = o["Op"], o["Y"]
    return outs


@pytest.mark.parametrize("B,H,W,C", [(2, 8, 8, 64), (2, 56, 56, 64), (2, 14, 14, 256), (1, 9, 7, 128)])
def test_conv_chain_three_blocks(bnn, B, H, W, C):
    X = workloads.normal_f32(10400 + C + H, (B, H, W, C))
    Ws = [workloads.normal_f32(10410 + i + C, (C, 3, 3, C)) for i in range(3)]
    betas = [_beta(10420 + i + C, C) for i in range(3)]
    banner(f"conv chain x3 B={B} H={H} W={W} C={C}")
    g = _gpu_chain(bnn, X, Ws, betas)
    torch.cuda.synchronize()
    ref = oracle.conv_chain(X, Ws, betas)
    M = B * H * W
    for l, ((Dg, Yg, Og), (Dr, Yr)) in enumerate(zip(g, ref)):
        np.testing.assert_array_equal(host(Dg), Dr, err_msg=f"block {l} D")
        _bits_equal(host(Yg), Yr.reshape(M, C), f"block {l} Y")
        if l + 1 < len(Ws):
            np.testing.assert_array_equal(
                host_u32(Og), oracle.pack_signs(oracle.rsign(Yr.reshape(M, C), betas[l + 1]), ld=Og.shape[1]),
                err_msg=f"block {l} next-layer bits")
