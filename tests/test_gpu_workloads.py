"""GPU parity on the five workloads at their full sizes, against the CPU oracle.

Where the oracle cannot compute every output in seconds, sampled rows are
compared element by element (first/last rows, rows at 256-row tile
boundaries and seeded random rows), and every output is checked for the
properties that hold at any size (D = K mod 2, |D| <= K, Y = fl32(alpha*D)).
The launch configurations are the ones ``bench.py`` times."""
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


def _sample_rows(M, seed, n_random=6):
    rng = np.random.default_rng(seed)
    rows = {0, 1, M - 1, M - 2}
    for b in (255, 256, 257, 4095, 4096, 8191, 8192):
        if b < M:
            rows.add(b)
    rows.update(int(r) for r in rng.integers(0, M, n_random))
    return np.array(sorted(rows))


def _check_dot_properties(D: torch.Tensor, K: int):
    Dl = D.to(torch.int64)
    assert bool(((Dl - K) % 2 == 0).all()), "D - K must be even"
    assert bool((Dl.abs() <= K).all()), "|D| must not exceed K"


# ---------------------------------------------------------------- workload 1
def test_workload1_single_binary_linear(bnn):
    c = workloads.WORKLOADS[1]
    M, N, K = c["M"], c["N"], c["K"]
    X = workloads.normal_f32(workloads.seed_for(1, 0), (M, K))
    W = workloads.normal_f32(workloads.seed_for(1, 1), (N, K))
    banner(f"workload1 M={M} N={N} K={K}")
    Wp, a = bnn.pack_weights(dev(W))
    Xp = bnn.pack_activations(dev(X))
    D, Y = bnn.xnor_gemm(Xp, Wp, K, alpha=a, want_scaled=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_u32(Wp), oracle.pack_signs(oracle.sign(W), ld=Wp.shape[1]))
    np.testing.assert_array_equal(host_u32(Xp), oracle.pack_signs(oracle.sign(X), ld=Xp.shape[1]))
    D_ref, Y_ref, a_ref = oracle.binary_linear(X, W)
    np.testing.assert_array_equal(host(D), D_ref)
    np.testing.assert_array_equal(host(a).view(np.uint32), a_ref.view(np.uint32))
    assert_f32_close(host(Y), Y_ref, what="Y")


# ---------------------------------------------------------------- workload 2
def _mlp_inputs():
    c = workloads.WORKLOADS[2]
    B, d_in, h, d_out = c["batch"], c["d_in"], c["hidden"], c["d_out"]
    X = workloads.uniform01_f32(workloads.seed_for(2, 0), (B, d_in))
    W1 = workloads.normal_f32(workloads.seed_for(2, 1), (h, d_in))
    hidden = []
    for i in range(c["n_hidden"]):
        Wh = workloads.normal_f32(workloads.seed_for(2, 2 + i), (h, h))
        hidden.append((Wh,) + workloads.bn_params(workloads.seed_for(2, 10 + i), h))
    W5 = workloads.normal_f32(workloads.seed_for(2, 20), (d_out, h))
    return X, W1, hidden, W5


def run_mlp_gpu(bnn, X, W1, hidden, W5):
    """The binary MLP on the GPU path; returns per-layer packed outputs, alphas
    and the logits (all device tensors)."""
    h = W1.shape[0]
    acts = [bnn.dense_f32_sign_pack(dev(X), dev(W1))]
    alphas, taus = [], []
    for (Wh, g, b, mu, var, eps) in hidden:
        Wp, a = bnn.pack_weights(dev(Wh))
        tau, d = bnn.fold_bn_thresholds(g, b, mu, var, eps, host(a))
        out = bnn.linear_fused(acts[-1], Wp, h, bnn.EPI_THRESH_PACK, tau=dev(tau), dir=dev(d))
        acts.append(out["Op"])
        alphas.append(a)
        taus.append((tau, d))
    logits = bnn.dense_binact_f32(acts[-1], dev(W5), h)
    return acts, alphas, taus, logits


def test_workload2_binary_mlp(bnn):
    X, W1, hidden, W5 = _mlp_inputs()
    banner("workload2 binary MLP batch 1024")
    acts, alphas, taus, logits = run_mlp_gpu(bnn, X, W1, hidden, W5)
    torch.cuda.synchronize()
    ref = oracle.binary_mlp(X, W1, hidden, W5)
    # first FP layer: a double sum of exact products in any order is within
    # K 2^-52 sum|x w| of the exact value, so with no output inside that bound
    # the signs are unique (and must match exactly)
    h1 = ref["h1"]
    bound = X.shape[1] * 2.0**-52 * (np.abs(X).astype(np.float64) @ np.abs(W1).astype(np.float64).T)
    assert int((np.abs(h1) <= bound).sum()) == 0, "first-layer near-ties present"
    for i, act in enumerate(acts):
        want = oracle.pack_signs(ref["signs"][i], ld=act.shape[1])
        np.testing.assert_array_equal(host_u32(act), want, err_msg=f"layer {i + 1} packed signs")
        if i < len(alphas):
            np.testing.assert_array_equal(host(alphas[i]).view(np.uint32), ref["alphas"][i].view(np.uint32))
            np.testing.assert_array_equal(taus[i][0].view(np.uint32), ref["taus"][i].view(np.uint32))
            np.testing.assert_array_equal(taus[i][1], ref["dirs"][i])
    W5sum = np.abs(W5).sum(axis=1)[None, :]
    assert_f32_close(host(logits), ref["logits"], scale=1e-3 * W5sum, what="logits")


# ---------------------------------------------------------------- workload 3
@pytest.mark.parametrize("shape", workloads.WORKLOADS[3]["shapes"], ids=lambda s: f"N{s['N']}_K{s['K']}")
def test_workload3_gemv_exact_shape(bnn, shape):
    N, K = shape["N"], shape["K"]
    W = workloads.normal_f32(workloads.seed_for(3, 0) + K, (N, K))
    x = workloads.normal_f32(workloads.seed_for(3, 1) + K, (1, K))
    banner(f"workload3 gemv N={N} K={K}")
    Wp, a = bnn.pack_weights(dev(W))
    xp = bnn.pack_activations(dev(x))
    D, Y = bnn.xnor_gemm(xp, Wp, K, alpha=a, want_scaled=True)
    torch.cuda.synchronize()
    D_ref, Y_ref, a_ref = oracle.binary_linear(x, W)
    np.testing.assert_array_equal(host(D), D_ref)
    np.testing.assert_array_equal(host(a).view(np.uint32), a_ref.view(np.uint32))
    np.testing.assert_array_equal(host(Y).view(np.uint32), Y_ref.view(np.uint32))


@pytest.mark.parametrize("shape", workloads.WORKLOADS[3]["shapes"], ids=lambda s: f"N{s['N']}_K{s['K']}")
def test_workload3_gemv_streaming_stack(bnn, shape):
    """The timed launch: 191 stacked copies of the weight matrix (> 1 GiB,
    larger than the 256 MB last-level cache) in one GEMV launch."""
    G = 191
    N, K = shape["N"], shape["K"]
    W = workloads.normal_f32(workloads.seed_for(3, 0) + K, (N, K))
    x = workloads.normal_f32(workloads.seed_for(3, 1) + K, (1, K))
    banner(f"workload3 gemv stack G={G} N={N} K={K}")
    Wp, a = bnn.pack_weights(dev(W))
    Wst = Wp.repeat(G, 1)
    ast = a.repeat(G)
    xp = bnn.pack_activations(dev(x))
    D, Y = bnn.xnor_gemm(xp, Wst, K, alpha=ast, want_scaled=True)
    torch.cuda.synchronize()
    D_ref, Y_ref, _ = oracle.binary_linear(x, W)
    Dh, Yh = host(D).reshape(G, N), host(Y).reshape(G, N)
    for g in (0, 1, G // 2, G - 1):
        np.testing.assert_array_equal(Dh[g], D_ref[0])
        np.testing.assert_array_equal(Yh[g].view(np.uint32), Y_ref[0].view(np.uint32))
    assert (Dh == Dh[0:1]).all()


# ---------------------------------------------------------------- workload 4
@pytest.mark.parametrize("shape", workloads.WORKLOADS[4]["shapes"], ids=lambda s: f"M{s['M']}")
def test_workload4_large_gemm_sampled(bnn, shape):
    M, N, K = shape["M"], shape["N"], shape["K"]
    X = workloads.normal_f32(workloads.seed_for(4, 0) + M, (M, K))
    W = workloads.normal_f32(workloads.seed_for(4, 1) + M, (N, K))
    banner(f"workload4 gemm M={M} N={N} K={K}")
    Wd, Xd = dev(W), dev(X)
    Wp, a = bnn.pack_weights(Wd)
    Xp = bnn.pack_activations(Xd)
    del Wd, Xd
    D, Y = bnn.xnor_gemm(Xp, Wp, K, alpha=a, want_scaled=True)
    torch.cuda.synchronize()
    _check_dot_properties(D, K)
    assert bool((Y == a[None, :] * D.to(torch.float32)).all()), "Y != fl32(alpha * D)"
    rows = _sample_rows(M, 4242 + M)
    ws = oracle.sign(W)
    a_ref = oracle.alpha(W)
    np.testing.assert_array_equal(host(a).view(np.uint32), a_ref.view(np.uint32))
    D_ref = oracle.dot(oracle.sign(X[rows]), ws)
    np.testing.assert_array_equal(host(D[torch.from_numpy(rows).cuda()]), D_ref)
    Y_ref = oracle.scale(D_ref, a_ref)
    np.testing.assert_array_equal(host(Y[torch.from_numpy(rows).cuda()]).view(np.uint32), Y_ref.view(np.uint32))
    # packed operands: sampled rows bit-exact
    np.testing.assert_array_equal(host_u32(Xp[torch.from_numpy(rows).cuda()]),
                                  oracle.pack_signs(oracle.sign(X[rows]), ld=Xp.shape[1]))
    cols = _sample_rows(N, 77 + N)
    np.testing.assert_array_equal(host_u32(Wp[torch.from_numpy(cols).cuda()]),
                                  oracle.pack_signs(ws[cols], ld=Wp.shape[1]))


# ---------------------------------------------------------------- workload 5
@pytest.mark.parametrize("shape", workloads.WORKLOADS[5]["shapes"], ids=lambda s: f"H{s['H']}_C{s['C']}")
def test_workload5_conv_block_sampled_images(bnn, shape):
    B, H, Wd, C, Co = shape["B"], shape["H"], shape["W"], shape["C"], shape["Cout"]
    X = workloads.normal_f32(workloads.seed_for(5, 0) + C, (B, H, Wd, C))
    Wt = workloads.normal_f32(workloads.seed_for(5, 1) + C, (Co, 3, 3, C))
    K = 9 * C
    banner(f"workload5 conv B={B} H={H} W={Wd} C={C}")
    Xd = dev(X)
    Wp, a = bnn.pack_weights(dev(Wt.reshape(Co, K)))
    Xp = bnn.pack_activations(Xd, conv3x3=True)
    R = Xd.reshape(B * H * Wd, C)
    out = bnn.linear_fused(Xp, Wp, K, bnn.EPI_SCALE_F32 | bnn.EPI_RESIDUAL_F32, alpha=a, R=R)
    torch.cuda.synchronize()
    Y = out["Y"]
    a_ref = oracle.alpha(Wt.reshape(Co, K))
    np.testing.assert_array_equal(host(a).view(np.uint32), a_ref.view(np.uint32))
    P = H * Wd
    for b in (0, 1, B - 1):
        Db, Yb, _ = oracle.conv_block(X[b:b + 1], Wt)
        sl = slice(b * P, (b + 1) * P)
        np.testing.assert_array_equal(host(Y[sl]).view(np.uint32), Yb.view(np.uint32), err_msg=f"image {b}")
        want_p = oracle.pack_signs(oracle.im2col_signs(X[b:b + 1]), ld=Xp.shape[1])
        np.testing.assert_array_equal(host_u32(Xp[sl]), want_p, err_msg=f"im2col image {b}")
