"""GPU parity on the five workloads at their full sizes, against the CPU oracle.

Every output is compared element by element with the oracle: packed
operands, int32 dot products and alpha-scaled fp32 outputs bit-exact, the
binary MLP's packed BatchNorm-then-sign outputs against the oracle's exact
decisions.  The properties that hold at any size (D = K mod 2, |D| <= K) are
checked as well.  The launch configurations are the ones ``bench.py`` times.
The largest case (16384^3) costs the oracle about half a minute on 16 host
threads."""
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


def _equal(got: np.ndarray, want: np.ndarray, what: str):
    """Element-by-element equality of two large arrays (bit patterns for
    floats), reporting the count and the first mismatches."""
    if got.dtype == np.float32:
        got, want = got.view(np.uint32), np.asarray(want, np.float32).view(np.uint32)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        raise AssertionError(f"{what}: {len(bad)} of {got.size} differ; first {bad[:5].tolist()}")


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
    """The library path (GPU alpha -> host BatchNorm fold -> THRESH_PACK) against
    the oracle's BatchNorm-then-sign decided exactly from its definition
    ("Binary Neural Network (BNN)" glossary; "Extreme Quantization" eq. (4))."""
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
        if i > 0:
            margin = float(ref["bn_margins"][i - 1].min())
            print(f"[workload2] layer {i + 1}: smallest |BN(alpha D)| of any output {margin:.3g}", flush=True)
        _equal(host_u32(act), want, f"layer {i + 1} packed signs")
        if i < len(alphas):
            _equal(host(alphas[i]), ref["alphas"][i], f"layer {i + 2} alpha")
    W5sum = np.abs(W5).sum(axis=1)[None, :]
    assert_f32_close(host(logits), ref["logits"], scale=1e-3 * W5sum, what="logits")


def test_workload2_mlp_graph_replay(bnn):
    """The MLP forward (first layer, three THRESH_PACK layers, last layer)
    captured once in a HIP graph and replayed three times, with eager work and
    synchronisation between the replays: every replay's packed activations and
    logits equal the eager run's bit for bit."""
    X, W1, hidden, W5 = _mlp_inputs()
    h = W1.shape[0]
    banner("workload2 MLP graph replay")
    acts_e, _, taus, logits_e = run_mlp_gpu(bnn, X, W1, hidden, W5)
    Xd, W1d, W5d = dev(X), dev(W1), dev(W5)
    layers = []
    for (Wh, *_), (tau, d) in zip(hidden, taus):
        Wp, _ = bnn.pack_weights(dev(Wh))
        layers.append((Wp, dev(tau), dev(d)))
    ld = bnn.padded_ld(h)
    acts = [torch.empty((X.shape[0], ld), dtype=torch.int32, device="cuda") for _ in range(4)]
    logits = torch.empty((X.shape[0], W5.shape[0]), dtype=torch.float32, device="cuda")

    def step():
        bnn.dense_f32_sign_pack(Xd, W1d, out=acts[0])
        for i, (Wp, tau, d) in enumerate(layers):
            bnn.linear_fused(acts[i], Wp, h, bnn.EPI_THRESH_PACK, tau=tau, dir=d, Op=acts[i + 1])
        bnn.dense_binact_f32(acts[3], W5d, h, out=logits)

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        for t in acts + [logits]:
            t.fill_(-1)                            # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i in range(4):
            _equal(host_u32(acts[i]), host_u32(acts_e[i]), f"replay {r} layer {i + 1} packed signs")
        _equal(host(logits).view(np.uint32), host(logits_e).view(np.uint32), f"replay {r} logits")


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
def test_workload4_large_gemm_full(bnn, shape):
    """Every element of D, Y and both packed operands against the oracle."""
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
    Dh, Yh, Xph, Wph, ah = host(D), host(Y), host_u32(Xp), host_u32(Wp), host(a)
    del D, Y, Xp, Wp
    torch.cuda.empty_cache()
    banner(f"workload4 oracle M={M} N={N} K={K} on {oracle.num_threads()} threads")
    xs, ws = oracle.sign(X), oracle.sign(W)
    del X
    _equal(Wph, oracle.pack_signs(ws, ld=Wph.shape[1]), "packed W")
    _equal(Xph, oracle.pack_signs(xs, ld=Xph.shape[1]), "packed X")
    a_ref = oracle.alpha(W)
    _equal(ah, a_ref, "alpha")
    D_ref = oracle.dot(xs, ws)
    del xs, ws
    _equal(Dh, D_ref, "D")
    _equal(Yh, oracle.scale(D_ref, a_ref), "Y")


# ---------------------------------------------------------------- workload 5
@pytest.mark.parametrize("shape", workloads.WORKLOADS[5]["shapes"], ids=lambda s: f"H{s['H']}_C{s['C']}")
def test_workload5_conv_block_full(bnn, shape):
    """All 256 images: the packed im2col matrix, the packed sign image, D, and
    Y = fl32(fl32(alpha D) + R) by the explicit and the implicit im2col."""
    B, H, Wd, C, Co = shape["B"], shape["H"], shape["W"], shape["C"], shape["Cout"]
    X = workloads.normal_f32(workloads.seed_for(5, 0) + C, (B, H, Wd, C))
    Wt = workloads.normal_f32(workloads.seed_for(5, 1) + C, (Co, 3, 3, C))
    K = 9 * C
    banner(f"workload5 conv B={B} H={H} W={Wd} C={C}")
    Xd = dev(X)
    Wp, a = bnn.pack_weights(dev(Wt.reshape(Co, K)))
    Xp = bnn.pack_activations(Xd, conv3x3=True)
    R = Xd.reshape(B * H * Wd, C)
    # the launches the benchmark times (Y only): explicit im2col + GEMM, and the
    # packed sign image + implicit-im2col conv; then the GEMM with D as well
    out = bnn.linear_fused(Xp, Wp, K, bnn.EPI_SCALE_F32 | bnn.EPI_RESIDUAL_F32, alpha=a, R=R)
    img = bnn.pack_activations(R)
    out_i = bnn.conv3x3_fused(img, Wp, (B, H, Wd, C), bnn.EPI_SCALE_F32 | bnn.EPI_RESIDUAL_F32, alpha=a, R=R)
    out_d = bnn.linear_fused(Xp, Wp, K, bnn.EPI_DOT_I32, alpha=a)
    torch.cuda.synchronize()
    _check_dot_properties(out_d["D"], K)
    Dh, Yh, Xph, ah = host(out_d["D"]), host(out["Y"]), host_u32(Xp), host(a)
    Yih, imgh = host(out_i["Y"]), host_u32(img)
    banner(f"workload5 oracle B={B} H={H} W={Wd} C={C}")
    D_ref, Y_ref, a_ref = oracle.conv_block(X, Wt)
    _equal(ah, a_ref, "alpha")
    _equal(Dh, D_ref, "D")
    _equal(Yh, Y_ref, "Y")
    _equal(Yih, Y_ref, "Y (implicit im2col)")
    _equal(Xph, oracle.pack_signs(oracle.im2col_signs(X), ld=Xph.shape[1]), "packed im2col")
    _equal(imgh, oracle.pack_signs(oracle.sign(X.reshape(B * H * Wd, C)), ld=imgh.shape[1]), "packed image")
