"""C-ABI checks that need no GPU: the library loads, exports every entry
point the header declares, rejects bad arguments before any launch, and its
host-side BatchNorm fold gives, for every integer dot product, the decision
that the oracle takes from the definition of BatchNorm followed by sign."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bnn.h")

OK, ERR_NULL, ERR_SHAPE, ERR_LD, ERR_ALIGN, ERR_UNSUPPORTED, ERR_HIP = range(7)

# Fake device addresses: validation never dereferences them, and every case
# below fails validation, so nothing is launched.
A16 = 0x10000          # 16-byte aligned
A4 = 0x10004           # 4-byte aligned, not 16
A2 = 0x10002           # misaligned


@pytest.fixture(scope="module")
def L():
    import xnor_popcount_gemm_amd as bnn
    return bnn.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bnn_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_are_exported(L):
    names = declared_functions()
    assert {"bnn_pack_weights", "bnn_pack_activations", "bnn_xnor_gemm", "bnn_linear_fused"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/bnn.h but not exported"


def test_packed_words_and_status_strings(L):
    assert [L.bnn_packed_words(k) for k in (0, 1, 31, 32, 33, 1000, 16384)] == [0, 1, 1, 1, 2, 32, 512]
    assert L.bnn_packed_words(-1) == -1
    for s in range(7):
        assert L.bnn_status_string(s).startswith(b"BNN_")


@pytest.mark.parametrize("args,want", [
    # (W, N, K, ldW, Wp, ldWp, alpha)
    ((0, 4, 64, 64, A16, 4, None), ERR_NULL),
    ((A16, 4, 64, 64, 0, 4, None), ERR_NULL),
    ((A16, 4, 0, 64, A16, 4, None), ERR_SHAPE),
    ((A16, 4, (1 << 24) + 1, (1 << 24) + 1, A16, 1 << 19, None), ERR_SHAPE),
    ((A16, -1, 64, 64, A16, 4, None), ERR_SHAPE),
    ((A16, 4, 64, 63, A16, 4, None), ERR_LD),
    ((A16, 4, 1000, 1000, A16, 28, None), ERR_LD),
    ((A16, 4, 64, 64, A4, 4, None), ERR_ALIGN),
    ((A16, 4, 64, 64, A16, 6, None), ERR_ALIGN),
    ((A2, 4, 64, 64, A16, 4, None), ERR_ALIGN),
    ((A16, 4, 64, 64, A16, 4, A2), ERR_ALIGN),
])
def test_pack_weights_validation(L, args, want):
    W, N, K, ldW, Wp, ldWp, a = args
    assert L.bnn_pack_weights(W, N, K, ldW, Wp, ldWp, a, None) == want


def test_pack_activations_validation(L):
    import xnor_popcount_gemm_amd as bnn
    bad = bnn._ConvGeom(2, 5, 5, 8, 3, 3, 2, 1)       # stride 2: unsupported
    assert L.bnn_pack_activations(A16, 50, 72, 8, ctypes.byref(bad), A16, 4, None) == ERR_UNSUPPORTED
    g2 = bnn._ConvGeom(2, 5, 5, 8, 3, 3, 1, 1)
    assert L.bnn_pack_activations(A16, 49, 72, 8, ctypes.byref(g2), A16, 4, None) == ERR_SHAPE   # M != B*H*W
    assert L.bnn_pack_activations(A16, 50, 71, 8, ctypes.byref(g2), A16, 4, None) == ERR_SHAPE   # K != 9*C
    assert L.bnn_pack_activations(0, 4, 64, 64, None, A16, 4, None) == ERR_NULL
    assert L.bnn_pack_activations(A16, 4, 64, 60, None, A16, 4, None) == ERR_LD
    assert L.bnn_pack_activations(A16, 4, 64, 64, None, A16 + 4, 4, None) == ERR_ALIGN


def test_conv_geom_struct_layout():
    import xnor_popcount_gemm_amd as bnn
    assert ctypes.sizeof(bnn._ConvGeom) == 8 * 8


@pytest.mark.parametrize("kw,want", [
    (dict(Xp=0), ERR_NULL),
    (dict(Wp=0), ERR_NULL),
    (dict(D=0, Y=0), ERR_NULL),
    (dict(K=0), ERR_SHAPE),
    (dict(M=-1), ERR_SHAPE),
    (dict(ldXp=1), ERR_LD),
    (dict(ldWp=0), ERR_LD),
    (dict(ldD=7), ERR_LD),
    (dict(Xp=A4), ERR_ALIGN),
    (dict(ldWp=6), ERR_ALIGN),
    (dict(D=A2), ERR_ALIGN),
    (dict(Y=A16, alpha=0), ERR_NULL),
    (dict(D=0, Y=A16, alpha=A16, ldY=3), ERR_LD),
])
def test_xnor_gemm_validation(L, kw, want):
    a = dict(Xp=A16, ldXp=4, Wp=A16, ldWp=4, M=3, N=8, K=100, D=A16, ldD=8, alpha=None, Y=None, ldY=0)
    a.update(kw)
    st = L.bnn_xnor_gemm(a["Xp"], a["ldXp"], a["Wp"], a["ldWp"], a["M"], a["N"], a["K"],
                         a["D"], a["ldD"], a["alpha"], a["Y"], a["ldY"], None)
    assert st == want


def _fused(**kw):
    import xnor_popcount_gemm_amd as bnn
    a = bnn._FusedArgs()
    base = dict(Xp=A16, ldXp=4, Wp=A16, ldWp=4, M=3, N=40, K=100, epilogue=bnn.EPI_DOT_I32,
                D=A16, ldD=40)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,want", [
    (dict(epilogue=0), ERR_UNSUPPORTED),
    (dict(epilogue=16), ERR_UNSUPPORTED),
    (dict(epilogue=4, Y=A16, ldY=40, R=A16, ldR=40, alpha=A16), ERR_UNSUPPORTED),   # residual without scale
    (dict(epilogue=8), ERR_NULL),                                                 # thresh without tau/dir/Op
    (dict(epilogue=8, tau=A16, dir=A16, Op=A16, ldOp=1), ERR_LD),                 # ldOp < ceil(40/32)
    (dict(epilogue=6, Y=A16, ldY=40, alpha=A16), ERR_NULL),                       # residual without R
    (dict(epilogue=6, Y=A16, ldY=40, alpha=A16, R=A16 + 64, ldR=40), ERR_UNSUPPORTED),  # R, Y overlap
    (dict(M=(1 << 31)), ERR_SHAPE),
    (dict(epilogue=32), ERR_UNSUPPORTED),                                          # bias without scale
    (dict(epilogue=64), ERR_UNSUPPORTED),                                          # unknown flag
    (dict(epilogue=34, Y=A16, ldY=40, alpha=A16), ERR_NULL),                       # bias pointer missing
    (dict(epilogue=34, Y=A16, ldY=40, alpha=A16, bias=A2), ERR_ALIGN),
    (dict(epilogue=18, Y=A16, ldY=40, alpha=A2), ERR_ALIGN),                       # per-tensor alpha, misaligned
    (dict(epilogue=65), ERR_NULL),                                                 # ternary without Zp
    (dict(epilogue=65, Zp=A16), ERR_NULL),                                         # ternary without nnz
    (dict(epilogue=65, Zp=A4, nnz=A16), ERR_ALIGN),
    (dict(epilogue=65, Zp=A16, nnz=A2), ERR_ALIGN),
    (dict(epilogue=64), ERR_UNSUPPORTED),                                          # a format flag is no output
    (dict(epilogue=128), ERR_UNSUPPORTED),
])
def test_linear_fused_validation(L, kw, want):
    a = _fused(**kw)
    assert L.bnn_linear_fused(ctypes.byref(a), None) == want
    assert L.bnn_linear_fused(None, None) == ERR_NULL


def test_dense_support_validation(L):
    assert L.bnn_dense_f32_sign_pack(0, 784, A16, 784, 4, 64, 784, A16, 4, None) == ERR_NULL
    assert L.bnn_dense_f32_sign_pack(A16, 783, A16, 784, 4, 64, 784, A16, 4, None) == ERR_LD
    assert L.bnn_dense_f32_sign_pack(A16, 784, A16, 784, 4, 64, 784, A16, 1, None) == ERR_LD
    assert L.bnn_dense_binact_f32(A4, 128, A16, 4096, 4, 10, 4096, A16, 10, None) == ERR_ALIGN
    assert L.bnn_dense_binact_f32(A16, 128, A16, 4096, 4, 10, 4096, A16, 9, None) == ERR_LD


def _i8(**kw):
    import xnor_popcount_gemm_amd as bnn
    a = bnn._I8Args()
    base = dict(Xb=A16, ldXb=4, xsum=A16, Wp=A16, ldWp=4, M=1, N=40, K=100,
                epilogue=bnn.EPI_DOT_I32, D=A16, ldD=40)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,want", [
    (dict(), OK),                                                   # valid: validation passes, M=0 below
    (dict(Xb=0), ERR_NULL),                                         # no activation form
    (dict(Xb=0, Xq=A16, ldXq=112), OK),                             # int8 rows (GEMM path)
    (dict(Xb=0, Xq=A16, ldXq=100), ERR_ALIGN),                      # ldXq % 16
    (dict(Xb=0, Xq=A16 + 4, ldXq=112), ERR_ALIGN),
    (dict(Xb=0, Xq=A16, ldXq=96), ERR_LD),
    (dict(Xb=0, Xq=A16, ldXq=112, xsum=A2), ERR_ALIGN),             # GEMM row sums are read too
    (dict(Xb=0, Xq=A16, ldXq=112, N=1 << 25, ldWp=16, ldD=1 << 25), ERR_SHAPE),   # past 32-bit offsets
    (dict(Xb=0, Xq=A16, ldXq=112, N=(1 << 25) - 1, ldWp=16, ldD=1 << 25), OK),
    (dict(M=3), ERR_NULL),                                          # planes serve M <= 2 only
    (dict(K=(1 << 17) + 1), ERR_SHAPE),
    (dict(K=0), ERR_SHAPE),
    (dict(ldXb=3), ERR_LD),
    (dict(Xb=A4), ERR_ALIGN),
    (dict(xsum=A2), ERR_ALIGN),
    (dict(epilogue=4), ERR_UNSUPPORTED),                            # residual is not offered here
    (dict(epilogue=16), ERR_UNSUPPORTED),                           # per-tensor alpha without scale
    (dict(epilogue=2), ERR_NULL),                                   # scale without Y / alpha
    (dict(epilogue=18, Y=A16, ldY=40, alpha=A16), OK),
    (dict(epilogue=2, Y=A16, ldY=39, alpha=A16), ERR_LD),
    (dict(xscale=A2), ERR_ALIGN),
    (dict(epilogue=65), ERR_NULL),                                  # ternary without Zp
    (dict(epilogue=65, Zp=A4), ERR_ALIGN),
    (dict(epilogue=65, Zp=A16, xsum=0), OK),                        # ternary planes need no row sums
    (dict(epilogue=1, xsum=0), ERR_NULL),                           # binary planes do
])
def test_bwn_i8_validation(L, kw, want):
    a = _i8(**kw)
    if want == OK:
        a.M = 0                      # nothing is launched on this host
    assert L.bnn_bwn_i8_linear(ctypes.byref(a), None) == want
    assert L.bnn_bwn_i8_linear(None, None) == ERR_NULL


def test_i8_activation_writers_validation(L):
    # quantize: X, M, K, ldX, Xq, ldXq, Xb, ldXb, xsum, xscale
    q = L.bnn_quantize_act_i8
    assert q(A16, 0, 100, 100, A16, 112, A16, 4, A16, A16, None) == OK
    assert q(0, 1, 100, 100, A16, 112, A16, 4, A16, A16, None) == ERR_NULL
    assert q(A16, 1, 100, 100, 0, 0, 0, 0, 0, A16, None) == ERR_NULL       # no output form
    assert q(A16, 1, 100, 100, A16, 112, A16, 4, A16, 0, None) == ERR_NULL  # xscale required
    assert q(A16, 1, 100, 100, 0, 0, A16, 4, 0, A16, None) == ERR_NULL      # planes need xsum
    assert q(A16, 0, 100, 100, A16, 112, 0, 0, A16, A16, None) == OK        # row sums without planes
    assert q(A16, 1, 100, 100, A16, 112, 0, 0, A2, A16, None) == ERR_ALIGN
    assert q(A16, 1, 100, 99, A16, 112, 0, 0, 0, A16, None) == ERR_LD
    assert q(A16, 1, 100, 100, A16, 99, 0, 0, 0, A16, None) == ERR_LD
    assert q(A16, 1, 100, 100, 0, 0, A16, 6, A16, A16, None) == ERR_ALIGN
    assert q(A16, 1, (1 << 17) + 1, 1 << 18, A16, 1 << 18, 0, 0, 0, A16, None) == ERR_SHAPE
    p = L.bnn_pack_act_i8                    # Xq, M, K, ldXq, Xb, ldXb, xsum
    assert p(A16, 0, 100, 100, A16, 4, A16, None) == OK
    assert p(A16, 1, 100, 100, 0, 4, A16, None) == ERR_NULL
    assert p(A16, 1, 100, 100, A16, 4, 0, None) == ERR_NULL
    assert p(A16, 1, 100, 99, A16, 4, A16, None) == ERR_LD
    assert p(A16, 1, 100, 100, A16 + 4, 4, A16, None) == ERR_ALIGN
    s = L.bnn_weight_scale_tensor            # W, N, K, ldW, work, alpha
    assert s(A16, 0, 100, 100, A16, A16, None) == ERR_SHAPE
    assert s(A16, 4, 100, 100, 0, A16, None) == ERR_NULL
    assert s(A16, 4, 100, 99, A16, A16, None) == ERR_LD
    assert s(A16, 4, 100, 100, A4, A16, None) == ERR_ALIGN


def test_pack_weights_ternary_validation(L):
    p = L.bnn_pack_weights_ternary          # W, N, K, ldW, gamma, delta, Sp, Zp, ld, nnz
    f = ctypes.c_float(0.5)
    assert p(A16, 0, 64, 64, None, f, A16, A16, 4, A16, None) == OK
    assert p(0, 4, 64, 64, None, f, A16, A16, 4, A16, None) == ERR_NULL
    assert p(A16, 4, 64, 64, None, f, A16, 0, 4, A16, None) == ERR_NULL
    assert p(A16, 4, 64, 64, None, f, A16, A16, 4, 0, None) == ERR_NULL
    assert p(A16, 4, 64, 63, None, f, A16, A16, 4, A16, None) == ERR_LD
    assert p(A16, 4, 200, 200, None, f, A16, A16, 4, A16, None) == ERR_LD     # ld < ceil(200/32)
    assert p(A16, 4, 64, 64, None, f, A4, A16, 4, A16, None) == ERR_ALIGN
    assert p(A16, 4, 64, 64, A2, f, A16, A16, 4, A16, None) == ERR_ALIGN
    assert p(A16, 4, 0, 64, None, f, A16, A16, 4, A16, None) == ERR_SHAPE


def test_xnor_gemm_mfma_validation(L):
    # Xp, ldXp, Wp, ldWp, M, N, K, D, ldD, alpha, Y, ldY, stream: the checks of bnn_xnor_gemm
    g = L.bnn_xnor_gemm_mfma
    assert g(A16, 4, A16, 4, 0, 8, 100, A16, 8, None, None, 0, None) == OK
    assert g(A16, 4, A16, 4, 3, 0, 100, A16, 8, None, None, 0, None) == OK
    assert g(A16, 4, A16, 4, 3, 8, 100, None, 8, None, None, 0, None) == ERR_NULL        # no output
    assert g(0, 4, A16, 4, 3, 8, 100, A16, 8, None, None, 0, None) == ERR_NULL
    assert g(A16, 4, A16, 4, 3, 8, 100, None, 0, None, A16, 8, None) == ERR_NULL         # Y without alpha
    assert g(A16, 4, A16, 4, 3, 8, 0, A16, 8, None, None, 0, None) == ERR_SHAPE
    assert g(A16, 4, A16, 4, 3, 8, (1 << 24) + 1, A16, 8, None, None, 0, None) == ERR_SHAPE
    assert g(A16, 3, A16, 4, 3, 8, 100, A16, 8, None, None, 0, None) == ERR_LD
    assert g(A16, 4, A16, 4, 3, 8, 100, A16, 7, None, None, 0, None) == ERR_LD
    assert g(A4, 4, A16, 4, 3, 8, 100, A16, 8, None, None, 0, None) == ERR_ALIGN
    assert g(A16, 4, A16, 6, 3, 8, 100, A16, 8, None, None, 0, None) == ERR_ALIGN


def test_bwn_f16_gemv_validation(L):
    # X, ldX, Wp, ldWp, M, N, K, epilogue, alpha, Y, ldY, stream
    g = L.bnn_bwn_f16_gemv
    SC, AT, DOT = 2, 16, 1
    assert g(A16, 104, A16, 4, 0, 8, 100, SC, A16, A16, 8, None) == OK            # M == 0: nothing to do
    assert g(A16, 104, A16, 4, 2, 0, 100, SC, A16, A16, 8, None) == OK            # N == 0
    assert g(0, 104, A16, 4, 1, 8, 100, SC, A16, A16, 8, None) == ERR_NULL
    assert g(A16, 104, 0, 4, 1, 8, 100, SC, A16, A16, 8, None) == ERR_NULL
    assert g(A16, 104, A16, 4, 1, 8, 100, SC, 0, A16, 8, None) == ERR_NULL
    assert g(A16, 104, A16, 4, 1, 8, 100, SC, A16, 0, 8, None) == ERR_NULL
    assert g(A16, 104, A16, 4, 1, 8, 100, DOT, A16, A16, 8, None) == ERR_UNSUPPORTED
    assert g(A16, 104, A16, 4, 1, 8, 100, SC | DOT, A16, A16, 8, None) == ERR_UNSUPPORTED
    assert g(A16, 104, A16, 4, 1, 8, 100, AT, A16, A16, 8, None) == ERR_UNSUPPORTED   # no SCALE
    assert g(A16, 104, A16, 4, 1, 8, 0, SC, A16, A16, 8, None) == ERR_SHAPE
    assert g(A16, 16384, A16, 512, 1, 8, 16385, SC, A16, A16, 8, None) == ERR_SHAPE
    assert g(A16, 96, A16, 4, 1, 8, 100, SC, A16, A16, 8, None) == ERR_LD         # ldX < K
    assert g(A16, 104, A16, 4, 1, 8, 100, SC, A16, A16, 7, None) == ERR_LD        # ldY < N
    assert g(A16, 104, A16, 3, 1, 8, 100, SC, A16, A16, 8, None) == ERR_LD        # ldWp < ceil(K/32)
    assert g(A4, 104, A16, 4, 1, 8, 100, SC, A16, A16, 8, None) == ERR_ALIGN      # X not 16-byte aligned
    assert g(A16, 100, A16, 4, 1, 8, 100, SC, A16, A16, 8, None) == ERR_ALIGN     # ldX % 8 != 0
    assert g(A16, 104, A4, 4, 1, 8, 100, SC, A16, A16, 8, None) == ERR_ALIGN      # Wp not 16-byte aligned
    assert g(A16, 104, A16, 4, 1, 8, 100, SC, A2, A16, 8, None) == ERR_ALIGN
    assert g(A16, 104, A16, 4, 1, 8, 100, SC, A16, A2, 8, None) == ERR_ALIGN


def test_empty_calls_launch_nothing(L):
    # M == 0 or N == 0 is a valid empty call that returns before any launch.
    assert L.bnn_xnor_gemm(A16, 4, A16, 4, 0, 8, 100, A16, 8, None, None, 0, None) == OK
    assert L.bnn_xnor_gemm(A16, 4, A16, 4, 3, 0, 100, A16, 8, None, None, 0, None) == OK
    assert L.bnn_pack_weights(A16, 0, 64, 64, A16, 4, None, None) == OK
    assert L.bnn_pack_activations(A16, 0, 64, 64, None, A16, 4, None) == OK


def _fold_decisions(tau, d, D):
    """The THRESH_PACK rule of the header: +1 iff (float)(dir * D) >= tau."""
    v = (d[None, :].astype(np.int64) * np.asarray(D, np.int64)).astype(np.float32)
    return np.where(v >= tau[None, :], 1, -1).astype(np.int8)


def _check_fold_against_rule(tau, d, a, g, b, mu, var, eps, K, extra_D=()):
    """The fold's decisions equal the oracle's exact rule (bisected over
    [-K, K]) for every D in [-min(K, 4096), min(K, 4096)] and every D of
    extra_D (all within [-K, K])."""
    kind, bound = oracle.bn_rule(a, g, b, mu, var, eps, K)
    N = a.shape[0]
    span = min(K, 4096)
    Ds = np.unique(np.concatenate([np.arange(-span, span + 1, dtype=np.int64),
                                   np.asarray(extra_D, np.int64).reshape(-1)]))
    assert np.abs(Ds).max() <= K
    D = np.broadcast_to(Ds[:, None], (Ds.size, N))
    got = _fold_decisions(tau, d, D)
    want = oracle.rule_signs(kind, bound, D)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} decisions differ; first (D, channel) {[(int(Ds[i]), int(n)) for i, n in bad[:5]]}"
    # tau is an integer-valued float (exact comparisons)
    assert np.all(tau == np.rint(tau))


@pytest.mark.parametrize("layer", [0, 1, 2])
def test_fold_bn_thresholds_exact_on_every_mlp_channel(layer):
    """The binary MLP's three hidden layers (4096 channels each, K = 4096):
    the fold's threshold rule equals the exact BatchNorm decision for every
    channel and every D in [-K, K] ("Binary Neural Network (BNN)" glossary,
    BatchNorm; "Extreme Quantization" eq. (4))."""
    import xnor_popcount_gemm_amd as bnn
    h = workloads.WORKLOADS[2]["hidden"]
    Wh = workloads.normal_f32(workloads.seed_for(2, 2 + layer), (h, h))
    a = oracle.alpha(Wh)
    g, b, mu, var, eps = workloads.bn_params(workloads.seed_for(2, 10 + layer), h)
    tau, d = bnn.fold_bn_thresholds(g, b, mu, var, eps, a)
    _check_fold_against_rule(tau, d, a, g, b, mu, var, eps, h)


def _hard_channels():
    """Channels built to be hard for a threshold fold: exact ties reached
    through a rational square root, boundaries off the data range, zero and
    negative slopes, tiny and huge magnitudes."""
    f = np.float32
    rows = [  # alpha, gamma, beta, mean, var, eps
        (0.5, 1.0, -1.0, 0.0, 1.0, 0.0),          # tie at D = 2
        (0.5, -1.0, -1.0, 0.0, 1.0, 0.0),         # tie at D = -2, negative slope
        (0.5, 2.0, -2.0, 0.0, 2.25, 0.0),         # sd = 1.5, tie at D = 3
        (0.25, 1.0, 0.0, 1.5, 2.25, 0.0),         # tie at D = 6 through the mean
        (0.25, -3.0, 0.0, 1.5, 0.0, 0.0625),      # sd = 0.25 from eps alone
        (0.5, 0.0, 0.3, 0.0, 1.0, 1e-5),          # gamma = 0: constant +1
        (0.0, 1.0, 0.2, 1.0, 1.0, 0.0),           # alpha = 0: constant -1
        (0.0, 1.0, 0.0, 0.0, 1.0, 0.0),           # BN = 0 for every D: +1
        (1e-30, 1.0, 0.0, 1e10, 1.0, 0.0),        # boundary far above 2^24: never +1
        (1e-30, -1.0, 0.0, 1e10, 1.0, 0.0),       # ... negative slope: always +1
        (2.0**-20, 1.0, -1.0, 0.0, 1.0, 0.0),     # boundary at 2^20
        (2.0**-24, 1.0, -1.0, 0.0, 1.0, 0.0),     # boundary at 2^24 exactly
        (2.0**-24, 1.0, -1.0, 2.0**-24, 1.0, 0.0),  # boundary at 2^24 + 1: never within range
        (3.0, 1.0, 0.0, 3.0 * 16777216.0, 1.0, 0.0),  # boundary at 2^24 via the mean
        (1.0, 1.0, 1e8, 0.0, 1.0, 0.0),           # boundary far below -2^24: always +1
        (1e-45, 1e-45, 1e-45, 1e-45, 1e-45, 1e-45),  # denormals everywhere
        (3e38, 3e38, -3e38, 3e38, 3e38, 0.0),     # near the top of the range
        (0.7, 1.3, -0.9, 1e-3, 1e-6, 1e-5),       # ordinary values
    ]
    cols = list(zip(*rows))
    a, g, b, mu, var = (np.array(c, np.float32) for c in cols[:5])
    eps_vals = np.array(cols[5], np.float32)
    return a, g, b, mu, var, eps_vals


def test_fold_bn_thresholds_exact_on_hard_channels():
    import xnor_popcount_gemm_amd as bnn
    a, g, b, mu, var, eps_vals = _hard_channels()
    K = 1 << 24        # the largest |D| the library produces
    big = [K, K - 1, K - 2, -K, -K + 1, -K + 2, 1 << 20, (1 << 20) - 1, (1 << 20) + 1]
    for n in range(a.shape[0]):       # eps is per call: one channel at a time
        sl = slice(n, n + 1)
        tau, d = bnn.fold_bn_thresholds(g[sl], b[sl], mu[sl], var[sl], eps_vals[n], a[sl])
        _check_fold_against_rule(tau, d, a[sl], g[sl], b[sl], mu[sl], var[sl], eps_vals[n], K, extra_D=big)


def test_fold_bn_thresholds_random_wide_parameters():
    import xnor_popcount_gemm_amd as bnn
    rng = np.random.default_rng(2001)
    N = 4096
    g, b, mu, var, eps = workloads.bn_params(2001, N)
    g = g * np.where(rng.random(N) < 0.1, -1, 1).astype(np.float32)
    g[:3] = 0.0
    mu = (rng.normal(0, 1, N) * 10.0 ** rng.integers(-3, 4, N)).astype(np.float32)
    var = (rng.random(N) * 3 + 0.01).astype(np.float32)
    a = (rng.random(N) + 0.1).astype(np.float32)
    a[5] = 0.0
    tau, d = bnn.fold_bn_thresholds(g, b, mu, var, eps, a)
    _check_fold_against_rule(tau, d, a, g, b, mu, var, eps, 2048)


def test_fold_bn_thresholds_errors():
    import xnor_popcount_gemm_amd as bnn
    f = lambda *v: np.array(v, np.float32)
    one = f(1.0)
    with pytest.raises(bnn.BnnError) as e:
        bnn.fold_bn_thresholds(one, one, one, f(0.0), 0.0, one)        # var + eps = 0
    assert e.value.status == ERR_UNSUPPORTED
    with pytest.raises(bnn.BnnError) as e:
        bnn.fold_bn_thresholds(one, one, one, f(-2.0), 1.0, one)       # var + eps < 0
    assert e.value.status == ERR_UNSUPPORTED
    for bad in (np.inf, np.nan):
        with pytest.raises(bnn.BnnError) as e:
            bnn.fold_bn_thresholds(f(bad), one, one, one, 0.0, one)
        assert e.value.status == ERR_UNSUPPORTED
    with pytest.raises(bnn.BnnError) as e:
        bnn.fold_bn_thresholds(one, one, one, one, np.inf, one)
    assert e.value.status == ERR_UNSUPPORTED
    L = bnn.lib()
    fp = ctypes.c_float(0.0)
    assert L.bnn_fold_bn_thresholds_host(None, None, None, None, fp, None, 0, None, None) == ERR_NULL
    assert L.bnn_fold_bn_thresholds_host(A16, A16, A16, A16, fp, A16, -1, A16, A16) == ERR_SHAPE


def test_weight_scale_tensor_noalloc_validation(L):
    f = L.bnn_weight_scale_tensor_noalloc      # W, N, K, ldW, alpha, stream
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    lim = 1 << 16
    assert f(A16, lim + 1, 64, 64, A16, None) == ERR_SHAPE      # beyond the static scratch
    assert f(A16, 0, 64, 64, A16, None) == ERR_SHAPE
    assert f(A16, 4, 0, 64, A16, None) == ERR_SHAPE
    assert f(0, 4, 64, 64, A16, None) == ERR_NULL
    assert f(A16, 4, 64, 64, 0, None) == ERR_NULL
    assert f(A16, 4, 64, 63, A16, None) == ERR_LD
    assert f(A2, 4, 64, 64, A16, None) == ERR_ALIGN
    assert f(A16, 4, 64, 64, A2, None) == ERR_ALIGN
