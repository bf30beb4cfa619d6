"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

None of these checks re-types an oracle formula: each compares the oracle with
a different formulation (the XOR-popcount identity on packed words, a numpy
float64 matmul, exact rational arithmetic, torch's conv2d, values derived by
hand from a worked example) or with an invariant.  Sources are cited by page
title and section/equation.
"""
from __future__ import annotations

import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from exact_math import round_to_f32, f32_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_kv(path):
    out = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split("=", 1)
            out[k.strip()] = v.strip()
    return out


def _popcount_identity(xw: np.ndarray, ww: np.ndarray, K: int) -> np.ndarray:
    """K - 2 * sum popcount(x xor w) over packed rows (page "First Principles",
    section "1. Arithmetic"; page "Extreme Quantization" eq. (6)), computed with
    numpy's bit count on uint32 words."""
    x = xw[:, None, :] ^ ww[None, :, :]
    return (K - 2 * np.bitwise_count(x).sum(axis=-1, dtype=np.int64)).astype(np.int64)


def _rand_signs(rng, shape):
    return np.where(rng.random(shape) < 0.5, 1, -1).astype(np.int8)


# ---------------------------------------------------------------- worked example
def test_exercise1_worked_example():
    g = _read_kv(os.path.join(GOLDEN, "exercise1.txt"))
    w = np.array([int(t) for t in g["w_b"].split()], dtype=np.float32)[None, :]
    x = np.array([int(t) for t in g["x_b"].split()], dtype=np.float32)[None, :]
    ws, xs = oracle.sign(w), oracle.sign(x)
    wp, xp = oracle.pack_signs(ws), oracle.pack_signs(xs)
    assert int(wp[0, 0]) == int(g["w_word"])
    assert int(xp[0, 0]) == int(g["x_word"])
    assert bin(int(wp[0, 0]) ^ int(xp[0, 0])).count("1") == int(g["xor_popcount"])
    assert int(oracle.dot(xs, ws)[0, 0]) == int(g["dot"])


# ---------------------------------------------------------------- sign
def test_sign_edge_table():
    rows = []
    with open(os.path.join(GOLDEN, "sign_table.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                h, s, *_ = line.split()
                rows.append((int(h, 16), int(s)))
    bits = np.array([r[0] for r in rows], dtype=np.uint32)
    want = np.array([r[1] for r in rows], dtype=np.int8)
    got = oracle.sign(bits.view(np.float32)[None, :])[0]
    np.testing.assert_array_equal(got, want)


def test_sign_random_values_match_definition_by_bits():
    # sign by the IEEE ordering of the bit pattern: x >= 0 iff (non-NaN and the
    # sign bit clear) or x is -0.0.
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    nonneg = ((bits <= 0x7F800000) | (bits == 0x80000000))
    want = np.where(nonneg, 1, -1).astype(np.int8)
    np.testing.assert_array_equal(oracle.sign(x[None, :])[0], want)


# ---------------------------------------------------------------- packing
def test_pack_layout_bit_order_and_pads():
    # element k -> word k//32, bit k%32; -1 is bit 1; pad bits/words are 0.
    K = 70
    s = np.ones((3, K), dtype=np.int8)
    s[0, 0] = -1
    s[1, 33] = -1
    s[2, 69] = -1
    p = oracle.pack_signs(s, ld=5)
    assert p.shape == (3, 5)
    assert p[0].tolist() == [1, 0, 0, 0, 0]
    assert p[1].tolist() == [0, 2, 0, 0, 0]
    assert p[2].tolist() == [0, 0, 1 << 5, 0, 0]
    allneg = -np.ones((1, K), dtype=np.int8)
    q = oracle.pack_signs(allneg, ld=4)
    assert q[0].tolist() == [0xFFFFFFFF, 0xFFFFFFFF, 0x3F, 0]   # 6 live bits in word 2


def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(3)
    for K in (1, 31, 32, 33, 63, 64, 65, 1000):
        s = _rand_signs(rng, (5, K))
        p = oracle.pack_signs(s, ld=(K + 31) // 32 + 3)
        np.testing.assert_array_equal(oracle.unpack_signs(p, K), s)


def test_packed_bytes_match_page_formula():
    # page "First Principles", "Bandwidth math": binary packed weights take
    # M*N/8 bytes (1/8 byte per weight, 32 binary values per 32-bit word).
    for (N, K) in ((11008, 4096), (4096, 11008)):
        p = oracle.pack_signs(np.ones((4, K), dtype=np.int8))
        assert p.shape[1] * 4 * N == N * K // 8


# ---------------------------------------------------------------- the dot identity
def test_identity_exhaustive_small_K():
    for K in range(1, 9):
        S = np.array(list(itertools.product([1, -1], repeat=K)), dtype=np.int8)
        D = oracle.dot(S, S)
        P = oracle.pack_signs(S)
        np.testing.assert_array_equal(D.astype(np.int64), _popcount_identity(P, P, K))


@pytest.mark.parametrize("K", list(range(1, 131)) + [576, 1000, 2304, 4096, 11008])
def test_identity_random_K(K):
    rng = np.random.default_rng(K)
    xs, ws = _rand_signs(rng, (6, K)), _rand_signs(rng, (5, K))
    D = oracle.dot(xs, ws)
    np.testing.assert_array_equal(
        D.astype(np.int64), _popcount_identity(oracle.pack_signs(xs), oracle.pack_signs(ws), K))


@pytest.mark.parametrize("K", [1, 31, 32, 33, 100, 1000, 4096])
def test_packed_identity_routine_equals_dot(K):
    """The oracle's packed routine (K - 2 popcount(x xor w)) against its plain
    +1/-1 multiply-add, with wider rows (pad words) on one side."""
    rng = np.random.default_rng(90 + K)
    xs, ws = _rand_signs(rng, (7, K)), _rand_signs(rng, (5, K))
    xw = oracle.pack_signs(xs, ld=(K + 31) // 32 + 4)
    ww = oracle.pack_signs(ws)
    np.testing.assert_array_equal(oracle.dot_packed(xw, ww, K), oracle.dot(xs, ws))


def test_dot_matches_float64_matmul():
    rng = np.random.default_rng(11)
    for (M, N, K) in ((64, 256, 1000), (7, 9, 4096), (33, 17, 11008)):
        xs, ws = _rand_signs(rng, (M, K)), _rand_signs(rng, (N, K))
        ref = xs.astype(np.float64) @ ws.astype(np.float64).T
        np.testing.assert_array_equal(oracle.dot(xs, ws), ref.astype(np.int32))


def test_dot_invariants():
    rng = np.random.default_rng(5)
    K = 1000
    xs, ws = _rand_signs(rng, (20, K)), _rand_signs(rng, (30, K))
    D = oracle.dot(xs, ws).astype(np.int64)
    assert np.all((D - K) % 2 == 0)
    assert np.all(np.abs(D) <= K)
    np.testing.assert_array_equal(np.diag(oracle.dot(xs, xs)), np.full(20, K))
    np.testing.assert_array_equal(np.diag(oracle.dot(xs, -xs)), np.full(20, -K))
    ws2 = ws.copy()
    ws2[4] = -ws2[4]
    D2 = oracle.dot(xs, ws2).astype(np.int64)
    np.testing.assert_array_equal(D2[:, 4], -D[:, 4])
    np.testing.assert_array_equal(np.delete(D2, 4, axis=1), np.delete(D, 4, axis=1))


def test_pad_bit_invariance_and_negative_control():
    # page "First Principles": pad bits must encode +1 so they do not add to the
    # disagreement count d.  Equal pad bits on both sides leave the identity's
    # value unchanged; mismatched pad bits lower it by 2 per mismatch.
    rng = np.random.default_rng(9)
    for K in (1, 5, 31, 33, 1000):
        xs, ws = _rand_signs(rng, (4, K)), _rand_signs(rng, (3, K))
        D = oracle.dot(xs, ws).astype(np.int64)
        xp, wp = oracle.pack_signs(xs), oracle.pack_signs(ws)
        live = K % 32
        if live == 0:
            continue
        padmask = np.uint32((0xFFFFFFFF << live) & 0xFFFFFFFF)
        pat = np.uint32(rng.integers(1, 2**32, dtype=np.uint64)) & padmask
        xq, wq = xp.copy(), wp.copy()
        xq[:, -1] |= pat
        wq[:, -1] |= pat
        np.testing.assert_array_equal(_popcount_identity(xq, wq, K), D)
        xr = xp.copy()
        xr[:, -1] |= pat
        mism = bin(int(pat)).count("1")
        np.testing.assert_array_equal(_popcount_identity(xr, wp, K), D - 2 * mism)


# ---------------------------------------------------------------- alpha
def test_alpha_equals_exact_rational_mean():
    # page "Extreme Quantization" eq. (1): alpha = (1/n) sum |w_i|.  The exact
    # rational mean, rounded once to fp32, must equal the oracle's value.
    for K in (576, 1000, 2304, 4096, 11008, 16384):
        W = workloads.normal_f32(90000 + K, (6, K))
        a = oracle.alpha(W)
        for n in range(W.shape[0]):
            exact = sum((Fraction(float(abs(v))) for v in W[n]), Fraction(0)) / K
            assert f32_bits(a[n]) == f32_bits(round_to_f32(exact)), (K, n)


def test_alpha_closed_forms():
    rng = np.random.default_rng(1)
    K = 1000
    W = (0.75 * _rand_signs(rng, (4, K))).astype(np.float32)
    np.testing.assert_array_equal(oracle.alpha(W), np.full(4, 0.75, np.float32))
    assert oracle.alpha(np.zeros((1, 33), np.float32))[0] == 0.0
    # mean of |1..K| = (K+1)/2
    W = np.arange(1, K + 1, dtype=np.float32)[None, :] * np.where(np.arange(K) % 3, 1, -1)
    assert oracle.alpha(W.astype(np.float32))[0] == np.float32((K + 1) / 2)


# ---------------------------------------------------------------- scaling epilogues
def test_scale_is_one_rounded_multiply():
    rng = np.random.default_rng(2)
    a = (rng.random(50) * 3).astype(np.float32)
    D = rng.integers(-2**24, 2**24 + 1, size=(40, 50)).astype(np.int32)
    D[0, :] = 0
    Y = oracle.scale(D, a)
    for m in range(0, 40, 3):
        for n in range(50):
            want = round_to_f32(Fraction(float(a[n])) * int(D[m, n]))
            assert f32_bits(Y[m, n]) == f32_bits(want)


def test_scale_residual_two_roundings():
    rng = np.random.default_rng(4)
    a = (rng.random(30) * 2).astype(np.float32)
    D = rng.integers(-5000, 5001, size=(20, 30)).astype(np.int32)
    R = workloads.normal_f32(44, (20, 30)) * np.float32(1e3)
    R[0, :5] = np.float32(1e-30)     # very different exponents
    Y = oracle.scale_residual(D, a, R)
    for m in range(20):
        for n in range(30):
            z = round_to_f32(Fraction(float(a[n])) * int(D[m, n]))
            want = round_to_f32(Fraction(float(z)) + Fraction(float(R[m, n])))
            assert f32_bits(Y[m, n]) == f32_bits(want)


# ---------------------------------------------------------------- BatchNorm + sign
# Page "Binary Neural Network (BNN)" glossary (BatchNorm around the binary
# layers) and page "Extreme Quantization", eq. (4) (the next layer takes the
# sign, +1 for >= 0).  The oracle decides sign(BN(alpha D)) exactly; these pins
# check it against an evaluation of the formula in 80-digit decimal arithmetic
# (square root included, no rearrangement) and against closed-form ties.
def _bn_decimal(D, a, g, b, mu, var, eps, digits=80):
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = digits
        q = lambda v: Decimal(float(np.float32(v)))          # exact value of the fp32
        sd = (q(var) + q(eps)).sqrt()
        return q(g) * (q(a) * int(D) - q(mu)) / sd + q(b)


def _decided_sign(D, a, g, b, mu, var, eps):
    """+1 / -1 from the decimal value; None when it is too close to call
    (the 80-digit evaluation is good to ~1e-75 relative to the terms)."""
    v = _bn_decimal(D, a, g, b, mu, var, eps)
    scale = abs(float(g) * float(a) * D) + abs(float(g) * float(mu)) + abs(float(b)) + 1e-300
    if abs(v) <= scale * 1e-70:
        return None
    return 1 if v > 0 else -1


def test_bn_sign_closed_form_ties_and_directions():
    f = np.float32
    col = lambda *v: np.array(v, np.int32)[:, None]
    # gamma=1, alpha=0.5, beta=-1, mean=0, var=1, eps=0: BN = 0.5 D - 1, tie at D=2 -> +1
    s, m = oracle.bn_next_sign(col(1, 2, 3), f(0.5), f(1), f(-1), f(0), f(1), f(0))
    assert s[:, 0].tolist() == [-1, 1, 1] and m[0] == 0.0
    # gamma=-1: BN = -0.5 D - 1 >= 0 iff D <= -2 (tie at -2 -> +1)
    s, _ = oracle.bn_next_sign(col(-3, -2, -1), f(0.5), f(-1), f(-1), f(0), f(1), f(0))
    assert s[:, 0].tolist() == [1, 1, -1]
    # gamma=0: the constant sign of beta (beta=0 is a tie -> +1)
    for beta, want in ((0.3, 1), (-0.3, -1), (0.0, 1)):
        s, _ = oracle.bn_next_sign(col(-7, 0, 9), f(0.5), f(0), f(beta), f(0), f(1), f(1e-5))
        assert s[:, 0].tolist() == [want] * 3
    # alpha=0 (all-zero weight row): BN = beta - gamma*mean/sd = 0.2 - 1 < 0
    s, _ = oracle.bn_next_sign(col(5, -5), f(0), f(1), f(0.2), f(1), f(1), f(0))
    assert s[:, 0].tolist() == [-1, -1]
    # eps enters sd = sqrt(var + eps): var=0, eps=4 -> sd=2, BN = 0.5 D/2 - 1, tie at D=4
    s, _ = oracle.bn_next_sign(col(2, 3, 4, 5), f(0.5), f(1), f(-1), f(0), f(0), f(4))
    assert s[:, 0].tolist() == [-1, -1, 1, 1]
    # the mean shifts the tie: BN = (0.25 D - 1.5)/1.5 + 0 -> tie at D = 6
    s, _ = oracle.bn_next_sign(col(5, 6, 7), f(0.25), f(1), f(0), f(1.5), f(2.25), f(0))
    assert s[:, 0].tolist() == [-1, 1, 1]
    # a tie reached through sqrt: var+eps = 2.25 -> sd = 1.5; BN = 2(0.5 D - 0)/1.5 - 2 -> tie at D = 3
    s, _ = oracle.bn_next_sign(col(2, 3, 4), f(0.5), f(2), f(-2), f(0), f(2.25), f(0))
    assert s[:, 0].tolist() == [-1, 1, 1]


def test_bn_sign_rejects_undefined_parameters():
    f = np.float32
    D = np.zeros((1, 1), np.int32)
    with pytest.raises(ValueError):        # sqrt(var + eps) = 0
        oracle.bn_next_sign(D, f(1), f(1), f(0), f(0), f(0), f(0))
    with pytest.raises(ValueError):
        oracle.bn_next_sign(D, f(1), f(np.inf), f(0), f(0), f(1), f(0))


def _bn_random_channels(seed, N):
    rng = np.random.default_rng(seed)
    g, b, mu, var, eps = workloads.bn_params(seed, N)
    g = g * np.where(np.arange(N) % 5 == 0, -1, 1).astype(np.float32)   # both directions
    g[7] = 0.0
    mu = rng.normal(0, 3, N).astype(np.float32)
    var = (rng.random(N) * 2 + 0.1).astype(np.float32)
    a = (rng.random(N) + 0.2).astype(np.float32)
    a[11] = 0.0
    return a, g, b, mu, var, eps


@pytest.mark.parametrize("eps_scale", [1.0, 1e4])
def test_bn_sign_matches_decimal_evaluation(eps_scale):
    N = 48
    a, g, b, mu, var, eps = _bn_random_channels(12, N)
    eps = np.float32(eps * eps_scale)        # 1e-5, and 0.1 where eps moves the boundaries
    K = 64
    rng = np.random.default_rng(13)
    D = rng.integers(-K, K + 1, size=(40, N)).astype(np.int32)
    s, margin = oracle.bn_next_sign(D, a, g, b, mu, var, eps)
    undecided = 0
    for m in range(D.shape[0]):
        for n in range(N):
            want = _decided_sign(int(D[m, n]), a[n], g[n], b[n], mu[n], var[n], eps)
            if want is None:
                undecided += 1
                continue
            assert s[m, n] == want, (m, n)
    assert undecided == 0
    for n in range(N):   # the reported margin is the smallest |BN| of the column
        mins = min(abs(float(_bn_decimal(int(d), a[n], g[n], b[n], mu[n], var[n], eps))) for d in D[:, n])
        assert margin[n] == pytest.approx(mins, rel=1e-12, abs=1e-300)


def test_bn_rule_boundaries_by_decimal_evaluation():
    """Each channel's integer boundary: the decimal value changes sign there."""
    N = 48
    a, g, b, mu, var, eps = _bn_random_channels(14, N)
    K = 200
    kind, bound = oracle.bn_rule(a, g, b, mu, var, eps, K)
    for n in range(N):
        args = (a[n], g[n], b[n], mu[n], var[n], eps)
        if kind[n] == 0:
            assert g[n] == 0 or a[n] == 0
            assert all(_decided_sign(d, *args) == bound[n] for d in (-K, 0, K))
        elif kind[n] > 0:
            if -K < bound[n] <= K:
                assert _decided_sign(int(bound[n]), *args) == 1
                assert _decided_sign(int(bound[n]) - 1, *args) == -1
        else:
            if -K <= bound[n] < K:
                assert _decided_sign(int(bound[n]), *args) == 1
                assert _decided_sign(int(bound[n]) + 1, *args) == -1
    # the rule applied to every D agrees with the per-output decisions
    Dall = np.broadcast_to(np.arange(-K, K + 1, dtype=np.int32)[:, None], (2 * K + 1, N))
    s, _ = oracle.bn_next_sign(Dall, a, g, b, mu, var, eps)
    np.testing.assert_array_equal(oracle.rule_signs(kind, bound, Dall), s)


def test_bn_brute_force_tiny_layer():
    """Every decision of a small binary layer against the decimal value."""
    rng = np.random.default_rng(15)
    M, N, K = 12, 14, 37
    xs, ws = _rand_signs(rng, (M, K)), _rand_signs(rng, (N, K))
    D = oracle.dot(xs, ws)
    a, g, b, mu, var, eps = _bn_random_channels(16, N)
    mu = (a * rng.integers(-3, 4, N)).astype(np.float32)   # boundaries near the data
    s, _ = oracle.bn_next_sign(D, a, g, b, mu, var, eps)
    for m in range(M):
        for n in range(N):
            assert s[m, n] == _decided_sign(int(D[m, n]), a[n], g[n], b[n], mu[n], var[n], eps)


def _mlp_layer_params(i):
    c = workloads.WORKLOADS[2]
    h = c["hidden"]
    Wh = workloads.normal_f32(workloads.seed_for(2, 2 + i), (h, h))
    return (oracle.alpha(Wh),) + workloads.bn_params(workloads.seed_for(2, 10 + i), h)


@pytest.mark.parametrize("layer", [0, 1, 2])
def test_full_bn_rule_every_mlp_channel(layer):
    """The binary MLP's hidden layers (batch 1024, 4096 -> 4096, K = 4096):
    for every one of the 4096 channels, the oracle's exact boundary is where
    the 80-digit value of BN(alpha D) changes sign.  Decisions on both sides
    of each boundary are also far from their ties (reported margin)."""
    a, g, b, mu, var, eps = _mlp_layer_params(layer)
    K = workloads.WORKLOADS[2]["hidden"]
    kind, bound = oracle.bn_rule(a, g, b, mu, var, eps, K)
    assert (kind == 1).all()              # gamma > 0 and alpha > 0 on every channel
    closest = np.inf
    for n in range(K):
        args = (a[n], g[n], b[n], mu[n], var[n], eps)
        hi = _bn_decimal(int(bound[n]), *args)
        lo = _bn_decimal(int(bound[n]) - 1, *args)
        assert hi >= 0 > lo, n
        closest = min(closest, float(hi), -float(lo))
    assert closest > 1e-6, f"a decision lies within {closest:.3g} of its tie"


# ---------------------------------------------------------------- conv im2col
def _direct_conv_pm1(xs_nhwc: np.ndarray, ws_ohwi: np.ndarray) -> np.ndarray:
    """3x3, stride 1, pad 1 with pad value +1, as direct loops over the
    padded +1/-1 image (no im2col)."""
    B, H, W, C = xs_nhwc.shape
    Co = ws_ohwi.shape[0]
    P = np.ones((B, H + 2, W + 2, C), dtype=np.int64)
    P[:, 1:-1, 1:-1, :] = xs_nhwc
    out = np.zeros((B, H, W, Co), dtype=np.int64)
    for b in range(B):
        for oh in range(H):
            for ow in range(W):
                for o in range(Co):
                    acc = 0
                    for kh in range(3):
                        for kw in range(3):
                            acc += int(np.dot(P[b, oh + kh, ow + kw, :], ws_ohwi[o, kh, kw, :].astype(np.int64)))
                    out[b, oh, ow, o] = acc
    return out


def test_im2col_dot_matches_direct_conv_and_torch():
    import torch
    import torch.nn.functional as F
    X = workloads.normal_f32(5100, (2, 5, 4, 3))
    Wt = workloads.normal_f32(5101, (4, 3, 3, 3))
    D = oracle.dot(oracle.im2col_signs(X), oracle.sign(Wt.reshape(4, 27)))
    xs = oracle.sign(X.reshape(-1, 3)).reshape(X.shape)
    ws = oracle.sign(Wt.reshape(-1, 3)).reshape(Wt.shape)
    direct = _direct_conv_pm1(xs, ws).reshape(-1, 4)
    np.testing.assert_array_equal(D.astype(np.int64), direct)
    xt = torch.from_numpy(xs.astype(np.float64)).permute(0, 3, 1, 2)
    wt = torch.from_numpy(ws.astype(np.float64)).permute(0, 3, 1, 2)
    ref = F.conv2d(F.pad(xt, (1, 1, 1, 1), value=1.0), wt)
    np.testing.assert_array_equal(D.astype(np.int64),
                                  ref.permute(0, 2, 3, 1).reshape(-1, 4).numpy().astype(np.int64))


def test_im2col_border_taps_are_plus_one():
    X = -np.ones((1, 2, 2, 2), dtype=np.float32)     # every in-image sign is -1
    cols = oracle.im2col_signs(X)
    # output pixel (0,0): taps with kh==0 or kw==0 are outside -> +1
    row = cols[0].reshape(3, 3, 2)
    for kh in range(3):
        for kw in range(3):
            want = 1 if (kh == 0 or kw == 0) else -1
            assert np.all(row[kh, kw] == want), (kh, kw)


def test_conv_block_residual_layout():
    X = workloads.normal_f32(5200, (1, 3, 3, 4))
    Wt = workloads.normal_f32(5201, (4, 3, 3, 4))
    D, Y, a = oracle.conv_block(X, Wt)
    np.testing.assert_array_equal(Y, oracle.scale_residual(D, a, X.reshape(9, 4)))


# ---------------------------------------------------------------- FP first/last layers
def test_dense_f64_matches_numpy_and_exact():
    X = workloads.uniform01_f32(2000, (8, 784))
    W = workloads.normal_f32(2001, (16, 784))
    H = oracle.dense_f64(X, W)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    bound = 784 * 2.0**-52 * (np.abs(X).astype(np.float64) @ np.abs(W).astype(np.float64).T)
    assert np.all(np.abs(H - ref) <= 2 * bound)
    for (m, n) in ((0, 0), (3, 7), (7, 15)):
        exact = sum((Fraction(float(X[m, k])) * Fraction(float(W[n, k])) for k in range(784)), Fraction(0))
        assert abs(Fraction(H[m, n]) - exact) <= Fraction(float(bound[m, n]))


def test_dense_pm1_f32out_is_rounded_exact_sum():
    rng = np.random.default_rng(8)
    s = _rand_signs(rng, (4, 300))
    W = workloads.normal_f32(2005, (3, 300))
    Y = oracle.dense_pm1_f32out(s, W)
    for m in range(4):
        for n in range(3):
            exact = sum((int(s[m, k]) * Fraction(float(W[n, k])) for k in range(300)), Fraction(0))
            # double accumulation error is far below half an fp32 ulp here
            assert abs(float(Y[m, n]) - float(exact)) <= abs(float(exact)) * 2.0**-23 + 1e-30
            assert f32_bits(Y[m, n]) == f32_bits(round_to_f32(exact))


def test_mlp_chain_small_composition():
    X = workloads.uniform01_f32(2100, (16, 40))
    W1 = workloads.normal_f32(2101, (64, 40))
    hidden = []
    for i in range(3):
        Wh = workloads.normal_f32(2110 + i, (64, 64))
        hidden.append((Wh,) + workloads.bn_params(2120 + i, 64))
    W5 = workloads.normal_f32(2130, (10, 64))
    r = oracle.binary_mlp(X, W1, hidden, W5)
    s = r["signs"][0]
    np.testing.assert_array_equal(s, np.where(X.astype(np.float64) @ W1.astype(np.float64).T >= 0, 1, -1))
    for i, (Wh, g, b, mu, var, eps) in enumerate(hidden):
        D = (s.astype(np.int64) @ np.where(Wh >= 0, 1, -1).T)
        np.testing.assert_array_equal(r["dots"][i], D)
        for m in range(0, 16, 5):
            for n in range(64):
                want = _decided_sign(int(D[m, n]), r["alphas"][i][n], g[n], b[n], mu[n], var[n], eps)
                assert r["signs"][i + 1][m, n] == want
        s = r["signs"][i + 1]
    assert r["logits"].shape == (16, 10)


# ---------------------------------------------------------------- binary weights x INT8 activations
# Page "Extreme Quantization", "Binary Neural Networks" eq. (1)-(2): with
# +1/-1 weights a dot product only adds or subtracts activations; its "BitNet"
# section keeps the activations at INT8.
def test_dot_i8_matches_int64_matmul():
    rng = np.random.default_rng(70)
    for K in (1, 7, 31, 32, 33, 100, 1000, 4096):
        xq = rng.integers(-128, 128, size=(5, K)).astype(np.int8)
        ws = _rand_signs(rng, (9, K))
        want = xq.astype(np.int64) @ ws.astype(np.int64).T
        np.testing.assert_array_equal(oracle.dot_i8(xq, ws).astype(np.int64), want)


def test_dot_i8_add_subtract_reading():
    # eq. (2): each weight either adds (+1) or subtracts (-1) its activation
    rng = np.random.default_rng(71)
    xq = rng.integers(-128, 128, size=(3, 37)).astype(np.int8)
    ws = _rand_signs(rng, (4, 37))
    D = oracle.dot_i8(xq, ws)
    for m in range(3):
        for n in range(4):
            acc = 0
            for k in range(37):
                if ws[n, k] == 1:
                    acc += int(xq[m, k])
                else:
                    acc -= int(xq[m, k])
            assert int(D[m, n]) == acc


def test_half_decode_every_finite_pattern():
    # the oracle decodes fp16 from the format's definition; numpy's IEEE
    # binary16 conversion is the independent reading of the same standard
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 10) & 0x1F) != 0x1F
    bits = bits[finite]
    U = oracle.bwn_f16_units(bits.reshape(-1, 1), np.ones((1, 1), np.int8))[:, 0]
    want = bits.view(np.float16).astype(np.float64)
    np.testing.assert_array_equal(U.astype(np.float64) * 2.0 ** -24, want)
    with pytest.raises(ValueError):
        oracle.bwn_f16_units(np.array([[0x7C00]], np.uint16), np.ones((1, 1), np.int8))


def test_bwn_f16_pm1_activations_equal_dot():
    # eq. (1)-(2) with +1/-1 activations is the binary dot product (eq. (6))
    rng = np.random.default_rng(73)
    for K in (1, 31, 33, 1000, 4096):
        xs = _rand_signs(rng, (3, K))
        ws = _rand_signs(rng, (5, K))
        U = oracle.bwn_f16_units(xs.astype(np.float16), ws)
        np.testing.assert_array_equal(U, oracle.dot(xs, ws).astype(np.int64) << 24)


def test_bwn_f16_exact_rational_sums():
    # brute force in exact rationals over values of every fp16 class
    # (subnormals, zeros of both signs, the largest finite value)
    rng = np.random.default_rng(74)
    x = (rng.standard_normal((4, 57)) * np.exp2(rng.integers(-26, 17, size=(4, 57)))).astype(np.float16)
    x[0, :5] = np.array([0.0, -0.0, 65504.0, -65504.0, 2.0 ** -24], np.float16)
    x[~np.isfinite(x)] = np.float16(1.5)
    W = rng.standard_normal((6, 57)).astype(np.float32)
    W[0, :3] = [0.0, -0.0, 1e-40]                # sign(0) = sign(-0) = +1, a denormal weight +1
    S, _ = oracle.bwn_f16(x, W, np.ones(6, np.float32))
    U = oracle.bwn_f16_units(x, oracle.sign(W))
    for m in range(4):
        for n in range(6):
            exact = sum((Fraction(float(x[m, k])) * (1 if (W[n, k] >= 0) else -1) for k in range(57)), Fraction(0))
            assert Fraction(int(U[m, n]), 1 << 24) == exact
            assert S[m, n] == float(exact)


def test_bwn_f16_invariants():
    rng = np.random.default_rng(75)
    x = rng.standard_normal((3, 300)).astype(np.float16)
    W = rng.standard_normal((7, 300)).astype(np.float32)
    W[W == 0] = 1.0
    U = oracle.bwn_f16_units(x, oracle.sign(W))
    np.testing.assert_array_equal(oracle.bwn_f16_units(x, oracle.sign(-W)), -U)          # negate weights
    np.testing.assert_array_equal(oracle.bwn_f16_units(-x, oracle.sign(W)), -U)          # negate activations
    ones = np.ones((1, 300), np.int8)
    tot = oracle.bwn_f16_units(x, ones)[:, 0]
    np.testing.assert_array_equal(tot.astype(np.float64) * 2.0 ** -24,
                                  x.astype(np.float64).sum(axis=1))     # all +1: the plain sum (exact here)
    _, y = oracle.bwn_f16(x, W, np.full(7, 0.5, np.float32))
    np.testing.assert_array_equal(y, 0.5 * U.astype(np.float64) * 2.0 ** -24)


def test_dot_i8_extremes_and_invariants():
    K = 1000
    lo = np.full((1, K), -128, np.int8)
    hi = np.full((1, K), 127, np.int8)
    plus = np.ones((1, K), np.int8)
    minus = -plus
    assert int(oracle.dot_i8(lo, minus)[0, 0]) == 128 * K
    assert int(oracle.dot_i8(lo, plus)[0, 0]) == -128 * K
    assert int(oracle.dot_i8(hi, minus)[0, 0]) == -127 * K
    rng = np.random.default_rng(72)
    xq = rng.integers(-128, 128, size=(4, 333)).astype(np.int8)
    ws = _rand_signs(rng, (6, 333))
    D = oracle.dot_i8(xq, ws)
    np.testing.assert_array_equal(oracle.dot_i8(xq, -ws), -D)          # negate weights
    np.testing.assert_array_equal(oracle.dot_i8(xq, ws[::-1]), D[:, ::-1])  # row n -> column n


def test_planes_layout_hand_example():
    # q = [1, -1, -128, 127, 0]; bytes 0x01, 0xFF, 0x80, 0x7F, 0x00.
    # plane 0 holds elements 0, 1, 3 -> 0b1011 = 11; planes 1..6 hold
    # elements 1, 3 -> 0b1010 = 10; plane 7 holds elements 1, 2 -> 0b110 = 6.
    words, xsum = oracle.pack_planes_i8(np.array([[1, -1, -128, 127, 0]], np.int8), ld=2)
    assert words.shape == (1, 8, 2)
    assert [int(v) for v in words[0, :, 0]] == [11, 10, 10, 10, 10, 10, 10, 6]
    assert not words[0, :, 1].any()
    assert int(xsum[0]) == -1


def test_planes_reconstruct_values_and_pads():
    rng = np.random.default_rng(73)
    for K in (1, 31, 32, 33, 1000):
        Q = rng.integers(-128, 128, size=(3, K)).astype(np.int8)
        words, xsum = oracle.pack_planes_i8(Q, ld=(K + 31) // 32 + 2)
        bits = (words[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1   # [M, 8, ld, 32]
        bits = bits.reshape(3, 8, -1).astype(np.int64)
        weight = np.array([1, 2, 4, 8, 16, 32, 64, -128], np.int64)      # two's complement
        vals = np.einsum("mbk,b->mk", bits, weight)
        np.testing.assert_array_equal(vals[:, :K], Q.astype(np.int64))
        assert not bits[:, :, K:].any()                                    # pads hold 0
        np.testing.assert_array_equal(xsum.astype(np.int64), Q.astype(np.int64).sum(axis=1))


def test_planes_popcount_identity_equals_dot_i8():
    # With weight bit 1 = -1: sum_k s_k x_k = sum_k x_k - 2 sum_{k: bit_k = 1} x_k,
    # and sum_{bit=1} x = sum_b c_b popcount(plane_b AND wbits), c_b = 2^b
    # (b < 7), c_7 = -128.
    rng = np.random.default_rng(74)
    for K in (5, 64, 1000, 4096):
        Q = rng.integers(-128, 128, size=(4, K)).astype(np.int8)
        ws = _rand_signs(rng, (7, K))
        planes, xsum = oracle.pack_planes_i8(Q)
        wp = oracle.pack_signs(ws)
        cnt = np.bitwise_count(planes[:, None, :, :] & wp[None, :, None, :]).sum(axis=-1, dtype=np.int64)
        weight = np.array([1, 2, 4, 8, 16, 32, 64, -128], np.int64)
        neg = (cnt * weight).sum(axis=-1)
        np.testing.assert_array_equal(xsum[:, None].astype(np.int64) - 2 * neg,
                                      oracle.dot_i8(Q, ws).astype(np.int64))


def test_quantize_integer_grid_is_exact():
    x = np.arange(-127, 128, dtype=np.float32)[None, :]
    Q, sc = oracle.quantize_absmax_i8(x)
    np.testing.assert_array_equal(Q[0].astype(np.int64), np.arange(-127, 128))
    assert sc[0] == np.float32(1.0)


def test_quantize_half_even_ties():
    # amax = 254 -> 127/254 = 0.5 exactly; x * 0.5 lands on .5 for odd x
    x = np.array([[254.0, 5.0, 7.0, -5.0, -7.0, 1.0, 3.0, -254.0]], np.float32)
    Q, sc = oracle.quantize_absmax_i8(x)
    assert Q[0].tolist() == [127, 2, 4, -2, -4, 0, 2, -127]
    assert sc[0] == np.float32(2.0)


def test_quantize_matches_exact_rounding_away_from_ties():
    # q is the integer nearest to x * 127 / amax; the single-precision
    # evaluation may differ from exact only within a few ulps of a .5 tie.
    rng = np.random.default_rng(75)
    X = workloads.normal_f32(75000, (6, 700)) * np.float32(3.0)
    X[1] *= np.float32(1e-30)                  # tiny magnitudes
    X[2] *= np.float32(1e30)
    Q, sc = oracle.quantize_absmax_i8(X)
    for m in range(X.shape[0]):
        amax = Fraction(float(np.abs(X[m]).max()))
        assert f32_bits(sc[m]) == f32_bits(round_to_f32(amax / 127))
        for k in range(X.shape[1]):
            t = Fraction(float(X[m, k])) * 127 / amax
            fl = math.floor(t)
            frac = t - fl
            if abs(frac - Fraction(1, 2)) > Fraction(1, 10000):
                assert int(Q[m, k]) == (fl + 1 if frac > Fraction(1, 2) else fl), (m, k)
            else:
                assert int(Q[m, k]) in (fl, fl + 1)
    # the largest magnitude always maps to +-127; the map is odd
    for m in range(X.shape[0]):
        k = int(np.abs(X[m]).argmax())
        assert abs(int(Q[m, k])) == 127
    Qn, scn = oracle.quantize_absmax_i8(-X)
    np.testing.assert_array_equal(Qn, -Q)
    np.testing.assert_array_equal(scn, sc)
    del rng


def test_quantize_special_rows():
    nan, inf = np.float32(np.nan), np.float32(np.inf)
    X = np.array([[0.0, -0.0, 0.0, 0.0],
                  [nan, 2.0, -1.0, nan],
                  [inf, 1.0, -3.0, 0.0]], np.float32)
    Q, sc = oracle.quantize_absmax_i8(X)
    assert Q[0].tolist() == [0, 0, 0, 0] and sc[0] == 0.0
    assert Q[1].tolist() == [0, 127, -64, 0] and sc[1] == np.float32(2.0 / 127.0)
    assert Q[2].tolist() == [0, 0, 0, 0] and np.isinf(sc[2])


def test_alpha_tensor_equals_exact_rational_mean():
    # page "Extreme Quantization" eq. (8): ||W||_1 / (nm), one scale
    for shape in ((3, 1000), (16, 576), (7, 33)):
        W = workloads.normal_f32(76000 + shape[1], shape)
        exact = sum((Fraction(float(abs(v))) for v in W.ravel()), Fraction(0)) / (shape[0] * shape[1])
        assert f32_bits(oracle.alpha_tensor(W)) == f32_bits(round_to_f32(exact))
    W = np.full((5, 40), -0.25, np.float32)
    assert oracle.alpha_tensor(W) == np.float32(0.25)
    # per-tensor scale differs from the per-row one when the rows differ
    W = np.vstack([np.full((1, 8), 1.0, np.float32), np.full((1, 8), 3.0, np.float32)])
    assert oracle.alpha_tensor(W) == np.float32(2.0)
    assert oracle.alpha(W).tolist() == [1.0, 3.0]


def test_scale_i8_two_roundings():
    rng = np.random.default_rng(77)
    D = rng.integers(-128 * 4096, 128 * 4096, size=(6, 20)).astype(np.int32)
    a = (rng.random(20) * 2).astype(np.float32)
    xs = (rng.random(6) * 0.1).astype(np.float32)
    for aa in (a, a[:1]):
        Y = oracle.scale_i8(D, aa, xs)
        for m in range(6):
            for n in range(20):
                an = aa[n] if aa.shape[0] > 1 else aa[0]
                z = round_to_f32(Fraction(float(an)) * int(D[m, n]))
                want = round_to_f32(Fraction(float(z)) * Fraction(float(xs[m])))
                assert f32_bits(Y[m, n]) == f32_bits(want)


def test_scale_bias_residual_roundings():
    rng = np.random.default_rng(78)
    D = rng.integers(-5000, 5001, size=(8, 12)).astype(np.int32)
    a = (rng.random(12) * 2).astype(np.float32)
    b = workloads.normal_f32(78001, (12,)) * np.float32(100.0)
    R = workloads.normal_f32(78002, (8, 12)) * np.float32(1e3)
    R[0, :3] = np.float32(1e-30)
    for aa in (a, a[:1]):
        for RR in (None, R):
            Y = oracle.scale_bias_residual(D, aa, b, RR)
            for m in range(8):
                for n in range(12):
                    an = aa[n] if aa.shape[0] > 1 else aa[0]
                    z = round_to_f32(Fraction(float(an)) * int(D[m, n]))
                    z = round_to_f32(Fraction(float(z)) + Fraction(float(b[n])))
                    if RR is not None:
                        z = round_to_f32(Fraction(float(z)) + Fraction(float(RR[m, n])))
                    assert f32_bits(Y[m, n]) == f32_bits(z)


# ---------------------------------------------------------------- ternary weights
# Page "Extreme Quantization": "Ternary Quantization" eq. (7) and "BitNet
# b1.58" eq. (9).
def test_ternary_threshold_cases():
    d = np.float32(0.25)
    up = np.nextafter(d, np.float32(1))
    W = np.array([[0.25, -0.25, up, -up, 0.0, -0.0, 1e-30, np.nan, np.inf, -np.inf, 3.0, -3.0]], np.float32)
    assert oracle.ternary_threshold(W, d)[0].tolist() == [0, 0, 1, -1, 0, 0, 0, 0, 1, -1, 1, -1]
    # Delta = 0 reduces to the sign with 0 kept as 0
    rng = np.random.default_rng(80)
    W = workloads.normal_f32(80001, (5, 300))
    np.testing.assert_array_equal(oracle.ternary_threshold(W, 0.0), np.sign(W).astype(np.int8))
    # huge Delta: everything is 0
    assert not oracle.ternary_threshold(W, 1e30).any()
    del rng


def test_ternary_roundclip_exact_rounding():
    # gamma a power of two makes w / gamma exact: ties at .5 go to even
    g = np.float32(0.5)
    W = np.array([[0.25, -0.25, 0.75, -0.75, 0.2499999, 0.2500001, 0.0, 100.0, -100.0, np.nan]], np.float32)
    assert oracle.ternary_roundclip(W, g)[0].tolist() == [0, 0, 1, -1, 0, 1, 0, 1, -1, 0]
    # random weights: equal to the exactly rounded quotient wherever it is
    # not within a few ulps of a .5 tie
    W = workloads.normal_f32(81001, (6, 400))
    gam = oracle.alpha_tensor(W)
    T = oracle.ternary_roundclip(W, gam)
    G = Fraction(float(gam))
    for n in range(W.shape[0]):
        for k in range(W.shape[1]):
            q = Fraction(float(W[n, k])) / G
            fl = math.floor(q)
            fr = q - fl
            if abs(fr - Fraction(1, 2)) < Fraction(1, 10**6):
                continue
            r = fl + 1 if fr > Fraction(1, 2) else fl
            assert int(T[n, k]) == max(-1, min(1, r)), (n, k)


def test_ternary_b158_gamma_is_tensor_mean_and_delta_relation():
    W = workloads.normal_f32(82001, (4, 1000))
    T, g = oracle.ternary_b158(W)
    exact = sum((Fraction(float(abs(v))) for v in W.ravel()), Fraction(0)) / W.size
    assert f32_bits(g) == f32_bits(round_to_f32(exact))
    # away from the rounding boundary, RoundClip(w / gamma) is eq. (7) with Delta = gamma / 2
    T7 = oracle.ternary_threshold(W, np.float32(g) / np.float32(2))
    far = np.abs(np.abs(W.astype(np.float64)) / float(g) - 0.5) > 1e-5
    np.testing.assert_array_equal(T[far], T7[far])
    # roughly the familiar share of zeros for a Gaussian at Delta = 0.4 sigma (~31%)
    assert 0.2 < (T == 0).mean() < 0.45


def test_pack_ternary_layout_and_roundtrip():
    T = np.array([[1, -1, 0, 0, 0, 0, 1, -1]], np.int8)
    S, Z, nnz = oracle.pack_ternary(T, ld=2)
    assert S.tolist() == [[0b10000010, 0]] and Z.tolist() == [[0b11000011, 0]] and nnz.tolist() == [4]
    rng = np.random.default_rng(83)
    for K in (1, 31, 32, 33, 100, 1000):
        T = rng.integers(-1, 2, size=(4, K)).astype(np.int8)
        S, Z, nnz = oracle.pack_ternary(T, ld=(K + 31) // 32 + 1)
        sb = ((S[..., None] >> np.arange(32, dtype=np.uint32)) & 1).reshape(4, -1).astype(np.int64)
        zb = ((Z[..., None] >> np.arange(32, dtype=np.uint32)) & 1).reshape(4, -1).astype(np.int64)
        back = zb * (1 - 2 * sb)
        np.testing.assert_array_equal(back[:, :K], T.astype(np.int64))
        assert not sb[:, K:].any() and not zb[:, K:].any()
        assert (sb <= zb).all()                      # a sign bit only where nonzero
        np.testing.assert_array_equal(nnz, (T != 0).sum(axis=1))


def test_ternary_dot_identities():
    # integer multiply-add vs numpy, and the two packed identities the GPU uses:
    #  binary x: sum t x = nnz - 2 popcount((xbits ^ S) & Z)
    #  int8 x:   sum t q = sum_b c_b (popc(P_b & Z) - 2 popc(P_b & Z & S))
    rng = np.random.default_rng(84)
    c = np.array([1, 2, 4, 8, 16, 32, 64, -128], np.int64)
    for K in (7, 64, 1000):
        T = rng.integers(-1, 2, size=(6, K)).astype(np.int8)
        xs = _rand_signs(rng, (5, K))
        Q = rng.integers(-128, 128, size=(5, K)).astype(np.int8)
        D1 = oracle.dot_i8(xs, T)
        D2 = oracle.dot_i8(Q, T)
        np.testing.assert_array_equal(D1.astype(np.int64), xs.astype(np.int64) @ T.astype(np.int64).T)
        np.testing.assert_array_equal(D2.astype(np.int64), Q.astype(np.int64) @ T.astype(np.int64).T)
        S, Z, nnz = oracle.pack_ternary(T)
        xp = oracle.pack_signs(xs)
        pc = np.bitwise_count((xp[:, None, :] ^ S[None]) & Z[None]).sum(axis=-1, dtype=np.int64)
        np.testing.assert_array_equal(nnz[None, :].astype(np.int64) - 2 * pc, D1.astype(np.int64))
        P, _ = oracle.pack_planes_i8(Q)
        a = np.bitwise_count(P[:, None, :, :] & Z[None, :, None, :]).sum(axis=-1, dtype=np.int64)
        b = np.bitwise_count(P[:, None, :, :] & (Z & S)[None, :, None, :]).sum(axis=-1, dtype=np.int64)
        np.testing.assert_array_equal(((a - 2 * b) * c).sum(axis=-1), D2.astype(np.int64))


# ---------------------------------------------------------------- RSign and chained conv blocks
# Page "State of the Art Survey", ReActNet row (RSign) and Bi-Real Net row
# (FP shortcut per block).
def test_rsign_is_sign_of_exact_difference():
    rng = np.random.default_rng(85)
    X = workloads.normal_f32(85001, (40, 24))
    beta = (rng.standard_normal(24) * 0.5).astype(np.float32)
    X[0, :] = beta                                   # ties: x == beta -> +1
    X[1, :3] = [np.nan, np.inf, -np.inf]
    s = oracle.rsign(X, beta)
    for r in range(X.shape[0]):
        for c in range(X.shape[1]):
            x, b = float(X[r, c]), float(beta[c])
            if math.isnan(x):
                want = -1
            elif math.isinf(x):
                want = 1 if x > 0 else -1
            else:
                want = 1 if Fraction(x) - Fraction(b) >= 0 else -1
            assert int(s[r, c]) == want, (r, c)
    # beta = 0 is the plain sign (Notation of "Extreme Quantization")
    np.testing.assert_array_equal(oracle.rsign(X, np.zeros(24, np.float32)), oracle.sign(X))


def test_im2col_pm1_matches_sign_im2col():
    X = workloads.normal_f32(86001, (2, 5, 4, 8))
    S = oracle.sign(X.reshape(-1, 8)).reshape(X.shape)
    np.testing.assert_array_equal(oracle.im2col_pm1(S), oracle.im2col_signs(X))


def test_conv_block_rsign_matches_torch_conv():
    import torch
    B, H, W, C = 2, 5, 6, 8
    X = workloads.normal_f32(87001, (B, H, W, C))
    Wt = workloads.normal_f32(87002, (C, 3, 3, C))
    beta = workloads.normal_f32(87003, (C,)) * np.float32(0.3)
    D, Y, a = oracle.conv_block_rsign(X, Wt, beta)
    # signs of (x - beta) decided exactly, then a float64 conv with +1 padding
    xs = np.where(X.astype(np.float64) - beta.astype(np.float64) >= 0, 1.0, -1.0)
    t = torch.from_numpy(xs).permute(0, 3, 1, 2)
    t = torch.nn.functional.pad(t, (1, 1, 1, 1), value=1.0)
    w = torch.from_numpy(np.where(Wt >= 0, 1.0, -1.0)).permute(0, 3, 1, 2)
    ref = torch.nn.functional.conv2d(t, w).permute(0, 2, 3, 1).reshape(B * H * W, C).numpy()
    np.testing.assert_array_equal(D.astype(np.float64), ref)
    np.testing.assert_array_equal(Y.reshape(-1, C), oracle.scale_residual(D, a, X.reshape(-1, C)))


def test_conv_chain_composes_blocks():
    B, H, W, C = 1, 4, 4, 8
    X = workloads.normal_f32(88001, (B, H, W, C))
    Ws = [workloads.normal_f32(88002 + i, (C, 3, 3, C)) for i in range(3)]
    bs = [workloads.normal_f32(88010 + i, (C,)) * np.float32(0.2) for i in range(3)]
    out = oracle.conv_chain(X, Ws, bs)
    x = X
    for (D, Y), Wl, bl in zip(out, Ws, bs):
        D2, Y2, _ = oracle.conv_block_rsign(x, Wl, bl)
        np.testing.assert_array_equal(D, D2)
        np.testing.assert_array_equal(Y, Y2)
        x = Y2
