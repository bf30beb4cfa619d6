"""CPU oracle for the binary XNOR-popcount path (numpy front end).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline may import this package; the product package never does.  It shares
no code with the HIP library.

The arithmetic lives in ``oracle.c`` (plain C, built with gcc into
``liboracle.so``); this module only marshals numpy arrays.  Each wrapper names
the passage of the source pages it follows (page title and section/equation):

* "First Principles: Why Binary Ops Can Be Exponentially Faster", section
  "1. Arithmetic: MAC -> XNOR + popcount": bit 0 encodes +1, bit 1 encodes -1,
  pad bits encode +1, and the dot identity <w,x> = N - 2 popcount(w xor x).
* "Extreme Quantization: Binary, Ternary & 1-bit LLMs": Notation (sign),
  eq. (1) (alpha = mean |w|), eq. (4)-(6) (XNOR-Net).
* "Binary Neural Network (BNN)" glossary: scaling factors and BatchNorm
  (BatchNorm followed by the sign is decided exactly in ``batchnorm.py``).
* "Perfected Concept", "What is binary vs not": FP first/last layers and FP
  residual streams; "State of the Art Survey", Bi-Real Net: FP shortcut.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .batchnorm import bn_next_sign, bn_rule, bn_value, rule_signs  # noqa: F401  (exact BatchNorm + sign)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


GCC_FLAGS = ["-std=c11", "-O3", "-fopenmp", "-fPIC", "-shared",
             "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra"]


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile ``oracle.c`` with gcc (never hipcc) into ``liboracle.so``."""
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp"
    subprocess.run(["gcc"] + GCC_FLAGS + [src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def _load(path: str):
    L = ctypes.CDLL(path)
    return L


def use_library(path: str | None):
    """Point the wrappers at another build of oracle.c (the mutation test
    compiles deliberately broken copies to check that the pins catch them);
    None restores the default library."""
    global _lib
    _lib = None if path is None else _configure(_load(path))


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _configure(_load(_LIB))
    return _lib


def _configure(L):
    """Declare the C signatures on a loaded oracle library."""
    sigs = {
        "oracle_sign": [_p, _i64, _i64, _i64, _p],
        "oracle_pack_signs": [_p, _i64, _i64, _p, _i64],
        "oracle_unpack_signs": [_p, _i64, _i64, _i64, _p],
        "oracle_alpha": [_p, _i64, _i64, _i64, _p],
        "oracle_dot": [_p, _p, _i64, _i64, _i64, _p],
        "oracle_dot_packed": [_p, _i64, _p, _i64, _i64, _i64, _i64, _p],
        "oracle_scale": [_p, _p, _i64, _i64, _p],
        "oracle_scale_residual": [_p, _p, _p, _i64, _i64, _i64, _p],
        "oracle_im2col_signs": [_p, _i64, _i64, _i64, _i64, _p],
        "oracle_dense_f64": [_p, _i64, _p, _i64, _i64, _i64, _i64, _p],
        "oracle_dense_pm1_f32out": [_p, _p, _i64, _i64, _i64, _i64, _p],
        "oracle_dot_i8": [_p, _p, _i64, _i64, _i64, _p],
        "oracle_quantize_absmax_i8": [_p, _i64, _i64, _i64, _p, _p],
        "oracle_pack_planes_i8": [_p, _i64, _i64, _p, _i64, _p],
        "oracle_scale_i8": [_p, _p, _i64, _p, _i64, _i64, _p],
        "oracle_scale_bias_residual": [_p, _p, _i64, _p, _p, _i64, _i64, _i64, _p],
        "oracle_ternary_threshold": [_p, _i64, _i64, _i64, ctypes.c_float, _p],
        "oracle_ternary_roundclip": [_p, _i64, _i64, _i64, ctypes.c_float, _p],
        "oracle_pack_ternary": [_p, _i64, _i64, _i64, _p, _p, _p],
        "oracle_rsign": [_p, _i64, _i64, _i64, _p, _p],
        "oracle_im2col_pm1": [_p, _i64, _i64, _i64, _i64, _p],
    }
    for name, args in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = None
    L.oracle_bwn_f16.argtypes = [_p, _i64, _p, _i64, _i64, _i64, _p]
    L.oracle_bwn_f16.restype = ctypes.c_int
    L.oracle_alpha_tensor.argtypes = [_p, _i64, _i64, _i64]
    L.oracle_alpha_tensor.restype = ctypes.c_float
    L.oracle_num_threads.argtypes = []
    L.oracle_num_threads.restype = ctypes.c_int
    return L


def num_threads() -> int:
    """OpenMP threads the oracle's loops run on."""
    return int(lib().oracle_num_threads())


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def sign(x: np.ndarray) -> np.ndarray:
    """sign(x) = +1 for x >= 0, -1 otherwise, as int8 (Notation, page
    "Extreme Quantization")."""
    x = _c(x, np.float32)
    x2 = x.reshape(-1, x.shape[-1]) if x.ndim > 1 else x.reshape(1, -1)
    s = np.empty(x2.shape, dtype=np.int8)
    lib().oracle_sign(_ptr(x2), x2.shape[0], x2.shape[1], x2.shape[1], _ptr(s))
    return s.reshape(x.shape)


def pack_signs(s: np.ndarray, ld: int | None = None) -> np.ndarray:
    """Pack a [rows, K] matrix of +1/-1 into uint32 words [rows, ld]
    (bit 0 = +1, bit 1 = -1, LSB first, pad bits and pad words 0)."""
    s = _c(s, np.int8)
    rows, K = s.shape
    kw = (K + 31) // 32
    ld = kw if ld is None else ld
    assert ld >= kw
    out = np.empty((rows, ld), dtype=np.uint32)
    lib().oracle_pack_signs(_ptr(s), rows, K, _ptr(out), ld)
    return out


def unpack_signs(words: np.ndarray, K: int) -> np.ndarray:
    words = _c(words, np.uint32)
    rows, ld = words.shape
    s = np.empty((rows, K), dtype=np.int8)
    lib().oracle_unpack_signs(_ptr(words), rows, K, ld, _ptr(s))
    return s


def alpha(W: np.ndarray) -> np.ndarray:
    """alpha_n = mean_k |W[n, k]| (eq. (1)), double sum, one rounding."""
    W = _c(W, np.float32)
    N, K = W.shape
    out = np.empty(N, dtype=np.float32)
    lib().oracle_alpha(_ptr(W), N, K, K, _ptr(out))
    return out


def dot(xs: np.ndarray, ws: np.ndarray) -> np.ndarray:
    """D[m, n] = sum_k xs[m, k] * ws[n, k] over +1/-1 int8 (eq. (6))."""
    xs = _c(xs, np.int8)
    ws = _c(ws, np.int8)
    M, K = xs.shape
    N, K2 = ws.shape
    assert K == K2
    D = np.empty((M, N), dtype=np.int32)
    lib().oracle_dot(_ptr(xs), _ptr(ws), M, N, K, _ptr(D))
    return D


def dot_packed(xw: np.ndarray, ww: np.ndarray, K: int) -> np.ndarray:
    """D = K - 2 sum popcount(x xor w) over packed rows (the identity of
    "First Principles" section "1. Arithmetic" / "Extreme Quantization"
    eq. (6)); CPU-baseline context, not an expected-value source."""
    xw = _c(xw, np.uint32)
    ww = _c(ww, np.uint32)
    M, ldx = xw.shape
    N, ldw = ww.shape
    assert min(ldx, ldw) >= (K + 31) // 32
    D = np.empty((M, N), dtype=np.int32)
    lib().oracle_dot_packed(_ptr(xw), ldx, _ptr(ww), ldw, M, N, K, _ptr(D))
    return D


def dot_i8(xq: np.ndarray, ws: np.ndarray) -> np.ndarray:
    """D[m, n] = sum_k xq[m, k] * ws[n, k]: int8 activations times +1/-1
    weights ("Extreme Quantization" eq. (1)-(2); INT8 activations of its
    BitNet section)."""
    xq = _c(xq, np.int8)
    ws = _c(ws, np.int8)
    M, K = xq.shape
    N, K2 = ws.shape
    assert K == K2
    D = np.empty((M, N), dtype=np.int32)
    lib().oracle_dot_i8(_ptr(xq), _ptr(ws), M, N, K, _ptr(D))
    return D


def bwn_f16_units(x16: np.ndarray, ws: np.ndarray) -> np.ndarray:
    """S[m, n] = sum_k ws[n, k] * x[m, k] with fp16 activations and +1/-1
    weights ("Extreme Quantization" eq. (1)-(2), BinaryConnect / BWN), taken
    exactly: int64 [M, N] in units of 2^-24 (S = units * 2^-24).  x16 holds
    fp16 values (np.float16) or their bit patterns (np.uint16); all finite."""
    x16 = np.ascontiguousarray(x16)
    bits = x16.view(np.uint16) if x16.dtype == np.float16 else _c(x16, np.uint16)
    ws = _c(ws, np.int8)
    M, K = bits.shape
    N, K2 = ws.shape
    assert K == K2 and K <= 1 << 14
    S = np.empty((M, N), dtype=np.int64)
    if lib().oracle_bwn_f16(_ptr(bits), K, _ptr(ws), M, N, K, _ptr(S)):
        raise ValueError("fp16 activations must be finite")
    return S


def bwn_f16(x16: np.ndarray, W: np.ndarray, a: np.ndarray):
    """Binary weights x fp16 activations, y = alpha_n * sum_k s(W[n, k]) x[m, k]
    (eq. (1)-(2)): returns (S float64 [M, N], y float64 [M, N]) with S exact
    up to its final rounding to double and y = alpha * S in double (the
    reference a tolerance is measured against)."""
    U = bwn_f16_units(x16, sign(W))
    S = U.astype(np.float64) * 2.0 ** -24
    return S, np.asarray(a, np.float64)[None, :] * S


def quantize_absmax_i8(X: np.ndarray):
    """Per-row symmetric absmax INT8 quantization (BitNet item 2; the
    quantizer itself is this module's reading): returns (Q int8 [M, K],
    scale fp32 [M]) with X ~= scale * Q."""
    X = _c(X, np.float32)
    M, K = X.shape
    Q = np.empty((M, K), dtype=np.int8)
    sc = np.empty(M, dtype=np.float32)
    lib().oracle_quantize_absmax_i8(_ptr(X), M, K, K, _ptr(Q), _ptr(sc))
    return Q, sc


def pack_planes_i8(Q: np.ndarray, ld: int | None = None):
    """Bit planes of int8 rows: words [M, 8, ld] (plane b = bit b of each
    two's-complement byte, packed LSB first along K, pads 0) and xsum [M]."""
    Q = _c(Q, np.int8)
    M, K = Q.shape
    kw = (K + 31) // 32
    ld = kw if ld is None else ld
    assert ld >= kw
    words = np.empty((M, 8, ld), dtype=np.uint32)
    xsum = np.empty(M, dtype=np.int32)
    lib().oracle_pack_planes_i8(_ptr(Q), M, K, _ptr(words), ld, _ptr(xsum))
    return words, xsum


def alpha_tensor(W: np.ndarray) -> np.float32:
    """One scale for the whole matrix, ||W||_1 / (N K) (eq. (8))."""
    W = _c(W, np.float32)
    N, K = W.shape
    return np.float32(lib().oracle_alpha_tensor(_ptr(W), N, K, K))


def scale_i8(D: np.ndarray, a: np.ndarray, xscale: np.ndarray) -> np.ndarray:
    """Y = fl(fl(alpha * D) * xscale_m); a of length N (per row) or 1 (per
    tensor)."""
    D = _c(D, np.int32)
    a = _c(np.atleast_1d(a), np.float32)
    xscale = _c(xscale, np.float32)
    M, N = D.shape
    stride = 0 if a.shape[0] == 1 else 1
    assert stride == 0 or a.shape[0] == N
    Y = np.empty((M, N), dtype=np.float32)
    lib().oracle_scale_i8(_ptr(D), _ptr(a), stride, _ptr(xscale), M, N, _ptr(Y))
    return Y


def scale_bias_residual(D: np.ndarray, a: np.ndarray, bias: np.ndarray,
                        R: np.ndarray | None = None) -> np.ndarray:
    """Y = fl(fl(fl(alpha * D) + b_n) + R) (bias of "y = Wx + b"; R optional);
    a of length N (per row) or 1 (per tensor, eq. (8))."""
    D = _c(D, np.int32)
    a = _c(np.atleast_1d(a), np.float32)
    bias = _c(bias, np.float32)
    M, N = D.shape
    stride = 0 if a.shape[0] == 1 else 1
    assert stride == 0 or a.shape[0] == N
    Y = np.empty((M, N), dtype=np.float32)
    if R is None:
        lib().oracle_scale_bias_residual(_ptr(D), _ptr(a), stride, _ptr(bias), None, 0, M, N, _ptr(Y))
    else:
        R = _c(R, np.float32)
        assert R.shape == (M, N)
        lib().oracle_scale_bias_residual(_ptr(D), _ptr(a), stride, _ptr(bias), _ptr(R), N, M, N, _ptr(Y))
    return Y


def binary_weight_linear_i8(X: np.ndarray, W: np.ndarray, per_tensor: bool = False):
    """fp32 activations X [M, K] quantized to INT8, times binary weights W
    [N, K]: returns (Q, xscale, D int32, Y fp32, alpha)."""
    Q, xs = quantize_absmax_i8(X)
    a = np.atleast_1d(alpha_tensor(W)) if per_tensor else alpha(W)
    D = dot_i8(Q, sign(W))
    return Q, xs, D, scale_i8(D, a, xs), a


def scale(D: np.ndarray, a: np.ndarray) -> np.ndarray:
    """Y = alpha_n * D (eq. (1)), one rounded single multiply."""
    D = _c(D, np.int32)
    a = _c(a, np.float32)
    M, N = D.shape
    Y = np.empty((M, N), dtype=np.float32)
    lib().oracle_scale(_ptr(D), _ptr(a), M, N, _ptr(Y))
    return Y


def scale_residual(D: np.ndarray, a: np.ndarray, R: np.ndarray) -> np.ndarray:
    """Y = fl(fl(alpha_n * D) + R) (FP shortcut of Bi-Real Net)."""
    D = _c(D, np.int32)
    a = _c(a, np.float32)
    R = _c(R, np.float32)
    M, N = D.shape
    assert R.shape == (M, N)
    Y = np.empty((M, N), dtype=np.float32)
    lib().oracle_scale_residual(_ptr(D), _ptr(a), _ptr(R), N, M, N, _ptr(Y))
    return Y


def im2col_signs(X: np.ndarray) -> np.ndarray:
    """[B*H*W, 9*C] signs of a 3x3/stride-1/pad-1 im2col of NHWC X, pad = +1."""
    X = _c(X, np.float32)
    B, H, W, C = X.shape
    cols = np.empty((B * H * W, 9 * C), dtype=np.int8)
    lib().oracle_im2col_signs(_ptr(X), B, H, W, C, _ptr(cols))
    return cols


def dense_f64(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """H = X W^T accumulated in double (first FP layer)."""
    X = _c(X, np.float32)
    W = _c(W, np.float32)
    M, K = X.shape
    N, K2 = W.shape
    assert K == K2
    H = np.empty((M, N), dtype=np.float64)
    lib().oracle_dense_f64(_ptr(X), K, _ptr(W), K, M, N, K, _ptr(H))
    return H


def dense_pm1_f32out(s: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Y = fl32(sum_k s[m,k] W[n,k]) with a double sum (last FP layer)."""
    s = _c(s, np.int8)
    W = _c(W, np.float32)
    M, K = s.shape
    N, K2 = W.shape
    assert K == K2
    Y = np.empty((M, N), dtype=np.float32)
    lib().oracle_dense_pm1_f32out(_ptr(s), _ptr(W), K, M, N, K, _ptr(Y))
    return Y


# ---------------------------------------------------------------------------
# Whole-workload chains, each composed only of the routines above.
# ---------------------------------------------------------------------------

def binary_linear(X: np.ndarray, W: np.ndarray):
    """Single binary linear layer: returns (D int32, Y = alpha*D fp32, alpha)."""
    a = alpha(W)
    D = dot(sign(X), sign(W))
    return D, scale(D, a), a


def binary_mlp(X, W1, hidden, W5):
    """Binary MLP: FP first layer (double accumulate) -> sign -> binary hidden
    layers with folded BatchNorm and sign -> FP last layer on the +1/-1 output.

    ``hidden`` is a list of (W, gamma, beta, mean, var, eps).  Returns a dict
    with the first-layer pre-activations, per-layer signs, alphas, integer
    dots, the BatchNorm margins (smallest |BN(alpha D)| per channel) and the
    logits.
    """
    h1 = dense_f64(X, W1)
    s = np.where(h1 >= 0.0, 1, -1).astype(np.int8)
    out = dict(h1=h1, signs=[s], alphas=[], dots=[], bn_margins=[])
    for (W, g, b, mu, var, eps) in hidden:
        a = alpha(W)
        D = dot(s, sign(W))
        s, margin = bn_next_sign(D, a, g, b, mu, var, eps)
        out["alphas"].append(a)
        out["dots"].append(D)
        out["bn_margins"].append(margin)
        out["signs"].append(s)
    out["logits"] = dense_pm1_f32out(s, W5)
    return out


def conv_block(X: np.ndarray, W_ohwi: np.ndarray):
    """Binary 3x3 conv (stride 1, pad 1, pad pixels +1) + alpha + FP residual.

    X is NHWC [B, H, W, C]; W_ohwi is [Cout, 3, 3, C]; the residual is X
    itself (Cout == C).  Returns (D [B*H*W, Cout], Y, alpha)."""
    B, H, Wd, C = X.shape
    Cout = W_ohwi.shape[0]
    Wf = np.ascontiguousarray(W_ohwi.reshape(Cout, 9 * C))
    a = alpha(Wf)
    D = dot(im2col_signs(X), sign(Wf))
    R = X.reshape(B * H * Wd, C)
    return D, scale_residual(D, a, R), a


def ternary_threshold(W: np.ndarray, delta: float) -> np.ndarray:
    """Eq. (7): +1 for w > Delta, -1 for w < -Delta, else 0 (int8 [N, K])."""
    W = _c(W, np.float32)
    N, K = W.shape
    T = np.empty((N, K), dtype=np.int8)
    lib().oracle_ternary_threshold(_ptr(W), N, K, K, ctypes.c_float(float(delta)), _ptr(T))
    return T


def ternary_roundclip(W: np.ndarray, gamma: float) -> np.ndarray:
    """Eq. (9): RoundClip(W / gamma, -1, 1) (int8 [N, K])."""
    W = _c(W, np.float32)
    N, K = W.shape
    T = np.empty((N, K), dtype=np.int8)
    lib().oracle_ternary_roundclip(_ptr(W), N, K, K, ctypes.c_float(float(gamma)), _ptr(T))
    return T


def pack_ternary(T: np.ndarray, ld: int | None = None):
    """Sign plane, nonzero plane (uint32 [N, ld] each) and nonzero counts [N]."""
    T = _c(T, np.int8)
    N, K = T.shape
    kw = (K + 31) // 32
    ld = kw if ld is None else ld
    assert ld >= kw
    S = np.empty((N, ld), dtype=np.uint32)
    Z = np.empty((N, ld), dtype=np.uint32)
    nnz = np.empty(N, dtype=np.int32)
    lib().oracle_pack_ternary(_ptr(T), N, K, ld, _ptr(S), _ptr(Z), _ptr(nnz))
    return S, Z, nnz


def ternary_b158(W: np.ndarray):
    """BitNet b1.58 weights (eq. (9)): (T int8 [N, K], gamma)."""
    g = alpha_tensor(W)
    return ternary_roundclip(W, g), g


def rsign(X: np.ndarray, beta: np.ndarray) -> np.ndarray:
    """RSign (ReActNet row): +1 where x >= beta_c (per column c), else -1."""
    X = _c(X, np.float32)
    beta = _c(beta, np.float32)
    rows, cols = X.shape
    assert beta.shape == (cols,)
    s = np.empty((rows, cols), dtype=np.int8)
    lib().oracle_rsign(_ptr(X), rows, cols, cols, _ptr(beta), _ptr(s))
    return s


def im2col_pm1(S: np.ndarray) -> np.ndarray:
    """[B*H*W, 9*C] im2col of NHWC signs S, taps outside the image +1."""
    S = _c(S, np.int8)
    B, H, W, C = S.shape
    cols = np.empty((B * H * W, 9 * C), dtype=np.int8)
    lib().oracle_im2col_pm1(_ptr(S), B, H, W, C, _ptr(cols))
    return cols


def conv_block_rsign(X: np.ndarray, W_ohwi: np.ndarray, beta: np.ndarray | None = None):
    """One binary 3x3 conv block with RSign input: D = conv(RSign(X, beta), sign W),
    Y = fl(fl(alpha * D) + X) (Bi-Real FP shortcut).  beta None means 0 (the
    plain sign).  Returns (D [B*H*W, Cout], Y [B, H, W, Cout], alpha)."""
    B, H, Wd, C = X.shape
    Cout = W_ohwi.shape[0]
    assert Cout == C
    b = np.zeros(C, np.float32) if beta is None else beta
    S = rsign(X.reshape(B * H * Wd, C), b).reshape(B, H, Wd, C)
    Wf = np.ascontiguousarray(W_ohwi.reshape(Cout, 9 * C))
    a = alpha(Wf)
    D = dot(im2col_pm1(S), sign(Wf))
    Y = scale_residual(D, a, X.reshape(B * H * Wd, C))
    return D, Y.reshape(B, H, Wd, Cout), a


def conv_chain(X: np.ndarray, weights, betas):
    """A chain of conv blocks: X_{l+1} = Y_l.  Returns the list of (D, Y)."""
    out = []
    for Wl, bl in zip(weights, betas):
        D, Y, _ = conv_block_rsign(X, Wl, bl)
        out.append((D, Y))
        X = Y
    return out
