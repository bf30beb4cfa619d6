"""Python binding of libbnn.so, the MI355X (gfx950) binary-network hot path.

Argument marshalling only: every step of the path (sign + bit-pack,
XNOR-popcount GEMM/GEMV, alpha / residual / folded-BatchNorm epilogues, the FP
first and last layers) runs in the HIP kernels behind the C ABI declared in
``include/bnn.h``.  PyTorch provides device memory and the current stream;
there is no CPU or PyTorch fallback: if the library is missing, importing the
binding's calls raises.

The functions keep the C names without the ``bnn_`` prefix.  Tensors passed
in must live on a HIP device; outputs are allocated here (or given with
``out=`` style arguments) with the layouts the C ABI documents:
packed matrices are uint32 ``[rows, ld]`` stored as ``torch.int32`` (same
bits), ``ld`` a multiple of 4, bit 0 = +1, bit 1 = -1, pad bits and words 0.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "BnnError", "lib", "packed_words", "padded_ld", "pack_weights", "pack_activations",
    "xnor_gemm", "xnor_gemm_mfma", "linear_fused", "fold_bn_thresholds", "dense_f32_sign_pack",
    "dense_binact_f32", "EPI_DOT_I32", "EPI_SCALE_F32", "EPI_RESIDUAL_F32",
    "EPI_THRESH_PACK", "EPI_ALPHA_TENSOR", "EPI_BIAS_F32", "LIB_PATH",
    "weight_scale_tensor", "weight_scale_tensor_noalloc", "NOALLOC_MAX_ROWS", "quantize_act_i8", "pack_act_i8", "bwn_i8_linear", "MAX_K_I8", "bwn_f16_gemv", "MAX_K_F16",
    "W_TERNARY", "pack_weights_ternary", "EPI_SIGN_PACK", "pack_activations_rsign", "conv3x3_fused",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbnn.so")

EPI_DOT_I32 = 1
EPI_SCALE_F32 = 2
EPI_RESIDUAL_F32 = 4
EPI_THRESH_PACK = 8
EPI_ALPHA_TENSOR = 16
EPI_BIAS_F32 = 32
W_TERNARY = 64
EPI_SIGN_PACK = 128
MAX_K_I8 = 1 << 17
MAX_K_F16 = 16384
NOALLOC_MAX_ROWS = 1 << 16

_STATUS = {
    0: "BNN_OK", 1: "BNN_ERR_NULL", 2: "BNN_ERR_SHAPE", 3: "BNN_ERR_LD",
    4: "BNN_ERR_ALIGN", 5: "BNN_ERR_UNSUPPORTED", 6: "BNN_ERR_HIP",
}


class BnnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)}")


class _ConvGeom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("B", "H", "W", "C", "R", "S", "stride", "pad")]


class _FusedArgs(ctypes.Structure):
    _fields_ = [
        ("Xp", ctypes.c_void_p), ("ldXp", ctypes.c_int64),
        ("Wp", ctypes.c_void_p), ("ldWp", ctypes.c_int64),
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("epilogue", ctypes.c_uint32),
        ("D", ctypes.c_void_p), ("ldD", ctypes.c_int64),
        ("alpha", ctypes.c_void_p),
        ("Y", ctypes.c_void_p), ("ldY", ctypes.c_int64),
        ("R", ctypes.c_void_p), ("ldR", ctypes.c_int64),
        ("tau", ctypes.c_void_p), ("dir", ctypes.c_void_p),
        ("Op", ctypes.c_void_p), ("ldOp", ctypes.c_int64),
        ("bias", ctypes.c_void_p),
        ("Zp", ctypes.c_void_p), ("nnz", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
    ]


class _I8Args(ctypes.Structure):
    _fields_ = [
        ("Xb", ctypes.c_void_p), ("ldXb", ctypes.c_int64),
        ("xsum", ctypes.c_void_p),
        ("Xq", ctypes.c_void_p), ("ldXq", ctypes.c_int64),
        ("xscale", ctypes.c_void_p),
        ("Wp", ctypes.c_void_p), ("ldWp", ctypes.c_int64),
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("epilogue", ctypes.c_uint32),
        ("D", ctypes.c_void_p), ("ldD", ctypes.c_int64),
        ("alpha", ctypes.c_void_p),
        ("Y", ctypes.c_void_p), ("ldY", ctypes.c_int64),
        ("Zp", ctypes.c_void_p),
    ]


_lib = None
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """Load libbnn.so (built in-tree by ``xnor_popcount_gemm_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m xnor_popcount_gemm_amd.build` "
                "(there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        L.bnn_packed_words.argtypes = [_i64]
        L.bnn_packed_words.restype = _i64
        L.bnn_status_string.argtypes = [ctypes.c_int]
        L.bnn_status_string.restype = ctypes.c_char_p
        sigs = {
            "bnn_pack_weights": [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp],
            "bnn_pack_activations": [_vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp],
            "bnn_xnor_gemm": [_vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _vp],
            "bnn_xnor_gemm_mfma": [_vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _vp],
            "bnn_linear_fused": [ctypes.POINTER(_FusedArgs), _vp],
            "bnn_fold_bn_thresholds_host": [_vp, _vp, _vp, _vp, ctypes.c_float, _vp, _i64, _vp, _vp],
            "bnn_dense_f32_sign_pack": [_vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _i64, _vp],
            "bnn_dense_binact_f32": [_vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _i64, _vp],
            "bnn_weight_scale_tensor": [_vp, _i64, _i64, _i64, _vp, _vp, _vp],
            "bnn_weight_scale_tensor_noalloc": [_vp, _i64, _i64, _i64, _vp, _vp],
            "bnn_quantize_act_i8": [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp],
            "bnn_pack_act_i8": [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp],
            "bnn_bwn_i8_linear": [ctypes.POINTER(_I8Args), _vp],
            "bnn_bwn_f16_gemv": [_vp, _i64, _vp, _i64, _i64, _i64, _i64, ctypes.c_uint32, _vp, _vp, _i64, _vp],
            "bnn_pack_weights_ternary": [_vp, _i64, _i64, _i64, _vp, ctypes.c_float, _vp, _vp, _i64, _vp, _vp],
            "bnn_pack_activations_rsign": [_vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp],
            "bnn_conv3x3_fused": [ctypes.POINTER(_FusedArgs), ctypes.POINTER(_ConvGeom), _vp],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise BnnError(status, where)


def packed_words(K: int) -> int:
    """ceil(K / 32)."""
    return int(lib().bnn_packed_words(int(K)))


def padded_ld(K: int) -> int:
    """Smallest valid leading dimension of a packed matrix: ceil(K/32) rounded
    up to a multiple of 4 words (16-byte rows)."""
    kw = (int(K) + 31) // 32
    return (kw + 3) // 4 * 4


def _dev(t: torch.Tensor, dtype, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    return t


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _packed_empty(rows: int, K: int, device, ld: int | None = None) -> torch.Tensor:
    ld = padded_ld(K) if ld is None else ld
    return torch.empty((rows, ld), dtype=torch.int32, device=device)


def pack_weights(W: torch.Tensor, *, alpha: bool = True, out: torch.Tensor | None = None,
                 alpha_out: torch.Tensor | None = None):
    """Sign + bit-pack fp32 weights [N, K]; returns (Wp [N, ld], alpha [N] or None)."""
    _dev(W, torch.float32, "W")
    N, K = W.shape
    Wp = _packed_empty(N, K, W.device) if out is None else out
    a = None
    if alpha:
        a = torch.empty(N, dtype=torch.float32, device=W.device) if alpha_out is None else alpha_out
    _check(lib().bnn_pack_weights(_ptr(W), N, K, _ld(W), _ptr(Wp), _ld(Wp), _ptr(a),
                                  _stream(W.device)), "bnn_pack_weights")
    return Wp, a


def pack_activations(X: torch.Tensor, *, conv3x3: bool = False, out: torch.Tensor | None = None):
    """Sign + bit-pack activations.

    Dense: X fp32 [M, K] -> packed [M, ld].  ``conv3x3=True``: X is an NHWC
    fp32 image [B, H, W, C] (contiguous) and the result is its packed 3x3 /
    stride 1 / pad 1 im2col matrix [B*H*W, ld] with K = 9*C, pad pixels +1.
    """
    _dev(X, torch.float32, "X")
    if conv3x3:
        if X.dim() != 4 or not X.is_contiguous():
            raise ValueError("conv3x3 input must be a contiguous NHWC tensor")
        B, H, Wd, C = X.shape
        M, K = B * H * Wd, 9 * C
        g = _ConvGeom(B, H, Wd, C, 3, 3, 1, 1)
        Xp = _packed_empty(M, K, X.device) if out is None else out
        _check(lib().bnn_pack_activations(_ptr(X), M, K, C, ctypes.byref(g), _ptr(Xp), _ld(Xp),
                                          _stream(X.device)), "bnn_pack_activations")
        return Xp
    M, K = X.shape
    Xp = _packed_empty(M, K, X.device) if out is None else out
    _check(lib().bnn_pack_activations(_ptr(X), M, K, _ld(X), None, _ptr(Xp), _ld(Xp),
                                      _stream(X.device)), "bnn_pack_activations")
    return Xp


def xnor_gemm(Xp: torch.Tensor, Wp: torch.Tensor, K: int, *, alpha: torch.Tensor | None = None,
              want_dot: bool = True, want_scaled: bool = False,
              D: torch.Tensor | None = None, Y: torch.Tensor | None = None):
    """D = K - 2 popcount(Xp xor Wp) (int32 [M, N]) and/or Y = alpha * D (fp32)."""
    _dev(Xp, torch.int32, "Xp")
    _dev(Wp, torch.int32, "Wp")
    M, N = Xp.shape[0], Wp.shape[0]
    if want_dot and D is None:
        D = torch.empty((M, N), dtype=torch.int32, device=Xp.device)
    if want_scaled and Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=Xp.device)
    if not want_dot:
        D = None
    if not want_scaled:
        Y = None
    _check(lib().bnn_xnor_gemm(_ptr(Xp), _ld(Xp), _ptr(Wp), _ld(Wp), M, N, int(K),
                               _ptr(D), _ld(D) if D is not None else 0, _ptr(alpha),
                               _ptr(Y), _ld(Y) if Y is not None else 0,
                               _stream(Xp.device)), "bnn_xnor_gemm")
    return D, Y


def xnor_gemm_mfma(Xp: torch.Tensor, Wp: torch.Tensor, K: int, *, alpha: torch.Tensor | None = None,
                   want_dot: bool = True, want_scaled: bool = False,
                   D: torch.Tensor | None = None, Y: torch.Tensor | None = None):
    """The same D and Y as ``xnor_gemm``, computed on the fp4 matrix cores
    (bnn_xnor_gemm_mfma: exact +-1 products)."""
    _dev(Xp, torch.int32, "Xp")
    _dev(Wp, torch.int32, "Wp")
    M, N = Xp.shape[0], Wp.shape[0]
    if want_dot and D is None:
        D = torch.empty((M, N), dtype=torch.int32, device=Xp.device)
    if want_scaled and Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=Xp.device)
    if not want_dot:
        D = None
    if not want_scaled:
        Y = None
    _check(lib().bnn_xnor_gemm_mfma(_ptr(Xp), _ld(Xp), _ptr(Wp), _ld(Wp), M, N, int(K),
                                    _ptr(D), _ld(D) if D is not None else 0, _ptr(alpha),
                                    _ptr(Y), _ld(Y) if Y is not None else 0,
                                    _stream(Xp.device)), "bnn_xnor_gemm_mfma")
    return D, Y


def _fused_struct(Xp, Wp, K, epilogue, M, *, alpha=None, R=None, tau=None, dir=None, D=None, Y=None,
                  Op=None, bias=None, Zp=None, nnz=None, beta=None):
    N = Wp.shape[0]
    dev = Xp.device
    if epilogue & EPI_DOT_I32 and D is None:
        D = torch.empty((M, N), dtype=torch.int32, device=dev)
    if epilogue & (EPI_SCALE_F32 | EPI_RESIDUAL_F32) and Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    if epilogue & (EPI_THRESH_PACK | EPI_SIGN_PACK) and Op is None:
        Op = _packed_empty(M, N, dev)
    a = _FusedArgs()
    a.Xp, a.ldXp = Xp.data_ptr(), _ld(Xp)
    a.Wp, a.ldWp = Wp.data_ptr(), _ld(Wp)
    a.M, a.N, a.K = M, N, int(K)
    a.epilogue = int(epilogue)
    if D is not None:
        a.D, a.ldD = D.data_ptr(), _ld(D)
    if alpha is not None:
        a.alpha = alpha.data_ptr()
    if Y is not None:
        a.Y, a.ldY = Y.data_ptr(), _ld(Y)
    if R is not None:
        a.R, a.ldR = R.data_ptr(), _ld(R)
    if tau is not None:
        a.tau = tau.data_ptr()
    if dir is not None:
        a.dir = dir.data_ptr()
    if Op is not None:
        a.Op, a.ldOp = Op.data_ptr(), _ld(Op)
    if bias is not None:
        a.bias = bias.data_ptr()
    if Zp is not None:
        a.Zp = Zp.data_ptr()
    if nnz is not None:
        a.nnz = nnz.data_ptr()
    if beta is not None:
        a.beta = beta.data_ptr()
    return a, {"D": D, "Y": Y, "Op": Op}


def linear_fused(Xp: torch.Tensor, Wp: torch.Tensor, K: int, epilogue: int, *,
                 alpha=None, R=None, tau=None, dir=None, D=None, Y=None, Op=None,
                 bias=None, Zp=None, nnz=None, beta=None, M: int | None = None):
    """XNOR-popcount GEMM with a fused epilogue (OR of EPI_* flags).

    Returns a dict with the outputs the flags ask for: ``D`` (int32 [M, N]),
    ``Y`` (fp32 [M, N]), ``Op`` (packed [M, ld] of the output signs).
    """
    _dev(Xp, torch.int32, "Xp")
    _dev(Wp, torch.int32, "Wp")
    M = Xp.shape[0] if M is None else M
    a, out = _fused_struct(Xp, Wp, K, epilogue, M, alpha=alpha, R=R, tau=tau, dir=dir, D=D, Y=Y, Op=Op,
                           bias=bias, Zp=Zp, nnz=nnz, beta=beta)
    _check(lib().bnn_linear_fused(ctypes.byref(a), _stream(Xp.device)), "bnn_linear_fused")
    return out


def conv3x3_fused(Ximg: torch.Tensor, Wp: torch.Tensor, geom, epilogue: int, **kw):
    """Binary 3x3 conv with implicit im2col: Ximg is the packed NHWC image
    [B*H*W, ld] (C bits per pixel), Wp the packed OHWI weights; geom =
    (B, H, W, C).  Epilogue keywords as for linear_fused."""
    _dev(Ximg, torch.int32, "Ximg")
    _dev(Wp, torch.int32, "Wp")
    B, H, W, C = geom
    M = B * H * W
    a, out = _fused_struct(Ximg, Wp, 9 * C, epilogue, M, **kw)
    g = _ConvGeom(B, H, W, C, 3, 3, 1, 1)
    _check(lib().bnn_conv3x3_fused(ctypes.byref(a), ctypes.byref(g), _stream(Ximg.device)), "bnn_conv3x3_fused")
    return out


def pack_activations_rsign(X: torch.Tensor, beta: torch.Tensor, *, out: torch.Tensor | None = None):
    """Packed RSign of fp32 rows [M, K]: bit = (x >= beta_k) ? 0 : 1."""
    _dev(X, torch.float32, "X")
    _dev(beta, torch.float32, "beta")
    M, K = X.shape
    Xp = _packed_empty(M, K, X.device) if out is None else out
    _check(lib().bnn_pack_activations_rsign(_ptr(X), M, K, _ld(X), _ptr(beta), _ptr(Xp), _ld(Xp),
                                            _stream(X.device)), "bnn_pack_activations_rsign")
    return Xp


def fold_bn_thresholds(gamma, beta, mean, var, eps, alpha):
    """Host-side BatchNorm fold -> (tau fp32 [N], dir int8 [N]) as numpy arrays."""
    import numpy as np
    g, b, mu, v, a = (np.ascontiguousarray(x, dtype=np.float32) for x in (gamma, beta, mean, var, alpha))
    N = a.shape[0]
    tau = np.empty(N, dtype=np.float32)
    d = np.empty(N, dtype=np.int8)
    P = lambda x: x.ctypes.data_as(ctypes.c_void_p)
    _check(lib().bnn_fold_bn_thresholds_host(P(g), P(b), P(mu), P(v), ctypes.c_float(float(eps)),
                                             P(a), N, P(tau), P(d)), "bnn_fold_bn_thresholds_host")
    return tau, d


def dense_f32_sign_pack(X: torch.Tensor, W: torch.Tensor, *, out: torch.Tensor | None = None):
    """FP first layer: packed signs of X W^T (double accumulation)."""
    _dev(X, torch.float32, "X")
    _dev(W, torch.float32, "W")
    M, K = X.shape
    N = W.shape[0]
    Op = _packed_empty(M, N, X.device) if out is None else out
    _check(lib().bnn_dense_f32_sign_pack(_ptr(X), _ld(X), _ptr(W), _ld(W), M, N, K,
                                         _ptr(Op), _ld(Op), _stream(X.device)),
           "bnn_dense_f32_sign_pack")
    return Op


def dense_binact_f32(Xp: torch.Tensor, W: torch.Tensor, K: int, *, out: torch.Tensor | None = None):
    """FP last layer on packed +1/-1 activations: fp32 [M, N]."""
    _dev(Xp, torch.int32, "Xp")
    _dev(W, torch.float32, "W")
    M, N = Xp.shape[0], W.shape[0]
    Y = torch.empty((M, N), dtype=torch.float32, device=Xp.device) if out is None else out
    _check(lib().bnn_dense_binact_f32(_ptr(Xp), _ld(Xp), _ptr(W), _ld(W), M, N, int(K),
                                      _ptr(Y), _ld(Y), _stream(Xp.device)), "bnn_dense_binact_f32")
    return Y


def weight_scale_tensor(W: torch.Tensor, *, out: torch.Tensor | None = None) -> torch.Tensor:
    """One scale for the whole matrix, ||W||_1 / (N K) (fp32 [1])."""
    _dev(W, torch.float32, "W")
    N, K = W.shape
    work = torch.empty(N, dtype=torch.float64, device=W.device)
    a = torch.empty(1, dtype=torch.float32, device=W.device) if out is None else out
    _check(lib().bnn_weight_scale_tensor(_ptr(W), N, K, _ld(W), _ptr(work), _ptr(a),
                                         _stream(W.device)), "bnn_weight_scale_tensor")
    return a


def weight_scale_tensor_noalloc(W: torch.Tensor, *, out: torch.Tensor) -> torch.Tensor:
    """The scale of weight_scale_tensor through the entry point that allocates
    nothing: the caller passes the output, the library's static per-GPU
    scratch holds the row sums (N <= NOALLOC_MAX_ROWS; overlapping calls on
    one GPU race)."""
    _dev(W, torch.float32, "W")
    _dev(out, torch.float32, "out")
    N, K = W.shape
    _check(lib().bnn_weight_scale_tensor_noalloc(_ptr(W), N, K, _ld(W), _ptr(out), _stream(W.device)),
           "bnn_weight_scale_tensor_noalloc")
    return out


def i8_ld(K: int) -> int:
    """Row stride of an int8 activation matrix: K rounded up to 16 bytes."""
    return (int(K) + 15) // 16 * 16


def _planes_ld(Xb: torch.Tensor) -> int:
    if Xb.dim() != 3 or Xb.shape[1] != 8 or Xb.stride(2) != 1 or Xb.stride(0) != 8 * Xb.stride(1):
        raise ValueError("bit planes must be an int32 tensor [M, 8, ld] with row stride 8*ld")
    return Xb.stride(1)


def quantize_act_i8(X: torch.Tensor, *, want_int8: bool = True, want_planes: bool = True,
                    want_xsum: bool | None = None):
    """Absmax INT8 quantization per row of fp32 X [M, K].

    Returns a dict: ``Xq`` int8 [M, K] (row stride a multiple of 16) or None,
    ``Xb`` int32 bit planes [M, 8, ld] (or None), ``xsum`` int32 [M] row
    sums (always with planes; else when ``want_xsum``), and ``xscale`` fp32
    [M] (X ~= xscale * Xq)."""
    _dev(X, torch.float32, "X")
    M, K = X.shape
    dev = X.device
    if want_xsum is None:
        want_xsum = want_planes
    if want_planes and not want_xsum:
        raise ValueError("bit planes come with their row sums")
    Xq = torch.empty((M, i8_ld(K)), dtype=torch.int8, device=dev)[:, :K] if want_int8 else None
    Xb = torch.empty((M, 8, padded_ld(K)), dtype=torch.int32, device=dev) if want_planes else None
    xsum = torch.empty(M, dtype=torch.int32, device=dev) if want_xsum else None
    xscale = torch.empty(M, dtype=torch.float32, device=dev)
    _check(lib().bnn_quantize_act_i8(_ptr(X), M, K, _ld(X),
                                     _ptr(Xq), Xq.stride(0) if Xq is not None else 0,
                                     _ptr(Xb), _planes_ld(Xb) if Xb is not None else 0, _ptr(xsum),
                                     _ptr(xscale), _stream(dev)), "bnn_quantize_act_i8")
    return {"Xq": Xq, "Xb": Xb, "xsum": xsum, "xscale": xscale}


def pack_act_i8(Xq: torch.Tensor):
    """Bit planes [M, 8, ld] and row sums [M] of int8 activations [M, K]."""
    _dev(Xq, torch.int8, "Xq")
    M, K = Xq.shape
    Xb = torch.empty((M, 8, padded_ld(K)), dtype=torch.int32, device=Xq.device)
    xsum = torch.empty(M, dtype=torch.int32, device=Xq.device)
    _check(lib().bnn_pack_act_i8(_ptr(Xq), M, K, _ld(Xq), _ptr(Xb), _planes_ld(Xb), _ptr(xsum),
                                 _stream(Xq.device)), "bnn_pack_act_i8")
    return Xb, xsum


def bwn_i8_linear(Wp: torch.Tensor, K: int, epilogue: int, *, Xb=None, xsum=None, Xq=None,
                  xscale=None, alpha=None, D=None, Y=None, Zp=None, M: int | None = None):
    """Binary weights x INT8 activations: D = sum q * s (int32) and/or
    Y = alpha * D (* xscale) (fp32), from bit planes (GEMV, M <= 2) or int8
    rows (MFMA GEMM).  Returns a dict with ``D`` and ``Y``."""
    _dev(Wp, torch.int32, "Wp")
    if M is None:
        M = (Xb if Xb is not None else Xq).shape[0]
    N = Wp.shape[0]
    dev = Wp.device
    if epilogue & EPI_DOT_I32 and D is None:
        D = torch.empty((M, N), dtype=torch.int32, device=dev)
    if epilogue & EPI_SCALE_F32 and Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    a = _I8Args()
    if Xb is not None:
        _dev(Xb, torch.int32, "Xb")
        a.Xb, a.ldXb = Xb.data_ptr(), _planes_ld(Xb)
    if xsum is not None:
        a.xsum = xsum.data_ptr()
    if Xq is not None:
        _dev(Xq, torch.int8, "Xq")
        a.Xq, a.ldXq = Xq.data_ptr(), _ld(Xq)
    if xscale is not None:
        a.xscale = xscale.data_ptr()
    a.Wp, a.ldWp = Wp.data_ptr(), _ld(Wp)
    a.M, a.N, a.K = M, N, int(K)
    a.epilogue = int(epilogue)
    if D is not None:
        a.D, a.ldD = D.data_ptr(), _ld(D)
    if alpha is not None:
        a.alpha = alpha.data_ptr()
    if Y is not None:
        a.Y, a.ldY = Y.data_ptr(), _ld(Y)
    if Zp is not None:
        a.Zp = Zp.data_ptr()
    _check(lib().bnn_bwn_i8_linear(ctypes.byref(a), _stream(dev)), "bnn_bwn_i8_linear")
    return {"D": D, "Y": Y}


def bwn_f16_gemv(Wp: torch.Tensor, K: int, X: torch.Tensor, alpha: torch.Tensor, *,
                 alpha_tensor: bool = False, Y: torch.Tensor | None = None):
    """Binary weights x fp16 activations: Y = fl32(alpha * sum_k s x_k) with
    an fp32 sum (bnn_bwn_f16_gemv).  X float16 [M, ldX >= K] (ldX % 8 == 0),
    alpha fp32 [N] (or [1] with ``alpha_tensor``).  Returns Y fp32 [M, N]."""
    _dev(Wp, torch.int32, "Wp")
    _dev(X, torch.float16, "X")
    _dev(alpha, torch.float32, "alpha")
    M, N = X.shape[0], Wp.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=Wp.device)
    fl = EPI_SCALE_F32 | (EPI_ALPHA_TENSOR if alpha_tensor else 0)
    _check(lib().bnn_bwn_f16_gemv(X.data_ptr(), _ld(X), Wp.data_ptr(), _ld(Wp), M, N, int(K), fl,
                                  alpha.data_ptr(), Y.data_ptr(), _ld(Y), _stream(Wp.device)), "bnn_bwn_f16_gemv")
    return Y


def pack_weights_ternary(W: torch.Tensor, *, gamma: torch.Tensor | None = None, delta: float = 0.0):
    """Ternary weights as (sign plane Sp [N, ld], nonzero plane Zp [N, ld],
    nnz int32 [N]): RoundClip(W / gamma) (eq. (9)) when ``gamma`` (a device
    fp32 [1]) is given, else the threshold ``delta`` (eq. (7))."""
    _dev(W, torch.float32, "W")
    N, K = W.shape
    Sp = _packed_empty(N, K, W.device)
    Zp = _packed_empty(N, K, W.device)
    nnz = torch.empty(N, dtype=torch.int32, device=W.device)
    _check(lib().bnn_pack_weights_ternary(_ptr(W), N, K, _ld(W), _ptr(gamma), ctypes.c_float(float(delta)),
                                          _ptr(Sp), _ptr(Zp), _ld(Sp), _ptr(nnz), _stream(W.device)),
           "bnn_pack_weights_ternary")
    return Sp, Zp, nnz
