"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of ``oracle/oracle.c`` (a
wrong comparison, a dropped term, a transposed index, a wrong divisor, a
missing rounding, a flipped sign, ...), builds it with gcc into a temporary
library, points the oracle at it, and runs the pin suite of
``test_oracle_pins.py``: at least one pin must fail.  A mutant that every pin
accepts would mean the pins do not constrain that part of the oracle.
"""
from __future__ import annotations

import importlib.util
import os
import tempfile

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.c")
BN_SRC = os.path.join(os.path.dirname(SRC), "batchnorm.py")

MUTATIONS = [
    ("sign: zero maps to -1",
     "(x[r * ldx + c] >= 0.0f)", "(x[r * ldx + c] > 0.0f)"),
    ("pack: bit 1 encodes +1",
     "if (s[r * K + k] == -1)", "if (s[r * K + k] == 1)"),
    ("pack: most significant bit first",
     "words[r * ld + k / 32] |= (uint32_t)1u << (k % 32);",
     "words[r * ld + k / 32] |= (uint32_t)1u << (31 - k % 32);"),
    ("planes: most significant bit first",
     "words[(m * 8 + b) * ld + k / 32] |= (uint32_t)1u << (k % 32);",
     "words[(m * 8 + b) * ld + k / 32] |= (uint32_t)1u << (31 - k % 32);"),
    ("pack: pad words left as ones",
     "for (int64_t w = 0; w < ld; ++w) words[r * ld + w] = 0u;",
     "for (int64_t w = 0; w < ld; ++w) words[r * ld + w] = (w * 32 >= K) ? ~0u : 0u;"),
    ("dot: last term dropped",
     "for (int64_t k = 0; k < K; ++k)\n                acc += (int32_t)xs",
     "for (int64_t k = 0; k + 1 < K; ++k)\n                acc += (int32_t)xs"),
    ("dot: operands paired in reverse order",
     "(int32_t)ws[n * K + k];", "(int32_t)ws[n * K + (K - 1 - k)];"),
    ("alpha: divided by K + 1",
     "alpha[n] = (float)(sum / (double)K);", "alpha[n] = (float)(sum / (double)(K + 1));"),
    ("alpha: summed in single precision",
     "double sum = 0.0;\n        for (int64_t k = 0; k < K; ++k) sum += fabs((double)W[n * ldw + k]);",
     "float sum = 0.0f;\n        for (int64_t k = 0; k < K; ++k) sum += fabsf(W[n * ldw + k]);"),
    ("alpha: signed mean",
     "sum += fabs((double)W[n * ldw + k]);", "sum += (double)W[n * ldw + k];"),
    ("scale: alpha indexed by row",
     "Y[m * N + n] = alpha[n] * (float)D[m * N + n];", "Y[m * N + n] = alpha[m % N] * (float)D[m * N + n];"),
    ("residual: fused multiply-add",
     "float z = alpha[n] * (float)D[m * N + n];\n            Y[m * N + n] = z + R[m * ldr + n];",
     "Y[m * N + n] = fmaf(alpha[n], (float)D[m * N + n], R[m * ldr + n]);"),
    ("im2col: pad pixels encode -1",
     "int8_t v = 1;\n                    if (inside)", "int8_t v = -1;\n                    if (inside)"),
    ("im2col: tap order transposed",
     "cols[p * K + (kh * 3 + kw) * C + c] = v;", "cols[p * K + (kw * 3 + kh) * C + c] = v;"),
    ("im2col: window not centred",
     "int64_t ih = oh - 1 + kh, iw = ow - 1 + kw;\n                int inside = (ih",
     "int64_t ih = oh + kh, iw = ow - 1 + kw;\n                int inside = (ih"),
    ("RSign im2col: window not centred",
     "int64_t ih = oh - 1 + kh, iw = ow - 1 + kw;\n                int inside = ih",
     "int64_t ih = oh - 1 + kh, iw = ow + kw;\n                int inside = ih"),
    ("first FP layer: single-precision accumulation",
     "acc += (double)X[m * ldx + k] * (double)W[n * ldw + k];", "acc += (double)(X[m * ldx + k] * W[n * ldw + k]);"),
    ("last FP layer: activation signs ignored",
     "acc += (double)s[m * K + k] * (double)W[n * ldw + k];", "acc += (double)W[n * ldw + k];"),
    ("last FP layer: no final rounding to single",
     "Y[m * N + n] = (float)acc;", "Y[m * N + n] = (float)(acc * (1.0 + 1e-6));"),
    ("int8 dot: activations read as unsigned",
     "acc += (int64_t)xq[m * K + k] * (int64_t)ws[n * K + k];",
     "acc += (int64_t)(uint8_t)xq[m * K + k] * (int64_t)ws[n * K + k];"),
    ("int8 dot: weight sign ignored",
     "acc += (int64_t)xq[m * K + k] * (int64_t)ws[n * K + k];",
     "acc += (int64_t)xq[m * K + k];"),
    ("quantize: 128 levels instead of 127",
     "float inv = (amax > 0.0f) ? 127.0f / amax : 0.0f;",
     "float inv = (amax > 0.0f) ? 128.0f / amax : 0.0f;"),
    ("quantize: truncation instead of rounding",
     "float r = rintf(v);", "float r = truncf(v);"),
    ("quantize: ties rounded away from zero",
     "float r = rintf(v);", "float r = roundf(v);"),
    ("quantize: scale inverted",
     "scale[m] = amax / 127.0f;", "scale[m] = 127.0f / amax;"),
    ("quantize: NaN taken as the maximum",
     "if (a > amax) amax = a;", "if (!(a <= amax)) amax = a;"),
    ("planes: sign plane dropped",
     "for (int64_t b = 0; b < 8; ++b)\n                if", "for (int64_t b = 0; b < 7; ++b)\n                if"),
    ("planes: sum of magnitudes",
     "total += Q[m * K + k];", "total += Q[m * K + k] < 0 ? -Q[m * K + k] : Q[m * K + k];"),
    ("per-tensor alpha: divided by K only",
     "return (float)(total / ((double)N * (double)K));", "return (float)(total / (double)K);"),
    ("per-tensor alpha: signed sum",
     "total += fabs((double)W[n * ldw + k]);", "total += (double)W[n * ldw + k];"),
    ("int8 dequant: activation scale ignored",
     "Y[m * N + n] = z * xscale[m];", "Y[m * N + n] = z;"),
    ("bias: added before the alpha scale",
     "float zb = z + bias[n];", "float zb = alpha[n * alpha_stride] * ((float)D[m * N + n] + bias[n]);"),
    ("bias: indexed by activation row",
     "float zb = z + bias[n];", "float zb = z + bias[m % N];"),
    ("ternary threshold: ties at Delta kept nonzero",
     "T[n * K + k] = (int8_t)((w > delta) - (w < -delta));",
     "T[n * K + k] = (int8_t)((w >= delta) - (w <= -delta));"),
    ("ternary RoundClip: truncation",
     "float r = rintf(W[n * ldw + k] / gamma);", "float r = truncf(W[n * ldw + k] / gamma);"),
    ("ternary RoundClip: ties away from zero",
     "float r = rintf(W[n * ldw + k] / gamma);", "float r = roundf(W[n * ldw + k] / gamma);"),
    ("ternary RoundClip: scaled by gamma instead of divided",
     "float r = rintf(W[n * ldw + k] / gamma);", "float r = rintf(W[n * ldw + k] * gamma);"),
    ("ternary pack: sign bit set for +1",
     "if (t == -1) S[n * ld + k / 32]", "if (t == 1) S[n * ld + k / 32]"),
    ("RSign: strict comparison at the tie",
     "s[r * cols + c] = (x[r * ldx + c] >= beta[c])", "s[r * cols + c] = (x[r * ldx + c] > beta[c])"),
    ("RSign: shift ignored",
     "s[r * cols + c] = (x[r * ldx + c] >= beta[c])", "s[r * cols + c] = (x[r * ldx + c] >= 0.0f)"),
    ("RSign im2col: pad taps -1",
     "inside ? S[((b * H + ih) * W + iw) * C + c] : (int8_t)1;",
     "inside ? S[((b * H + ih) * W + iw) * C + c] : (int8_t)-1;"),
    ("half: exponent bias off by one",
     "else u = (1024 + f) << (e - 1);", "else u = (1024 + f) << e;"),
    ("half: sign bit ignored",
     "return (h & 0x8000) ? -u : u;", "return u;"),
    ("half: subnormals given the implicit leading one",
     "if (e == 0) u = f;", "if (e == 0) u = 1024 + f;"),
    ("fp16 activations: last term dropped",
     "for (int64_t k = 0; k < K; ++k)\n                acc += (int64_t)ws[n * K + k] * half_units",
     "for (int64_t k = 0; k + 1 < K; ++k)\n                acc += (int64_t)ws[n * K + k] * half_units"),
    ("fp16 activations: weight sign ignored",
     "acc += (int64_t)ws[n * K + k] * half_units(x[m * ldx + k], &dummy);",
     "acc += half_units(x[m * ldx + k], &dummy);"),
    ("ternary pack: zeros counted as nonzero",
     "if (t != 0) {\n                Z[n * ld + k / 32]", "if (t != 2) {\n                Z[n * ld + k / 32]"),
]


# Mistakes planted in the exact BatchNorm + sign module (oracle/batchnorm.py).
BN_MUTATIONS = [
    ("bn: strict comparison at the tie",
     "return u * u >= b * b * self.s", "return u * u > b * b * self.s"),
    ("bn: zero sum with zero beta read as negative",
     "if u >= 0 and b >= 0:", "if u > 0 and b >= 0:"),
    ("bn: eps ignored",
     'self.s = _exact(var, "var") + _exact(eps, "eps")', 'self.s = _exact(var, "var")'),
    ("bn: sign of beta flipped",
     "        b = self.b\n        if u >= 0", "        b = -self.b\n        if u >= 0"),
    ("bn: mean added instead of subtracted",
     "u = self.g * (self.a * int(D) - self.mu)\n        b = self.b",
     "u = self.g * (self.a * int(D) + self.mu)\n        b = self.b"),
    ("bn: negative slope treated as positive",
     "if ch.slope_sign > 0:       # decisions False", "if ch.slope_sign != 0:      # decisions False"),
    ("bn rule: boundary of a negative slope off by one",
     "-K + _first_true(lambda d: not ch.nonneg(d), ints) - 1", "-K + _first_true(lambda d: not ch.nonneg(d), ints)"),
    ("bn: margin from one side of the boundary only",
     "for j in (i - 1, i) if", "for j in (i,) if"),
]
_BN_NAMES = ("bn_next_sign", "bn_rule", "bn_value", "rule_signs")


def _pin_calls():
    """The pin suite; parametrized pins run with their own parameter lists
    (the random-K identity with a representative subset).  The full-size pins
    (test_full_*) are left out of the sweep for time; smaller pins cover the
    same code."""
    calls = []
    for name in sorted(dir(pins)):
        fn = getattr(pins, name)
        if not (name.startswith("test_") and callable(fn)) or name.startswith("test_full_"):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            calls.append((name, fn))
            continue
        argnames, values = marks[0].args[0], marks[0].args[1]
        if name == "test_identity_random_K":
            values = [1, 5, 31, 32, 33, 64, 100, 1000]
        keys = [a.strip() for a in argnames.split(",")]
        for v in values:
            args = v if len(keys) > 1 else (v,)
            calls.append((f"{name}{list(args)}", lambda fn=fn, args=args: fn(*args)))
    return calls


@pytest.fixture(scope="module")
def workdir():
    with tempfile.TemporaryDirectory(prefix="oracle_mut_") as d:
        yield d


def test_pins_pass_on_the_real_oracle():
    oracle.use_library(None)
    for name, call in _pin_calls():
        call()


@pytest.mark.parametrize("label,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_each_planted_mistake_fails_a_pin(workdir, label, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique or missing: {label}"
    mutated = src.replace(old, new)
    tag = "".join(ch if ch.isalnum() else "_" for ch in label)
    csrc = os.path.join(workdir, f"{tag}.c")
    lib = os.path.join(workdir, f"{tag}.so")
    with open(csrc, "w") as f:
        f.write(mutated)
    oracle.build(src=csrc, out=lib)
    failed = []
    try:
        oracle.use_library(lib)
        for name, call in _pin_calls():
            try:
                call()
            except Exception:        # AssertionError, or a numpy comparison error
                failed.append(name)
    finally:
        oracle.use_library(None)
    assert failed, f"no pin caught the planted mistake: {label}"


@pytest.mark.parametrize("label,old,new", BN_MUTATIONS, ids=[m[0] for m in BN_MUTATIONS])
def test_each_planted_batchnorm_mistake_fails_a_pin(workdir, label, old, new):
    src = open(BN_SRC).read()
    assert src.count(old) == 1, f"mutation site not unique or missing: {label}"
    tag = "".join(ch if ch.isalnum() else "_" for ch in label)
    path = os.path.join(workdir, f"{tag}.py")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"bn_mutant_{tag}", path)
    mutant = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mutant)
    saved = {n: getattr(oracle, n) for n in _BN_NAMES}
    failed = []
    try:
        for n in _BN_NAMES:
            setattr(oracle, n, getattr(mutant, n))
        for name, call in _pin_calls():
            try:
                call()
            except Exception:
                failed.append(name)
    finally:
        for n, v in saved.items():
            setattr(oracle, n, v)
    assert failed, f"no pin caught the planted mistake: {label}"
