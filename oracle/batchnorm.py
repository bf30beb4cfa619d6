"""Inference BatchNorm followed by the sign, decided from its definition.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline may use this module; the product package never does.  It shares no
code with the HIP library (whose host helper folds BatchNorm into integer
thresholds by its own method).

Sources (page title, section / equation):
  * "Binary Neural Network (BNN)" glossary: BatchNorm sits around the
    binarized layers.
  * "Extreme Quantization: Binary, Ternary & 1-bit LLMs", eq. (4): the next
    binary layer takes the sign of its input; "Notation": sign(x) = +1 for
    x >= 0, -1 otherwise.

What is decided, for an output D[m, n] of a binary layer with per-row scale
alpha_n (eq. (1)), is the plain definition of inference BatchNorm then sign:

    BN(z) = gamma_n * (z - mean_n) / sqrt(var_n + eps) + beta_n,   z = alpha_n * D
    next sign = +1  iff  BN(z) >= 0,

in exact real arithmetic on the given fp32 values of alpha, gamma, beta,
mean, var and eps (the pages fix no precision for it; var + eps is the exact
sum, not a rounded one).  It is decided with rationals (``fractions``):
multiplying BN(z) by sqrt(var + eps) > 0 keeps its sign, so the question is
the sign of  u + beta * r  with  u = gamma (alpha D - mean)  rational and
r = sqrt(var + eps) > 0.  When u and beta do not have opposite signs the
answer is read off; otherwise |u| and |beta| r are compared through their
squares u^2 and beta^2 (var + eps), both rational.

BN(alpha * D) is an affine function of D whose slope has the sign of
gamma * alpha, so along one output column the decision is monotone in D.
The column's decisions are therefore fixed by one boundary value, found by
bisection over the column's distinct D values with the exact test above at
each probe; every output's decision is the exact one.
"""
from __future__ import annotations

from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np

__all__ = ["bn_next_sign", "bn_rule", "bn_value", "rule_signs"]


def _exact(x, what: str) -> Fraction:
    v = float(np.float32(x))
    if not np.isfinite(v):
        raise ValueError(f"BatchNorm {what} must be finite, got {v}")
    return Fraction(v)


class _Channel:
    """One output channel's alpha and BatchNorm parameters as exact rationals."""

    def __init__(self, alpha, gamma, beta, mean, var, eps):
        self.a = _exact(alpha, "alpha")
        self.g = _exact(gamma, "gamma")
        self.b = _exact(beta, "beta")
        self.mu = _exact(mean, "mean")
        self.s = _exact(var, "var") + _exact(eps, "eps")
        if self.s <= 0:
            raise ValueError("BatchNorm needs var + eps > 0")
        self.slope_sign = (self.g * self.a > 0) - (self.g * self.a < 0)

    def nonneg(self, D: int) -> bool:
        """BN(alpha * D) >= 0, exactly (see the module docstring)."""
        u = self.g * (self.a * int(D) - self.mu)
        b = self.b
        if u >= 0 and b >= 0:
            return True
        if u <= 0 and b <= 0:          # not both zero here, so the sum is < 0
            return False
        if u > 0:                      # b < 0:  u >= |b| r  iff  u^2 >= b^2 s
            return u * u >= b * b * self.s
        return b * b * self.s >= u * u  # u < 0 < b:  b r >= |u|

    def value(self, D: int, digits: int = 60) -> float:
        """BN(alpha * D) to ``digits`` significant digits (for reporting how
        far a decision is from its tie; the decision itself uses nonneg)."""
        with localcontext() as ctx:
            ctx.prec = digits
            u = self.g * (self.a * int(D) - self.mu)
            num = Decimal(u.numerator) / Decimal(u.denominator)
            s = Decimal(self.s.numerator) / Decimal(self.s.denominator)
            b = Decimal(self.b.numerator) / Decimal(self.b.denominator)
            return float(num / s.sqrt() + b)


def _first_true(pred, values):
    """Index of the first element of ``values`` for which the monotone
    (False ... False True ... True) predicate holds; len(values) if none."""
    lo, hi = 0, len(values)
    while lo < hi:
        mid = (lo + hi) // 2
        if pred(values[mid]):
            hi = mid
        else:
            lo = mid + 1
    return lo


def _params(alpha, gamma, beta, mean, var, eps):
    a = np.atleast_1d(np.asarray(alpha, np.float32))
    N = a.shape[0]
    g, b, mu, v = (np.broadcast_to(np.asarray(x, np.float32), (N,)) for x in (gamma, beta, mean, var))
    return N, [(a[n], g[n], b[n], mu[n], v[n], eps) for n in range(N)]


def bn_next_sign(D, alpha, gamma, beta, mean, var, eps):
    """Next-layer signs after inference BatchNorm of alpha * D.

    D int [M, N]; alpha, gamma, beta, mean, var fp32 [N]; eps a scalar.
    Returns (s, margin): s int8 [M, N] with s = +1 iff BN(alpha_n D[m, n]) >= 0,
    decided exactly; margin float64 [N], the smallest |BN(alpha_n D)| over the
    column's outputs (0.0 marks an exact tie, decided +1)."""
    D = np.asarray(D)
    M, N = D.shape
    n_par, par = _params(alpha, gamma, beta, mean, var, eps)
    assert n_par == N
    s = np.empty((M, N), dtype=np.int8)
    margin = np.full(N, np.inf)
    for n in range(N):
        ch = _Channel(*par[n])
        col = D[:, n].astype(np.int64)
        vals = [int(v) for v in np.unique(col)]          # ascending
        if not vals:
            continue
        if ch.slope_sign == 0:
            plus = ch.nonneg(0)
            s[:, n] = 1 if plus else -1
            margin[n] = abs(ch.value(0))
            continue
        if ch.slope_sign > 0:       # decisions False ... True along ascending D
            i = _first_true(ch.nonneg, vals)
            s[:, n] = np.where(col >= (vals[i] if i < len(vals) else vals[-1] + 1), 1, -1)
        else:                       # True ... False along ascending D
            i = _first_true(lambda d: not ch.nonneg(d), vals)
            s[:, n] = np.where(col < (vals[i] if i < len(vals) else vals[-1] + 1), 1, -1)
        near = [vals[j] for j in (i - 1, i) if 0 <= j < len(vals)]
        margin[n] = min(abs(ch.value(d)) for d in near)
    return s, margin


def bn_rule(alpha, gamma, beta, mean, var, eps, K: int):
    """The exact decision rule of each channel over every integer |D| <= K.

    Returns (kind int8 [N], bound int64 [N]):
      kind +1: the sign is +1 iff D >= bound   (bound = K + 1: never)
      kind -1: the sign is +1 iff D <= bound   (bound = -K - 1: never)
      kind  0: the sign does not depend on D; bound is +1 or -1, that sign.
    Each bound is found by bisection over the integers in [-K, K] with the
    exact test (the decision is monotone in D, as above)."""
    N, par = _params(alpha, gamma, beta, mean, var, eps)
    kind = np.zeros(N, dtype=np.int8)
    bound = np.zeros(N, dtype=np.int64)
    ints = range(-K, K + 1)
    for n in range(N):
        ch = _Channel(*par[n])
        if ch.slope_sign == 0:
            kind[n], bound[n] = 0, (1 if ch.nonneg(0) else -1)
        elif ch.slope_sign > 0:
            kind[n], bound[n] = 1, -K + _first_true(ch.nonneg, ints)
        else:
            kind[n], bound[n] = -1, -K + _first_true(lambda d: not ch.nonneg(d), ints) - 1
    return kind, bound


def bn_value(D: int, alpha, gamma, beta, mean, var, eps, digits: int = 60) -> float:
    """BN(alpha * D) of one channel, to ``digits`` significant digits."""
    return _Channel(alpha, gamma, beta, mean, var, eps).value(D, digits)


def rule_signs(kind, bound, D):
    """Apply bn_rule's (kind, bound) to D int [M, N]: int8 signs [M, N]."""
    D = np.asarray(D, dtype=np.int64)
    kind = np.asarray(kind)[None, :]
    bound = np.asarray(bound)[None, :]
    plus = np.where(kind > 0, D >= bound, np.where(kind < 0, D <= bound, bound > 0))
    return np.where(plus, 1, -1).astype(np.int8)

