// Host-side fold of inference BatchNorm + sign into integer thresholds for the
// THRESH_PACK epilogue ("Binary Neural Network (BNN)" glossary: BatchNorm
// around the binary layers; "Extreme Quantization", eq. (4): the next layer
// takes the sign).  Host code only, no kernels.
//
// For one output channel with scale alpha (eq. (1)) and BatchNorm parameters
// (gamma, beta, mean, var, eps), the next sign of an integer dot product D is
//     +1  iff  BN(alpha D) = gamma (alpha D - mean) / sqrt(var + eps) + beta >= 0.
// BN(alpha D) is affine in D with a slope of the sign of c = gamma * alpha, so
// over the integers the rule is  D >= B  (c > 0),  D <= B'  (c < 0)  or a
// constant (c = 0).  The fold finds the integer boundary and stores it as an
// integer-valued float, so the kernel's single-precision test
// (float)(dir * D) >= tau is exact for every |D| <= 2^24.
//
// The boundary is first estimated in double, tau ~ (gamma mean - beta sd) / c,
// then certified (and moved if the estimate was off) by evaluating the sign of
// BN at integer points exactly: every fp32 input is a dyadic rational
// m * 2^e, so sqrt(var + eps) * BN(alpha D) = u + beta sqrt(var + eps) with
// u = gamma (alpha D - mean) is decided with big-integer arithmetic (u and
// beta read off when their signs agree, else u^2 against beta^2 (var + eps)).
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "bnn.h"

namespace {

// A dyadic rational (-1)^neg * mag * 2^exp; mag is little-endian 32-bit limbs.
struct Dyadic {
    std::vector<uint32_t> mag;
    int exp = 0;
    bool neg = false;
    bool zero() const { return mag.empty(); }
};

void trim(std::vector<uint32_t>& m) {
    while (!m.empty() && m.back() == 0u) m.pop_back();
}

Dyadic from_u64(uint64_t v, int exp, bool neg) {
    Dyadic d;
    d.mag = {static_cast<uint32_t>(v), static_cast<uint32_t>(v >> 32)};
    trim(d.mag);
    d.exp = exp;
    d.neg = neg && !d.mag.empty();
    return d;
}

// Exact value of a finite float: |f| = mant * 2^(e - 24) with mant < 2^24.
Dyadic from_float(float f) {
    if (f == 0.0f) return Dyadic{};
    int e = 0;
    const float m = frexpf(fabsf(f), &e);               // m in [0.5, 1)
    const uint64_t mant = static_cast<uint64_t>(ldexpf(m, 24));
    return from_u64(mant, e - 24, f < 0.0f);
}

Dyadic from_i64(int64_t v) {
    const uint64_t a = v < 0 ? static_cast<uint64_t>(-(v + 1)) + 1u : static_cast<uint64_t>(v);
    return from_u64(a, 0, v < 0);
}

std::vector<uint32_t> shifted(const std::vector<uint32_t>& m, int bits) {
    if (m.empty()) return m;
    const int limbs = bits / 32, rem = bits % 32;
    std::vector<uint32_t> r(m.size() + limbs + 1, 0u);
    for (size_t i = 0; i < m.size(); ++i) {
        const uint64_t v = static_cast<uint64_t>(m[i]) << rem;
        r[i + limbs] |= static_cast<uint32_t>(v);
        r[i + limbs + 1] |= static_cast<uint32_t>(v >> 32);
    }
    trim(r);
    return r;
}

int cmp_mag(const std::vector<uint32_t>& a, const std::vector<uint32_t>& b) {
    if (a.size() != b.size()) return a.size() < b.size() ? -1 : 1;
    for (size_t i = a.size(); i-- > 0;)
        if (a[i] != b[i]) return a[i] < b[i] ? -1 : 1;
    return 0;
}

std::vector<uint32_t> add_mag(const std::vector<uint32_t>& a, const std::vector<uint32_t>& b) {
    std::vector<uint32_t> r(std::max(a.size(), b.size()) + 1, 0u);
    uint64_t carry = 0;
    for (size_t i = 0; i < r.size(); ++i) {
        const uint64_t s = carry + (i < a.size() ? a[i] : 0u) + (i < b.size() ? b[i] : 0u);
        r[i] = static_cast<uint32_t>(s);
        carry = s >> 32;
    }
    trim(r);
    return r;
}

// a - b for a >= b.
std::vector<uint32_t> sub_mag(const std::vector<uint32_t>& a, const std::vector<uint32_t>& b) {
    std::vector<uint32_t> r(a.size(), 0u);
    int64_t borrow = 0;
    for (size_t i = 0; i < a.size(); ++i) {
        int64_t s = static_cast<int64_t>(a[i]) - borrow - (i < b.size() ? static_cast<int64_t>(b[i]) : 0);
        borrow = s < 0 ? 1 : 0;
        r[i] = static_cast<uint32_t>(s + (borrow << 32));
    }
    trim(r);
    return r;
}

Dyadic mul(const Dyadic& a, const Dyadic& b) {
    Dyadic r;
    if (a.zero() || b.zero()) return r;
    std::vector<uint64_t> acc(a.mag.size() + b.mag.size() + 1, 0u);
    for (size_t i = 0; i < a.mag.size(); ++i) {
        uint64_t carry = 0;
        for (size_t j = 0; j < b.mag.size(); ++j) {
            const uint64_t t = static_cast<uint64_t>(a.mag[i]) * b.mag[j] + acc[i + j] + carry;
            acc[i + j] = t & 0xFFFFFFFFu;
            carry = t >> 32;
        }
        acc[i + b.mag.size()] += carry;
    }
    r.mag.assign(acc.size(), 0u);
    for (size_t i = 0; i < acc.size(); ++i) r.mag[i] = static_cast<uint32_t>(acc[i]);
    trim(r.mag);
    r.exp = a.exp + b.exp;
    r.neg = a.neg != b.neg;
    return r;
}

Dyadic add(const Dyadic& a, const Dyadic& b) {
    if (a.zero()) return b;
    if (b.zero()) return a;
    const int e = std::min(a.exp, b.exp);
    const std::vector<uint32_t> A = shifted(a.mag, a.exp - e), B = shifted(b.mag, b.exp - e);
    Dyadic r;
    r.exp = e;
    if (a.neg == b.neg) {
        r.mag = add_mag(A, B);
        r.neg = a.neg;
    } else {
        const int c = cmp_mag(A, B);
        if (c == 0) return Dyadic{};
        r.mag = c > 0 ? sub_mag(A, B) : sub_mag(B, A);
        r.neg = c > 0 ? a.neg : b.neg;
    }
    return r;
}

Dyadic negated(Dyadic a) {
    a.neg = !a.neg && !a.zero();
    return a;
}

// Compares two non-negative dyadics.
int cmp_nonneg(const Dyadic& a, const Dyadic& b) {
    if (a.zero() || b.zero()) return a.zero() ? (b.zero() ? 0 : -1) : 1;
    const int e = std::min(a.exp, b.exp);
    return cmp_mag(shifted(a.mag, a.exp - e), shifted(b.mag, b.exp - e));
}

int sign_of(const Dyadic& a) { return a.zero() ? 0 : (a.neg ? -1 : 1); }

struct Channel {
    Dyadic alpha, gamma, beta, neg_mean, beta2_s;   // beta2_s = beta^2 (var + eps)

    // BN(alpha * D) >= 0, decided exactly.
    bool bn_nonneg(int64_t D) const {
        const Dyadic u = mul(gamma, add(mul(alpha, from_i64(D)), neg_mean));
        const int su = sign_of(u), sb = sign_of(beta);
        if (su >= 0 && sb >= 0) return true;
        if (su <= 0 && sb <= 0) return false;
        const int c = cmp_nonneg(mul(u, u), beta2_s);      // u^2 vs beta^2 (var + eps)
        return su > 0 ? c >= 0 : c <= 0;
    }
};

constexpr int64_t kLo = -(int64_t(1) << 24);       // the smallest D the library produces
constexpr int64_t kHi = (int64_t(1) << 24) + 1;    // one past the largest: "never"

// Smallest t in [kLo, kHi] with pred(t) true, pred monotone (false ... true)
// and pred(kHi) taken as true; the search starts from the estimate t0.
template <class Pred>
int64_t first_true(const Pred& pred, int64_t t0) {
    auto p = [&](int64_t t) { return t >= kHi || pred(t); };
    t0 = std::min(std::max(t0, kLo), kHi);
    int64_t lo, hi;                // invariant: p(lo) false (or lo = kLo - 1), p(hi) true
    if (p(t0)) {
        hi = t0;
        int64_t step = 1;
        lo = t0 - step;
        while (lo >= kLo && p(lo)) {
            hi = lo;
            step *= 2;
            lo = hi - step;
        }
        lo = std::max(lo, kLo - 1);
    } else {
        lo = t0;
        int64_t step = 1;
        hi = std::min(t0 + step, kHi);
        while (!p(hi)) {
            lo = hi;
            step *= 2;
            hi = std::min(lo + step, kHi);
        }
    }
    while (hi - lo > 1) {
        const int64_t mid = lo + (hi - lo) / 2;
        if (p(mid)) hi = mid; else lo = mid;
    }
    return hi;
}

// Estimate of the first D with BN(alpha D) >= 0 (c > 0), or of the first
// -D with it (c < 0): the real boundary in double, rounded up.
int64_t estimate(double rhs_over_c) {
    if (!(rhs_over_c == rhs_over_c)) return 0;
    if (rhs_over_c >= static_cast<double>(kHi)) return kHi;
    if (rhs_over_c <= static_cast<double>(kLo)) return kLo;
    return static_cast<int64_t>(ceil(rhs_over_c));
}

bool finite_f(float v) { return isfinite(v) != 0; }

}  // namespace

extern "C" __attribute__((visibility("default")))
bnn_status bnn_fold_bn_thresholds_host(const float* gamma, const float* beta,
                                       const float* mean, const float* var, float eps,
                                       const float* alpha, int64_t N, float* tau, int8_t* dir)
{
    if (N < 0) return BNN_ERR_SHAPE;
    if (!gamma || !beta || !mean || !var || !alpha || !tau || !dir) return BNN_ERR_NULL;
    if (!finite_f(eps)) return BNN_ERR_UNSUPPORTED;
    for (int64_t n = 0; n < N; ++n) {
        if (!finite_f(gamma[n]) || !finite_f(beta[n]) || !finite_f(mean[n]) || !finite_f(var[n]) ||
            !finite_f(alpha[n]))
            return BNN_ERR_UNSUPPORTED;
        // var + eps of two floats: its double sum has the sign of the exact sum
        if (!((double)var[n] + (double)eps > 0.0)) return BNN_ERR_UNSUPPORTED;
    }
    const Dyadic e = from_float(eps);
    for (int64_t n = 0; n < N; ++n) {
        Channel ch;
        ch.alpha = from_float(alpha[n]);
        ch.gamma = from_float(gamma[n]);
        ch.beta = from_float(beta[n]);
        ch.neg_mean = negated(from_float(mean[n]));
        ch.beta2_s = mul(mul(ch.beta, ch.beta), add(from_float(var[n]), e));
        const int cs = sign_of(ch.gamma) * sign_of(ch.alpha);
        if (cs == 0) {                       // BN does not depend on D
            dir[n] = 0;
            tau[n] = ch.bn_nonneg(0) ? 0.0f : 1.0f;
            continue;
        }
        const double sd = sqrt((double)var[n] + (double)eps);
        const double c = (double)gamma[n] * (double)alpha[n];
        const double est = ((double)gamma[n] * (double)mean[n] - (double)beta[n] * sd) / c;
        int64_t t;
        if (cs > 0) {                        // +1 iff D >= t
            t = first_true([&](int64_t d) { return ch.bn_nonneg(d); }, estimate(est));
            dir[n] = 1;
        } else {                             // +1 iff D <= -t, i.e. -D >= t
            t = first_true([&](int64_t d) { return ch.bn_nonneg(-d); }, estimate(-est));
            dir[n] = -1;
        }
        // t in [-2^24, 2^24 + 1]; 2^24 + 1 (never) is stored as 2^25, which
        // no |D| <= 2^24 reaches; every other value is exact in fp32.
        tau[n] = t >= kHi ? 33554432.0f : static_cast<float>(t);
    }
    return BNN_OK;
}
