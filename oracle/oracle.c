/*
 * CPU oracle for the binary (XNOR-popcount) inference path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no source, header, table or helper with the HIP
 * library; the two meet only through the seeded inputs.
 *
 * Every routine is the plain definition written out: signs are stored
 * unpacked as int8 (+1 / -1) and a binary dot product is an integer
 * multiply-add over them.  Floating point uses IEEE single/double arithmetic
 * as written in C (built without fast-math and without FMA contraction).
 * Loops over independent outputs run under OpenMP; no loop is blocked, fused
 * or reordered.
 *
 * Sources (page title, section / equation):
 *  [P2] "First Principles: Why Binary Ops Can Be Exponentially Faster",
 *       section "1. Arithmetic: MAC -> XNOR + popcount" (encoding bit0 -> +1,
 *       bit1 -> -1; dot identity; pad bits encode +1; 64 bits per word).
 *  [P5] "Extreme Quantization: Binary, Ternary & 1-bit LLMs": "Notation"
 *       (sign(x) = +1 for x >= 0, -1 for x < 0), "Binary Neural Networks"
 *       eq. (1) (alpha = mean |w|, y = alpha * w_b^T x), "XNOR-Net" eq. (4)-(6).
 *  [P1] "Binary Neural Network (BNN)" glossary: per-filter scaling factors and
 *       BatchNorm around the binarized layers.
 *  [P3] "Perfected Concept", table "What is binary vs not": first/last layers
 *       and BatchNorm scales stay in higher precision; residual streams stay FP.
 *  [P4] "State of the Art Survey", Bi-Real Net row: FP residual shortcut.
 *  [P5] "BitNet: 1-bit Transformer": activations kept at INT8 next to binary
 *       weights; eq. (8) (one mean-|W| scale for the whole matrix).
 *  [P5] "Ternary Quantization" eq. (7) (threshold Delta) and "BitNet b1.58"
 *       eq. (9) (RoundClip(W / gamma, -1, 1), gamma = ||W||_1 / (nm)).
 *  [P4] "State of the Art Survey", ReActNet row: RSign (a learnable shift of
 *       the activation distribution before the sign).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stddef.h>

#define API __attribute__((visibility("default")))

/* [P5] Notation: sign(x) = +1 if x >= 0, else -1.  The comparison is the IEEE
 * one: -0.0 >= 0 holds (+1); NaN compares false (-1); denormals compare by
 * value.  Output s is dense [rows, cols]. */
API void oracle_sign(const float* x, int64_t rows, int64_t cols, int64_t ldx, int8_t* s)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            s[r * cols + c] = (x[r * ldx + c] >= 0.0f) ? (int8_t)1 : (int8_t)-1;
}

/* [P2] encoding: a sign of +1 is bit value 0, a sign of -1 is bit value 1.
 * Element k of a row sits in word k / 32 at bit k % 32 (least significant
 * bit first).  Bits at positions k >= K and words from ceil(K/32) up to ld-1
 * are written as 0, i.e. they encode +1 as [P2] requires of pad bits. */
API void oracle_pack_signs(const int8_t* s, int64_t rows, int64_t K, uint32_t* words, int64_t ld)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t w = 0; w < ld; ++w) words[r * ld + w] = 0u;
        for (int64_t k = 0; k < K; ++k) {
            if (s[r * K + k] == -1)
                words[r * ld + k / 32] |= (uint32_t)1u << (k % 32);
        }
    }
}

/* Inverse of oracle_pack_signs over the first K positions. */
API void oracle_unpack_signs(const uint32_t* words, int64_t rows, int64_t K, int64_t ld, int8_t* s)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k)
            s[r * K + k] = ((words[r * ld + k / 32] >> (k % 32)) & 1u) ? (int8_t)-1 : (int8_t)1;
}

/* [P5] eq. (1): alpha = (1/n) * sum_i |w_i|, one value per output row (per
 * filter, [P1]).  n is the real row length K.  The sum runs in double in
 * index order, is divided by K in double and rounded once to float. */
API void oracle_alpha(const float* W, int64_t N, int64_t K, int64_t ldw, float* alpha)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double sum = 0.0;
        for (int64_t k = 0; k < K; ++k) sum += fabs((double)W[n * ldw + k]);
        alpha[n] = (float)(sum / (double)K);
    }
}

/* [P5] eq. (4)-(6): the binary dot product w_b^T x_b, computed here as the
 * plain integer multiply-add of the +1/-1 values.  xs is [M, K], ws is
 * [N, K] (both dense), D is [M, N]. */
API void oracle_dot(const int8_t* xs, const int8_t* ws, int64_t M, int64_t N, int64_t K, int32_t* D)
{
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int32_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int32_t)xs[m * K + k] * (int32_t)ws[n * K + k];
            D[m * N + n] = acc;
        }
    }
}

/* [P2] section "1. Arithmetic" and [P5] eq. (6): the same dot products
 * through the packed identity, D = K - 2 * sum_w popcount(x_w xor w_w) over
 * the Kw = ceil(K/32) words of each packed row (pad bits equal on both
 * operands contribute nothing).  Not used for any expected value: it is
 * timed next to oracle_dot as context for the CPU baseline, and pinned to
 * oracle_dot by the tests.  xw is [M, ldx] words, ww is [N, ldw] words. */
__attribute__((target("popcnt")))
API void oracle_dot_packed(const uint32_t* xw, int64_t ldx, const uint32_t* ww, int64_t ldw,
                           int64_t M, int64_t N, int64_t K, int32_t* D)
{
    const int64_t Kw = (K + 31) / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t ones = 0;
            for (int64_t w = 0; w < Kw; ++w)
                ones += __builtin_popcount(xw[m * ldx + w] ^ ww[n * ldw + w]);
            D[m * N + n] = (int32_t)(K - 2 * ones);
        }
}

/* [P5] eq. (1): y = alpha * (w_b^T x_b), one rounded single multiply. */
API void oracle_scale(const int32_t* D, const float* alpha, int64_t M, int64_t N, float* Y)
{
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            Y[m * N + n] = alpha[n] * (float)D[m * N + n];
}

/* [P4] Bi-Real Net row and [P3] "residual streams stay FP": the scaled binary
 * output plus the fp32 shortcut, as two rounded single operations (scale,
 * then add).  R is [M, N] with leading dimension ldr. */
API void oracle_scale_residual(const int32_t* D, const float* alpha, const float* R, int64_t ldr,
                               int64_t M, int64_t N, float* Y)
{
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            float z = alpha[n] * (float)D[m * N + n];
            Y[m * N + n] = z + R[m * ldr + n];
        }
}

/* im2col of the signs of an NHWC input for a 3x3 convolution with stride 1
 * and padding 1.  Output row p = (b * H + oh) * W + ow; column
 * k = (kh * 3 + kw) * C + c (tap-major, channel-minor).  A tap that falls
 * outside the image contributes +1 for every channel (pad pixels encode +1,
 * the pad-bit rule of [P2] applied to the spatial border).  Inside the image
 * the entry is sign(X[b, oh - 1 + kh, ow - 1 + kw, c]) per [P5] Notation. */
API void oracle_im2col_signs(const float* X, int64_t B, int64_t H, int64_t W, int64_t C, int8_t* cols)
{
    const int64_t K = 9 * C;
    #pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < B * H * W; ++p) {
        int64_t b = p / (H * W);
        int64_t oh = (p / W) % H;
        int64_t ow = p % W;
        for (int64_t kh = 0; kh < 3; ++kh)
            for (int64_t kw = 0; kw < 3; ++kw) {
                int64_t ih = oh - 1 + kh, iw = ow - 1 + kw;
                int inside = (ih >= 0 && ih < H && iw >= 0 && iw < W);
                for (int64_t c = 0; c < C; ++c) {
                    int8_t v = 1;
                    if (inside)
                        v = (X[((b * H + ih) * W + iw) * C + c] >= 0.0f) ? (int8_t)1 : (int8_t)-1;
                    cols[p * K + (kh * 3 + kw) * C + c] = v;
                }
            }
    }
}

/* [P3] "What is binary vs not": the first layer stays in floating point.
 * H[m, n] = sum_k X[m, k] * W[n, k] accumulated in double in index order
 * (each product of two floats is exact in double). */
API void oracle_dense_f64(const float* X, int64_t ldx, const float* W, int64_t ldw,
                          int64_t M, int64_t N, int64_t K, double* H)
{
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += (double)X[m * ldx + k] * (double)W[n * ldw + k];
            H[m * N + n] = acc;
        }
}

/* [P3]: the last layer stays in floating point and reads the +1/-1 outputs
 * of the last binary layer.  Y[m, n] = (float)(sum_k s[m, k] * W[n, k]) with
 * the sum in double in index order, rounded once to float. */
API void oracle_dense_pm1_f32out(const int8_t* s, const float* W, int64_t ldw,
                                 int64_t M, int64_t N, int64_t K, float* Y)
{
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += (double)s[m * K + k] * (double)W[n * ldw + k];
            Y[m * N + n] = (float)acc;
        }
}

/* [P5] "Binary Neural Networks" eq. (1)-(2) (binary weights times real
 * activations: only additions and subtractions) with the activations
 * quantized to 8-bit integers as in the BitNet section of [P5]:
 * D[m, n] = sum_k x[m, k] * s[n, k], an exact integer multiply-add over int8
 * values (|D| <= 128 K fits int32 for K <= 2^24).  The weights s are +1/-1
 * (binary) or -1/0/+1 (ternary, eq. (7) / (9)); the activations are int8
 * codes or +1/-1 signs.  xq is [M, K] (dense), ws is [N, K], D is [M, N]. */
API void oracle_dot_i8(const int8_t* xq, const int8_t* ws, int64_t M, int64_t N, int64_t K, int32_t* D)
{
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)xq[m * K + k] * (int64_t)ws[n * K + k];
            D[m * N + n] = (int32_t)acc;
        }
}

/* IEEE half precision (binary16) as an exact multiple of 2^-24, decoded from
 * the format's definition: sign bit 15, biased exponent e = bits 14..10,
 * fraction f = bits 9..0.  Normal (1 <= e <= 30): (1024 + f) * 2^(e - 25)
 * = (1024 + f) * 2^(e - 1) units of 2^-24; subnormal or zero (e = 0):
 * f units.  Returns 0 and sets *bad for infinities and NaNs (e = 31). */
static int64_t half_units(uint16_t h, int* bad)
{
    const int64_t e = (h >> 10) & 0x1F, f = h & 0x3FF;
    int64_t u;
    if (e == 31) { *bad = 1; return 0; }
    if (e == 0) u = f;
    else u = (1024 + f) << (e - 1);
    return (h & 0x8000) ? -u : u;
}

/* [P5] "Binary Neural Networks" eq. (1)-(2) with real activations
 * (BinaryConnect / BWN): each +1/-1 weight adds or subtracts its activation,
 * S[m, n] = sum_k s[n, k] * x[m, k].  x is fp16 (bit patterns, [M, ldx]); the
 * sum is taken exactly, in integer units of 2^-24 (every fp16 value is one:
 * |x| < 2^16, so |S| < 2^54 units for K <= 2^14 and int64 cannot overflow).
 * S_units[m * N + n] = S[m, n] * 2^24.  Returns 1 if any x is not finite. */
API int oracle_bwn_f16(const uint16_t* x, int64_t ldx, const int8_t* ws, int64_t M, int64_t N, int64_t K,
                       int64_t* S_units)
{
    int bad = 0;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) (void)half_units(x[m * ldx + k], &bad);
    if (bad) return 1;
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int dummy = 0;
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)ws[n * K + k] * half_units(x[m * ldx + k], &dummy);
            S_units[m * N + n] = acc;
        }
    return 0;
}

/* [P5] "BitNet: 1-bit Transformer", item 2 (activations quantized to INT8).
 * The page names no quantizer; the reading taken is symmetric per-row absmax:
 *   amax = max_k |x[m,k]| (NaN elements skipped),
 *   inv  = fl32(127 / amax)  (0 when amax is 0),
 *   q    = rint(fl32(x * inv)) clamped to [-127, 127]  (round half to even;
 *          NaN products give 0),
 *   scale[m] = fl32(amax / 127), so x ~= scale * q.
 * All arithmetic is IEEE single precision as written (one rounding per op).
 * Q is dense [M, K]. */
API void oracle_quantize_absmax_i8(const float* X, int64_t M, int64_t K, int64_t ldx,
                                   int8_t* Q, float* scale)
{
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(X[m * ldx + k]);
            if (a > amax) amax = a;
        }
        float inv = (amax > 0.0f) ? 127.0f / amax : 0.0f;
        scale[m] = amax / 127.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = X[m * ldx + k] * inv;
            float r = rintf(v);
            int8_t q;
            if (isnan(r)) q = 0;
            else if (r > 127.0f) q = 127;
            else if (r < -127.0f) q = -127;
            else q = (int8_t)r;
            Q[m * K + k] = q;
        }
    }
}

/* Bit-plane layout of int8 activations (a storage convention, not stated by
 * the pages): plane b (0..7) of row m holds bit b of the two's-complement
 * byte of Q[m,k], packed like a sign row (element k in word k / 32 at bit
 * k % 32); plane b of row m starts at words + (m * 8 + b) * ld.  Pad bits and
 * pad words are 0, i.e. the value 0.  xsum[m] = sum_k Q[m,k]. */
API void oracle_pack_planes_i8(const int8_t* Q, int64_t M, int64_t K, uint32_t* words, int64_t ld,
                               int32_t* xsum)
{
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        int64_t total = 0;
        for (int64_t b = 0; b < 8; ++b)
            for (int64_t w = 0; w < ld; ++w) words[(m * 8 + b) * ld + w] = 0u;
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = (uint8_t)Q[m * K + k];
            total += Q[m * K + k];
            for (int64_t b = 0; b < 8; ++b)
                if ((byte >> b) & 1u)
                    words[(m * 8 + b) * ld + k / 32] |= (uint32_t)1u << (k % 32);
        }
        xsum[m] = (int32_t)total;
    }
}

/* [P5] eq. (8): one scale for the whole matrix, the mean magnitude over all
 * N * K weights (||W||_1 / (nm)), summed in double in index order and
 * rounded once to float. */
API float oracle_alpha_tensor(const float* W, int64_t N, int64_t K, int64_t ldw)
{
    double total = 0.0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) total += fabs((double)W[n * ldw + k]);
    return (float)(total / ((double)N * (double)K));
}

/* Dequantized output of binary weights times absmax-int8 activations:
 * Y[m,n] = fl32(fl32(alpha[n] * (float)D[m,n]) * xscale[m]), two rounded
 * multiplies, no FMA.  alpha_stride 1: one scale per output row n; 0: one
 * scale for the whole matrix (alpha[0]). */
API void oracle_scale_i8(const int32_t* D, const float* alpha, int64_t alpha_stride,
                         const float* xscale, int64_t M, int64_t N, float* Y)
{
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            float z = alpha[n * alpha_stride] * (float)D[m * N + n];
            Y[m * N + n] = z * xscale[m];
        }
}

/* [P2] "y = Wx + b": the layer's bias after the alpha scale, then the
 * optional residual: Y = fl32(fl32(fl32(alpha * D) + b[n]) + R[m,n]), each
 * step one rounded op, no FMA.  alpha_stride as above; R may be NULL. */
API void oracle_scale_bias_residual(const int32_t* D, const float* alpha, int64_t alpha_stride,
                                    const float* bias, const float* R, int64_t ldr,
                                    int64_t M, int64_t N, float* Y)
{
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            float z = alpha[n * alpha_stride] * (float)D[m * N + n];
            float zb = z + bias[n];
            Y[m * N + n] = R ? zb + R[m * ldr + n] : zb;
        }
}

/* [P5] eq. (7): t = +1 for w > Delta, -1 for w < -Delta, 0 for |w| <= Delta.
 * The comparisons are IEEE single; a NaN satisfies none of the three cases
 * and is read as 0 (t = (w > Delta) - (w < -Delta)).  T is dense [N, K]. */
API void oracle_ternary_threshold(const float* W, int64_t N, int64_t K, int64_t ldw, float delta, int8_t* T)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            float w = W[n * ldw + k];
            T[n * K + k] = (int8_t)((w > delta) - (w < -delta));
        }
}

/* [P5] eq. (9): t = RoundClip(w / gamma, -1, 1) = max(-1, min(1, round(w / gamma))),
 * with w / gamma one IEEE single division and round() to nearest, ties to
 * even (rintf); a NaN quotient (gamma = 0 with w = 0, or a NaN weight) gives 0. */
API void oracle_ternary_roundclip(const float* W, int64_t N, int64_t K, int64_t ldw, float gamma, int8_t* T)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            float r = rintf(W[n * ldw + k] / gamma);
            int8_t t;
            if (isnan(r)) t = 0;
            else if (r > 1.0f) t = 1;
            else if (r < -1.0f) t = -1;
            else t = (int8_t)r;
            T[n * K + k] = t;
        }
}

/* Two-plane storage of ternary rows (a storage convention): in the sign plane
 * S a bit is 1 where t = -1; in the nonzero plane Z a bit is 1 where t != 0;
 * element k sits in word k / 32 at bit k % 32 of row n (row stride ld); pad
 * bits and pad words are 0 in both planes.  nnz[n] = number of nonzero t. */
API void oracle_pack_ternary(const int8_t* T, int64_t N, int64_t K, int64_t ld,
                             uint32_t* S, uint32_t* Z, int32_t* nnz)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        int32_t cnt = 0;
        for (int64_t w = 0; w < ld; ++w) { S[n * ld + w] = 0u; Z[n * ld + w] = 0u; }
        for (int64_t k = 0; k < K; ++k) {
            int8_t t = T[n * K + k];
            if (t != 0) {
                Z[n * ld + k / 32] |= (uint32_t)1u << (k % 32);
                ++cnt;
            }
            if (t == -1) S[n * ld + k / 32] |= (uint32_t)1u << (k % 32);
        }
        nnz[n] = cnt;
    }
}

/* [P4] ReActNet row, RSign: the sign of an activation after a per-channel
 * shift.  The page gives no formula; the reading taken is
 * s = sign(x - beta_c) with sign as in [P5] Notation (+1 for >= 0), decided
 * as the IEEE single comparison x >= beta_c (for finite values the same as
 * the sign of the rounded difference; NaN gives -1).  X is [rows, cols] with
 * row stride ldx, beta has cols entries, s is dense [rows, cols]. */
API void oracle_rsign(const float* x, int64_t rows, int64_t cols, int64_t ldx, const float* beta, int8_t* s)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            s[r * cols + c] = (x[r * ldx + c] >= beta[c]) ? (int8_t)1 : (int8_t)-1;
}

/* im2col of a 3x3 / stride 1 / pad 1 convolution over an NHWC tensor of
 * signs S [B, H, W, C] (+1 / -1): the same gather as oracle_im2col_signs,
 * with taps outside the image read as +1. */
API void oracle_im2col_pm1(const int8_t* S, int64_t B, int64_t H, int64_t W, int64_t C, int8_t* cols)
{
    const int64_t K = 9 * C;
    #pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < B * H * W; ++p) {
        int64_t b = p / (H * W), oh = (p / W) % H, ow = p % W;
        for (int64_t kh = 0; kh < 3; ++kh)
            for (int64_t kw = 0; kw < 3; ++kw) {
                int64_t ih = oh - 1 + kh, iw = ow - 1 + kw;
                int inside = ih >= 0 && ih < H && iw >= 0 && iw < W;
                for (int64_t c = 0; c < C; ++c)
                    cols[p * K + (kh * 3 + kw) * C + c] =
                        inside ? S[((b * H + ih) * W + iw) * C + c] : (int8_t)1;
            }
    }
}

/* Number of OpenMP threads the routines above use (for reporting). */
API int oracle_num_threads(void) { return omp_get_max_threads(); }
