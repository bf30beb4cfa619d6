/*
 * bnn.h - C ABI of libbnn.so, the MI355X (gfx950) binary-neural-network
 * inference path: sign + bit-pack, XNOR-popcount GEMM / GEMV, and fused
 * epilogues (alpha scale, fp32 residual, folded-BatchNorm threshold with
 * re-sign and re-pack).
 *
 * Sources (page title, section / equation):
 *  [P2] "First Principles: Why Binary Ops Can Be Exponentially Faster",
 *       section "1. Arithmetic: MAC -> XNOR + popcount": bit 0 encodes +1,
 *       bit 1 encodes -1; <w,x> = N - 2 popcount(w_bit xor x_bit); pad bits
 *       encode +1; pack bits into machine words.  Section "Bandwidth math":
 *       batch-1 y = Wx moves about MN/8 bytes of packed weights.
 *  [P5] "Extreme Quantization: Binary, Ternary & 1-bit LLMs": "Notation"
 *       (sign(x) = +1 for x >= 0, else -1), "Binary Neural Networks" eq. (1)
 *       (y = alpha * w_b^T x, alpha = mean |w|), "XNOR-Net" eq. (4)-(6).
 *  [P1] "Binary Neural Network (BNN)" glossary: activations are binarized
 *       before each binary layer; per-filter scaling factors; BatchNorm.
 *  [P3] "Perfected Concept", "What is binary vs not": first/last layers and
 *       BatchNorm scales stay FP; residual streams stay FP.
 *  [P4] "State of the Art Survey", Bi-Real Net row: FP residual shortcut.
 *  [P5] "BitNet: 1-bit Transformer": binary weights next to INT8
 *       activations; eq. (8) one mean-|W| scale for the whole matrix.
 *
 * Conventions (all entry points):
 *  - Data pointers are DEVICE pointers unless the name ends in _host.  The
 *    caller owns every buffer; the library never allocates, frees or
 *    synchronizes.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  Argument structs are host memory, read during the call only.
 *  - Arguments are validated before anything is launched.  A non-OK status
 *    means nothing was launched and no memory was touched.  BNN_ERR_HIP means
 *    the HIP runtime refused a launch.  Faults inside kernels surface at the
 *    caller's next synchronization.
 *  - No global mutable state, except the per-GPU scratch array of
 *    bnn_weight_scale_tensor_noalloc: calls may be issued from several host
 *    threads (that one entry point's calls must not overlap on one GPU).
 *  - Sizes: 1 <= K <= 2^24 (so every dot product is exact as an fp32 and an
 *    int32).  M == 0 or N == 0 is a valid empty call (nothing launched); its
 *    pointers are validated like those of any other call (non-null, aligned),
 *    so a zero-size buffer still needs a valid base address.
 *
 * Packed layout (the "packed operand" of every call):
 *  - A packed matrix [rows, ld] of uint32 words holds row r's element k at
 *    word r*ld + k/32, bit k%32 (least significant bit first); bit value 0
 *    is +1 and 1 is -1 [P2].  Kw = ceil(K/32) words carry data.
 *  - Pad bits (k >= K in word Kw-1) and pad words (Kw .. ld-1) hold 0, i.e.
 *    +1 [P2]; the pack calls always write them.  The GEMM/GEMV read words
 *    0..Kw-1 only and need the pad bits of the two operands to be equal.
 *  - Packed operands: base pointer 16-byte aligned and ld a multiple of 4
 *    (rows are read in 16-byte units), else BNN_ERR_ALIGN.
 */
#ifndef BNN_H
#define BNN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* bnn_stream_t; /* a hipStream_t; NULL selects the null stream */

typedef enum bnn_status {
    BNN_OK = 0,
    BNN_ERR_NULL = 1,        /* a required pointer is NULL */
    BNN_ERR_SHAPE = 2,       /* a size is negative or out of range */
    BNN_ERR_LD = 3,          /* a leading dimension is smaller than the row */
    BNN_ERR_ALIGN = 4,       /* a packed operand is misaligned */
    BNN_ERR_UNSUPPORTED = 5, /* unknown flag, flag combination or geometry */
    BNN_ERR_HIP = 6          /* the HIP runtime reported an error at launch */
} bnn_status;

#define BNN_MAX_K ((int64_t)1 << 24)

/* Epilogue flags of bnn_linear_fused (OR them together). */
#define BNN_EPI_DOT_I32      1u /* D[m,n] = K - 2*popcount(...)  (int32)              */
#define BNN_EPI_SCALE_F32    2u /* Y[m,n] = fl32(alpha[n] * D[m,n])  [P5] eq. (1)       */
#define BNN_EPI_RESIDUAL_F32 4u /* Y[m,n] = fl32(fl32(alpha[n]*D) + R[m,n])  [P4], [P3]  */
#define BNN_EPI_THRESH_PACK  8u /* Op bit (m,n) = ((float)(dir[n]*D) >= tau[n]) ? 0 : 1  */
#define BNN_EPI_ALPHA_TENSOR 16u /* with SCALE: one scale alpha[0] for every n  [P5] eq. (8) */
#define BNN_EPI_BIAS_F32     32u /* with SCALE: + bias[n] after the scale, before R  [P2]  */
/* Weight-format flag (OR it into the same field): ternary weights {-1,0,+1},
 * [P5] "Ternary Quantization" eq. (7) / "BitNet b1.58" eq. (9), stored as
 * the sign plane Wp and the nonzero plane Zp of bnn_pack_weights_ternary.  */
#define BNN_W_TERNARY        64u
/* With SCALE_F32: after the final Y (scale, bias, residual), also write the
 * next layer's packed input, Op bit (m,n) = (Y[m,n] >= beta[n]) ? 0 : 1
 * (RSign of [P4] "State of the Art Survey", ReActNet row, as a per-channel
 * shift before the sign of [P5] Notation; beta NULL means 0, the plain sign),
 * packed along n like THRESH_PACK.  Not together with THRESH_PACK.          */
#define BNN_EPI_SIGN_PACK   128u

/* Longest row of the INT8-activation calls: |D| <= 128 K stays exact in fp32. */
#define BNN_MAX_K_I8 ((int64_t)1 << 17)
#define BNN_MAX_K_F16 ((int64_t)16384)

/* Geometry of a binary 3x3 convolution lowered to a GEMM by im2col.
 * Input NHWC [B, H, W, C] fp32, contiguous.  Only R = S = 3, stride 1,
 * pad 1 is supported; the pad pixels encode +1 (bit 0), the pad-bit rule of
 * [P2] applied to the image border.  The im2col row of output pixel
 * p = (b*H + oh)*W + ow has K = 9*C entries, k = (kh*3 + kw)*C + c. */
typedef struct bnn_conv_geom {
    int64_t B, H, W, C;
    int64_t R, S;        /* kernel height, width: must be 3, 3 */
    int64_t stride, pad; /* must be 1, 1 */
} bnn_conv_geom;

/* Arguments of bnn_linear_fused.  Host struct; every pointer is device
 * memory.  Pointers an epilogue does not use may be NULL. */
typedef struct bnn_fused_args {
    const uint32_t* Xp; int64_t ldXp; /* packed activations [M, ldXp]           */
    const uint32_t* Wp; int64_t ldWp; /* packed weights     [N, ldWp]           */
    int64_t M, N, K;
    uint32_t epilogue;                /* OR of BNN_EPI_* (at least one)         */
    int32_t* D; int64_t ldD;          /* DOT_I32: int32 [M, ldD], ldD >= N      */
    const float* alpha;               /* SCALE/RESIDUAL: fp32 [N]               */
    float* Y; int64_t ldY;            /* SCALE/RESIDUAL: fp32 [M, ldY]          */
    const float* R; int64_t ldR;      /* RESIDUAL: fp32 [M, ldR]; may not alias Y
                                         unless R == Y and ldR == ldY           */
    const float* tau;                 /* THRESH_PACK: fp32 [N]                  */
    const int8_t* dir;                /* THRESH_PACK: int8 [N] in {+1, -1, 0}   */
    uint32_t* Op; int64_t ldOp;       /* THRESH_PACK: packed [M, ldOp],
                                         ldOp >= ceil(N/32); pad bits/words 0   */
    const float* bias;                /* BIAS_F32: fp32 [N]                     */
    const uint32_t* Zp;               /* W_TERNARY: nonzero plane [N, ldWp]     */
    const int32_t* nnz;               /* W_TERNARY: nonzero count per row [N]   */
    const float* beta;                /* SIGN_PACK: RSign shift per column [N],
                                         or NULL                                */
} bnn_fused_args;

/* Arguments of bnn_bwn_i8_linear (binary weights x INT8 activations).  Host
 * struct; every pointer is device memory.  The activations come in either
 * (or both) of two forms written by bnn_quantize_act_i8 / bnn_pack_act_i8:
 *   bit planes  Xb [M, 8, ldXb] + xsum [M]  (read by the bit-plane GEMV);
 *   int8 rows   Xq [M, ldXq]                (read by the MFMA GEMM, with
 *                                            xsum too when given). */
typedef struct bnn_i8_args {
    const uint32_t* Xb; int64_t ldXb; /* planes: 16-byte aligned, ldXb % 4 == 0,
                                         ldXb >= ceil(K/32); plane pad bits 0  */
    const int32_t* xsum;              /* [M] row sums of the int8 values: sum
                                         over k < K of q[m,k] (4-byte aligned);
                                         required by the GEMV with binary
                                         weights; optional for the GEMM, which
                                         with binary weights then trusts it
                                         (a cheaper weight expansion)         */
    const int8_t* Xq; int64_t ldXq;   /* int8 rows: 16-byte aligned, ldXq % 16
                                         == 0, ldXq >= K; the GEMM reads whole
                                         16-byte pieces of a row below ldXq
                                         (bytes from K on are ignored);
                                         M * ldXq < 2^31                      */
    const float* xscale;              /* [M] activation scales, or NULL (1.0)   */
    const uint32_t* Wp; int64_t ldWp; /* packed weights [N, ldWp] (packed layout);
                                         the GEMM needs N * ldWp < 2^29      */
    int64_t M, N, K;                  /* 1 <= K <= BNN_MAX_K_I8                 */
    uint32_t epilogue;                /* DOT_I32 | SCALE_F32 [| ALPHA_TENSOR]   */
    int32_t* D; int64_t ldD;          /* DOT_I32: int32 [M, ldD], ldD >= N      */
    const float* alpha;               /* SCALE: fp32 [N] (or [1], ALPHA_TENSOR) */
    float* Y; int64_t ldY;            /* SCALE: fp32 [M, ldY], ldY >= N         */
    const uint32_t* Zp;               /* W_TERNARY: nonzero plane [N, ldWp]     */
} bnn_i8_args;

/* Number of 32-bit words that carry K packed bits: ceil(K/32); -1 if K < 0. */
int64_t bnn_packed_words(int64_t K);

/* Static, human-readable name of a status code. */
const char* bnn_status_string(bnn_status status);

/* Binarize and pack weights, and compute the per-output-row scale.
 * [P1] weights are binarized once for inference; [P5] Notation for sign;
 * [P2] encoding; [P5] eq. (1) alpha = (1/K) sum_k |W[n,k]| per output row.
 *  W     fp32 [N, ldW] (row-major, ldW >= K, 4-byte aligned).
 *  Wp    packed [N, ldWp] output (16-byte aligned, ldWp % 4 == 0,
 *        ldWp >= Kw); bits, pad bits and pad words are all written.
 *  alpha fp32 [N] output, or NULL to skip.  The sum of |W| runs in double
 *        and is rounded once to fp32 after the division by K.
 * sign(x) is decided on the bit pattern: +1 for +0.0, -0.0 and every x > 0
 * including +inf and positive denormals; -1 for x < 0 and for NaN. */
bnn_status bnn_pack_weights(const float* W, int64_t N, int64_t K, int64_t ldW,
                            uint32_t* Wp, int64_t ldWp, float* alpha,
                            bnn_stream_t stream);

/* Binarize and pack activations.  [P1] each layer's activations are
 * binarized before the next binary layer; [P5] eq. (4) x_b = sign(x).
 *  geom == NULL: X is fp32 [M, ldX] (ldX >= K), packed row by row.
 *  geom != NULL: X is the NHWC image of *geom; the call writes its packed
 *        im2col matrix (see bnn_conv_geom).  M must equal B*H*W and K must
 *        equal 9*C; ldX is ignored.
 *  Xp    packed [M, ldXp] output (16-byte aligned, ldXp % 4 == 0,
 *        ldXp >= Kw); pad bits and pad words written as 0. */
bnn_status bnn_pack_activations(const float* X, int64_t M, int64_t K, int64_t ldX,
                                const bnn_conv_geom* geom,
                                uint32_t* Xp, int64_t ldXp, bnn_stream_t stream);

/* XNOR-popcount binary matrix multiply [P2], [P5] eq. (6):
 *     D[m,n] = K - 2 * sum_{w < Kw} popcount(Xp[m,w] xor Wp[n,w])
 *     Y[m,n] = fl32(alpha[n] * (float)D[m,n])          ([P5] eq. (1))
 *  Xp [M, ldXp], Wp [N, ldWp]: packed operands (see the layout above).
 *  D  int32 [M, ldD] (ldD >= N) or NULL; Y fp32 [M, ldY] (ldY >= N) or NULL;
 *  alpha fp32 [N], required when Y is given.  At least one of D, Y.
 *  Small M (M <= 4, the batch-1 decode case of [P2] "Bandwidth math") runs
 *  an HBM-streaming GEMV kernel; larger M the register-blocked GEMM. */
bnn_status bnn_xnor_gemm(const uint32_t* Xp, int64_t ldXp,
                         const uint32_t* Wp, int64_t ldWp,
                         int64_t M, int64_t N, int64_t K,
                         int32_t* D, int64_t ldD,
                         const float* alpha, float* Y, int64_t ldY,
                         bnn_stream_t stream);

/* The same D and Y as bnn_xnor_gemm, computed on the matrix cores: every sign
 * becomes the FP4 (e2m1) value +1.0 or -1.0, so each product is exactly +-1
 * and the fp32 accumulation of integers below 2^24 is exact (K <= 2^24):
 * D[m,n] = sum_k s(X[m,k]) s(W[n,k]) bit for bit, the integer of [P2]
 * section "1. Arithmetic" and [P5] eq. (6) (not an approximation).  One
 * kernel for every M (no batch-1 GEMV path); arguments, layouts, limits and
 * errors as bnn_xnor_gemm. */
bnn_status bnn_xnor_gemm_mfma(const uint32_t* Xp, int64_t ldXp,
                              const uint32_t* Wp, int64_t ldWp,
                              int64_t M, int64_t N, int64_t K,
                              int32_t* D, int64_t ldD,
                              const float* alpha, float* Y, int64_t ldY,
                              bnn_stream_t stream);

/* The XNOR-popcount GEMM with a fused epilogue (see BNN_EPI_*):
 *  DOT_I32      D as in bnn_xnor_gemm.
 *  SCALE_F32    Y = fl32(alpha[n] * D)                               [P5] eq. (1)
 *  RESIDUAL_F32 with SCALE_F32: Y = fl32(fl32(alpha[n] * D) + R[m,n]), two
 *               rounded operations, no fused multiply-add      [P4] Bi-Real, [P3]
 *  THRESH_PACK  folded BatchNorm followed by sign [P1], [P5] eq. (4): the
 *               output bit of (m,n) is 0 (+1) iff (float)(dir[n]*D) >= tau[n],
 *               else 1 (-1); packed along n (bit n%32 of word n/32 of row m),
 *               so Op is the packed activation matrix of the next binary
 *               layer (its K is N).  Bits n >= N and words ceil(N/32)..ldOp-1
 *               are written as 0.  tau/dir come from
 *               bnn_fold_bn_thresholds_host.
 *  W_TERNARY    the weights are ternary (Wp = sign plane, Zp, nnz): every
 *               epilogue above uses D = nnz[n] - 2 popcount((x ^ S) & Z)
 *  ALPHA_TENSOR with SCALE_F32: alpha[0] scales every column, the single
 *               scale ||W||_1 / (nm) of [P5] eq. (8) (bnn_weight_scale_tensor)
 *  BIAS_F32     with SCALE_F32: Y = fl32(fl32(alpha * D) + bias[n]), then
 *               the residual (if any) is added: the "y = Wx + b" of [P2]
 *               section "The cost of a neural network step"
 * Errors: RESIDUAL, BIAS or ALPHA_TENSOR without SCALE, no flag, or unknown
 * flag bits -> BNN_ERR_UNSUPPORTED. */
bnn_status bnn_linear_fused(const bnn_fused_args* args, bnn_stream_t stream);

/* Sign + pack of activations with a per-column shift, RSign of [P4] "State
 * of the Art Survey" (ReActNet row): bit (m,k) = (X[m,k] >= beta[k]) ? 0 : 1,
 * an IEEE single comparison (for finite values the sign of X - beta; NaN
 * gives 1, i.e. -1).  An NHWC image viewed as [B*H*W, C] with beta per
 * channel gives the packed image that bnn_conv3x3_fused reads.
 *  X fp32 [M, ldX] (ldX >= K); beta fp32 [K]; Xp packed [M, ldXp] (pad bits
 *  and pad words written 0). */
bnn_status bnn_pack_activations_rsign(const float* X, int64_t M, int64_t K, int64_t ldX, const float* beta,
                                     uint32_t* Xp, int64_t ldXp, bnn_stream_t stream);

/* Binary 3x3 convolution (stride 1, pad 1, pad pixels +1) with implicit
 * im2col: the XNOR-popcount GEMM of bnn_linear_fused whose activation rows
 * are gathered on the fly from the packed image instead of read from a
 * packed im2col matrix ([P2] section "1. Arithmetic": pad bits +1; [P4]
 * Bi-Real Net row: FP shortcut; the config's ResNet-style block).
 *  geom   B, H, W, C with R = S = 3, stride = pad = 1; C in {64, 128, 256, 512}
 *  args   Xp/ldXp = packed NHWC image [B*H*W, ldXp] (C bits per pixel, from
 *         bnn_pack_activations / bnn_pack_activations_rsign on the image
 *         viewed as [B*H*W, C], or from a previous call's SIGN_PACK output);
 *         M = B*H*W; K = 9*C; Wp = packed OHWI weights [N, ldWp >= 9C/32]
 *         (k = (kh*3 + kw)*C + c, as bnn_pack_weights gives for the
 *         flattened OHWI tensor); every epilogue flag of bnn_linear_fused
 *         except W_TERNARY.  M * ldXp < 2^31.
 * Results are those of bnn_linear_fused on the explicit packed im2col. */
bnn_status bnn_conv3x3_fused(const bnn_fused_args* args, const bnn_conv_geom* geom, bnn_stream_t stream);

/* Ternary weights, [P5] "Ternary Quantization" eq. (7) and "BitNet b1.58"
 * eq. (9), packed as two planes with the packed layout above:
 *     gamma != NULL:  t = RoundClip(W / gamma[0], -1, 1)   (eq. (9): one IEEE
 *                     single division, round half to even; NaN -> 0); gamma
 *                     is device memory, normally ||W||_1 / (nm) from
 *                     bnn_weight_scale_tensor
 *     gamma == NULL:  t = +1 if W > delta, -1 if W < -delta, else 0 (eq. (7);
 *                     NaN -> 0)
 *  Sp   sign plane    [N, ld]: bit 1 where t = -1
 *  Zp   nonzero plane [N, ld]: bit 1 where t != 0
 *  nnz  int32 [N]: number of nonzero t per row
 *  (pad bits and pad words 0 in both planes; both 16-byte aligned, ld % 4
 *  == 0, ld >= ceil(K/32)).  The dot products then follow from
 *     binary x: D = nnz[n] - 2 popcount((x ^ S) & Z)
 *     int8 q:   D = sum_b c_b (popcount(P_b & Z) - 2 popcount(P_b & Z & S))
 *  W fp32 [N, ldW], ldW >= K.  Errors as for bnn_pack_weights. */
bnn_status bnn_pack_weights_ternary(const float* W, int64_t N, int64_t K, int64_t ldW,
                                    const float* gamma, float delta,
                                    uint32_t* Sp, uint32_t* Zp, int64_t ld, int32_t* nnz,
                                    bnn_stream_t stream);

/* One scale for the whole weight matrix, [P5] eq. (8):
 *     alpha[0] = fl32( (sum_{n,k} |W[n,k]|) / (N*K) )
 *  the sums in fp64 (per row, then over rows in a fixed order; the same on
 *  every run), one rounding to fp32 at the end.
 *  W fp32 [N, ldW] (ldW >= K, 4-byte aligned); work: device scratch of N
 *  doubles owned by the caller (8-byte aligned); alpha: device fp32 [1].
 *  N >= 1.  Errors: NULL -> BNN_ERR_NULL; sizes -> BNN_ERR_SHAPE / _LD. */
bnn_status bnn_weight_scale_tensor(const float* W, int64_t N, int64_t K, int64_t ldW,
                                   double* work, float* alpha, bnn_stream_t stream);

/* The same scale as bnn_weight_scale_tensor with no workspace argument and
 * no allocation, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The N per-row partial sums live in a static device array of
 * BNN_NOALLOC_MAX_ROWS doubles (512 KiB), one per GPU, held until the
 * process ends; its address is looked up once per device, on the first call
 * made with that device current.  Every call on a GPU uses that GPU's one
 * array: calls that overlap on one GPU (other streams, other host threads)
 * race and must be ordered by the caller.  Each call writes all N partial
 * sums before reading them, so nothing from an earlier call is read.
 *  W fp32 [N, ldW] (ldW >= K, 4-byte aligned); alpha: device fp32 [1].
 *  1 <= N <= BNN_NOALLOC_MAX_ROWS, else BNN_ERR_SHAPE; NULL -> BNN_ERR_NULL;
 *  BNN_ERR_HIP if the array's device address cannot be obtained. */
#define BNN_NOALLOC_MAX_ROWS 65536
bnn_status bnn_weight_scale_tensor_noalloc(const float* W, int64_t N, int64_t K, int64_t ldW,
                                           float* alpha, bnn_stream_t stream);

/* Quantize fp32 activations to INT8, one scale per row, [P5] "BitNet"
 * item 2 (activations at INT8; the quantizer is not given there, this is
 * symmetric absmax):
 *     amax = max_k |X[m,k]|  (NaN skipped);  inv = fl32(127 / amax), 0 if amax == 0
 *     q[m,k] = rint(fl32(X[m,k] * inv)) clamped to [-127, 127] (ties to even;
 *              a NaN product gives 0);       xscale[m] = fl32(amax / 127)
 *  so X ~= xscale * q.  Outputs (any of Xq, Xb may be NULL, not both):
 *  Xq    int8 [M, ldXq] (ldXq >= K);
 *  Xb    bit planes [M, 8, ldXb]: plane b of row m starts at word
 *        (m*8 + b)*ldXb and holds bit b of each two's-complement byte q[m,k]
 *        at word k/32, bit k%32; pad bits and pad words are written 0;
 *        16-byte aligned, ldXb % 4 == 0, ldXb >= ceil(K/32);
 *  xsum  int32 [M] = sum_k q[m,k] (required with Xb; else written when
 *        non-NULL);
 *  xscale fp32 [M] (required).
 *  X fp32 [M, ldX], ldX >= K.  1 <= K <= BNN_MAX_K_I8. */
bnn_status bnn_quantize_act_i8(const float* X, int64_t M, int64_t K, int64_t ldX,
                               int8_t* Xq, int64_t ldXq,
                               uint32_t* Xb, int64_t ldXb, int32_t* xsum,
                               float* xscale, bnn_stream_t stream);

/* Bit planes (and row sums) of int8 activations that are already quantized;
 * the same plane layout and xsum as bnn_quantize_act_i8.
 *  Xq int8 [M, ldXq] (ldXq >= K); Xb, ldXb, xsum as above (all required). */
bnn_status bnn_pack_act_i8(const int8_t* Xq, int64_t M, int64_t K, int64_t ldXq,
                           uint32_t* Xb, int64_t ldXb, int32_t* xsum, bnn_stream_t stream);

/* Binary weights x INT8 activations, [P5] eq. (1)-(2) (each +1/-1 weight
 * adds or subtracts its activation) with the INT8 activations of [P5]
 * "BitNet":
 *     D[m,n] = sum_k q[m,k] * s(n,k)     (exact int32; s = +1 for bit 0)
 *     Y[m,n] = fl32( fl32(alpha_n * (float)D) * xscale[m] )   (xscale given)
 *            = fl32( alpha_n * (float)D )                      (xscale NULL)
 *  alpha_n = alpha[n], or alpha[0] with BNN_EPI_ALPHA_TENSOR.
 *  With BNN_W_TERNARY the weights are ternary (Wp = sign plane, Zp) and
 *  s(n,k) is -1, 0 or +1; xsum is then not needed.
 *  Path: M <= 2 with Xb (and xsum, for binary weights) given, and
 *  ceil(ceil(K/32)/4) <= 256/M (K <= 32768 for one row, 16384 for two): the
 *  bit-plane streaming GEMV (the batch-1 decode case of [P2] "Bandwidth
 *  math"); otherwise the int8 MFMA GEMM, which needs Xq.  Flags other than
 *  DOT_I32, SCALE_F32, ALPHA_TENSOR and W_TERNARY -> BNN_ERR_UNSUPPORTED;
 *  neither usable activation form -> BNN_ERR_NULL. */
bnn_status bnn_bwn_i8_linear(const bnn_i8_args* args, bnn_stream_t stream);

/* Binary weights x fp16 activations (BinaryConnect / BWN), [P5] "Binary
 * Neural Networks" eq. (1)-(2): real activations, +1/-1 weights, so each
 * weight adds or subtracts its activation:
 *     S[m,n] = sum_{k<K} s(n,k) * x[m,k]        (s = +1 for bit 0)
 *     Y[m,n] = fl32(alpha_n * S[m,n])
 *  The products +-x are exact; S is summed in fp32 in a fixed order of the
 *  kernel's: no term passes through more than n = 128 ceil(ceil(K/128) / G)
 *  + 6 rounded additions (G = lanes per weight row: the smallest power of
 *  two >= ceil(K/128), at most 64), so |S - S_exact| <= n u / (1 - n u) *
 *  sum_k |x[m,k]| with u = 2^-24.
 *  (The default kernel's sums are shallower: at most 22 additions.)
 *  One launch per activation row (two for K > 8192: the first leaves its
 *  partial sum in Y): the packed weights stream once per row (the batch-1
 *  decode case of [P2] "Bandwidth math").
 *  X     fp16 bit patterns [M, ldX]: 16-byte aligned, ldX % 8 == 0, ldX >= K;
 *  Wp    packed weights [N, ldWp] (packed layout, ldWp % 4 == 0);
 *  alpha fp32 [N], or [1] with BNN_EPI_ALPHA_TENSOR;
 *  Y     fp32 [M, ldY], ldY >= N, 4-byte aligned.
 *  epilogue: BNN_EPI_SCALE_F32 [| BNN_EPI_ALPHA_TENSOR]; anything else ->
 *  BNN_ERR_UNSUPPORTED.  1 <= K <= BNN_MAX_K_F16. */
bnn_status bnn_bwn_f16_gemv(const uint16_t* X, int64_t ldX, const uint32_t* Wp, int64_t ldWp,
                            int64_t M, int64_t N, int64_t K, uint32_t epilogue,
                            const float* alpha, float* Y, int64_t ldY, bnn_stream_t stream);

/* Fold inference BatchNorm of z = alpha[n] * D followed by sign into the
 * (tau, dir) pair consumed by BNN_EPI_THRESH_PACK.  [P1] BatchNorm around
 * binary layers; [P3] BatchNorm scales stay FP; [P5] eq. (4) the next layer
 * takes the sign.  HOST memory, synchronous.
 *   BN(z) = gamma (z - mean) / sqrt(var + eps) + beta ; next sign = +1 iff BN >= 0,
 * taken in exact real arithmetic on the given fp32 values.  BN(alpha D) is
 * affine in D, so over the integers the rule is one threshold:
 *   gamma*alpha > 0: dir = +1, tau = the smallest integer D with BN >= 0
 *   gamma*alpha < 0: dir = -1, tau = -(the largest integer D with BN >= 0)
 *   gamma*alpha = 0: dir =  0, tau = 0 if BN (a constant) >= 0, else 1
 * so that (float)(dir * D) >= tau holds exactly when BN(alpha D) >= 0, for
 * every |D| <= 2^24.  tau is an integer-valued float (a boundary beyond
 * +2^24 is stored as 2^25, one below -2^24 as -2^24).  The boundary is
 * estimated in double and certified with exact big-integer arithmetic, so
 * ties (BN = 0 exactly) give +1.
 * Errors: NULL pointer (also for N == 0) -> BNN_ERR_NULL; N < 0 ->
 * BNN_ERR_SHAPE; a non-finite parameter or var[n] + eps <= 0 ->
 * BNN_ERR_UNSUPPORTED (nothing written). */
bnn_status bnn_fold_bn_thresholds_host(const float* gamma, const float* beta,
                                       const float* mean, const float* var, float eps,
                                       const float* alpha, int64_t N,
                                       float* tau, int8_t* dir);

/* First FP layer of a binary network [P3] ("first / last layers stay higher
 * precision"), fused with the sign + pack of its output [P5] eq. (4):
 *     h[m,n] = sum_k X[m,k] * W[n,k]   (products exact, accumulated in double)
 *     Op bit (m,n) = (h >= 0) ? 0 : 1, packed along n as in THRESH_PACK.
 *  X fp32 [M, ldX], W fp32 [N, ldW] (ldX, ldW >= K; 4-byte aligned);
 *  Op packed [M, ldOp], ldOp >= ceil(N/32), pad bits/words written 0.
 *  K may exceed 2^24 here only up to 2^31-1 (no exactness claim on h). */
bnn_status bnn_dense_f32_sign_pack(const float* X, int64_t ldX,
                                   const float* W, int64_t ldW,
                                   int64_t M, int64_t N, int64_t K,
                                   uint32_t* Op, int64_t ldOp, bnn_stream_t stream);

/* Last FP layer of a binary network [P3], reading the +1/-1 outputs of the
 * last binary layer in packed form:
 *     Y[m,n] = fl32( sum_k s(m,k) * W[n,k] ),  s = +1 for bit 0, -1 for bit 1,
 *  the sum in double (exact terms), rounded once.
 *  Xp packed [M, ldXp] (16-byte aligned, ldXp % 4 == 0, ldXp >= Kw);
 *  W fp32 [N, ldW] (ldW >= K); Y fp32 [M, ldY] (ldY >= N). */
bnn_status bnn_dense_binact_f32(const uint32_t* Xp, int64_t ldXp,
                                const float* W, int64_t ldW,
                                int64_t M, int64_t N, int64_t K,
                                float* Y, int64_t ldY, bnn_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BNN_H */
