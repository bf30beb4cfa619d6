// Sign + bit-pack kernels for gfx950 (weights with per-row alpha, dense
// activations, and the 3x3 im2col of an NHWC image).
//
// Method (cited by page title and section / equation):
//  - sign(x) = +1 for x >= 0, -1 otherwise: "Extreme Quantization: Binary,
//    Ternary & 1-bit LLMs", Notation; weights binarized once, activations
//    before each binary layer: "Binary Neural Network (BNN)" glossary and
//    eq. (4) of the "Extreme Quantization" page.
//  - encoding bit 0 = +1, bit 1 = -1, pad bits +1, bits packed into words:
//    "First Principles: Why Binary Ops Can Be Exponentially Faster",
//    section "1. Arithmetic: MAC -> XNOR + popcount".
//  - alpha = (1/n) sum |w_i| per output row: "Extreme Quantization", eq. (1).
//
// Mapping: per step the 64 lanes of a wave read 64 x 16 B of consecutive
// source floats (1 KiB, fully coalesced; the im2col variant gathers the 16-B
// pieces of the neighbouring pixels) and each aligned group of 8 lanes folds
// its 32 sign bits into one word with three DPP row shifts; the last lane of
// the group stores the word.  Four steps (eight in the ternary pack) are
// issued before any is consumed; the loads are nontemporal, as every source
// element is read once.  The dense pack hands out 4 KiB chunks of rows (the
// waves in flight read neighbouring chunks); the other packs give a wave one
// output row at a time (grid-stride over rows).  alpha's |w| sum is fp64 per
// lane, then a fixed-order butterfly per wave and a fixed-order sum over the
// workgroup's waves: no atomics, the same result on every run.
#include "bnn_device.hpp"
#include "bnn_launch.hpp"

namespace bnn {
namespace {

constexpr int kThreads = 256;
constexpr int kSteps = 4;      // 8-word steps issued back to back per wave
constexpr int kRowSteps = 8;   // the same for the row-per-wave ternary pack
                               // (8 KiB in flight per wave)
constexpr int kChunkSteps = 4; // 8-word steps per chunk of the dense pack (4 KiB
                               // of source per chunk: 0.197 -> 0.183 ms for
                               // 16384 x 16384 fp32 activations on MI355X)

struct Frag {                  // four consecutive source elements as bit patterns
    uint32_t u[4];
};

__device__ __forceinline__ uint32_t nibble(const Frag& f) {
    return neg_bit(f.u[0]) | (neg_bit(f.u[1]) << 1) | (neg_bit(f.u[2]) << 2) | (neg_bit(f.u[3]) << 3);
}

__device__ __forceinline__ double abs_sum4(const Frag& f, double acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += (double)__uint_as_float(f.u[i] & 0x7FFFFFFFu);
    return acc;
}

// Elements k .. k+3 of a row; positions >= K read as +0.0 (bit 0, |x| = 0).
template <bool VEC>
__device__ __forceinline__ Frag load_frag(const float* __restrict__ row, int k, int K) {
    Frag f;
    if (VEC && k + 4 <= K) {
        // each source element is read once: nontemporal, so the stream does
        // not displace cached data
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + k));
        f.u[0] = v.x; f.u[1] = v.y; f.u[2] = v.z; f.u[3] = v.w;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            f.u[i] = (k + i < K) ? __float_as_uint(row[k + i]) : 0u;
    }
    return f;
}

// One chunk of a row: words w0 .. w0 + 8 kChunkSteps - 1 (clipped to ldp);
// returns the chunk's sum of |x| in double when ALPHA.
template <bool VEC, bool ALPHA>
__device__ __forceinline__ double pack_chunk(const float* __restrict__ xr, uint32_t* __restrict__ pr, int w0,
                                             int ldp, int K, int sub, int grp)
{
    double asum = 0.0;
    Frag f[kChunkSteps];
#pragma unroll
    for (int u = 0; u < kChunkSteps; ++u)
        f[u] = load_frag<VEC>(xr, 32 * (w0 + 8 * u + grp) + 4 * sub, K);
#pragma unroll
    for (int u = 0; u < kChunkSteps; ++u) {
        const int w = w0 + 8 * u + grp;
        const uint32_t word = or_reduce8_to_last(nibble(f[u]) << (4 * sub));
        if (sub == 7 && w < ldp) pr[w] = word;
        if (ALPHA) asum = abs_sum4(f[u], asum);
    }
    return asum;
}

// The work unit is a chunk of 8 kChunkSteps words (4 KiB of fp32 source) of a
// row.  Without alpha the waves take the chunks in row-major order, grid
// stride, so the waves in flight read neighbouring chunks.  With alpha a
// workgroup owns one row at a time: its waves take the row's chunks in turn
// and add their |w| sums through LDS in a fixed order (the same result on
// every run).  Measured on MI355X for a 1 GiB read: waves reading
// neighbouring blocks stream 6.6-6.8 TB/s, while waves spread over the
// whole buffer (as with one row per wave) get 5.6-5.9.
template <bool VEC, bool ALPHA>
__global__ __launch_bounds__(kThreads) void k_pack_dense(
    const float* __restrict__ X, int64_t rows, int K, int64_t ldX,
    uint32_t* __restrict__ P, int64_t ldP, float* __restrict__ alpha)
{
    // Each row writes words 0 .. ldP-1: its ceil(K/32) data words and its pad words.
    const int lane = threadIdx.x & 63;
    const int sub = lane & 7;
    const int grp = lane >> 3;
    const int ldp = (int)ldP;
    constexpr int kChunk = 8 * kChunkSteps;
    const int nch = (ldp + kChunk - 1) / kChunk;
    if (!ALPHA) {
        const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
        const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
        const int64_t units = rows * nch;
        for (int64_t u = wave; u < units; u += nwaves) {
            const int64_t r = u / nch;
            const int c = (int)(u - r * nch);
            pack_chunk<VEC, false>(X + r * ldX, P + r * ldP, c * kChunk, ldp, K, sub, grp);
        }
    } else {
        constexpr int kW = kThreads / 64;
        __shared__ double red[kW];
        const int wv = threadIdx.x >> 6;
        for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
            double asum = 0.0;
            for (int c = wv; c < nch; c += kW)
                asum += pack_chunk<VEC, true>(X + r * ldX, P + r * ldP, c * kChunk, ldp, K, sub, grp);
            asum = wave_sum_f64(asum);
            if (lane == 0) red[wv] = asum;
            __syncthreads();
            if (threadIdx.x == 0) {
                double t = red[0];
#pragma unroll
                for (int i = 1; i < kW; ++i) t += red[i];
                alpha[r] = (float)(t / (double)K);
            }
            __syncthreads();
        }
    }
}

// im2col of a 3x3 / stride 1 / pad 1 convolution over NHWC input, packed.
// Output row p = (b*H + oh)*W + ow; element k = (kh*3 + kw)*C + c.  Taps
// outside the image are +1 (bit 0).  CT is C when fixed at compile time
// (cheap tap / channel split), 0 for a runtime C.
template <bool VEC, int CT>
__global__ __launch_bounds__(kThreads) void k_pack_im2col3x3(
    const float* __restrict__ X, int B, int H, int W, int Crt,
    uint32_t* __restrict__ P, int64_t ldP)
{
    const int C = CT > 0 ? CT : Crt;
    const int K = 9 * C;
    const int lane = threadIdx.x & 63;
    const int sub = lane & 7;
    const int grp = lane >> 3;
    const int64_t rows = (int64_t)B * H * W;
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
    const int ldp = (int)ldP;

    for (int64_t p = wave; p < rows; p += nwaves) {
        const int ow = (int)(p % W);
        const int64_t t = p / W;
        const int oh = (int)(t % H);
        const int64_t b = t / H;
        uint32_t* __restrict__ pr = P + p * ldP;
        for (int w0 = 0; w0 < ldp; w0 += 8 * kSteps) {
            Frag f[kSteps];
#pragma unroll
            for (int u = 0; u < kSteps; ++u) {
                const int k = 32 * (w0 + 8 * u + grp) + 4 * sub;
#pragma unroll
                for (int i = 0; i < 4; ++i) f[u].u[i] = 0u;
                if (VEC) {
                    if (k < K) {                 // C % 4 == 0: k..k+3 share one tap
                        const int tap = k / C;
                        const int c = k - tap * C;
                        const int kh = tap / 3, kw = tap - 3 * (tap / 3);
                        const int ih = oh - 1 + kh, iw = ow - 1 + kw;
                        if (ih >= 0 && ih < H && iw >= 0 && iw < W) {
                            const uint4 v = *reinterpret_cast<const uint4*>(
                                X + ((b * H + ih) * W + iw) * C + c);
                            f[u].u[0] = v.x; f[u].u[1] = v.y; f[u].u[2] = v.z; f[u].u[3] = v.w;
                        }
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int kk = k + i;
                        if (kk < K) {
                            const int tap = kk / C;
                            const int c = kk - tap * C;
                            const int kh = tap / 3, kw = tap - 3 * (tap / 3);
                            const int ih = oh - 1 + kh, iw = ow - 1 + kw;
                            if (ih >= 0 && ih < H && iw >= 0 && iw < W)
                                f[u].u[i] = __float_as_uint(X[((b * H + ih) * W + iw) * C + c]);
                        }
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < kSteps; ++u) {
                const int w = w0 + 8 * u + grp;
                const uint32_t word = or_reduce8_to_last(nibble(f[u]) << (4 * sub));
                if (sub == 7 && w < ldp) pr[w] = word;
            }
        }
    }
}

// Banded im2col for C % 32 == 0 (every tap is CW = C/32 whole words).
// One workgroup owns R consecutive output rows (oh0 .. oh0+R-1) of one
// image.  Phase 1 packs the input rows oh0-1 .. oh0+R they need -- a
// contiguous stretch of the NHWC image, read as one coalesced stream -- into
// LDS (rows outside the image are 0, i.e. +1).  Phase 2 writes the R*W
// output rows, ld words each, in 16-byte pieces: word w < 9*CW is tap w/CW,
// read from LDS (0 for columns outside the image); words from 9*CW are pad.
template <int CWLOG2>
__global__ __launch_bounds__(kThreads) void k_im2col_band(
    const float* __restrict__ X, int H, int W, int R, int bands,
    uint32_t* __restrict__ P, int ldP)
{
    constexpr int CW = 1 << CWLOG2;
    extern __shared__ uint32_t band[];                  // (R+2) x W x CW words
    const int b = blockIdx.x / bands;
    const int oh0 = (blockIdx.x - b * bands) * R;
    const int rows_out = min(R, H - oh0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane & 7, grp = lane >> 3;

    // phase 1: words g of band rows 0 .. rows_out+1 (input row oh0-1+i)
    const int nwords = (rows_out + 2) * W * CW;
    const int row_words = W * CW;
    for (int g0 = wave * 8 * kSteps; g0 < nwords; g0 += 4 * 8 * kSteps) {
        Frag f[kSteps];
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            const int g = g0 + 8 * u + grp;
            const int i = g / row_words;
            const int ih = oh0 - 1 + i;
            f[u].u[0] = f[u].u[1] = f[u].u[2] = f[u].u[3] = 0u;
            if (g < nwords && ih >= 0 && ih < H) {
                const int64_t e = ((int64_t)b * H + ih) * W * (32 * CW) + (int64_t)(g - i * row_words) * 32 + 4 * sub;
                const uint4 v = *reinterpret_cast<const uint4*>(X + e);
                f[u].u[0] = v.x; f[u].u[1] = v.y; f[u].u[2] = v.z; f[u].u[3] = v.w;
            }
        }
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            const int g = g0 + 8 * u + grp;
            const uint32_t word = or_reduce8_to_last(nibble(f[u]) << (4 * sub));
            if (sub == 7 && g < nwords) band[g] = word;
        }
    }
    __syncthreads();

    // phase 2: the output rows of this band, 4 words per thread and step
    const int quads = ldP >> 2;                          // ldP % 4 == 0
    const int total = rows_out * W * quads;
    uint32_t* __restrict__ out = P + ((int64_t)b * H + oh0) * W * ldP;
    for (int t = threadIdx.x; t < total; t += kThreads) {
        const int px = t / quads;                        // pixel within the band
        const int w0 = (t - px * quads) * 4;
        const int r = px / W, ow = px - (px / W) * W;
        uint32_t v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int w = w0 + i;
            uint32_t x = 0u;
            if (w < 9 * CW) {
                const int tap = w >> CWLOG2, j = w & (CW - 1);
                const int kh = tap / 3, kw = tap - 3 * (tap / 3);
                const int iw = ow - 1 + kw;
                if (iw >= 0 && iw < W) x = band[((r + kh) * W + iw) * CW + j];
            }
            v[i] = x;
        }
        *reinterpret_cast<uint4*>(out + (int64_t)px * ldP + w0) = make_uint4(v[0], v[1], v[2], v[3]);
    }
}

// Ternary weights ("Extreme Quantization", eq. (7) and eq. (9)), packed as a
// sign plane S (bit 1 where t = -1) and a nonzero plane Z (bit 1 where
// t != 0), with nnz[n] = number of nonzero t of row n.  ROUNDCLIP: t =
// RoundClip(w / gamma, -1, 1) with gamma read from device memory (one IEEE
// division, round half to even, NaN -> 0); otherwise t = (w > delta) -
// (w < -delta).  Elements past K and the pad words are 0 in both planes.
// Same mapping as k_pack_dense: a wave per row, 8 lanes per word.
template <bool VEC, bool ROUNDCLIP>
__global__ __launch_bounds__(kThreads) void k_pack_ternary(
    const float* __restrict__ W, int64_t rows, int K, int64_t ldW, const float* __restrict__ gamma,
    float delta, uint32_t* __restrict__ S, uint32_t* __restrict__ Z, int64_t ld, int32_t* __restrict__ nnz)
{
    const int lane = threadIdx.x & 63;
    const int sub = lane & 7;
    const int grp = lane >> 3;
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
    const int ldi = (int)ld;
    const float gm = ROUNDCLIP ? gamma[0] : 0.0f;
    for (int64_t r = wave; r < rows; r += nwaves) {
        const float* __restrict__ wr = W + r * ldW;
        int32_t cnt = 0;
        for (int w0 = 0; w0 < ldi; w0 += 8 * kRowSteps) {
            Frag f[kRowSteps];
#pragma unroll
            for (int u = 0; u < kRowSteps; ++u)
                f[u] = load_frag<VEC>(wr, 32 * (w0 + 8 * u + grp) + 4 * sub, K);
#pragma unroll
            for (int u = 0; u < kRowSteps; ++u) {
                const int w = w0 + 8 * u + grp;
                uint32_t sn = 0u, zn = 0u;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = __uint_as_float(f[u].u[i]);
                    int t;
                    if (ROUNDCLIP) {
                        const float q = rintf(v / gm);
                        t = (q != q) ? 0 : (q > 1.0f ? 1 : (q < -1.0f ? -1 : (int)q));
                    } else {
                        t = (v > delta ? 1 : 0) - (v < -delta ? 1 : 0);
                    }
                    if (32 * w + 4 * sub + i >= K) t = 0;
                    sn |= (t < 0 ? 1u : 0u) << i;
                    zn |= (t != 0 ? 1u : 0u) << i;
                }
                const uint32_t sw = or_reduce8_to_last(sn << (4 * sub));
                const uint32_t zw = or_reduce8_to_last(zn << (4 * sub));
                if (sub == 7 && w < ldi) {
                    S[r * ld + w] = sw;
                    Z[r * ld + w] = zw;
                    cnt += __popc(zw);
                }
            }
        }
#pragma unroll
        for (int s2 = 32; s2 >= 1; s2 >>= 1) cnt += __shfl_xor(cnt, s2, 64);
        if (lane == 0) nnz[r] = cnt;
    }
}

// RSign ("State of the Art Survey", ReActNet row): the sign of x - beta_k,
// decided as the IEEE single comparison x >= beta_k (bit 0 for +1; NaN -> 1),
// with one shift per column k (per channel of an NHWC image viewed as
// [pixels, C]).  Same mapping as k_pack_dense; positions >= K are +1 (0).
// LDP = 4 or 8 (packed rows of that many words, C <= 256 channels): the 8
// lane groups of a wave cover 8 / LDP rows per step, so no lane group idles
// past the end of a short row; LDP = 0 walks any row length.  RSIGN = false
// (short rows only): the plain sign of the dense pack, beta unused.
template <bool VEC, int LDP, int DW = 0, bool RSIGN = true>
__global__ __launch_bounds__(kThreads) void k_pack_dense_rsign(
    const float* __restrict__ X, int64_t rows, int K, int64_t ldX, const float* __restrict__ beta,
    uint32_t* __restrict__ P, int64_t ldP)
{
    const int lane = threadIdx.x & 63;
    const int sub = lane & 7;
    const int grp = lane >> 3;
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
    const int ldp = (int)ldP;
    auto nibble_rs = [&](const Frag& f, int k0) {
        uint32_t nib = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = k0 + i;
            const bool neg = k < K && !(__uint_as_float(f.u[i]) >= beta[k]);
            nib |= (neg ? 1u : 0u) << i;
        }
        return nib;
    };
    static_assert(RSIGN || LDP > 0, "the plain sign takes the short-row mapping only");
    if constexpr (LDP > 0) {
        // step u of a wave pass: rows r0 + RS u + grp / WL, word grp % WL,
        // with WL = LDP words per row, or DW when the lane groups cover only
        // the first DW = LDP / 2 words (the rest of the row is pad: its
        // zeros are stored by the same lanes, with no loads spent on them);
        // the lane's four columns, and so its four shifts, never change
        static_assert(DW == 0 || 2 * DW == LDP, "data words are half the row");
        constexpr int WL = DW > 0 ? DW : (LDP > 0 ? LDP : 8);
        constexpr int RS = 8 / WL;
        const int w = grp % WL;
        const int k0 = 32 * w + 4 * sub;
        float bt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) bt[i] = (RSIGN && k0 + i < K) ? beta[k0 + i] : 0.0f;
        for (int64_t r0 = RS * kSteps * wave; r0 < rows; r0 += RS * kSteps * nwaves) {
            Frag f[kSteps];
#pragma unroll
            for (int u = 0; u < kSteps; ++u) {
                const int64_t r = r0 + RS * u + grp / WL;
                f[u] = Frag{};
                if (r < rows) f[u] = load_frag<VEC>(X + r * ldX, k0, K);
            }
#pragma unroll
            for (int u = 0; u < kSteps; ++u) {
                const int64_t r = r0 + RS * u + grp / WL;
                uint32_t nib = 0u;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool neg = RSIGN ? !(__uint_as_float(f[u].u[i]) >= bt[i]) : neg_bit(f[u].u[i]) != 0u;
                    nib |= ((k0 + i < K && neg) ? 1u : 0u) << i;
                }
                const uint32_t word = or_reduce8_to_last(nib << (4 * sub));
                if (sub == 7 && r < rows) {
                    P[r * ldP + w] = word;
                    if (DW > 0) P[r * ldP + w + DW] = 0u;
                }
            }
        }
        return;
    }
    for (int64_t r = wave; r < rows; r += nwaves) {
        const float* __restrict__ xr = X + r * ldX;
        uint32_t* __restrict__ pr = P + r * ldP;
        for (int w0 = 0; w0 < ldp; w0 += 8 * kSteps) {
            Frag f[kSteps];
#pragma unroll
            for (int u = 0; u < kSteps; ++u)
                f[u] = load_frag<VEC>(xr, 32 * (w0 + 8 * u + grp) + 4 * sub, K);
#pragma unroll
            for (int u = 0; u < kSteps; ++u) {
                const int w = w0 + 8 * u + grp;
                const uint32_t word = or_reduce8_to_last(nibble_rs(f[u], 32 * w + 4 * sub) << (4 * sub));
                if (sub == 7 && w < ldp) pr[w] = word;
            }
        }
    }
}

int grid_for_rows(int64_t rows) {
    const int64_t waves_per_block = kThreads / 64;
    int64_t blocks = (rows + waves_per_block - 1) / waves_per_block;
    const int64_t cap = 256 * 32;   // 32 blocks per CU of a 256-CU device
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    return (int)blocks;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// One scale for the whole weight matrix, ||W||_1 / (N K) ("Extreme
// Quantization", eq. (8)).  Pass 1: one wave per row sums |W| in fp64 (the
// same per-lane order and butterfly as alpha above) into work[n].  Pass 2:
// one workgroup adds work[0 .. N) in a fixed order (thread-strided partial
// sums, then a fixed butterfly and a fixed sum over waves), divides by N*K in
// fp64 and rounds once to fp32.  The same on every run; the fp64 error is
// far below the final fp32 rounding step.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void k_row_abs_sum(
    const float* __restrict__ W, int64_t rows, int K, int64_t ldW, double* __restrict__ work)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
    for (int64_t r = wave; r < rows; r += nwaves) {
        const float* __restrict__ wr = W + r * ldW;
        double asum = 0.0;
        for (int k = 4 * lane; k < K; k += 4 * 64) asum = abs_sum4(load_frag<VEC>(wr, k, K), asum);
        asum = wave_sum_f64(asum);
        if (lane == 0) work[r] = asum;
    }
}

__global__ __launch_bounds__(kThreads) void k_tensor_alpha(
    const double* __restrict__ work, int64_t rows, double count, float* __restrict__ alpha)
{
    __shared__ double part[kThreads / 64];
    double s = 0.0;
    for (int64_t r = threadIdx.x; r < rows; r += kThreads) s += work[r];
    s = wave_sum_f64(s);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = part[0];
        for (int w = 1; w < kThreads / 64; ++w) t += part[w];
        alpha[0] = (float)(t / count);
    }
}

}  // namespace

hipError_t launch_pack_dense(const float* X, int64_t rows, int64_t K, int64_t ldX,
                             uint32_t* P, int64_t ldP, float* alpha, hipStream_t s)
{
    const bool vec = aligned16(X) && (ldX % 4 == 0);
    if (!alpha && (ldP == 4 || ldP == 8)) {
        // short rows (C <= 256 channels of an NHWC image): 8 / ldP rows per
        // wave step, as in the RSign pack; with 2 data words in a 4-word row
        // the pad words are stored without loads.  A chunk per row would
        // leave 3/4 of the lanes idle: 19 -> 8 us for 50176 x 256 fp32 on MI355X.
        const dim3 block(kThreads);
        const int kk = (int)K;
        const float* nob = nullptr;
        if (ldP == 4 && (K + 31) / 32 <= 2) {
            const dim3 grid(grid_for_rows((rows + 4 * kSteps - 1) / (4 * kSteps)));
            if (vec) hipLaunchKernelGGL((k_pack_dense_rsign<true, 4, 2, false>), grid, block, 0, s, X, rows, kk, ldX, nob, P, ldP);
            else     hipLaunchKernelGGL((k_pack_dense_rsign<false, 4, 2, false>), grid, block, 0, s, X, rows, kk, ldX, nob, P, ldP);
        } else if (ldP == 4) {
            const dim3 grid(grid_for_rows((rows + 2 * kSteps - 1) / (2 * kSteps)));
            if (vec) hipLaunchKernelGGL((k_pack_dense_rsign<true, 4, 0, false>), grid, block, 0, s, X, rows, kk, ldX, nob, P, ldP);
            else     hipLaunchKernelGGL((k_pack_dense_rsign<false, 4, 0, false>), grid, block, 0, s, X, rows, kk, ldX, nob, P, ldP);
        } else {
            const dim3 grid(grid_for_rows((rows + kSteps - 1) / kSteps));
            if (vec) hipLaunchKernelGGL((k_pack_dense_rsign<true, 8, 0, false>), grid, block, 0, s, X, rows, kk, ldX, nob, P, ldP);
            else     hipLaunchKernelGGL((k_pack_dense_rsign<false, 8, 0, false>), grid, block, 0, s, X, rows, kk, ldX, nob, P, ldP);
        }
        return hipGetLastError();
    }
    // without alpha: one wave per 4 KiB chunk (grid-stride); with alpha: one
    // workgroup per row at a time
    const int64_t nch = (ldP + 8 * kChunkSteps - 1) / (8 * kChunkSteps);
    int64_t blocks = alpha ? rows : (rows * nch + kThreads / 64 - 1) / (kThreads / 64);
    const int64_t cap = 256 * 32;
    blocks = blocks > cap ? cap : (blocks < 1 ? 1 : blocks);
    const dim3 grid((unsigned)blocks), block(kThreads);
    const int k = (int)K;
    if (alpha) {
        if (vec) hipLaunchKernelGGL((k_pack_dense<true, true>), grid, block, 0, s, X, rows, k, ldX, P, ldP, alpha);
        else     hipLaunchKernelGGL((k_pack_dense<false, true>), grid, block, 0, s, X, rows, k, ldX, P, ldP, alpha);
    } else {
        if (vec) hipLaunchKernelGGL((k_pack_dense<true, false>), grid, block, 0, s, X, rows, k, ldX, P, ldP, alpha);
        else     hipLaunchKernelGGL((k_pack_dense<false, false>), grid, block, 0, s, X, rows, k, ldX, P, ldP, alpha);
    }
    return hipGetLastError();
}

hipError_t launch_pack_im2col3x3(const float* X, int64_t B, int64_t H, int64_t W, int64_t C,
                                 uint32_t* P, int64_t ldP, hipStream_t s)
{
    const int64_t rows = B * H * W;
    const int64_t cw = C / 32;
    // banded path: whole-word taps, 16-byte rows, band in <= 32 KiB of LDS
    if (C % 32 == 0 && aligned16(X) && aligned16(P) && ldP % 4 == 0 && (cw & (cw - 1)) == 0 && cw <= 16 &&
        W * cw * 3 <= 8192 && ldP < ((int64_t)1 << 20) && W * ldP < ((int64_t)1 << 24)) {
        int cwlog2 = 0;
        while ((1 << cwlog2) < cw) ++cwlog2;
        // rows per band: enough bands for ~1024 workgroups (4 per CU), within
        // the LDS budget; each band re-reads 2 input rows, so taller is cheaper
        const int64_t r_lds = 8192 / (W * cw) - 2;
        int64_t R = (B * H + 1023) / 1024;
        if (R < 1) R = 1;
        if (R > r_lds) R = r_lds;
        if (R > H) R = H;
        const int64_t bands = (H + R - 1) / R;
        const size_t lds = (size_t)(R + 2) * W * cw * sizeof(uint32_t);
        const dim3 grid((unsigned)(B * bands)), block(kThreads);
        const int hh = (int)H, ww = (int)W, rr = (int)R, nb = (int)bands, ldp = (int)ldP;
#define BNN_BAND(L) hipLaunchKernelGGL((k_im2col_band<L>), grid, block, lds, s, X, hh, ww, rr, nb, P, ldp)
        switch (cwlog2) {
            case 0: BNN_BAND(0); break;
            case 1: BNN_BAND(1); break;
            case 2: BNN_BAND(2); break;
            case 3: BNN_BAND(3); break;
            default: BNN_BAND(4); break;
        }
#undef BNN_BAND
        return hipGetLastError();
    }
    const bool vec = aligned16(X) && (C % 4 == 0);
    const dim3 grid(grid_for_rows(rows)), block(kThreads);
    const int b = (int)B, h = (int)H, w = (int)W, c = (int)C;
#define BNN_IM2COL(VEC, CT) hipLaunchKernelGGL((k_pack_im2col3x3<VEC, CT>), grid, block, 0, s, X, b, h, w, c, P, ldP)
    if (vec) {
        switch (C) {
            case 32: BNN_IM2COL(true, 32); break;
            case 64: BNN_IM2COL(true, 64); break;
            case 128: BNN_IM2COL(true, 128); break;
            case 256: BNN_IM2COL(true, 256); break;
            case 512: BNN_IM2COL(true, 512); break;
            default: BNN_IM2COL(true, 0); break;
        }
    } else {
        BNN_IM2COL(false, 0);
    }
#undef BNN_IM2COL
    return hipGetLastError();
}

hipError_t launch_alpha_tensor(const float* W, int64_t N, int64_t K, int64_t ldW,
                               double* work, float* alpha, hipStream_t s)
{
    const bool vec = (reinterpret_cast<uintptr_t>(W) & 15u) == 0 && ldW % 4 == 0;
    int64_t blocks = (N + 3) / 4;
    if (blocks > 8192) blocks = 8192;
    const dim3 grid((unsigned)blocks), block(kThreads);
    if (vec) hipLaunchKernelGGL((k_row_abs_sum<true>), grid, block, 0, s, W, N, (int)K, ldW, work);
    else     hipLaunchKernelGGL((k_row_abs_sum<false>), grid, block, 0, s, W, N, (int)K, ldW, work);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_tensor_alpha, dim3(1), block, 0, s, (const double*)work, N,
                       (double)N * (double)K, alpha);
    return hipGetLastError();
}

hipError_t launch_pack_ternary(const float* W, int64_t N, int64_t K, int64_t ldW, const float* gamma,
                               float delta, uint32_t* S, uint32_t* Z, int64_t ld, int32_t* nnz,
                               hipStream_t s)
{
    const bool vec = aligned16(W) && (ldW % 4 == 0);
    const dim3 grid(grid_for_rows(N)), block(kThreads);
    const int k = (int)K;
#define BNN_TPACK(V, R) hipLaunchKernelGGL((k_pack_ternary<V, R>), grid, block, 0, s, W, N, k, ldW, gamma, delta, S, Z, ld, nnz)
    if (gamma) { if (vec) BNN_TPACK(true, true); else BNN_TPACK(false, true); }
    else       { if (vec) BNN_TPACK(true, false); else BNN_TPACK(false, false); }
#undef BNN_TPACK
    return hipGetLastError();
}

hipError_t launch_pack_dense_rsign(const float* X, int64_t rows, int64_t K, int64_t ldX, const float* beta,
                                   uint32_t* P, int64_t ldP, hipStream_t s)
{
    const bool vec = aligned16(X) && (ldX % 4 == 0);
    const dim3 block(kThreads);
    if (ldP == 4 && (K + 31) / 32 <= 2) {           // 2 data words + 2 pad words per row
        const int64_t rs = 4;
        const dim3 grid(grid_for_rows((rows + rs * kSteps - 1) / (rs * kSteps)));
        if (vec) hipLaunchKernelGGL((k_pack_dense_rsign<true, 4, 2>), grid, block, 0, s, X, rows, (int)K, ldX, beta, P, ldP);
        else     hipLaunchKernelGGL((k_pack_dense_rsign<false, 4, 2>), grid, block, 0, s, X, rows, (int)K, ldX, beta, P, ldP);
        return hipGetLastError();
    }
    if (ldP == 4 || ldP == 8) {                      // 8 / ldP rows per wave step
        const int64_t rs = 8 / ldP;
        const dim3 grid(grid_for_rows((rows + rs * kSteps - 1) / (rs * kSteps)));
        if (ldP == 4) {
            if (vec) hipLaunchKernelGGL((k_pack_dense_rsign<true, 4>), grid, block, 0, s, X, rows, (int)K, ldX, beta, P, ldP);
            else     hipLaunchKernelGGL((k_pack_dense_rsign<false, 4>), grid, block, 0, s, X, rows, (int)K, ldX, beta, P, ldP);
        } else {
            if (vec) hipLaunchKernelGGL((k_pack_dense_rsign<true, 8>), grid, block, 0, s, X, rows, (int)K, ldX, beta, P, ldP);
            else     hipLaunchKernelGGL((k_pack_dense_rsign<false, 8>), grid, block, 0, s, X, rows, (int)K, ldX, beta, P, ldP);
        }
        return hipGetLastError();
    }
    const dim3 grid(grid_for_rows(rows));
    if (vec) hipLaunchKernelGGL((k_pack_dense_rsign<true, 0>), grid, block, 0, s, X, rows, (int)K, ldX, beta, P, ldP);
    else     hipLaunchKernelGGL((k_pack_dense_rsign<false, 0>), grid, block, 0, s, X, rows, (int)K, ldX, beta, P, ldP);
    return hipGetLastError();
}

}  // namespace bnn
