// Floating-point first and last layers around the binary layers (gfx950).
//
// Page "Perfected Concept", table "What is binary vs not": first/last layers
// stay in higher precision; the first layer's output is binarized for the
// next binary layer (eq. (4) of "Extreme Quantization: Binary, Ternary &
// 1-bit LLMs", sign per its Notation), and the last layer reads the +1/-1
// outputs of the last binary layer.
//
// First layer: 64 x 8 NJ output tile per one-wave workgroup, 8 x NJ outputs
// per lane (lane (tx, ty) owns rows 8 ty .. +7 and columns tx + 8 j), K
// staged through LDS in 16-wide slices already widened to double: 8 + NJ LDS
// doubles per 8 NJ FMAs, against 8 per 16 of a 4x4 tile (LDS-bound at 37% of
// the fp64 peak).  NJ = 4 when 8-column lanes would leave fewer than two
// waves per SIMD.  Every product of two floats is exact in double and each output
// accumulates its K products in index order with one rounding per step (an
// FMA of an exact product equals a rounded add), so the sign decision sees
// the same double sum as a plain sequential loop.  The signs of each row's
// 32-column groups are folded into packed words with DPP row shifts, as in
// the pack kernels.
//
// Last layer: one workgroup per activation row, K split over its waves,
// double accumulators, fixed-order reductions (deterministic on every run).
#include "bnn_device.hpp"
#include "bnn_launch.hpp"

namespace bnn {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int kSlice = 16;

template <bool VEC, int NJ>
__global__ __launch_bounds__(64) void k_dense_f32_sign_pack(
    const float* __restrict__ X, int64_t ldX, const float* __restrict__ W, int64_t ldW,
    int M, int N, int K, uint32_t* __restrict__ Op, int64_t ldOp, int tiles_n)
{
    constexpr int kTN = 8 * NJ;                     // tile columns
    __shared__ double xs[kSlice][kTile];
    __shared__ double ws[kSlice][kTN];
    const int lane = threadIdx.x;
    const int tx = lane & 7, ty = lane >> 3;
    const int tn = blockIdx.x % tiles_n, tm = blockIdx.x / tiles_n;
    const int m0 = tm * kTile, n0 = tn * kTN;
    // staging: lane l widens 16 consecutive k of tile row l (of X and of W)
    const int gm = m0 + lane, gn = n0 + lane;
    const float* __restrict__ xrow = X + (int64_t)min(gm, M - 1) * ldX;
    const float* __restrict__ wrow = W + (int64_t)min(min(gn, n0 + kTN - 1), N - 1) * ldW;

    double acc[8][NJ];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = 0.0;

    // global loads of a slice go out one slice ahead (registers), LDS reads
    // of a k one k ahead
    float xv[kSlice], wv[kSlice];
    auto fetch = [&](int k0) {
        if (VEC && k0 + kSlice <= K) {
#pragma unroll
            for (int q = 0; q < kSlice / 4; ++q) {
                const float4 x4 = *reinterpret_cast<const float4*>(xrow + k0 + 4 * q);
                const float4 w4 = *reinterpret_cast<const float4*>(wrow + k0 + 4 * q);
                xv[4 * q] = x4.x; xv[4 * q + 1] = x4.y; xv[4 * q + 2] = x4.z; xv[4 * q + 3] = x4.w;
                wv[4 * q] = w4.x; wv[4 * q + 1] = w4.y; wv[4 * q + 2] = w4.z; wv[4 * q + 3] = w4.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kSlice; ++i) {
                xv[i] = (k0 + i < K) ? xrow[k0 + i] : 0.0f;
                wv[i] = (k0 + i < K) ? wrow[k0 + i] : 0.0f;
            }
        }
    };
    fetch(0);
    for (int k0 = 0; k0 < K; k0 += kSlice) {
        __syncthreads();                             // the previous slice has been read
#pragma unroll
        for (int i = 0; i < kSlice; ++i) {
            xs[i][lane] = gm < M ? (double)xv[i] : 0.0;
            if (lane < kTN) ws[i][lane] = gn < N ? (double)wv[i] : 0.0;
        }
        __syncthreads();
        if (k0 + kSlice < K) fetch(k0 + kSlice);
        double a[2][8], b[2][NJ];
        auto rd = [&](int kk, int p) {
#pragma unroll
            for (int i = 0; i < 8; ++i) a[p][i] = xs[kk][8 * ty + i];
#pragma unroll
            for (int j = 0; j < NJ; ++j) b[p][j] = ws[kk][tx + 8 * j];
        };
        rd(0, 0);
#pragma unroll
        for (int kk = 0; kk < kSlice; ++kk) {
            if (kk + 1 < kSlice) rd(kk + 1, (kk + 1) & 1);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_fma(a[kk & 1][i], b[kk & 1][j], acc[i][j]);
        }
    }

    // Padded k (k >= K) contributed exact zeros, so each acc is the in-order
    // double sum over k < K.  Columns >= N hold 0.0 -> bit 0 (+1), the pad
    // rule.  Word h of a row (columns 32 h .. +31 of the tile) takes bit
    // tx + 8 j' from column tx + 8 (4 h + j') of lane tx: an OR over the 8
    // lanes of the row group.
    const int nw = (N + 31) >> 5;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int m = m0 + 8 * ty + i;
#pragma unroll
        for (int h = 0; h < NJ / 4; ++h) {
            uint32_t bits = 0u;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) bits |= (acc[i][4 * h + jj] >= 0.0 ? 0u : 1u) << (tx + 8 * jj);
            const uint32_t word = or_reduce8_to_last(bits);
            const int widx = (n0 >> 5) + h;
            if (tx == 7 && m < M && widx < nw) Op[(int64_t)m * ldOp + widx] = word;
        }
        if (tn == tiles_n - 1 && tx == 0 && m < M)
            for (int64_t w = nw; w < ldOp; ++w) Op[(int64_t)m * ldOp + w] = 0u;
    }
}

// Last layer: one workgroup per activation row; its 4 waves take interleaved
// 256-element slices of K (lane: 4 consecutive k), every lane keeps one
// double per output column (NB per pass), each wave reduces with a
// fixed-order butterfly and wave 0 adds the 4 wave sums in order.
template <int NB, bool VEC>
__global__ __launch_bounds__(kThreads) void k_dense_binact_f32(
    const uint32_t* __restrict__ Xp, int64_t ldXp, const float* __restrict__ W, int64_t ldW,
    int M, int N, int K, float* __restrict__ Y, int64_t ldY)
{
    __shared__ double part[4][NB];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t m = blockIdx.x;
    const uint32_t* __restrict__ xr = Xp + m * ldXp;
    for (int n0 = 0; n0 < N; n0 += NB) {
        double acc[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[j] = 0.0;
        for (int kb = 256 * wave; kb < K; kb += 1024) {
            const int k = kb + 4 * lane;
            if (k < K) {
                const uint32_t bits = xr[k >> 5] >> (k & 31);
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    if (n0 + j < N) {
                        const float* wr = W + (int64_t)(n0 + j) * ldW + k;
                        float w[4];
                        if (VEC && k + 4 <= K) {
                            const float4 v = *reinterpret_cast<const float4*>(wr);
                            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i) w[i] = (k + i < K) ? wr[i] : 0.0f;
                        }
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const double d = (double)w[i];
                            acc[j] = ((bits >> i) & 1u) ? acc[j] - d : acc[j] + d;
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const double tot = wave_sum_f64(acc[j]);
            if (lane == 0) part[wave][j] = tot;
        }
        __syncthreads();
        if (threadIdx.x < NB && n0 + (int)threadIdx.x < N) {
            const int j = threadIdx.x;
            Y[m * ldY + n0 + j] = (float)(((part[0][j] + part[1][j]) + part[2][j]) + part[3][j]);
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_dense_f32_sign_pack(const float* X, int64_t ldX, const float* W, int64_t ldW,
                                      int64_t M, int64_t N, int64_t K,
                                      uint32_t* Op, int64_t ldOp, hipStream_t s)
{
    const bool vec = (reinterpret_cast<uintptr_t>(X) & 15u) == 0 && (reinterpret_cast<uintptr_t>(W) & 15u) == 0 &&
                     ldX % 4 == 0 && ldW % 4 == 0;
    const int64_t tiles_m = (M + kTile - 1) / kTile;
    const bool wide = tiles_m * ((N + 63) / 64) >= (int64_t)num_cus() * 8;   // two waves per SIMD at NJ = 8
    const int tn_cols = wide ? 64 : 32;
    const int tiles_n = (int)((N + tn_cols - 1) / tn_cols);
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(64);
#define BNN_DENSE(V, NJ) hipLaunchKernelGGL((k_dense_f32_sign_pack<V, NJ>), grid, block, 0, s, X, ldX, W, ldW, \
                                            (int)M, (int)N, (int)K, Op, ldOp, tiles_n)
    if (vec) { if (wide) BNN_DENSE(true, 8); else BNN_DENSE(true, 4); }
    else     { if (wide) BNN_DENSE(false, 8); else BNN_DENSE(false, 4); }
#undef BNN_DENSE
    return hipGetLastError();
}

hipError_t launch_dense_binact_f32(const uint32_t* Xp, int64_t ldXp, const float* W, int64_t ldW,
                                   int64_t M, int64_t N, int64_t K,
                                   float* Y, int64_t ldY, hipStream_t s)
{
    const dim3 grid((unsigned)M), block(kThreads);
    const bool vec = (reinterpret_cast<uintptr_t>(W) & 15u) == 0 && ldW % 4 == 0;
    if (vec) hipLaunchKernelGGL((k_dense_binact_f32<16, true>), grid, block, 0, s, Xp, ldXp, W, ldW,
                                (int)M, (int)N, (int)K, Y, ldY);
    else     hipLaunchKernelGGL((k_dense_binact_f32<16, false>), grid, block, 0, s, Xp, ldXp, W, ldW,
                                (int)M, (int)N, (int)K, Y, ldY);
    return hipGetLastError();
}

}  // namespace bnn
