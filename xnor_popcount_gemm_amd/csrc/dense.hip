// Floating-point first and last layers around the binary layers (gfx950).
//
// Page "Perfected Concept", table "What is binary vs not": first/last layers
// stay in higher precision; the first layer's output is binarized for the
// next binary layer (eq. (4) of "Extreme Quantization: Binary, Ternary &
// 1-bit LLMs", sign per its Notation), and the last layer reads the +1/-1
// outputs of the last binary layer.
//
// First layer, 16-byte aligned rows: the fp64 matrix cores (see
// k_dense_f64_mfma_sign_pack).  Other rows: 64 x 8 NJ output tile per
// one-wave workgroup, 8 x NJ outputs
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
// Last layer: 4 activation rows per workgroup (one per 16-lane group of
// each wave, the groups sharing every weight load), K split over the waves,
// double accumulators, fixed-order reductions (deterministic on every run).
#include <stdio.h>
#include <stdlib.h>

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

// Last layer: a workgroup of 16 waves owns 4 activation rows.  In each wave the 16
// lanes of row group g (lanes 16 g .. 16 g + 15) take row 4 b + g, lane
// 16 g + l the 4 consecutive k = 64 (w + 16 t) + 4 l of wave w, t = 0, 1, ...
// The 4 row groups read the same weight addresses, which the memory
// pipeline serves once per instruction, so each weight travels from L2 once
// per 4 rows.  Per k: acc += s * (double)w with s = +1.0 / -1.0 from the
// row's bit: an fma with an exact product, i.e. the exactly rounded
// acc +- w.  Each output's lane sums meet in a fixed 16-lane DPP scan,
// then the 16 waves' sums are added in wave order; NB columns per pass.
// (With 4 waves per workgroup, 16 K steps per wave, one wave per SIMD: 48
// us for the binary MLP's 1024 x 4096 -> 10 layer, latency-bound.)
constexpr int kBinactThreads = 1024;

// Sum of a double over each aligned 16-lane row, complete in the row's last
// lane: an inclusive scan by DPP row shifts of 1, 2, 4, 8 (both 32-bit
// halves moved, lanes shifted in from outside the row read +0.0), a fixed
// order with no LDS traffic.
__device__ __forceinline__ double dsum16_to_last(double v) {
#define BNN_DSTEP(CTRL)                                                                              \
    {                                                                                                \
        const uint64_t b = (uint64_t)__double_as_longlong(v);                                        \
        const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, true); \
        const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, true); \
        v += __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));                          \
    }
    BNN_DSTEP(0x111) BNN_DSTEP(0x112) BNN_DSTEP(0x114) BNN_DSTEP(0x118)
#undef BNN_DSTEP
    return v;
}
template <int NB, bool VEC>
__global__ __launch_bounds__(kBinactThreads) void k_dense_binact_f32(
    const uint32_t* __restrict__ Xp, int64_t ldXp, const float* __restrict__ W, int64_t ldW,
    int M, int N, int K, float* __restrict__ Y, int64_t ldY)
{
    constexpr int RB = 4;                         // rows per workgroup (one per 16-lane group)
    constexpr int WPG = kBinactThreads / 64;      // waves per workgroup
    __shared__ double part[WPG][RB][NB];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rg = lane >> 4, li = lane & 15;
    const int64_t m0 = (int64_t)blockIdx.x * RB;
    const int64_t mc = min(m0 + rg, (int64_t)M - 1);
    const uint32_t* __restrict__ xr = Xp + mc * ldXp;
    for (int n0 = 0; n0 < N; n0 += NB) {
        double acc[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[j] = 0.0;
        for (int kb = 64 * wave; kb < K; kb += 64 * WPG) {
            const int k = kb + 4 * li;
            if (k < K) {
                const uint32_t bits = xr[k >> 5] >> (k & 31);
                double sg[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) sg[i] = ((bits >> i) & 1u) ? -1.0 : 1.0;
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
                        for (int i = 0; i < 4; ++i) acc[j] = __builtin_fma(sg[i], (double)w[i], acc[j]);
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if (n0 + j < N) {
                const double v = dsum16_to_last(acc[j]);
                if (li == 15) part[wave][rg][j] = v;
            }
        }
        __syncthreads();
        if (threadIdx.x < RB * NB) {
            const int r = threadIdx.x / NB, j = threadIdx.x % NB;
            const int64_t m = m0 + r;
            if (m < M && n0 + j < N) {
                double t = part[0][r][j];
#pragma unroll
                for (int w = 1; w < WPG; ++w) t += part[w][r][j];
                Y[m * ldY + n0 + j] = (float)t;
            }
        }
        __syncthreads();
    }
}

// First layer on the fp64 matrix cores (v_mfma_f64_16x16x4_f64): the same
// h = X W^T with exact float products in double, for 16-byte aligned rows.
// A wave owns a 32 x 64 tile: 2 row blocks (m) x 4 column blocks (n) of
// 16 x 16 accumulators, 8 MFMAs per k-step.  Operands: A = a block of X
// (lane l: row m = l % 16), B = a block of W (lane l: column n = l % 16),
// both at k = 16 t + 4 (l / 16) + s in sub-step s of K-chunk t, so each lane
// loads its 4 consecutive k of a chunk as one float4 and every k < K enters
// once.  Result element r of lane l is D[4 r + l / 16][l % 16] (A's row
// first; the lane layout measured on MI355X), i.e. h[m = 4 r + l / 16]
// [n = l % 16] of the block, so one ballot over the 64 lanes gives
// the sign bits of 4 rows x 16 columns in 16-bit fields.  Each output's sum
// runs over the chunks in order; within a k-step the matrix core adds its 4
// products in its own order, so h can differ from a sequential double sum
// in the last bits (a sign differs only for |h| within that rounding error).
typedef double v4d __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_k4(const float* __restrict__ row, int k, int K) {
    if (k + 4 <= K) return *reinterpret_cast<const float4*>(row + k);
    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (k < K) v.x = row[k];
    if (k + 1 < K) v.y = row[k + 1];
    if (k + 2 < K) v.z = row[k + 2];
    if (k + 3 < K) v.w = row[k + 3];
    return v;
}

__device__ __forceinline__ float comp(const float4& v, int s) {
    return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

template <int BM, int BN>
__global__ __launch_bounds__(kThreads) void k_dense_f64_mfma_sign_pack(
    const float* __restrict__ X, int64_t ldX, const float* __restrict__ W, int64_t ldW,
    int M, int N, int K, uint32_t* __restrict__ Op, int64_t ldOp, int tiles_n, int tiles)
{
    const int lane = threadIdx.x & 63;
    const int tile = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (tile >= tiles) return;                       // no barriers below
    const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
    const int m0 = 16 * BM * tm, n0 = 16 * BN * tn;
    const int g = lane >> 4, c = lane & 15;
    const float* xr[BM];
    const float* wr[BN];
#pragma unroll
    for (int bm = 0; bm < BM; ++bm) xr[bm] = X + (int64_t)min(m0 + 16 * bm + c, M - 1) * ldX;
#pragma unroll
    for (int bn = 0; bn < BN; ++bn) wr[bn] = W + (int64_t)min(n0 + 16 * bn + c, N - 1) * ldW;

    v4d acc[BM][BN];
#pragma unroll
    for (int bm = 0; bm < BM; ++bm)
#pragma unroll
        for (int bn = 0; bn < BN; ++bn) acc[bm][bn] = (v4d){0.0, 0.0, 0.0, 0.0};

    // Full 16-k chunks run with unguarded loads and only uniform branches
    // (guarded loads inside the loop made the compiler move the accumulators
    // between AGPRs and VGPRs around every chunk: 4 extra VALU ops per MFMA);
    // the two operand buffers swap roles each chunk (no register copies).
    // A last partial chunk (K % 16 != 0) takes guarded loads after the loop.
    const int nfull = K >> 4;
    float4 x0[BM], w0[BN], x1[BM], w1[BN];
    auto ld_full = [&](float4 (&xv)[BM], float4 (&wv)[BN], int t) {
        const int k = 16 * t + 4 * g;
#pragma unroll
        for (int bm = 0; bm < BM; ++bm) xv[bm] = *reinterpret_cast<const float4*>(xr[bm] + k);
#pragma unroll
        for (int bn = 0; bn < BN; ++bn) wv[bn] = *reinterpret_cast<const float4*>(wr[bn] + k);
    };
    auto mma_chunk = [&](const float4 (&xa)[BM], const float4 (&wa)[BN]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            double xd[BM], wd[BN];
#pragma unroll
            for (int bm = 0; bm < BM; ++bm) xd[bm] = (double)comp(xa[bm], s);
#pragma unroll
            for (int bn = 0; bn < BN; ++bn) wd[bn] = (double)comp(wa[bn], s);
#pragma unroll
            for (int bm = 0; bm < BM; ++bm)
#pragma unroll
                for (int bn = 0; bn < BN; ++bn)
                    acc[bm][bn] = __builtin_amdgcn_mfma_f64_16x16x4f64(xd[bm], wd[bn], acc[bm][bn], 0, 0, 0);
        }
    };
    if (nfull > 0) ld_full(x0, w0, 0);
    int t = 0;
    for (; t + 2 <= nfull; t += 2) {              // chunk t from buffer 0, t + 1 from buffer 1
        ld_full(x1, w1, t + 1);
        mma_chunk(x0, w0);
        if (t + 2 < nfull) ld_full(x0, w0, t + 2);
        mma_chunk(x1, w1);
    }
    if (t < nfull) mma_chunk(x0, w0);             // an odd last full chunk, already loaded
    if (K & 15) {                                 // the partial chunk: k >= K reads as 0
        const int k = 16 * nfull + 4 * g;
#pragma unroll
        for (int bm = 0; bm < BM; ++bm) x1[bm] = load_k4(xr[bm], k, K);
#pragma unroll
        for (int bn = 0; bn < BN; ++bn) w1[bn] = load_k4(wr[bn], k, K);
        mma_chunk(x1, w1);
    }

    // Sign bits: bit 1 for h < 0; columns >= N give 0 (+1, the pad rule).
    // For block row bm and element r, ballot bn holds rows m0 + 16 bm + 4 r
    // + q (q = 0..3) in bits 16 q .. 16 q + 15, columns n0 + 16 bn + 0..15;
    // lanes 0 .. 4 BN/2 - 1 write the 4 rows' BN/2 words.
    static_assert(BN % 2 == 0, "whole 32-column words per tile");
    constexpr int WPR = BN / 2;
    const int nw = (N + 31) >> 5;
#pragma unroll
    for (int bm = 0; bm < BM; ++bm)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            uint64_t b[BN];
#pragma unroll
            for (int bn = 0; bn < BN; ++bn)
                b[bn] = __builtin_amdgcn_ballot_w64(acc[bm][bn][r] < 0.0 && n0 + 16 * bn + c < N);
            if (lane < 4 * WPR) {
                const int q = lane / WPR, w = lane - q * WPR;
                uint64_t lo = b[0], hi = b[1];
#pragma unroll
                for (int i = 1; i < WPR; ++i)
                    if (w == i) { lo = b[2 * i]; hi = b[2 * i + 1]; }
                const uint32_t word = (uint32_t)((lo >> (16 * q)) & 0xFFFFu) |
                                      ((uint32_t)((hi >> (16 * q)) & 0xFFFFu) << 16);
                const int m = m0 + 16 * bm + 4 * r + q;
                const int widx = (n0 >> 5) + w;
                if (m < M && widx < nw) Op[(int64_t)m * ldOp + widx] = word;
            }
        }
    if (tn == tiles_n - 1 && lane < 16 * BM && m0 + lane < M)
        for (int64_t w = nw; w < ldOp; ++w) Op[(int64_t)(m0 + lane) * ldOp + w] = 0u;
}

}  // namespace

hipError_t launch_dense_f32_sign_pack(const float* X, int64_t ldX, const float* W, int64_t ldW,
                                      int64_t M, int64_t N, int64_t K,
                                      uint32_t* Op, int64_t ldOp, hipStream_t s)
{
    const bool vec = (reinterpret_cast<uintptr_t>(X) & 15u) == 0 && (reinterpret_cast<uintptr_t>(W) & 15u) == 0 &&
                     ldX % 4 == 0 && ldW % 4 == 0;
    if (vec) {                                       // 16-byte rows: the matrix cores
        int bm = 2, bn = 4;
        if (const char* v = getenv("BNN_DENSE_TILE")) {  // tuning override "BM,BN" (16-row / 16-column blocks)
            int a = 0, c = 0;
            if (sscanf(v, "%d,%d", &a, &c) == 2 && (a == 1 || a == 2 || a == 4) && (c == 2 || c == 4)) { bm = a; bn = c; }
        }
        const int tn = (int)((N + 16 * bn - 1) / (16 * bn));
        const int64_t tiles = ((M + 16 * bm - 1) / (16 * bm)) * tn;
        const dim3 g((unsigned)((tiles + kThreads / 64 - 1) / (kThreads / 64))), b(kThreads);
#define BNN_DMF(A, C) hipLaunchKernelGGL((k_dense_f64_mfma_sign_pack<A, C>), g, b, 0, s, X, ldX, W, ldW, \
                                         (int)M, (int)N, (int)K, Op, ldOp, tn, (int)tiles)
        switch (bm * 8 + bn) {
            case 1 * 8 + 2: BNN_DMF(1, 2); break;
            case 1 * 8 + 4: BNN_DMF(1, 4); break;
            case 2 * 8 + 2: BNN_DMF(2, 2); break;
            case 4 * 8 + 2: BNN_DMF(4, 2); break;
            case 4 * 8 + 4: BNN_DMF(4, 4); break;
            default: BNN_DMF(2, 4); break;
        }
#undef BNN_DMF
        return hipGetLastError();
    }
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
    const dim3 grid((unsigned)((M + 3) / 4)), block(kBinactThreads);
    const bool vec = (reinterpret_cast<uintptr_t>(W) & 15u) == 0 && ldW % 4 == 0;
    if (vec) hipLaunchKernelGGL((k_dense_binact_f32<16, true>), grid, block, 0, s, Xp, ldXp, W, ldW,
                                (int)M, (int)N, (int)K, Y, ldY);
    else     hipLaunchKernelGGL((k_dense_binact_f32<16, false>), grid, block, 0, s, Xp, ldXp, W, ldW,
                                (int)M, (int)N, (int)K, Y, ldY);
    return hipGetLastError();
}

}  // namespace bnn
