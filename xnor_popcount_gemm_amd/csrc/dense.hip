// Floating-point first and last layers around the binary layers (gfx950).
//
// Page "Perfected Concept", table "What is binary vs not": first/last layers
// stay in higher precision; the first layer's output is binarized for the
// next binary layer (eq. (4) of "Extreme Quantization: Binary, Ternary &
// 1-bit LLMs", sign per its Notation), and the last layer reads the +1/-1
// outputs of the last binary layer.
//
// First layer: 64x64 output tile per 256-thread workgroup, 4x4 per thread,
// K staged through LDS in 16-wide slices already widened to double.  Every
// product of two floats is exact in double and each output accumulates its
// K products in index order with one rounding per step (an FMA of an exact
// product equals a rounded add), so the sign decision sees the same double
// sum as a plain sequential loop.  The signs of each row's 32-column groups
// are folded into packed words with DPP row shifts, as in the pack kernels.
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

__global__ __launch_bounds__(kThreads) void k_dense_f32_sign_pack(
    const float* __restrict__ X, int64_t ldX, const float* __restrict__ W, int64_t ldW,
    int M, int N, int K, uint32_t* __restrict__ Op, int64_t ldOp, int tiles_n)
{
    __shared__ double xs[kSlice][kTile];
    __shared__ double ws[kSlice][kTile];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int tn = blockIdx.x % tiles_n, tm = blockIdx.x / tiles_n;
    const int m0 = tm * kTile, n0 = tn * kTile;
    // staging map: thread -> (tile row, 4 consecutive k)
    const int sr = tid >> 2, sk = (tid & 3) * 4;

    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;

    for (int k0 = 0; k0 < K; k0 += kSlice) {
        {
            const int gm = m0 + sr, gn = n0 + sr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k = k0 + sk + i;
                xs[sk + i][sr] = (gm < M && k < K) ? (double)X[(int64_t)gm * ldX + k] : 0.0;
                ws[sk + i][sr] = (gn < N && k < K) ? (double)W[(int64_t)gn * ldW + k] : 0.0;
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kSlice; ++kk) {
            double a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = xs[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = ws[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fma(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }

    // Padded k (k >= K) contributed exact zeros, so each acc is the in-order
    // double sum over k < K.  Columns >= N hold 0.0 -> bit 0 (+1), the pad rule.
    const int nw = (N + 31) >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t nib = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) nib |= (acc[i][j] >= 0.0 ? 0u : 1u) << j;
        const uint32_t word = or_reduce8_to_last(nib << (4 * (tx & 7)));
        const int m = m0 + ty * 4 + i;
        const int widx = (n0 >> 5) + (tx >> 3);
        if ((tx & 7) == 7 && m < M && widx < nw) Op[(int64_t)m * ldOp + widx] = word;
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
    const int tiles_n = (int)((N + kTile - 1) / kTile);
    const int64_t tiles_m = (M + kTile - 1) / kTile;
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(kThreads);
    hipLaunchKernelGGL(k_dense_f32_sign_pack, grid, block, 0, s, X, ldX, W, ldW,
                       (int)M, (int)N, (int)K, Op, ldOp, tiles_n);
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
