// Binary weights x fp16 activations on gfx950: the streaming GEMV of a
// BinaryConnect / BWN layer (real activations, +1/-1 weights, one scale per
// output row).
//
// Method (cited by page title and section / equation):
//  - y = alpha * (w_b^T x) with w_b in {-1, +1}: "Extreme Quantization:
//    Binary, Ternary & 1-bit LLMs", "Binary Neural Networks" eq. (1); each
//    weight only adds or subtracts its activation, eq. (2).
//  - bit 0 = +1, bit 1 = -1 along K, as for the XNOR path: "First
//    Principles: Why Binary Ops Can Be Exponentially Faster", section "1.
//    Arithmetic: MAC -> XNOR + popcount".
//  - batch-1 inference is bound by fetching the packed weights: "First
//    Principles", sections "The cost of a neural network step" and
//    "Bandwidth math".
//
// Arithmetic.  A weight word W covers activations x[32w .. 32w+31].  They sit
// in a lane's registers as 16 fp16 pairs, pair p = (x[32w+p], x[32w+p+16]),
// so the two sign bits of pair p are bits p and p+16 of W, and one shift by
// 15-p moves them onto the two fp16 sign bits (15 and 31):
//     flip_p = (W << (15 - p)) & 0x80008000
//     acc    = dot2(pair_p XOR flip_p, (1.0, 1.0), acc)     (v_dot2_f32_f16)
// The products are +-x exactly; only the fp32 additions round.  Activations
// past K are 0, so the weights' pad bits add nothing.
//
// Mapping (as the binary GEMV): G lanes (a power of two covering the row's
// 16-byte weight granules, at most 64) share one weight row, 64/G rows per
// wave step, U row-steps' weight loads in flight before the first is used.
// A lane keeps its granules' 128 activations per granule as 64 pair
// registers for the whole kernel and sums a row in four dot2 chains (one per
// word of a granule, added pairwise at the end); the G partial sums of a
// row meet in a fixed DPP tree and the group's last lane writes y.  The
// deepest term passes through 2 * 16 CPL additions of its chain (a dot2 may
// round twice), 2 of the pairwise sum and GLOG2 <= 6 of the tree: within
// the 128 CPL + 6 the interface states.
#include <stdlib.h>

#include "bnn_device.hpp"
#include "bnn_launch.hpp"

namespace bnn {
namespace {

constexpr int kThreads = 256;
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_pm(uint32_t pair, uint32_t flip, float acc) {
    const uint32_t v = pair ^ flip;
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, v), __builtin_bit_cast(h2, 0x3C003C00u), acc, false);
}

// fp32 sum over each aligned group of 2^GLOG2 lanes, complete in the group's
// last lane (the same DPP steps as the integer group sum; a fixed order).
template <int GLOG2>
__device__ __forceinline__ float fsum_to_last(float v) {
#define BNN_FDPP(CTRL, RM, BC) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, RM, 0xF, BC))
    if (GLOG2 >= 1) BNN_FDPP(0x111, 0xF, true);   // row_shr:1
    if (GLOG2 >= 2) BNN_FDPP(0x112, 0xF, true);   // row_shr:2
    if (GLOG2 >= 3) BNN_FDPP(0x114, 0xF, true);   // row_shr:4
    if (GLOG2 >= 4) BNN_FDPP(0x118, 0xF, true);   // row_shr:8
    if (GLOG2 >= 5) BNN_FDPP(0x142, 0xA, false);  // row_bcast:15 -> rows 1, 3
    if (GLOG2 >= 6) BNN_FDPP(0x143, 0xC, false);  // row_bcast:31 -> rows 2, 3
#undef BNN_FDPP
    return v;
}

// The 16 pairs of activation word w of row x (elements >= K read as 0).
__device__ __forceinline__ void load_pairs(uint32_t (&pr)[16], const uint16_t* __restrict__ x, int w, int K) {
    const int k0 = 32 * w;
    uint32_t d[16];                                // d[q] = (x[k0+2q], x[k0+2q+1])
    if (k0 + 32 <= K) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(x + k0 + 8 * q);
            d[4 * q] = v.x; d[4 * q + 1] = v.y; d[4 * q + 2] = v.z; d[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const uint32_t lo = (k0 + 2 * q < K) ? x[k0 + 2 * q] : 0u;
            const uint32_t hi = (k0 + 2 * q + 1 < K) ? x[k0 + 2 * q + 1] : 0u;
            d[q] = lo | (hi << 16);
        }
    }
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        // lo half: element p (half p&1 of d[p/2]); hi half: element p+16 (of d[8+p/2])
        const uint32_t a = d[p >> 1], b = d[8 + (p >> 1)];
        pr[p] = (p & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
    }
}

template <int GLOG2, int CPL, int U>
__global__ __launch_bounds__(kThreads) void k_bwn_f16_gemv(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ Wp, int64_t ldW, int N, int K,
    const float* __restrict__ alpha, int astr, float* __restrict__ Y)
{
    constexpr int G = 1 << GLOG2;
    constexpr int RPS = 64 / G;                   // rows per wave step
    const int lane = threadIdx.x & 63;
    const int gl = lane & (G - 1);
    const int go = lane >> GLOG2;
    const int Kw = (K + 31) >> 5;
    const int Kw4 = (Kw + 3) >> 2;

    // activation pairs of granules c = gl + G i (words 4c .. 4c+3)
    uint32_t xp[CPL][4][16];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = gl + G * i;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (c < Kw4 && 4 * c + j < Kw) load_pairs(xp[i][j], X, 4 * c + j, K);
            else {
#pragma unroll
                for (int p = 0; p < 16; ++p) xp[i][j][p] = 0u;
            }
        }
    }

    const int64_t nsteps = ((int64_t)N + RPS - 1) / RPS;
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
    for (int64_t s0 = wave * U; s0 < nsteps; s0 += nwaves * U) {
        u32x4 wv[U][CPL];
        float av[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = (s0 + u) * RPS + go;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = gl + G * i;
                wv[u][i] = (u32x4){0u, 0u, 0u, 0u};
                if (row < N && c < Kw4)
                    wv[u][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Wp + row * ldW + 4 * c));
            }
            av[u] = row < N ? alpha[row * astr] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = (s0 + u) * RPS + go;
            // one accumulator per word position: four independent dot2 chains
            float acc4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const uint32_t wj[4] = {wv[u][i].x, wv[u][i].y, wv[u][i].z, wv[u][i].w};
#pragma unroll
                for (int p = 0; p < 16; ++p) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc4[j] = dot2_pm(xp[i][j][p], (wj[j] << (15 - p)) & 0x80008000u, acc4[j]);
                }
            }
            float acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
            acc = fsum_to_last<GLOG2>(acc);
            if (gl == G - 1 && row < N) Y[row] = av[u] * acc;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

}  // namespace

int64_t f16_gemv_max_k() { return 64 * 2 * 128; }

hipError_t launch_bwn_f16_gemv(const uint16_t* X, const uint32_t* Wp, int64_t ldW, int64_t N, int64_t K,
                               const float* alpha, bool alpha_tensor, float* Y, hipStream_t s)
{
    const int64_t kw4 = ((K + 31) / 32 + 3) / 4;
    int glog2 = 0;
    while ((1 << glog2) < kw4 && glog2 < 6) ++glog2;
    const int G = 1 << glog2;
    const int cpl = (int)((kw4 + G - 1) / G);     // 1 or 2 (K <= f16_gemv_max_k())
    const int rps = 64 / G;
    const int64_t steps = (N + rps - 1) / rps;
    const int cus = num_cus();
    const bool unroll = steps >= (int64_t)cus * 4 * 8 * 4;
    const int U = unroll ? (cpl == 1 ? 4 : 2) : 1;
    const int64_t waves = (steps + U - 1) / U;
    int64_t blocks = (waves + 3) / 4;
    const int64_t cap = (int64_t)cus * 64;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    const dim3 grid((unsigned)blocks), block(kThreads);
    const int n = (int)N, k = (int)K, astr = alpha_tensor ? 0 : 1;
#define BNN_F16(GL, C, UU) hipLaunchKernelGGL((k_bwn_f16_gemv<GL, C, UU>), grid, block, 0, s, X, Wp, ldW, n, k, alpha, astr, Y)
#define BNN_F16_U(GL, C) \
    if (U == 4) BNN_F16(GL, C, 4); else if (U == 2) BNN_F16(GL, C, 2); else BNN_F16(GL, C, 1)
#define BNN_F16_G(C) \
    switch (glog2) { case 0: BNN_F16_U(0, C); break; case 1: BNN_F16_U(1, C); break; case 2: BNN_F16_U(2, C); break; \
                     case 3: BNN_F16_U(3, C); break; case 4: BNN_F16_U(4, C); break; case 5: BNN_F16_U(5, C); break; \
                     default: BNN_F16_U(6, C); break; }
    if (cpl == 1) { BNN_F16_G(1) } else { BNN_F16_G(2) }
#undef BNN_F16_G
#undef BNN_F16_U
#undef BNN_F16
    return hipGetLastError();
}

}  // namespace bnn
