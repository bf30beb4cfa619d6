// Streaming XNOR-popcount GEMV for gfx950 (batch 1 to 4 activation rows).
//
// Method (cited by page title and section / equation):
//  - <w,x> = N - 2 popcount(w_bit xor x_bit), bit 0 = +1, pad bits +1:
//    "First Principles: Why Binary Ops Can Be Exponentially Faster", section
//    "1. Arithmetic: MAC -> XNOR + popcount"; eq. (6) of "Extreme
//    Quantization: Binary, Ternary & 1-bit LLMs".
//  - y = alpha * (w_b^T x): "Extreme Quantization", eq. (1).
//  - batch-1 inference is bound by fetching the packed weights (about MN/8
//    bytes): "First Principles", sections "The cost of a neural network
//    step" and "Bandwidth math".
//
// Design: G lanes (the smallest power of two covering a weight row's 16-byte
// granules, at most 64) share one row, 64/G rows per wave step.  The U
// row-steps of a wave issue all their loads (nontemporal 16-byte weight
// granules, alpha, residual) before any is consumed; each row's popcount is
// summed over its G lanes with DPP row shifts and row broadcasts (no LDS) and
// the last lane of the group writes the epilogue.  HBM streaming of the
// packed weights dominates.
#include <stdlib.h>

#include "bnn_device.hpp"
#include "bnn_launch.hpp"

namespace bnn {
namespace {

constexpr int kThreads = 256;

// Streaming load of one 16-byte weight granule: the weights are read once per
// call, so the load is marked nontemporal and does not displace cached data.
__device__ __forceinline__ u32x4 load_stream(const uint32_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// TERN: ternary weights -- Wp is the sign plane, e.Zp the nonzero plane and
// e.nnz the nonzero count per row; a word contributes popcount((x ^ s) & z)
// (one v_bitop3 + one v_bcnt) and D = nnz - 2 * sum ("Extreme
// Quantization", eq. (7)).
// XEPI: the epilogue may take the per-tensor alpha or a bias (checked at run
// time); without it those branches are compiled out, which keeps the
// binary streaming loop as short as it can be.
template <int MR, int CPL, int U, bool TERN, bool XEPI>
__global__ __launch_bounds__(kThreads) void k_xnor_gemv(
    const uint32_t* __restrict__ Xp, int64_t ldX, const uint32_t* __restrict__ Wp, int64_t ldW,
    int N, int K, int glog2, Epilogue e)
{
    const int lane = threadIdx.x & 63;
    const int G = 1 << glog2;
    const int RPS = 64 >> glog2;                  // rows per wave step
    const int gl = lane & (G - 1);
    const int go = lane >> glog2;
    const int Kw = (K + 31) >> 5;
    const int Kw4 = (Kw + 3) >> 2;
    const bool ragged = (Kw & 3) != 0;

    // activation granules c = gl + G*i, words >= Kw zeroed
    u32x4 xg[MR][CPL];
    u32x4 wm[CPL];                                // word masks (all ones except pad words)
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = gl + G * i;
        wm[i] = (u32x4){0u, 0u, 0u, 0u};
        if (c < Kw4) {
            wm[i].x = (4 * c + 0 < Kw) ? ~0u : 0u;
            wm[i].y = (4 * c + 1 < Kw) ? ~0u : 0u;
            wm[i].z = (4 * c + 2 < Kw) ? ~0u : 0u;
            wm[i].w = (4 * c + 3 < Kw) ? ~0u : 0u;
        }
#pragma unroll
        for (int mr = 0; mr < MR; ++mr) {
            u32x4 v = (u32x4){0u, 0u, 0u, 0u};
            if (c < Kw4) v = *reinterpret_cast<const u32x4*>(Xp + (int64_t)mr * ldX + 4 * c);
            xg[mr][i] = v & wm[i];
        }
    }

    const int64_t nsteps = ((int64_t)N + RPS - 1) / RPS;
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
    const bool last = gl == G - 1;                // the lane that ends with a row's total
    for (int64_t s0 = wave * U; s0 < nsteps; s0 += nwaves * U) {
        u32x4 wv[U][CPL], zv[U][CPL];
        float av[U], bv[U], rv[U][MR];
        int32_t kb[U];
        // all loads of the U row-steps (weights, alpha, residual) go out
        // before the first is consumed
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = (s0 + u) * RPS + go;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = gl + G * i;
                wv[u][i] = (u32x4){0u, 0u, 0u, 0u};
                zv[u][i] = (u32x4){0u, 0u, 0u, 0u};
                if (row < N && c < Kw4) {
                    wv[u][i] = load_stream(Wp + row * ldW + 4 * c);
                    if (TERN) zv[u][i] = load_stream(e.Zp + row * ldW + 4 * c);
                }
            }
            kb[u] = K;
            if (TERN && row < N) kb[u] = e.nnz[row];
            av[u] = 0.0f;
            bv[u] = 0.0f;
            if ((e.flags & EPI_SCALE) && row < N) av[u] = e.alpha[(XEPI && (e.flags & EPI_ALPHA_TENSOR)) ? 0 : row];
            if (XEPI && (e.flags & EPI_BIAS) && row < N) bv[u] = e.bias[row];
#pragma unroll
            for (int mr = 0; mr < MR; ++mr) {
                rv[u][mr] = 0.0f;
                if ((e.flags & EPI_RESIDUAL) && row < N) rv[u][mr] = e.R[(int64_t)mr * e.ldR + row];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = (s0 + u) * RPS + go;
            if (ragged || TERN) {
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    if (TERN) zv[u][i] &= wm[i];
                    else      wv[u][i] &= wm[i];
                }
            }
#pragma unroll
            for (int mr = 0; mr < MR; ++mr) {
                uint32_t pc = 0u;
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    u32x4 t = xg[mr][i] ^ wv[u][i];
                    if (TERN) t &= zv[u][i];
                    pc = popc_acc(t.x, pc);
                    pc = popc_acc(t.y, pc);
                    pc = popc_acc(t.z, pc);
                    pc = popc_acc(t.w, pc);
                }
                pc = sum_reduce_to_last(pc, glog2);
                if (last && row < N) {
                    const int32_t d = kb[u] - 2 * (int32_t)pc;
                    if (e.flags & EPI_DOT) e.D[(int64_t)mr * e.ldD + row] = d;
                    if (e.flags & EPI_SCALE) {
                        float y = av[u] * (float)d;
                        if (XEPI && (e.flags & EPI_BIAS)) y = y + bv[u];
                        if (e.flags & EPI_RESIDUAL) y = y + rv[u][mr];
                        e.Y[(int64_t)mr * e.ldY + row] = y;
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);   // finish row-step u before u+1 (bounded live ranges)
        }
    }
}

}  // namespace

bool gemv_eligible(int64_t M, int64_t K, uint32_t flags) {
    const int64_t kw4 = ((K + 31) / 32 + 3) / 4;
    return M >= 1 && M <= 4 && !(flags & (EPI_THRESH | EPI_SIGN_PACK)) && kw4 <= 64 * 8;
}

hipError_t launch_xnor_gemv(const uint32_t* Xp, int64_t ldX, const uint32_t* Wp, int64_t ldW,
                            int64_t M, int64_t N, int64_t K, const Epilogue& e, hipStream_t s)
{
    // G lanes per weight row: the smallest power of two covering its 16-byte
    // granules (at most 64); CPL granules per lane.  Large calls unroll U
    // row-steps per wave (4 KiB of weight loads in flight per wave at
    // CPL = 1); calls too small to fill the chip keep U = 1 for more waves.
    const int64_t kw4 = ((K + 31) / 32 + 3) / 4;
    int glog2 = 0;
    while ((1 << glog2) < kw4 && glog2 < 6) ++glog2;
    const int G = 1 << glog2;
    const int cpl_needed = (int)((kw4 + G - 1) / G);
    const int cpl = cpl_needed <= 1 ? 1 : cpl_needed <= 2 ? 2 : cpl_needed <= 4 ? 4 : 8;
    // 4 row-steps per wave measured best on MI355X for both decode shapes
    // (K = 4096: 6.65 TB/s at U = 4 vs 6.0 at U = 8, which needs more VGPRs)
    int umax = cpl <= 2 ? 4 : 8 / cpl;
    if (const char* v = getenv("BNN_GEMV_U")) {       // tuning override: 1, 2, 4 or 8 (capped by 8/cpl)
        const int u = atoi(v);
        if (u == 1 || u == 2 || u == 4 || u == 8) umax = u < umax ? u : umax;
    }
    const int rps = 64 / G;
    const int64_t steps = (N + rps - 1) / rps;
    const int cus = num_cus();
    const int64_t full_chip_waves = (int64_t)cus * 4 * 8;
    const bool unroll = umax > 1 && steps >= full_chip_waves * umax;
    const int U = unroll ? umax : 1;
    const int64_t waves = (steps + U - 1) / U;
    int64_t blocks = (waves + 3) / 4;
    const int64_t cap = (int64_t)cus * 64;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    const dim3 grid((unsigned)blocks), block(kThreads);
    const int n = (int)N, k = (int)K;
    const bool xepi = (e.flags & (EPI_BIAS | EPI_ALPHA_TENSOR)) != 0;
#define BNN_GEMV(MR, CPL, UU) \
    if (e.flags & W_TERNARY) hipLaunchKernelGGL((k_xnor_gemv<MR, CPL, UU, true, true>), grid, block, 0, s, Xp, ldX, Wp, ldW, n, k, glog2, e); \
    else if (xepi)           hipLaunchKernelGGL((k_xnor_gemv<MR, CPL, UU, false, true>), grid, block, 0, s, Xp, ldX, Wp, ldW, n, k, glog2, e); \
    else                     hipLaunchKernelGGL((k_xnor_gemv<MR, CPL, UU, false, false>), grid, block, 0, s, Xp, ldX, Wp, ldW, n, k, glog2, e)
#define BNN_GEMV_MR(CPL, UU) \
    switch (M) { case 1: BNN_GEMV(1, CPL, UU); break; case 2: BNN_GEMV(2, CPL, UU); break; \
                 case 3: BNN_GEMV(3, CPL, UU); break; default: BNN_GEMV(4, CPL, UU); break; }
    if (unroll) {
        switch (cpl * 16 + U) {
            case 1 * 16 + 8: BNN_GEMV_MR(1, 8); break;
            case 1 * 16 + 4: BNN_GEMV_MR(1, 4); break;
            case 1 * 16 + 2: BNN_GEMV_MR(1, 2); break;
            case 2 * 16 + 4: BNN_GEMV_MR(2, 4); break;
            case 2 * 16 + 2: BNN_GEMV_MR(2, 2); break;
            default: BNN_GEMV_MR(4, 2); break;
        }
    } else {
        switch (cpl) {
            case 1: BNN_GEMV_MR(1, 1); break;
            case 2: BNN_GEMV_MR(2, 1); break;
            case 4: BNN_GEMV_MR(4, 1); break;
            default: BNN_GEMV_MR(8, 1); break;
        }
    }
#undef BNN_GEMV_MR
#undef BNN_GEMV
    return hipGetLastError();
}

}  // namespace bnn
