// Launcher of the XNOR-popcount GEMM for dense packed rows (binary and ternary
// weights).  The kernel and its design notes are in gemm_kernel.hpp.
#include "gemm_kernel.hpp"

namespace bnn {

hipError_t launch_xnor_gemm(const uint32_t* Xp, int64_t ldX, const uint32_t* Wp, int64_t ldW,
                            int64_t M, int64_t N, int64_t K, const Epilogue& e, hipStream_t s)
{
    const int tn = pick_tile_cols(M, N);
    // Epilogue: D and Y staged through LDS, so that stores cover whole row
    // segments (row-per-lane stores from registers write partial lines:
    // 1.29x the algorithmic bytes at 16384^3, and 9% slower at 8192^3).
    // THRESH_PACK stores its bits from registers.
    const int epi = pick_epilogue(e);
    // Waves per workgroup: all waves of a workgroup read the same TN weight
    // rows through the CU's scalar cache, so bigger workgroups put fewer
    // distinct weight streams on a CU.  Measured on MI355X: 8 waves for
    // 32-wide staged tiles with long rows (8192^3: 749 -> 731 us), 4
    // otherwise (8 waves lose 8% on the 64-wide tiles of 16384^3 and 15% on
    // the 14x14x256 conv GEMM, K = 2304).
    const int64_t kw = (K + 31) / 32;
    int waves = (tn == 32 && epi != EPI_DIRECT && kw > 128) ? 8 : 4;
    if (const char* v = getenv("BNN_GEMM_WAVES")) {       // tuning override: 4, 8 or 16
        const int w = atoi(v);
        if (w == 4 || w == 8 || w == 16) waves = w;
    }
    if (e.flags & W_TERNARY) waves = 4;
    const int64_t row_tiles = (M + waves * 64 - 1) / (waves * 64);
    const int tiles_n = (int)((N + tn - 1) / tn);
    const dim3 grid((unsigned)(row_tiles * tiles_n)), block(waves * 64);
    const int m = (int)M, n = (int)N, k = (int)K;
    // ternary weights: two SGPR planes per word, so 8-word chunks (the same
    // SGPR budget as the binary 16-word chunks) and 4-wave workgroups
#define BNN_GEMM(T, L, WV) hipLaunchKernelGGL((k_xnor_gemm<T, 16, L, WV, false, 0>), grid, block, 0, s, Xp, ldX, Wp, ldW, m, n, k, tiles_n, e, 0, 0)
#define BNN_GEMM_T(T, L) hipLaunchKernelGGL((k_xnor_gemm<T, 8, L, 4, true, 0>), grid, block, 0, s, Xp, ldX, Wp, ldW, m, n, k, tiles_n, e, 0, 0)
#define BNN_GEMM_W(T, L) \
    if (e.flags & W_TERNARY) BNN_GEMM_T(T, L); \
    else switch (waves) { case 8: BNN_GEMM(T, L, 8); break; case 16: BNN_GEMM(T, L, 16); break; default: BNN_GEMM(T, L, 4); break; }
#define BNN_GEMM_E(T) \
    if (epi == EPI_STAGED) { BNN_GEMM_W(T, EPI_STAGED); } else { BNN_GEMM_W(T, EPI_DIRECT); }
    switch (tn) {
        case 64: BNN_GEMM_E(64); break;
        case 32: BNN_GEMM_E(32); break;
        case 16: BNN_GEMM_E(16); break;
        default: BNN_GEMM_E(8); break;
    }
#undef BNN_GEMM_E
#undef BNN_GEMM_T
#undef BNN_GEMM_W
#undef BNN_GEMM
    return hipGetLastError();
}

}  // namespace bnn
