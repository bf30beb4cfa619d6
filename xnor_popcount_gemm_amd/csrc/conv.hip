// Launcher of the implicit-im2col binary 3x3 convolution (the XNOR-popcount
// GEMM kernel of gemm_kernel.hpp reading its activation rows from a packed
// NHWC image).
#include "gemm_kernel.hpp"

namespace bnn {

hipError_t launch_xnor_conv3x3(const uint32_t* Xp, int64_t ldX, const uint32_t* Wp, int64_t ldW,
                               int64_t M, int64_t N, int64_t H, int64_t W, int cw,
                               const Epilogue& e, hipStream_t s)
{
    // the same column-tile choice and epilogue rule as the dense GEMM
    const int tn = pick_tile_cols(M, N);
    const int64_t kw = 9 * (int64_t)cw;
    const int epi = pick_epilogue(e);
    // The residual tile is touched once the last K chunk has arrived, so it
    // streams in during that chunk's VALU work (staged epilogue only;
    // measured on MI355X: 94.5 -> 89.3 us on the 56x56x64 block's GEMM,
    // within noise on 14x14x256).
    Epilogue ec = e;
    const char* pfv = getenv("BNN_CONV_PREFETCH");          // tuning override: "0" turns it off
    if (epi != EPI_DIRECT && (e.flags & EPI_RESIDUAL) && !(pfv && pfv[0] == '0')) ec.flags |= EPI_PREFETCH_R;
    const int64_t row_tiles = (M + 255) / 256;
    const int tiles_n = (int)((N + tn - 1) / tn);
    const dim3 grid((unsigned)(row_tiles * tiles_n)), block(256);
    const int m = (int)M, n = (int)N, k = (int)(32 * kw), h = (int)H, w = (int)W;
#define BNN_CONV(T, L, C) hipLaunchKernelGGL((k_xnor_gemm<T, 16, L, 4, false, C>), grid, block, 0, s, Xp, ldX, Wp, ldW, m, n, k, tiles_n, ec, h, w)
#define BNN_CONV_C(T, L) switch (cw) { case 2: BNN_CONV(T, L, 2); break; case 4: BNN_CONV(T, L, 4); break; \
                                       case 8: BNN_CONV(T, L, 8); break; default: BNN_CONV(T, L, 16); break; }
#define BNN_CONV_T(L) switch (tn) { case 64: BNN_CONV_C(64, L); break; case 32: BNN_CONV_C(32, L); break; \
                                    case 16: BNN_CONV_C(16, L); break; default: BNN_CONV_C(8, L); break; }
    if (epi == EPI_STAGED) { BNN_CONV_T(EPI_STAGED) } else { BNN_CONV_T(EPI_DIRECT) }
#undef BNN_CONV_T
#undef BNN_CONV_C
#undef BNN_CONV
    return hipGetLastError();
}

}  // namespace bnn
