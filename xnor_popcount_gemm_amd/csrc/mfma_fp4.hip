// The XNOR-popcount GEMM on the fp4 matrix cores of gfx950: the +-1 dot
// product evaluated exactly as a dense contraction of FP4 (e2m1) values.
//
// Method (cited by page title and section / equation):
//  - <w,x> = sum_k s(w_k) s(x_k) with s = +1 for bit 0 and -1 for bit 1; the
//    XNOR-popcount form N - 2 popcount(w xor x) is the same integer: "First
//    Principles: Why Binary Ops Can Be Exponentially Faster", section "1.
//    Arithmetic: MAC -> XNOR + popcount"; "Extreme Quantization: Binary,
//    Ternary & 1-bit LLMs", eq. (6).
//  - y = alpha * (w_b^T x): "Extreme Quantization", eq. (1).
//
// Exactness.  +1 and -1 are e2m1 codes 0x2 and 0xA, so every product is +-1
// exactly; a 16x16x128 step adds 128 of them (an integer of magnitude <= 128)
// to an fp32 accumulator, and every partial sum is an integer below 2^24
// (K <= 2^24), so the accumulated value is the exact dot product.  Positions
// past K hold +1 on both sides (pad bits and pad words are 0 in the packed
// layout, and words past the row's last data word are replaced by 0 here),
// each adding exactly 1: D = S - (positions processed - K).
//
// Operand expansion.  One packed word holds 32 signs; a lane's share of a
// 16x16x128 operand is 32 fp4 values (4 dwords).  Nibble i of dword q takes
// bit 4i + q of the word:  dword_q = ((w << (3 - q)) & 0x88888888) | 0x22222222
// (7 VALU ops per word: three shifts and four and-ors).  The element order
// this gives is a fixed permutation
// of the word's bits; both operands use the same one, and lane group g (lanes
// 16g .. 16g+15) of both operands takes the same word, so every product
// pairs equal k.
//
// Tiling: a workgroup of 2 x 2 waves; each wave owns RB x CB blocks of 16 x 16
// outputs (4 fp32 accumulators per block and lane), 8 x 4 by default (a 256 x
// 128 workgroup tile).  Per K step of 16 words the workgroup loads its
// activation and weight rows once (64 bytes of a row per 4 threads) into LDS
// (row stride 20 words: 16-byte reads without bank conflicts), double
// buffered, one barrier per step; each wave reads its granules, expands them
// (7 VALU ops per word and fragment, so (RB + CB) / (RB CB) expansions per
// MFMA) and runs 4 RB CB MFMAs.
#include <stdlib.h>

#include "bnn_device.hpp"
#include "bnn_launch.hpp"

namespace bnn {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

// sgn = 0x88888888 and one = 0x22222222 are passed in registers (one VGPR
// each): with both as literals the compiler splits every and-or into a
// v_and and a v_or (VOP2 literals), 11 VALU ops per word instead of 7.
__device__ __forceinline__ i32x8 expand_fp4(uint32_t w, uint32_t sgn, uint32_t one) {
    i32x8 r;
    r[0] = (int)(((w << 3) & sgn) | one);
    r[1] = (int)(((w << 2) & sgn) | one);
    r[2] = (int)(((w << 1) & sgn) | one);
    r[3] = (int)((w & sgn) | one);
    r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;     // unused by the fp4 form
    return r;
}

__device__ __forceinline__ uint32_t word_of(const u32x4& g, int s) {
    return s == 0 ? g.x : s == 1 ? g.y : s == 2 ? g.z : g.w;
}

// A 16-byte granule of packed words w .. w+3 of a row, words >= Kw read as 0.
__device__ __forceinline__ u32x4 granule(const uint32_t* __restrict__ row, int w, int Kw) {
    u32x4 v = (u32x4){0u, 0u, 0u, 0u};
    if (w < Kw) v = *reinterpret_cast<const u32x4*>(row + w);
    if (w + 4 > Kw) {
        if (w + 1 >= Kw) v.y = 0u;
        if (w + 2 >= Kw) v.z = 0u;
        if (w + 3 >= Kw) v.w = 0u;
    }
    return v;
}

constexpr int WM = 2, WN = 2;                         // waves per workgroup
constexpr int NT = WM * WN * 64;
constexpr int RS = 20;                                // LDS row stride in words

// RB x CB MFMA blocks of 16 x 16 per wave; MINW resident waves per SIMD.
template <int RB, int CB, int MINW>
__global__ __launch_bounds__(NT, MINW) void k_xnor_gemm_fp4(
    const uint32_t* __restrict__ Xp, int64_t ldX, const uint32_t* __restrict__ Wp, int64_t ldW,
    int M, int N, int K, int tiles_n, int32_t* __restrict__ D, int64_t ldD,
    const float* __restrict__ alpha, int astr, float* __restrict__ Y, int64_t ldY)
{
    constexpr int TM = WM * RB * 16, TNC = WN * CB * 16;  // workgroup tile
    constexpr int GA = TM * 4 / NT, GB = TNC * 4 / NT;    // 16-byte granules per thread and step
    __shared__ uint32_t sa[2][TM * RS];
    __shared__ uint32_t sb[2][TNC * RS];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int tn = blockIdx.x % tiles_n, tm = blockIdx.x / tiles_n;
    const int mrow0 = tm * TM, ncol0 = tn * TNC;
    const int i = lane & 15, g = lane >> 4;
    const int Kw = (K + 31) >> 5;
    const int nsteps = (Kw + 15) >> 4;

    // this thread's granules of a step: index j = tid + NT u -> strip row j / 4, quarter j % 4
    const uint32_t* gpa[GA];
    const uint32_t* gpb[GB];
    int la[GA], lb[GB], qa[GA], qb[GB];
#pragma unroll
    for (int u = 0; u < GA; ++u) {
        const int j = tid + NT * u, row = j >> 2;
        qa[u] = j & 3;
        gpa[u] = Xp + (int64_t)min(mrow0 + row, M - 1) * ldX;    // rows past M: results not stored
        la[u] = row * RS + 4 * qa[u];
    }
#pragma unroll
    for (int u = 0; u < GB; ++u) {
        const int j = tid + NT * u, row = j >> 2;
        qb[u] = j & 3;
        gpb[u] = Wp + (int64_t)min(ncol0 + row, N - 1) * ldW;
        lb[u] = row * RS + 4 * qb[u];
    }
    u32x4 ra[GA], rb[GB];
    // a step whose 16 words all lie inside the rows (every step but a last,
    // partial one; a uniform test) loads without the per-granule guards, so
    // the loop carries no exec-masked branches
    auto gload = [&](int t) {
        if (16 * t + 16 <= Kw) {
#pragma unroll
            for (int u = 0; u < GA; ++u) ra[u] = *reinterpret_cast<const u32x4*>(gpa[u] + 16 * t + 4 * qa[u]);
#pragma unroll
            for (int u = 0; u < GB; ++u) rb[u] = *reinterpret_cast<const u32x4*>(gpb[u] + 16 * t + 4 * qb[u]);
        } else {
#pragma unroll
            for (int u = 0; u < GA; ++u) ra[u] = granule(gpa[u], 16 * t + 4 * qa[u], Kw);
#pragma unroll
            for (int u = 0; u < GB; ++u) rb[u] = granule(gpb[u], 16 * t + 4 * qb[u], Kw);
        }
    };
    auto swrite = [&](int b) {
#pragma unroll
        for (int u = 0; u < GA; ++u) *reinterpret_cast<u32x4*>(&sa[b][la[u]]) = ra[u];
#pragma unroll
        for (int u = 0; u < GB; ++u) *reinterpret_cast<u32x4*>(&sb[b][lb[u]]) = rb[u];
    };

    f32x4v acc[RB][CB];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int c = 0; c < CB; ++c) acc[r][c] = (f32x4v){0.f, 0.f, 0.f, 0.f};

    uint32_t sgn = 0x88888888u, one = 0x22222222u;
    asm volatile("" : "+v"(sgn), "+v"(one));
    gload(0);
    swrite(0);
    __syncthreads();
    for (int t = 0; t < nsteps; ++t) {
        const int b = t & 1;
        if (t + 1 < nsteps) gload(t + 1);          // in flight during this step's MFMAs
        u32x4 ga[RB], gb[CB];
#pragma unroll
        for (int r = 0; r < RB; ++r)
            ga[r] = *reinterpret_cast<const u32x4*>(&sa[b][(wm * RB * 16 + 16 * r + i) * RS + 4 * g]);
#pragma unroll
        for (int c = 0; c < CB; ++c)
            gb[c] = *reinterpret_cast<const u32x4*>(&sb[b][(wn * CB * 16 + 16 * c + i) * RS + 4 * g]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {                // word 4g + s of the step for lane group g
            i32x8 fb[CB];
#pragma unroll
            for (int c = 0; c < CB; ++c) fb[c] = expand_fp4(word_of(gb[c], s), sgn, one);
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const i32x8 fa = expand_fp4(word_of(ga[r], s), sgn, one);
#pragma unroll
                for (int c = 0; c < CB; ++c)
                    // fp4 (e2m1) for both operands, unit scales (E8M0 127 = 2^0)
                    acc[r][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, fb[c], acc[r][c], 4, 4,
                                                                                   0, 127, 0, 127);
            }
        }
        if (t + 1 < nsteps) swrite(b ^ 1);
        __syncthreads();
    }

    // accumulator element v of block (r, c): row 16 r + 4 g + v, column 16 c + i of the wave's tile
    const int corr = nsteps * 512 - K;
    const int row0 = mrow0 + wm * RB * 16, col0 = ncol0 + wn * CB * 16;
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            const int col = col0 + 16 * c + i;
            const float a = (Y && col < N) ? alpha[col * astr] : 0.0f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = row0 + 16 * r + 4 * g + v;
                if (row < M && col < N) {
                    const int32_t d = (int32_t)acc[r][c][v] - corr;
                    if (D) D[(int64_t)row * ldD + col] = d;
                    if (Y) Y[(int64_t)row * ldY + col] = a * (float)d;
                }
            }
        }
}

}  // namespace

hipError_t launch_xnor_gemm_fp4(const uint32_t* Xp, int64_t ldX, const uint32_t* Wp, int64_t ldW,
                                int64_t M, int64_t N, int64_t K, int32_t* D, int64_t ldD,
                                const float* alpha, bool alpha_tensor, float* Y, int64_t ldY, hipStream_t s)
{
    // 8 x 4 blocks per wave (a 256 x 128 workgroup tile, 2 waves per SIMD):
    // measured on MI355X 2.23 ms at 16384^3 against 2.31 for 4 x 4, 2.74
    // for 4 x 8 and 4.88 for 8 x 8 (1 wave per SIMD, spills)
    int rb = 8, cb = 4;
    if (const char* v = getenv("BNN_MFMA_TILE")) {   // tuning override: "4x4", "8x4", "4x8" or "8x8"
        rb = v[0] == '8' ? 8 : 4;
        cb = (v[0] && v[1] == 'x' && v[2] == '8') ? 8 : 4;
    }
    const int64_t TM = WM * rb * 16, TNC = WN * cb * 16;
    const int64_t tiles_m = (M + TM - 1) / TM, tiles_n = (N + TNC - 1) / TNC;
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(NT);
    const int m = (int)M, n = (int)N, k = (int)K, tn = (int)tiles_n, astr = alpha_tensor ? 0 : 1;
#define BNN_FP4(R, C, W) hipLaunchKernelGGL((k_xnor_gemm_fp4<R, C, W>), grid, block, 0, s, Xp, ldX, Wp, ldW, m, n, k, tn, \
                                            D, ldD, alpha, astr, Y, ldY)
    if (rb == 8 && cb == 8) BNN_FP4(8, 8, 1);
    else if (rb == 8) BNN_FP4(8, 4, 2);
    else if (cb == 8) BNN_FP4(4, 8, 2);
    else BNN_FP4(4, 4, 2);
#undef BNN_FP4
    return hipGetLastError();
}

}  // namespace bnn
