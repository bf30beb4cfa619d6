// Ternary weights x binary activations as a GEMM with one weight row per lane.
//
// Method (cited by page title and section / equation):
//  - ternary weights w in {-1, 0, +1} held as a sign plane s (bit 1: -1) and
//    a nonzero plane z: "Extreme Quantization: Binary, Ternary & 1-bit LLMs",
//    "Ternary Quantization" eq. (7) and "BitNet b1.58" eq. (8)-(9).
//  - with binary activations (bit 1: -1; "First Principles: Why Binary Ops
//    Can Be Exponentially Faster", section "1. Arithmetic: MAC -> XNOR +
//    popcount") a product is 0 where z = 0 and -1 where x and s differ, so
//    D[m, n] = nnz[n] - 2 sum_k popcount((x_m ^ s_n) & z_n).
//
// Mapping.  The row-per-lane GEMM puts activation rows on the lanes and
// broadcasts the weight words from SGPRs; with ternary weights both planes
// would then be SGPR operands of one v_bitop3_b32, which takes at most one,
// so every word costs an extra v_mov.  Here the roles are swapped: lane l
// holds weight row n = n0 + l (both planes, in VGPRs, a KC-word chunk at a
// time, the next chunk's loads in flight), the activation words of two rows
// at a time arrive by scalar loads into SGPRs (the next pair's loads issued
// before the current pair is used), and each word of each output costs one
// v_bitop3_b32 (x ^ s) & z with a single SGPR operand and one
// v_bcnt_u32_b32.  A wave owns 64 weight rows x TM activation rows; the 4
// waves of a workgroup take consecutive 64-row slices of 256 weight rows
// and share the activation rows (one scalar-cache stream per workgroup).
// Outputs: for each activation row m the 64 lanes store consecutive n, so
// every store instruction writes a whole 256-byte row segment; the packed
// outputs (THRESH_PACK, SIGN_PACK) are one ballot per row m, its two 32-bit
// words stored by lanes 0 and 1.
#include <stdlib.h>

#include "bnn_device.hpp"
#include "bnn_launch.hpp"

namespace bnn {
namespace {

// Measured on MI355X at 8192^3 (D + Y): 32 rows x 8-word chunks with at most
// 128 VGPRs (4 waves per SIMD) 1.02 ms; 96 VGPRs (5 waves) 1.05 ms; 16 rows
// 1.31-1.34 ms; 16-word chunks (114 VGPRs, no VGPR spill) 1.04 against 0.95
// ms for 8 in the same run; 64 rows spill SGPRs.
constexpr int kTM = 32;      // activation rows per wave
constexpr int kKC = 8;       // words per chunk
constexpr int kMinWaves = 4; // resident waves per SIMD the registers must allow

__device__ __forceinline__ void load_planes(uint32_t* s, uint32_t* z, const uint32_t* __restrict__ srow,
                                            const uint32_t* __restrict__ zrow, int k, int n4)
{
#pragma unroll
    for (int q = 0; q < n4; ++q) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(srow + k + 4 * q);
        const u32x4 b = *reinterpret_cast<const u32x4*>(zrow + k + 4 * q);
        s[4 * q] = a.x; s[4 * q + 1] = a.y; s[4 * q + 2] = a.z; s[4 * q + 3] = a.w;
        z[4 * q] = b.x; z[4 * q + 1] = b.y; z[4 * q + 2] = b.z; z[4 * q + 3] = b.w;
    }
}

// c0 += popcount((u[i] ^ s[i]) & z[i]), c1 += popcount((v[i] ^ s[i]) & z[i])
// over NW words (u, v: two activation rows' words, uniform, in SGPRs; s, z:
// this lane's weight planes).  v_bitop3_b32 takes the truth table of its
// three sources (index src0 * 4 + src1 * 2 + src2); (src0 ^ src2) & src1 is
// 0x48.  One s_nop 0 separates each bitop3 from the bit count that reads it
// (back to back, the bit count issues markedly slower).
#define BNN_BP(X, Z, S, C) "v_bitop3_b32 %[t], " X ", " Z ", " S " bitop3:0x48\n\ts_nop 0\n\t" \
                           "v_bcnt_u32_b32 " C ", %[t], " C "\n\t"
#define BNN_BP2(I) BNN_BP("%[u" #I "]", "%[z" #I "]", "%[s" #I "]", "%[c0]") \
                   BNN_BP("%[v" #I "]", "%[z" #I "]", "%[s" #I "]", "%[c1]")
#define BNN_BIN(I) [u##I] "s"(u[I]), [v##I] "s"(v[I]), [s##I] "v"(s[I]), [z##I] "v"(z[I])
template <int NW>
__device__ __forceinline__ void tern_popc_2rows(uint32_t& c0, uint32_t& c1, const uint32_t* u, const uint32_t* v,
                                                const uint32_t* s, const uint32_t* z)
{
    uint32_t t;
    if constexpr (NW == 8) {
        asm(BNN_BP2(0) BNN_BP2(1) BNN_BP2(2) BNN_BP2(3) BNN_BP2(4) BNN_BP2(5) BNN_BP2(6) BNN_BP2(7)
            : [c0] "+v"(c0), [c1] "+v"(c1), [t] "=&v"(t)
            : BNN_BIN(0), BNN_BIN(1), BNN_BIN(2), BNN_BIN(3), BNN_BIN(4), BNN_BIN(5), BNN_BIN(6), BNN_BIN(7));
    } else {
        static_assert(NW == 4, "blocks of 8 or 4 words");
        asm(BNN_BP2(0) BNN_BP2(1) BNN_BP2(2) BNN_BP2(3)
            : [c0] "+v"(c0), [c1] "+v"(c1), [t] "=&v"(t)
            : BNN_BIN(0), BNN_BIN(1), BNN_BIN(2), BNN_BIN(3));
    }
}
#undef BNN_BIN
#undef BNN_BP2
#undef BNN_BP

// One chunk of KCC words for all TM activation rows: the words of rows
// (j, j + 1) are scalar loads into one of two SGPR sets, the next pair's
// issued (and pinned there by a scheduling barrier) before the current
// pair's VALU work.  Rows past the last (FULLM false) re-read it.
template <int KCC, bool FULLM>
__device__ __forceinline__ void tern_chunk(uint32_t (&acc)[kTM], const uint32_t (&s)[KCC], const uint32_t (&z)[KCC],
                                           const uint32_t* __restrict__ xbase, int64_t ldX, int k0, int mlast)
{
    int64_t ldx = ldX;
    asm volatile("" : "+s"(ldx));   // keep the row offsets out of the loop preheader
    // full tiles walk the rows with one running pointer (two 64-bit adds per
    // pair, not a multiply per row); a partial tile clamps each row
    cptr_u32 pr = (cptr_u32)(xbase + k0);
    auto load_x = [&](uint32_t (&u)[2][KCC], int j) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const cptr_u32 p = FULLM ? pr + c * ldx : (cptr_u32)(xbase + (int64_t)min(j + c, mlast) * ldx + k0);
#pragma unroll
            for (int kk = 0; kk < KCC; ++kk) u[c][kk] = p[kk];
        }
        if (FULLM) pr += 2 * ldx;
    };
    uint32_t xc[2][KCC];
    load_x(xc, 0);
#pragma unroll
    for (int j = 0; j < kTM; j += 2) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int kk = 0; kk < KCC; ++kk) asm volatile("" : : "s"(xc[c][kk]));
        uint32_t xn[2][KCC];
        if (j + 2 < kTM) load_x(xn, j + 2);
        __builtin_amdgcn_sched_barrier(0);
        constexpr int NB = KCC % 8 == 0 ? 8 : 4;
#pragma unroll
        for (int k = 0; k < KCC; k += NB)
            tern_popc_2rows<NB>(acc[j], acc[j + 1], &xc[0][k], &xc[1][k], &s[k], &z[k]);
        if (j + 2 < kTM) {
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int kk = 0; kk < KCC; ++kk) xc[c][kk] = xn[c][kk];
        }
    }
}

template <bool FULLM>
__device__ __forceinline__ void tern_mainloop(uint32_t (&acc)[kTM], const uint32_t* __restrict__ xbase, int64_t ldX,
                                              const uint32_t* __restrict__ srow, const uint32_t* __restrict__ zrow,
                                              int Kw, int mlast)
{
    constexpr int KC = kKC;
    const int kfull = (Kw / KC) * KC;
    // weight chunks double-buffered, two per iteration with the roles swapped
    uint32_t s0[KC], z0[KC], s1[KC], z1[KC];
    if (kfull > 0) load_planes(s0, z0, srow, zrow, 0, KC / 4);
    int k0 = 0;
    for (; k0 + 2 * KC <= kfull; k0 += 2 * KC) {
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) asm volatile("" : : "v"(s0[kk]), "v"(z0[kk]));
        load_planes(s1, z1, srow, zrow, k0 + KC, KC / 4);
        tern_chunk<KC, FULLM>(acc, s0, z0, xbase, ldX, k0, mlast);
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) asm volatile("" : : "v"(s1[kk]), "v"(z1[kk]));
        if (k0 + 2 * KC < kfull) load_planes(s0, z0, srow, zrow, k0 + 2 * KC, KC / 4);
        tern_chunk<KC, FULLM>(acc, s1, z1, xbase, ldX, k0 + KC, mlast);
    }
    if (k0 < kfull) {                             // an odd last chunk, already in s0 / z0
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) asm volatile("" : : "v"(s0[kk]), "v"(z0[kk]));
        tern_chunk<KC, FULLM>(acc, s0, z0, xbase, ldX, k0, mlast);
    }
    // tail: 16-byte granules (rows hold ld >= roundup(Kw, 4) words); words at
    // or past Kw get a zero nonzero-plane word, so they add nothing
    for (int kt = kfull; kt < Kw; kt += 4) {
        uint32_t s[4], z[4];
        load_planes(s, z, srow, zrow, kt, 1);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) z[kk] = (kt + kk < Kw) ? z[kk] : 0u;
        tern_chunk<4, FULLM>(acc, s, z, xbase, ldX, kt, mlast);
    }
}

__global__ __launch_bounds__(256, kMinWaves) void k_tern_gemm_t(
    const uint32_t* __restrict__ Xp, int64_t ldX, const uint32_t* __restrict__ Sp, const uint32_t* __restrict__ Zp,
    int64_t ldW, int M, int N, int K, int tiles_n, Epilogue e)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int tn = blockIdx.x % tiles_n, tm = blockIdx.x / tiles_n;
    const int n0 = tn * 256 + wave * 64;
    if (n0 >= N) return;                          // whole wave past the last weight row
    const int m0 = tm * kTM;
    const int n = n0 + lane;
    const bool live = n < N;
    const int nc = min(n, N - 1);
    const int Kw = (K + 31) >> 5;
    const int mlast = M - 1 - m0;                 // last live row of this tile
    const uint32_t* __restrict__ xbase = Xp + (int64_t)m0 * ldX;

    uint32_t acc[kTM];
#pragma unroll
    for (int j = 0; j < kTM; ++j) acc[j] = 0u;
    if (m0 + kTM <= M) tern_mainloop<true>(acc, xbase, ldX, Sp + (int64_t)nc * ldW, Zp + (int64_t)nc * ldW, Kw, mlast);
    else               tern_mainloop<false>(acc, xbase, ldX, Sp + (int64_t)nc * ldW, Zp + (int64_t)nc * ldW, Kw, mlast);

    // epilogue: this lane's channel constants, then one output row at a time
    const uint32_t f = e.flags;
    const int32_t nnzv = e.nnz[nc];
    const float al = (f & EPI_SCALE) ? e.alpha[(f & EPI_ALPHA_TENSOR) ? 0 : nc] : 0.0f;
    const float bi = (f & EPI_BIAS) ? e.bias[nc] : 0.0f;
    const float bt = ((f & EPI_SIGN_PACK) && e.beta) ? e.beta[nc] : 0.0f;
    const float tau = (f & EPI_THRESH) ? e.tau[nc] : 0.0f;
    const int dir = (f & EPI_THRESH) ? (int)e.dir[nc] : 0;
    const bool packed = (f & (EPI_THRESH | EPI_SIGN_PACK)) != 0;
    const int wi = (n0 >> 5) + (lane & 1);        // the packed word of lanes 0 and 1
    const bool owrite = packed && lane < 2 && wi < e.ldOp;
    const bool lastw = n0 + 64 >= N;              // this wave holds the row's last channel
#pragma unroll
    for (int j = 0; j < kTM; ++j) {
        const int m = m0 + j;
        if (m >= M) break;
        const int32_t d = nnzv - 2 * (int32_t)acc[j];
        uint32_t vote = 0u;
        if ((f & EPI_DOT) && live) e.D[(int64_t)m * e.ldD + n] = d;
        if (f & EPI_SCALE) {
            float y = al * (float)d;
            if (f & EPI_BIAS) y = y + bi;
            if (f & EPI_RESIDUAL) y = y + e.R[(int64_t)m * e.ldR + nc];
            if (live) e.Y[(int64_t)m * e.ldY + n] = y;
            if (f & EPI_SIGN_PACK) vote = (live && !(y >= bt)) ? 1u : 0u;
        }
        if (f & EPI_THRESH) {
            const float v = (float)(dir * d);
            vote = (live && !(v >= tau)) ? 1u : 0u;
        }
        if (packed) {
            const uint64_t bits = __ballot(vote);
            uint32_t* orow = e.Op + (int64_t)m * e.ldOp;
            if (owrite) orow[wi] = (uint32_t)(bits >> (32 * (lane & 1)));
            if (lastw)                             // the row's pad words
                for (int w = (n0 >> 5) + 2 + lane; w < e.ldOp; w += 64) orow[w] = 0u;
        }
    }
}

}  // namespace

bool tern_gemm_t_eligible() {
    const char* v = getenv("BNN_TERN_KERNEL");        // tuning override: "rows" = row-per-lane kernel
    return !(v && v[0] == 'r');
}

hipError_t launch_tern_gemm_t(const uint32_t* Xp, int64_t ldX, const uint32_t* Sp, int64_t ldW,
                              int64_t M, int64_t N, int64_t K, const Epilogue& e, hipStream_t s)
{
    const int64_t tiles_n = (N + 255) / 256, tiles_m = (M + kTM - 1) / kTM;
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(256);
    hipLaunchKernelGGL(k_tern_gemm_t, grid, block, 0, s, Xp, ldX, Sp, e.Zp, ldW, (int)M, (int)N, (int)K,
                       (int)tiles_n, e);
    return hipGetLastError();
}

}  // namespace bnn
