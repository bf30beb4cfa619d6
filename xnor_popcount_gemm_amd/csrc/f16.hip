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
// Two kernels compute S = sum_k s_k x_k (s_k = +1 for bit 0, -1 for bit 1)
// with exact products and fp32 additions in a fixed order; Y = fl32(alpha S).
//
// Table kernel (the default, every K).  The signs of 4 consecutive
// activations are one nibble of a weight word, so S is a sum of one of 16
// signed sums per nibble.  A workgroup writes all 16 sums of every group of
// 4 activations into LDS (512 bytes per weight word), then streams weight
// rows: per nibble one SDWA op (the nibble into the LDS address), one LDS
// read and one fp32 add -- 16 VALU ops and 8 LDS reads per weight word.  The entries
// of one table sit in one bank and the lanes of a read use distinct banks,
// so a read costs what a conflict-free one does.  Rows longer than 8192 run
// as passes over 8192-wide K pieces (the tables of a piece fill 128 KiB).
//
// Register kernel (BNN_F16_KERNEL=regs).  A weight word W covers
// activations x[32w .. 32w+31].  They sit in a lane's registers as 16 fp16
// pairs, pair p = (x[32w+p], x[32w+p+16]), so the two sign bits of pair p
// are bits p and p+16 of W, and one shift by 15-p moves them onto the two
// fp16 sign bits (15 and 31):
//     flip_p = (W << (15 - p)) & 0x80008000
//     acc    = dot2(pair_p XOR flip_p, (1.0, 1.0), acc)     (v_dot2_f32_f16)
// 47 VALU ops per weight word.
//
// In both, activations past K are 0, so the weights' pad bits add nothing.
//
// Mapping (as the binary GEMV): G lanes (a power of two covering the row's
// 16-byte weight granules, at most 64) share one weight row, 64/G rows per
// wave step, U row-steps' weight loads in flight before the first is used.
// The register kernel keeps a lane's 128 activations per granule as 64 pair
// registers and sums a row in four dot2 chains (one per word of a granule,
// added pairwise at the end); the G partial sums of a row meet in a fixed
// DPP tree and the group's last lane writes y.  The deepest term passes
// through 2 * 16 CPL additions of its chain (a dot2 may round twice), 2 of
// the pairwise sum and GLOG2 <= 6 of the tree: within the 128 CPL + 6 the
// interface states.  The table kernel's depth is smaller (see
// k_bwn_f16_lut).
#include <stdlib.h>

#include <algorithm>

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

// ---------------------------------------------------------------------------
// Table variant.  Each weight nibble (4 consecutive bits of a word, i.e. the
// signs of 4 consecutive activations) selects one of 16 signed sums of those
// activations; a workgroup computes all of them once into LDS and then each
// nibble of each weight row costs one address op, one LDS read and one fp32
// add instead of 4 sign flips and 2 dot2 halves.
//   entry(w, i, nib) = ((s0 x0 + s1 x1) + s2 x2) + s3 x3,  x_q = x[32w+4i+q],
//   s_q = -1 if bit q of nib is set, else +1 (activations past K are 0).
// Layout (byte address of an entry):
//   h 65536 + (g / 2) 4096 + nib 256 + (g % 2) 128 + s 4
// for word j of 16-byte granule c (w = 4c + j), nibble i, g = 8 j + i; with
// >= 32 lanes per row s = c % 32 and h = c / 32, with fewer (row copies)
// s = (row group * G) % 32 + c and h = 0, the tables stored once per copy.
//  - The 16 entries of one table sit in one bank (s), and the lanes of a read
//    use distinct banks but for pairs: any nibbles cost a conflict-free read.
//  - A lane's address register holds h, nib and s; g is the read's immediate
//    offset, so per nibble one SDWA op writes the nibble into byte 1 of the
//    register (the other bytes stay): an and with 15 of byte k of the weight
//    word for nibble 2k, a shift right by 4 of it for nibble 2k + 1.
// A lane sums 4 chains (one per word of its granule), each adding the 8
// entries of its word in nibble order: a term passes through at most 3 (its
// entry) + 8 (its chain) + 2 (the pairwise sum) + GLOG2 <= 6 (the lane
// tree) rounded additions, plus one per later K piece (at most 3), i.e. at
// most 22 -- below the 128 ceil(ceil(K/128) / G) + 6 >= 134 of the
// register variant, which the interface states.
// A long row runs in passes over K pieces (mode: 0 single pass, Y = alpha S;
// 1 first pass, Y = S; 3 middle pass, Y = Y + S; 2 last pass,
// Y = alpha (Y + S)), X and Wp then pointing at the piece.
#define BNN_NIB_LO(K) "v_and_b32_sdwa %0, 15, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:BYTE_" #K
#define BNN_NIB_HI(K) "v_lshrrev_b32_sdwa %0, 4, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:BYTE_" #K
template <int I>
__device__ __forceinline__ void nib_to_byte1(uint32_t& a, uint32_t w) {
    if constexpr (I == 0) asm(BNN_NIB_LO(0) : "+v"(a) : "v"(w));
    else if constexpr (I == 1) asm(BNN_NIB_HI(0) : "+v"(a) : "v"(w));
    else if constexpr (I == 2) asm(BNN_NIB_LO(1) : "+v"(a) : "v"(w));
    else if constexpr (I == 3) asm(BNN_NIB_HI(1) : "+v"(a) : "v"(w));
    else if constexpr (I == 4) asm(BNN_NIB_LO(2) : "+v"(a) : "v"(w));
    else if constexpr (I == 5) asm(BNN_NIB_HI(2) : "+v"(a) : "v"(w));
    else if constexpr (I == 6) asm(BNN_NIB_LO(3) : "+v"(a) : "v"(w));
    else asm(BNN_NIB_HI(3) : "+v"(a) : "v"(w));
}
#undef BNN_NIB_LO
#undef BNN_NIB_HI

template <int I, int J>
__device__ __forceinline__ float lut_read(const char* tb, uint32_t a) {
    constexpr int g = 8 * J + I;
    return *reinterpret_cast<const float*>(tb + a + (g >> 1) * 4096 + (g & 1) * 128);
}

template <int I>
__device__ __forceinline__ void lut_nibble(float (&acc4)[4], uint32_t (&A)[2][4], const uint32_t (&wj)[4],
                                           const char* tb) {
    nib_to_byte1<I>(A[I & 1][0], wj[0]);
    nib_to_byte1<I>(A[I & 1][1], wj[1]);
    nib_to_byte1<I>(A[I & 1][2], wj[2]);
    nib_to_byte1<I>(A[I & 1][3], wj[3]);
    acc4[0] += lut_read<I, 0>(tb, A[I & 1][0]);
    acc4[1] += lut_read<I, 1>(tb, A[I & 1][1]);
    acc4[2] += lut_read<I, 2>(tb, A[I & 1][2]);
    acc4[3] += lut_read<I, 3>(tb, A[I & 1][3]);
}

template <int GLOG2, int U, int NH>
__global__ __launch_bounds__(1024) void k_bwn_f16_lut(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ Wp, int64_t ldW, int N, int K,
    const float* __restrict__ alpha, int astr, float* __restrict__ Y, int mode)
{
    constexpr int G = 1 << GLOG2;
    constexpr int RPS = 64 / G;                   // rows per wave step
    static_assert(G >= 32 || NH == 1, "narrow rows: one granule group, row copies");
    __shared__ float tab[NH * 16384];
    const int Kw = (K + 31) >> 5;
    const int Kw4 = (Kw + 3) >> 2;

    // one thread per (w, i) table: its 4 activations in one 8-byte load, the
    // 16 entries by extending the 2, 4 and 8 partial sums of the first 1, 2
    // and 3 terms (28 additions, each entry in the order above)
    for (int tix = threadIdx.x; tix < NH * 1024; tix += blockDim.x) {
        const int h = tix >> 10, g = (tix >> 5) & 31, sl = tix & 31;
        const int j = g >> 3, i = g & 7;
        const int c = G >= 32 ? h * 32 + sl : (sl & (G - 1));
        const int k0 = 32 * (4 * c + j) + 4 * i;
        float x[4];
        if (k0 + 4 <= K) {
            const uint2 v = *reinterpret_cast<const uint2*>(X + k0);
            x[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v.x & 0xFFFFu));
            x[1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v.x >> 16));
            x[2] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v.y & 0xFFFFu));
            x[3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v.y >> 16));
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) x[q] = (k0 + q < K) ? (float)__builtin_bit_cast(_Float16, X[k0 + q]) : 0.0f;
        }
        float p[16];
        p[0] = x[0]; p[1] = -x[0];
#pragma unroll
        for (int q = 1; q < 4; ++q) {
#pragma unroll
            for (int n = (1 << q) - 1; n >= 0; --n) {      // bit q of the entry index: the sign of x[q]
                p[n + (1 << q)] = p[n] - x[q];
                p[n] = p[n] + x[q];
            }
        }
        float* t = tab + h * 16384 + (g >> 1) * 1024 + (g & 1) * 32 + sl;
#pragma unroll
        for (int nib = 0; nib < 16; ++nib) t[nib * 64] = p[nib];
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int gl = lane & (G - 1);
    const int go = lane >> GLOG2;
    const uint32_t sl = G >= 32 ? (uint32_t)(gl & 31) : (uint32_t)(((go * G) & 31) | gl);
    const uint32_t h = G >= 32 ? (uint32_t)(gl >> 5) : 0u;
    // address registers (byte 1 rewritten per nibble): [nibble parity][word]
    uint32_t A[2][4];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) A[q][j] = (h << 16) | (sl << 2);
    const char* tb = reinterpret_cast<const char*>(tab);

    const int64_t nsteps = ((int64_t)N + RPS - 1) / RPS;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t s0 = wave * U; s0 < nsteps; s0 += nwaves * U) {
        u32x4 wv[U];
        float av[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = (s0 + u) * RPS + go;
            wv[u] = (u32x4){0u, 0u, 0u, 0u};
            if (row < N && gl < Kw4)
                wv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Wp + row * ldW + 4 * gl));
            av[u] = row < N ? alpha[row * astr] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = (s0 + u) * RPS + go;
            float acc4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            const uint32_t wj[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
            lut_nibble<0>(acc4, A, wj, tb);
            lut_nibble<1>(acc4, A, wj, tb);
            lut_nibble<2>(acc4, A, wj, tb);
            lut_nibble<3>(acc4, A, wj, tb);
            lut_nibble<4>(acc4, A, wj, tb);
            lut_nibble<5>(acc4, A, wj, tb);
            lut_nibble<6>(acc4, A, wj, tb);
            lut_nibble<7>(acc4, A, wj, tb);
            float acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
            acc = fsum_to_last<GLOG2>(acc);
            if (gl == G - 1 && row < N) {
                if (mode == 0) Y[row] = av[u] * acc;
                else if (mode == 1) Y[row] = acc;
                else if (mode == 3) Y[row] = Y[row] + acc;
                else Y[row] = av[u] * (Y[row] + acc);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

}  // namespace

int64_t f16_gemv_max_k() { return 64 * 2 * 128; }

namespace {

// Tuning override: BNN_F16_KERNEL=regs keeps the register variant for every K.
bool f16_regs_from_env() {
    const char* v = getenv("BNN_F16_KERNEL");
    return v && v[0] == 'r';
}

// The table variant: 32 blocks of 2 KiB per group of 32 granules (64 KiB
// up to K = 4096, two 1024-thread workgroups per CU; 128 KiB up to 8192,
// one).  Longer rows run as passes over pieces of 8192 (at most two: K is
// at most 16384), the first leaving its raw sum in Y.
hipError_t launch_lut_piece(const uint16_t* X, const uint32_t* Wp, int64_t ldW, int64_t N, int64_t K,
                            const float* alpha, int astr, float* Y, int mode, hipStream_t s, int cus)
{
    const int64_t kw4 = ((K + 31) / 32 + 3) / 4;
    int glog2 = 0;
    while ((1 << glog2) < kw4 && glog2 < 6) ++glog2;
    const int rps = 64 >> glog2;
    const int64_t steps = (N + rps - 1) / rps;
    const int nh = kw4 <= 32 ? 1 : 2;                  // 64 KiB of tables per 32 granules
    const int per_cu = nh == 1 ? 2 : 1;
    const bool unroll = steps >= (int64_t)cus * per_cu * 16 * 8;
    const int U = unroll ? 4 : 1;
    const int64_t waves = (steps + U - 1) / U;
    int64_t blocks = (waves + 15) / 16;
    const int64_t cap = (int64_t)cus * per_cu;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    const dim3 grid((unsigned)blocks), block(1024);
    const int n = (int)N, k = (int)K;
#define BNN_LUT(GL, UU, NHH) hipLaunchKernelGGL((k_bwn_f16_lut<GL, UU, NHH>), grid, block, 0, s, X, Wp, ldW, n, k, alpha, astr, Y, mode)
#define BNN_LUT_U(GL, NHH) do { if (U == 1) BNN_LUT(GL, 1, NHH); else BNN_LUT(GL, 4, NHH); } while (0)
    switch (glog2) {
        case 0: BNN_LUT_U(0, 1); break;
        case 1: BNN_LUT_U(1, 1); break;
        case 2: BNN_LUT_U(2, 1); break;
        case 3: BNN_LUT_U(3, 1); break;
        case 4: BNN_LUT_U(4, 1); break;
        case 5: BNN_LUT_U(5, 1); break;
        default: BNN_LUT_U(6, 2); break;
    }
#undef BNN_LUT_U
#undef BNN_LUT
    return hipGetLastError();
}

hipError_t launch_lut(const uint16_t* X, const uint32_t* Wp, int64_t ldW, int64_t N, int64_t K,
                      const float* alpha, bool alpha_tensor, float* Y, hipStream_t s, int cus)
{
    int64_t piece = 8192;                         // 64 granules: the 128 KiB table
    if (const char* v = getenv("BNN_F16_PIECE")) {          // tuning override: 4096 or 8192
        const int64_t p = atoll(v);
        if (p == 4096 || p == 8192) piece = p;
    }
    const int astr = alpha_tensor ? 0 : 1;
    if (K <= piece) return launch_lut_piece(X, Wp, ldW, N, K, alpha, astr, Y, 0, s, cus);
    for (int64_t k0 = 0; k0 < K; k0 += piece) {
        const int mode = k0 == 0 ? 1 : (k0 + piece >= K ? 2 : 3);
        const hipError_t e = launch_lut_piece(X + k0, Wp + k0 / 32, ldW, N, std::min(piece, K - k0), alpha, astr, Y,
                                              mode, s, cus);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

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
    if (!f16_regs_from_env()) return launch_lut(X, Wp, ldW, N, K, alpha, alpha_tensor, Y, s, cus);
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
