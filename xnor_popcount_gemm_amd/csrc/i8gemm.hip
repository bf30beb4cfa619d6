// Binary weights x INT8 activations as an MFMA GEMM on gfx950 (many
// activation rows, e.g. a prefill batch).
//
// Method (cited by page title and section / equation): with +1/-1 weights
// the product only adds or subtracts activations ("Extreme Quantization:
// Binary, Ternary & 1-bit LLMs", "Binary Neural Networks" eq. (1)-(2)); its
// "BitNet: 1-bit Transformer" section keeps activations at INT8.  The result
// D[m,n] = sum_k q[m,k] s[n,k] is an exact integer.
//
// With many activation rows this is a dense contraction, so it runs on the
// int8 matrix cores: v_mfma_i32_16x16x64_i8 (16 rows x 16 columns x 64 k per
// instruction, exact int32 accumulation).  The weights stay 1-bit in memory;
// each lane expands the 16 weight bits of its B fragment to 16 bytes of
// +1 / -1 right before the MFMA (a multiply spreads a nibble into bytes; an
// XOR turns 0/1 bytes into 0x01/0xFF without borrows between bytes).
//
// Fragment layout used for both operands: lane l holds row (A) or column (B)
// l % 16 and the 16 consecutive k of group l / 16 within the 64-wide step.
// A and B use the same k assignment, so each output is the full sum over k.
// The int32 result of lane l, register r is row 4*(l/16) + r, column l % 16.
//
// Tiling: a 256-thread workgroup computes 256 activation rows x 128 weight
// rows; wave w takes rows 128*(w/2) .. +127 and columns 64*(w%2) .. +63,
// i.e. 8 x 4 fragments (32 MFMAs per 64-wide k-half against 4 weight
// expansions, two halves per 128-wide k-step).  The workgroup's A tile
// (256 rows x 128 bytes per k-step) is staged through LDS, double-buffered
// with one barrier per k-step; 16-byte piece j of row r sits at slot
// j ^ ((r / 2) % 8) of the row's eight slots, so the 16 lanes of a fragment
// read (16 rows, one k-group) hit 16 distinct 4-bank groups.  The next
// k-step's A pieces go straight from global memory into the other LDS
// buffer, and its weight words into registers, before the current step's
// MFMAs.
#include <type_traits>

#include "bnn_device.hpp"
#include "bnn_launch.hpp"

namespace bnn {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 256, kBN = 128, kKS = 128;   // kKS: two MFMA k-widths per step

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// 16 bytes of an int8 row starting at k (a multiple of 16); bytes at k >= K
// read as 0.  A piece that starts below K ends at or below the row stride
// (both multiples of 16), so the 16-byte load stays inside the row; pieces
// that start at or past K are not loaded.
template <bool TAIL>
__device__ __forceinline__ v4i load_a(const int8_t* __restrict__ row, int k, int K) {
    if (!TAIL) return *reinterpret_cast<const v4i*>(row + k);
    v4i v = (v4i){0, 0, 0, 0};
    if (k < K) v = *reinterpret_cast<const v4i*>(row + k);
    const int valid = K - k;                       // bytes of the piece inside the row
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int vd = valid - 4 * d;
        const uint32_t m = vd >= 4 ? ~0u : vd <= 0 ? 0u : (1u << (8 * vd)) - 1u;
        v[d] = (int)((uint32_t)v[d] & m);
    }
    return v;
}

// 16 weight bits (bit i = element i; 1 means -1) to 16 bytes of +1 / -1.
__device__ __forceinline__ v4i expand_signs(uint32_t bits16) {
    v4i r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t nib = (bits16 >> (4 * q)) & 0xFu;
        // nib * (1 + 2^7 + 2^14 + 2^21) puts bit i at 8i (the other partial
        // products land at distinct positions outside the 0x01010101 mask)
        const uint32_t t = (nib * 0x00204081u) & 0x01010101u;
        r[q] = (int)(0x01010101u ^ (t * 0xFEu));   // 0 -> 0x01 (+1), 1 -> 0xFF (-1)
    }
    return r;
}

// Ternary weights ("Extreme Quantization", eq. (7) / (9)): c holds the
// lane's 16 nonzero bits (Z) in its low half and its 16 bits of -1 weights
// (S & Z) in its high half; each byte becomes 0x01 (+1), 0xFF (-1) or 0.
__device__ __forceinline__ v4i expand_ternary(uint32_t c) {
    v4i r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t zn = (c >> (4 * q)) & 0xFu;
        const uint32_t mn = (c >> (16 + 4 * q)) & 0xFu;
        const uint32_t tz = (zn * 0x00204081u) & 0x01010101u;
        const uint32_t tm = (mn * 0x00204081u) & 0x01010101u;
        r[q] = (int)(tz ^ (tm * 0xFEu));           // z=1: 0x01, then m=1 turns it into 0xFF
    }
    return r;
}

constexpr int kAPieces = kBM * kKS / 16 / kThreads;   // 16-byte A pieces per lane per k-step

typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// TERN: Wp is the sign plane, e.Zp the nonzero plane of ternary weights.
template <bool TERN>
__global__ __launch_bounds__(kThreads, 2) void k_bwn_i8_gemm(
    const int8_t* __restrict__ Xq, int64_t ldX, const uint32_t* __restrict__ Wp, int64_t ldW,
    int M, int N, int K, int tiles_n, EpilogueI8 e)
{
    __shared__ __attribute__((aligned(16))) int8_t lds_a[2][kBM * kKS];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int tn = blockIdx.x % tiles_n, tm = blockIdx.x / tiles_n;
    const int m_blk = tm * kBM, n_blk = tn * kBN;
    const int wm = wave >> 1, wn = wave & 1;
    const int r16 = lane & 15, g = lane >> 4;

    // A staging.  Instruction i of wave w fills tile rows 8 (8 w + i) ..
    // +7 (1 KiB of LDS): lane l takes row r = 8 (8 w + i) + l / 8, LDS slot
    // l % 8, and loads the piece j stored there, j = slot ^ ((r / 2) % 8).
    // Full k-steps load straight into LDS (global_load_lds_dwordx4 writes
    // lane l's 16 bytes at the instruction's LDS base + 16 l); the step
    // holding the end of the row goes through registers, masked past K.
    int aoff[kAPieces];                            // byte offset of row r (M * ldX < 2^31)
    int apiece[kAPieces];                          // byte offset of piece j in the row
#pragma unroll
    for (int i = 0; i < kAPieces; ++i) {
        const int r = 8 * (8 * wave + i) + (lane >> 3);
        aoff[i] = min(m_blk + r, M - 1) * (int)ldX;
        apiece[i] = (((lane & 7) ^ ((r >> 1) & 7)) << 4);
    }
    auto stage_direct = [&](int buf, int k0) {
#pragma unroll
        for (int i = 0; i < kAPieces; ++i)
            __builtin_amdgcn_global_load_lds((gptr_t)(Xq + aoff[i] + k0 + apiece[i]),
                                             (lptr_t)(&lds_a[buf][(8 * wave + i) * 1024]), 16, 0, 0);
    };
    auto stage_masked = [&](int buf, int k0) {
#pragma unroll
        for (int i = 0; i < kAPieces; ++i) {
            const v4i v = load_a<true>(Xq + aoff[i], k0 + apiece[i], K);
            *reinterpret_cast<v4i*>(&lds_a[buf][(8 * wave + i) * 1024 + 16 * lane]) = v;
        }
    };
    // fragment reads: row 16 f + r16 of the wave's 128, piece 4 h + g of the
    // step (h: first or second 64-wide half)
    int roff[2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            const int r = wm * 128 + 16 * f + r16;
            roff[h][f] = r * kKS + (((4 * h + g) ^ ((r >> 1) & 7)) << 4);
        }
    const uint32_t* wrow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) wrow[q] = Wp + (int64_t)min(n_blk + wn * 64 + 16 * q + r16, N - 1) * ldW;
    const int64_t zdelta = TERN ? e.Zp - Wp : 0;   // nonzero plane: same layout, other base
    // combined ternary word of lane group g: Z bits low, (S & Z) bits high
    auto tern_word = [](uint32_t sw, uint32_t zw, int gg) {
        const int sh = 16 * (gg & 1);
        return ((zw >> sh) & 0xFFFFu) | (((sw & zw) >> sh) << 16);
    };

    v4i acc[8][4];
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[f][q] = (v4i){0, 0, 0, 0};

    // weight words of a step: half h of column q is word (k0 / 32) + 2 h + g / 2
    const int steps = (K + kKS - 1) / kKS;
    const int full_steps = K / kKS;
    uint32_t bw[2][4];
    if (full_steps > 0) stage_direct(0, 0);
    else                stage_masked(0, 0);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            bw[h][q] = wrow[q][2 * h + (g >> 1)];
            if (TERN) bw[h][q] = tern_word(bw[h][q], (wrow[q] + zdelta)[2 * h + (g >> 1)], g);
        }
    __builtin_amdgcn_s_waitcnt(0);
    // the first step's words are complete before the loop, so no load is
    // pending on the loop-carried registers when an iteration begins
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 4; ++q) asm volatile("" : : "v"(bw[h][q]));
    __syncthreads();

    // One k-step: prefetch step s+1 (DIRECT: straight into LDS), run the 64
    // MFMAs of step s, wait for the prefetch, barrier.
    auto kstep = [&](int s, auto direct_tag) {
        constexpr bool DIRECT = decltype(direct_tag)::value;
        const int cur = s & 1;
        const bool more = s + 1 < steps;
        const int kn = (s + 1) * kKS;
        uint32_t bn[2][4], zn[2][4];
        if (more) {
            if (DIRECT) stage_direct(cur ^ 1, kn);
            else        stage_masked(cur ^ 1, kn);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    bn[h][q] = wrow[q][(kn >> 5) + 2 * h + (g >> 1)];
                    if (TERN) zn[h][q] = (wrow[q] + zdelta)[(kn >> 5) + 2 * h + (g >> 1)];
                }
        }
        const int8_t* la = lds_a[cur];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v4i bx[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                bx[q] = TERN ? expand_ternary(bw[h][q]) : expand_signs(bw[h][q] >> (16 * (g & 1)));
#pragma unroll
            for (int f = 0; f < 8; ++f) {
                const v4i a = *reinterpret_cast<const v4i*>(la + roff[h][f]);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[f][q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bx[q], acc[f][q], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);         // the step's MFMAs stay ahead of the waits below
        if (more) {
            __builtin_amdgcn_s_waitcnt(0);        // the prefetched A pieces are in LDS
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    asm volatile("" : : "v"(bn[h][q]));
                    if (TERN) asm volatile("" : : "v"(zn[h][q]));
                    bw[h][q] = TERN ? tern_word(bn[h][q], zn[h][q], g) : bn[h][q];
                }
        }
        __syncthreads();
    };
    // steps whose successor lies wholly inside K prefetch straight into LDS;
    // the prefetch of the step holding the end of the row is masked
    int s = 0;
    for (; s + 1 < full_steps; ++s) kstep(s, std::true_type{});
    for (; s < steps; ++s) kstep(s, std::false_type{});

    // Epilogue.  Full tiles with 16-byte aligned output rows go through LDS
    // (the A buffers are free now): in two passes of 4 fragment rows, each
    // wave parks its 64 x 64 int32 block (16 KiB; column c of row r at word
    // r * 64 + (c ^ 16 ((r / 4) % 4)), so the 4 lane groups of a fragment
    // write disjoint 16-bank groups) and reads it back as 16-byte row
    // pieces, so every store instruction writes 4 whole 256-byte row
    // segments.  Other tiles store element by element.
    const bool full = m_blk + kBM <= M && n_blk + kBN <= N &&
                      (!(e.flags & EPI_DOT) || ((reinterpret_cast<uintptr_t>(e.D) & 15u) == 0 && e.ldD % 4 == 0)) &&
                      (!(e.flags & EPI_SCALE) || ((reinterpret_cast<uintptr_t>(e.Y) & 15u) == 0 && e.ldY % 4 == 0));
    if (full) {
        int32_t* park = reinterpret_cast<int32_t*>(&lds_a[0][0]) + wave * (64 * 64);   // 4 x 16 KiB = both A buffers
        const int pc = 4 * (lane & 15);            // read-back: 4 columns of row lane/16 (+4 per pass)
        float an[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (e.flags & EPI_SCALE) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                an[c] = e.alpha[(e.flags & EPI_ALPHA_TENSOR) ? 0 : n_blk + wn * 64 + pc + c];
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int f = 0; f < 4; ++f)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        park[(16 * f + 4 * g + r) * 64 + ((16 * q + r16) ^ (16 * g))] = acc[4 * half + f][q][r];
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int p = 0; p < 16; ++p) {
                const int row = 4 * p + (lane >> 4);
                const v4i d = *reinterpret_cast<const v4i*>(&park[row * 64 + (pc ^ (16 * ((row >> 2) & 3)))]);
                const int64_t m = m_blk + wm * 128 + 64 * half + row;
                const int n = n_blk + wn * 64 + pc;
                if (e.flags & EPI_DOT)
                    __builtin_nontemporal_store(d, reinterpret_cast<v4i*>(e.D + m * e.ldD + n));
                if (e.flags & EPI_SCALE) {
                    v4f y = {an[0] * (float)d[0], an[1] * (float)d[1], an[2] * (float)d[2], an[3] * (float)d[3]};
                    if (e.xscale) {
                        const float xs = e.xscale[m];
                        y[0] = y[0] * xs; y[1] = y[1] * xs; y[2] = y[2] * xs; y[3] = y[3] * xs;
                    }
                    __builtin_nontemporal_store(y, reinterpret_cast<v4f*>(e.Y + m * e.ldY + n));
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
        return;
    }
    // lane holds rows 4g + r of each 16-row fragment, column r16
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int n = n_blk + wn * 64 + 16 * q + r16;
        if (n >= N) continue;
        float an = 0.0f;
        if (e.flags & EPI_SCALE) an = e.alpha[(e.flags & EPI_ALPHA_TENSOR) ? 0 : n];
#pragma unroll
        for (int f = 0; f < 8; ++f)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m_blk + wm * 128 + 16 * f + 4 * g + r;
                if (m >= M) continue;
                const int32_t d = acc[f][q][r];
                if (e.flags & EPI_DOT) e.D[(int64_t)m * e.ldD + n] = d;
                if (e.flags & EPI_SCALE) {
                    float y = an * (float)d;
                    if (e.xscale) y = y * e.xscale[m];
                    e.Y[(int64_t)m * e.ldY + n] = y;
                }
            }
    }
}

}  // namespace

hipError_t launch_bwn_i8_gemm(const int8_t* Xq, int64_t ldXq, const uint32_t* Wp, int64_t ldW,
                              int64_t M, int64_t N, int64_t K, const EpilogueI8& e, hipStream_t s)
{
    const int tiles_n = (int)((N + kBN - 1) / kBN);
    const int64_t tiles_m = (M + kBM - 1) / kBM;
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(kThreads);
    if (e.flags & W_TERNARY)
        hipLaunchKernelGGL((k_bwn_i8_gemm<true>), grid, block, 0, s, Xq, ldXq, Wp, ldW, (int)M, (int)N, (int)K, tiles_n, e);
    else
        hipLaunchKernelGGL((k_bwn_i8_gemm<false>), grid, block, 0, s, Xq, ldXq, Wp, ldW, (int)M, (int)N, (int)K, tiles_n, e);
    return hipGetLastError();
}

}  // namespace bnn
