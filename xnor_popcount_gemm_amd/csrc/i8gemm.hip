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
// Tiling: a 256-thread workgroup computes 128 activation rows x 128 weight
// rows; its 4 waves take 64 x 64 quarters (4 x 4 fragments each).  The next
// k-step's A fragments and weight words are loaded before the current
// step's MFMAs (register double buffering).
#include "bnn_device.hpp"
#include "bnn_launch.hpp"

namespace bnn {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 128, kBN = 128, kKS = 64;

typedef int v4i __attribute__((ext_vector_type(4)));

// 16 bytes of an int8 row starting at k; bytes at k >= K read as 0.
template <bool TAIL>
__device__ __forceinline__ v4i load_a(const int8_t* __restrict__ row, int k, int K) {
    if (!TAIL || k + 16 <= K) return *reinterpret_cast<const v4i*>(row + k);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    for (int i = 0; i < 16; ++i)
        if (k + i < K) w[i >> 2] |= ((uint32_t)(uint8_t)row[k + i]) << (8 * (i & 3));
    return (v4i){(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
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

template <bool TAIL>
__device__ __forceinline__ void load_step(v4i (&a)[4], uint32_t (&b)[4],
                                          const int8_t* const (&arow)[4], const uint32_t* const (&wrow)[4],
                                          int k0, int g, int K)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = load_a<TAIL>(arow[i], k0 + 16 * g, K);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = wrow[j][(k0 >> 5) + (g >> 1)];
}

__global__ __launch_bounds__(kThreads) void k_bwn_i8_gemm(
    const int8_t* __restrict__ Xq, int64_t ldX, const uint32_t* __restrict__ Wp, int64_t ldW,
    int M, int N, int K, int tiles_n, EpilogueI8 e)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int tn = blockIdx.x % tiles_n, tm = blockIdx.x / tiles_n;
    const int m0 = tm * kBM + (wave >> 1) * 64;
    const int n0 = tn * kBN + (wave & 1) * 64;
    const int r16 = lane & 15, g = lane >> 4;

    const int8_t* arow[4];
    const uint32_t* wrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) arow[i] = Xq + (int64_t)min(m0 + 16 * i + r16, M - 1) * ldX;
#pragma unroll
    for (int j = 0; j < 4; ++j) wrow[j] = Wp + (int64_t)min(n0 + 16 * j + r16, N - 1) * ldW;

    v4i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (v4i){0, 0, 0, 0};

    const int steps = (K + kKS - 1) / kKS;
    const int full_steps = K / kKS;                // steps with all 64 k inside the row
    v4i a[4];
    uint32_t b[4];
    if (full_steps > 0) load_step<false>(a, b, arow, wrow, 0, g, K);
    else                load_step<true>(a, b, arow, wrow, 0, g, K);
    for (int s = 0; s < steps; ++s) {
        v4i an[4];
        uint32_t bn[4];
        const int kn = (s + 1) * kKS;
        if (s + 1 < full_steps)   load_step<false>(an, bn, arow, wrow, kn, g, K);
        else if (s + 1 < steps)   load_step<true>(an, bn, arow, wrow, kn, g, K);
        v4i bx[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bx[j] = expand_signs(b[j] >> (16 * (g & 1)));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], bx[j], acc[i][j], 0, 0, 0);
        if (s + 1 < steps) {
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = an[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = bn[j];
        }
    }

    // epilogue: lane holds rows 4g + r of each 16-row fragment, column r16
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = n0 + 16 * j + r16;
        if (n >= N) continue;
        float an = 0.0f;
        if (e.flags & EPI_SCALE) an = e.alpha[(e.flags & EPI_ALPHA_TENSOR) ? 0 : n];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 16 * i + 4 * g + r;
                if (m >= M) continue;
                const int32_t d = acc[i][j][r];
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
    hipLaunchKernelGGL(k_bwn_i8_gemm, grid, block, 0, s, Xq, ldXq, Wp, ldW,
                       (int)M, (int)N, (int)K, tiles_n, e);
    return hipGetLastError();
}

}  // namespace bnn
