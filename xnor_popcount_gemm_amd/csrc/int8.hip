// Binary weights x INT8 activations on gfx950: activation quantization and
// bit-plane packing, and the bit-plane streaming GEMV (decode).
//
// Method (cited by page title and section / equation):
//  - With +1/-1 weights a dot product only adds or subtracts activations:
//    "Extreme Quantization: Binary, Ternary & 1-bit LLMs", "Binary Neural
//    Networks" eq. (1)-(2); its "BitNet: 1-bit Transformer" section keeps the
//    activations at INT8 next to binary weights (eq. (8) gives the weight
//    scale).
//  - batch-1 inference is bound by fetching the packed weights: "First
//    Principles: Why Binary Ops Can Be Exponentially Faster", sections "The
//    cost of a neural network step" and "Bandwidth math".
//
// Bit planes.  An int8 row q is stored as 8 packed bit rows: plane b holds
// bit b of every two's-complement byte, so q = sum_b c_b * plane_b with
// c_b = 2^b (b < 7) and c_7 = -128.  With the weight bit 1 meaning -1,
//     sum_k s_k q_k = sum_k q_k - 2 * sum_{k: wbit_k = 1} q_k
//                   = xsum - 2 * sum_b c_b * popcount(plane_b AND wbits),
// an exact integer identity: 8 (AND, popcount-accumulate) pairs per 32
// weights instead of 32 multiply-adds, so the GEMV stays bound by the 1-bit
// weight stream.  Plane pad bits are 0 (value 0), so weight pad bits never
// contribute.
#include <stdio.h>
#include <stdlib.h>

#include "bnn_device.hpp"
#include "bnn_launch.hpp"

namespace bnn {
namespace {

constexpr int kThreads = 256;

// Absmax quantization of one value (IEEE single, one rounding per step):
// q = rint(x * inv) clamped to [-127, 127]; a NaN product gives 0.
__device__ __forceinline__ int quant_i8(float x, float inv) {
    const float r = rintf(x * inv);
    if (r != r) return 0;
    if (r > 127.0f) return 127;
    if (r < -127.0f) return -127;
    return (int)r;
}

// Bit b of each of the 4 bytes of v, gathered into 4 consecutive bits:
// the masked bits sit at 0, 8, 16, 24; multiplying by 2^24 + 2^17 + 2^10 +
// 2^3 moves them to 24..27 with every other partial product at a distinct
// lower (or discarded) position, so no carry reaches bits 24..27.
__device__ __forceinline__ uint32_t gather_bit_of_bytes(uint32_t v, int b) {
    return (((v >> b) & 0x01010101u) * 0x01020408u) >> 24;
}

// One workgroup per activation row.  FROM_F32: quantize X (absmax per row);
// otherwise re-lay int8 input rows.  Writes any of: int8 Q, bit planes, row
// sum, row scale.  Each thread owns 16 consecutive elements per 4096-wide
// block of the row; a pair of lanes forms one 32-bit plane word (DPP).
template <bool FROM_F32>
__global__ __launch_bounds__(kThreads) void k_act_i8(
    const float* __restrict__ X, int64_t ldX, const int8_t* __restrict__ Qin, int64_t ldQin, int K,
    int8_t* __restrict__ Q, int64_t ldQ, uint32_t* __restrict__ Xb, int64_t ldXb,
    int32_t* __restrict__ xsum, float* __restrict__ xscale, int vecX, int vecQ)
{
    __shared__ float red_f[kThreads / 64];
    __shared__ int32_t red_i[kThreads / 64];
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const float* __restrict__ xr = X + m * ldX;
    const int8_t* __restrict__ qr = Qin + m * ldQin;

    float inv = 0.0f;
    if (FROM_F32) {
        float amax = 0.0f;                         // NaN compares false: skipped
        for (int k = 4 * tid; k < K; k += 4 * kThreads) {
            float v[4];
            if (vecX && k + 4 <= K) {
                const float4 t = *reinterpret_cast<const float4*>(xr + k);
                v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = (k + i < K) ? xr[k + i] : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float a = fabsf(v[i]);
                amax = a > amax ? a : amax;
            }
        }
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) {
            const float o = __shfl_xor(amax, s, 64);
            amax = o > amax ? o : amax;
        }
        if (lane == 0) red_f[wave] = amax;
        __syncthreads();
        amax = red_f[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) amax = red_f[w] > amax ? red_f[w] : amax;
        inv = amax > 0.0f ? 127.0f / amax : 0.0f;
        if (tid == 0) xscale[m] = amax / 127.0f;
    }

    const int Kw = (K + 31) >> 5;
    int32_t tsum = 0;
    const int iters = (K + 16 * kThreads - 1) / (16 * kThreads);
    for (int it = 0; it < iters; ++it) {           // uniform trip count: DPP partners stay active
        const int k0 = it * 16 * kThreads + 16 * tid;
        uint32_t qw[4];
        if (!FROM_F32 && vecX && k0 + 16 <= K) {
            const uint4 t = *reinterpret_cast<const uint4*>(qr + k0);
            qw[0] = t.x; qw[1] = t.y; qw[2] = t.z; qw[3] = t.w;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) tsum += (int32_t)(int8_t)(qw[j] >> (8 * i));
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k = k0 + 4 * j;
                float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if (FROM_F32) {
                    if (vecX && k + 4 <= K) {
                        const float4 t = *reinterpret_cast<const float4*>(xr + k);
                        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) v[i] = (k + i < K) ? xr[k + i] : 0.0f;
                    }
                }
                uint32_t word = 0u;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    int q = 0;
                    if (FROM_F32) q = (k + i < K) ? quant_i8(v[i], inv) : 0;
                    else q = (k + i < K) ? (int)qr[k + i] : 0;
                    tsum += q;
                    word |= ((uint32_t)q & 0xFFu) << (8 * i);
                }
                qw[j] = word;
            }
        }
        if (Q && k0 < K) {
            int8_t* __restrict__ qo = Q + m * ldQ + k0;
            if (vecQ && k0 + 16 <= K) *reinterpret_cast<uint4*>(qo) = make_uint4(qw[0], qw[1], qw[2], qw[3]);
            else
                for (int i = 0; i < 16 && k0 + i < K; ++i) qo[i] = (int8_t)(qw[i >> 2] >> (8 * (i & 3)));
        }
        if (Xb) {
            const int w = (k0 - 16 * (tid & 1)) >> 5;   // the pair's word
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                uint32_t h = 0u;
#pragma unroll
                for (int j = 0; j < 4; ++j) h |= gather_bit_of_bytes(qw[j], b) << (4 * j);
                // even lane: low 16 bits; the odd lane receives them (row_shr:1)
                const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, 0x111, 0xF, 0xF, true);
                if ((tid & 1) && w < Kw) Xb[(m * 8 + b) * ldXb + w] = lo | (h << 16);
            }
        }
    }
    if (Xb) {
        const int64_t pad = ldXb - Kw;             // pad words hold 0
        for (int64_t i = tid; i < 8 * pad; i += kThreads)
            Xb[(m * 8 + i / pad) * ldXb + Kw + i % pad] = 0u;
    }
    if (xsum) {
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) tsum += __shfl_xor(tsum, s, 64);
        if (lane == 0) red_i[wave] = tsum;
        __syncthreads();
        if (tid == 0) {
            int32_t t = 0;
#pragma unroll
            for (int w2 = 0; w2 < kThreads / 64; ++w2) t += red_i[w2];
            xsum[m] = t;
        }
    }
}

// Bit-plane GEMV: G = 2^GLOG2 lanes share one weight row and read it in
// consecutive 16-byte granules (coalesced), 64/G rows per wave step, CPL
// granules per lane, U row-steps per group with all their loads issued
// first.  The 8 planes of the MR activation rows sit in LDS for the whole
// kernel (holding them in registers took 96 VGPRs per lane at K = 11008 and
// limited the kernel to 3 waves per SIMD).  Per row-step a lane does
// 8 (v_and, v_bcnt) per word, 7 shift-adds to weigh the planes, and the
// group sum takes GLOG2 DPP adds.
// TERN: ternary weights -- Wp is the sign plane S and e.Zp the nonzero plane
// Z; sum_k t_k q_k = sum_b c_b (popcount(P_b & Z) - 2 popcount(P_b & Z & S))
// (no row sum needed), two (v_and, v_bcnt) pairs per plane and word.
template <int MR, int CPL, int U, int GLOG2, bool TERN>
__global__ __launch_bounds__(kThreads) void k_bwn_i8_gemv(
    const uint32_t* __restrict__ Xb, int64_t ldXb, const int32_t* __restrict__ xsum,
    const uint32_t* __restrict__ Wp, int64_t ldW, int N, int K, EpilogueI8 e)
{
    constexpr int G = 1 << GLOG2;
    constexpr int RPS = 64 >> GLOG2;
    const int lane = threadIdx.x & 63;
    const int gl = lane & (G - 1);
    const int go = lane >> GLOG2;
    const int Kw = (K + 31) >> 5;
    const int Kw4 = (Kw + 3) >> 2;

    // The 8 planes of the MR activation rows, granule slot c = gl + G i of
    // plane (mr, b) at lds_x[((mr * 8 + b) * CPL + i) * G + gl]; words >= Kw
    // are stored as 0.  Lanes of one group read consecutive 16-byte slots
    // (distinct banks), the groups of a wave the same slots (broadcast).
    __shared__ u32x4 lds_x[MR * 8 * CPL * G];
    for (int idx = threadIdx.x; idx < MR * 8 * CPL * G; idx += kThreads) {
        const int slot = idx % (CPL * G);              // = i * G + gl
        const int pl = idx / (CPL * G);                // = mr * 8 + b
        const int c = (slot % G) + G * (slot / G);     // granule index gl + G i
        u32x4 v = (u32x4){0u, 0u, 0u, 0u};
        if (c < Kw4) {
            v = *reinterpret_cast<const u32x4*>(Xb + (int64_t)pl * ldXb + 4 * c);
            v.x = (4 * c + 0 < Kw) ? v.x : 0u;
            v.y = (4 * c + 1 < Kw) ? v.y : 0u;
            v.z = (4 * c + 2 < Kw) ? v.z : 0u;
            v.w = (4 * c + 3 < Kw) ? v.w : 0u;
        }
        lds_x[idx] = v;
    }
    __syncthreads();
    // Weight loads are branch-free: a lane's granule past the row reads the
    // row's last granule instead (the activation planes of that slot are 0 in
    // LDS, so it adds nothing) and a row past N reads row N - 1 (its result is
    // not stored).  With the loads under a per-lane branch, the exec-masked
    // blocks sat in the streaming loop.
    int coff[CPL];                                // word offset of granule slot i in a row
#pragma unroll
    for (int i = 0; i < CPL; ++i) coff[i] = 4 * min(gl + G * i, Kw4 - 1);
    int32_t xs[MR];
    float xsc[MR];
#pragma unroll
    for (int mr = 0; mr < MR; ++mr) {
        xs[mr] = TERN ? 0 : xsum[mr];
        xsc[mr] = e.xscale ? e.xscale[mr] : 1.0f;
    }

    const int64_t nsteps = ((int64_t)N + RPS - 1) / RPS;
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t stride = (((int64_t)gridDim.x * kThreads) >> 6) * U;
    const bool last = gl == G - 1;
    for (int64_t s0 = wave * U; s0 < nsteps; s0 += stride) {
        const int64_t row0 = s0 * RPS + go;
        u32x4 w[U][CPL], z[U][CPL];
        float av[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = row0 + (int64_t)u * RPS;
            const int64_t roff = min(row, (int64_t)N - 1) * ldW;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                w[u][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Wp + roff + coff[i]));
                z[u][i] = (u32x4){0u, 0u, 0u, 0u};
                if (TERN) z[u][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(e.Zp + roff + coff[i]));
            }
            av[u] = 0.0f;
            if ((e.flags & EPI_SCALE) && row < N) av[u] = e.alpha[(e.flags & EPI_ALPHA_TENSOR) ? 0 : row];
        }
#pragma unroll
        for (int mr = 0; mr < MR; ++mr) {
            // binary: count the -1 weights (bit 1); ternary: the -1 weights
            // are S & Z, the nonzero ones Z.  Each pair of planes is read
            // from LDS once and used for all U row-steps.
            uint32_t acc[U][8], acz[U][8];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int b = 0; b < 8; ++b) { acc[u][b] = 0u; acz[u][b] = 0u; }
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
#pragma unroll
                for (int b = 0; b < 8; b += 2) {
                    const u32x4 x0 = lds_x[((mr * 8 + b) * CPL + i) * G + gl];
                    const u32x4 x1 = lds_x[((mr * 8 + b + 1) * CPL + i) * G + gl];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const u32x4 wn = TERN ? (w[u][i] & z[u][i]) : w[u][i];
                        and_popc_2x4(acc[u][b], acc[u][b + 1], x0, x1, wn);
                        if (TERN) and_popc_2x4(acz[u][b], acz[u][b + 1], x0, x1, z[u][i]);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t row = row0 + (int64_t)u * RPS;
                // sum over the planes with their two's-complement weights:
                // neg = sum of q over the -1 weights, nzs = over the nonzero ones
                uint32_t neg = acc[u][0], nzs = acz[u][0];
#pragma unroll
                for (int b = 1; b < 7; ++b) { neg += acc[u][b] << b; if (TERN) nzs += acz[u][b] << b; }
                neg -= acc[u][7] << 7;
                if (TERN) nzs -= acz[u][7] << 7;
                neg = sum_reduce_to_last_t<GLOG2>(neg);
                if (TERN) nzs = sum_reduce_to_last_t<GLOG2>(nzs);
                if (last && row < N) {
                    const int32_t d = (TERN ? (int32_t)nzs : xs[mr]) - 2 * (int32_t)neg;
                    if (e.flags & EPI_DOT) e.D[(int64_t)mr * e.ldD + row] = d;
                    if (e.flags & EPI_SCALE) {
                        float y = av[u] * (float)d;
                        if (e.xscale) y = y * xsc[mr];
                        e.Y[(int64_t)mr * e.ldY + row] = y;
                    }
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

}  // namespace

hipError_t launch_act_i8(const float* X, int64_t ldX, const int8_t* Xq_in, int64_t ldXq_in,
                         int64_t M, int64_t K,
                         int8_t* Q, int64_t ldQ, uint32_t* Xb, int64_t ldXb, int32_t* xsum,
                         float* xscale, hipStream_t s)
{
    const dim3 grid((unsigned)M), block(kThreads);
    const int vecQ = Q && (reinterpret_cast<uintptr_t>(Q) & 15u) == 0 && ldQ % 16 == 0;
    if (X) {
        const int vecX = (reinterpret_cast<uintptr_t>(X) & 15u) == 0 && ldX % 4 == 0;
        hipLaunchKernelGGL((k_act_i8<true>), grid, block, 0, s, X, ldX, (const int8_t*)nullptr, (int64_t)0,
                           (int)K, Q, ldQ, Xb, ldXb, xsum, xscale, vecX, vecQ);
    } else {
        const int vecX = (reinterpret_cast<uintptr_t>(Xq_in) & 15u) == 0 && ldXq_in % 16 == 0;
        hipLaunchKernelGGL((k_act_i8<false>), grid, block, 0, s, (const float*)nullptr, (int64_t)0, Xq_in, ldXq_in,
                           (int)K, Q, ldQ, Xb, ldXb, xsum, xscale, vecX, vecQ);
    }
    return hipGetLastError();
}

namespace {
// Lane-group shape of the G-lanes GEMV for a row of K: G = 2^glog2 lanes and
// CPL granules per lane, the fewest lane slots G * CPL covering the row's
// ceil(Kw/4) granules (G in 16..64, CPL * M <= 4, which bounds the planes'
// LDS space to 32 KB per workgroup); among equal slot counts the larger CPL
// (fewer group sums).
struct I8Shape { int glog2, cpl; };

bool i8_shape(int64_t M, int64_t K, I8Shape* out) {
    const int64_t kw4 = ((K + 31) / 32 + 3) / 4;
    I8Shape best = {0, 0};
    int64_t best_slots = 0;
    for (int cpl = 4; cpl >= 1; --cpl) {
        if (cpl * M > 4) continue;
        for (int g = 4; g <= 6; ++g) {
            const int64_t slots = (int64_t)cpl << g;
            if (slots < kw4) continue;
            if (best.cpl == 0 || slots < best_slots) { best = {g, cpl}; best_slots = slots; }
        }
    }
    if (best.cpl == 0) return false;
    if (const char* v = getenv("BNN_I8_SHAPE")) {     // tuning override "glog2,cpl"
        int g = 0, c = 0;
        if (sscanf(v, "%d,%d", &g, &c) == 2 && g >= 4 && g <= 6 && c >= 1 && c <= 4 && c * M <= 4 &&
            ((int64_t)c << g) >= kw4) best = {g, c};
    }
    *out = best;
    return true;
}
}  // namespace

bool i8_gemv_eligible(int64_t M, int64_t K) {
    I8Shape sh;
    return M >= 1 && M <= 2 && i8_shape(M, K, &sh);
}

hipError_t launch_bwn_i8_gemv(const uint32_t* Xb, int64_t ldXb, const int32_t* xsum,
                              const uint32_t* Wp, int64_t ldW,
                              int64_t M, int64_t N, int64_t K, const EpilogueI8& e, hipStream_t s)
{
    const int cus = num_cus();
    I8Shape sh;
    i8_shape(M, K, &sh);
    int umax = 2;
    if (const char* v = getenv("BNN_GEMV_U")) {       // tuning override: 1 or 2
        const int u = atoi(v);
        if (u == 1 || u == 2) umax = u;
    }
    const int rps = 64 >> sh.glog2;
    const int64_t steps = (N + rps - 1) / rps;
    const bool unroll = umax > 1 && steps >= (int64_t)cus * 4 * 8 * umax;
    const int U = unroll ? umax : 1;
    const int64_t waves = (steps + U - 1) / U;
    int64_t blocks = (waves + 3) / 4;
    const int64_t cap = (int64_t)cus * 64;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    const dim3 grid((unsigned)blocks), block(kThreads);
    const int n = (int)N, k = (int)K;
#define BNN_I8GEMV(MR, CPL, UU, GL) \
    if (e.flags & W_TERNARY) hipLaunchKernelGGL((k_bwn_i8_gemv<MR, CPL, UU, GL, true>), grid, block, 0, s, Xb, ldXb, xsum, Wp, ldW, n, k, e); \
    else                     hipLaunchKernelGGL((k_bwn_i8_gemv<MR, CPL, UU, GL, false>), grid, block, 0, s, Xb, ldXb, xsum, Wp, ldW, n, k, e)
#define BNN_I8GEMV_G(MR, CPL, UU) \
    switch (sh.glog2) { case 4: BNN_I8GEMV(MR, CPL, UU, 4); break; case 5: BNN_I8GEMV(MR, CPL, UU, 5); break; \
                        default: BNN_I8GEMV(MR, CPL, UU, 6); break; }
#define BNN_I8GEMV_U(MR, CPL) \
    if (U == 2) { BNN_I8GEMV_G(MR, CPL, 2) } else { BNN_I8GEMV_G(MR, CPL, 1) }
    if (M == 1) {
        switch (sh.cpl) { case 1: BNN_I8GEMV_U(1, 1); break; case 2: BNN_I8GEMV_U(1, 2); break;
                          case 3: BNN_I8GEMV_U(1, 3); break; default: BNN_I8GEMV_U(1, 4); break; }
    } else {
        switch (sh.cpl) { case 1: BNN_I8GEMV_U(2, 1); break; default: BNN_I8GEMV_U(2, 2); break; }
    }
#undef BNN_I8GEMV_U
#undef BNN_I8GEMV_G
#undef BNN_I8GEMV
    return hipGetLastError();
}

}  // namespace bnn
