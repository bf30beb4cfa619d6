// Host-side launchers of the gfx950 kernels (internal to libbnn).  The C ABI
// in bnn_api.hip validates every argument before calling these; the
// launchers assume valid, non-empty shapes and report only launch errors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bnn {

// Epilogue parameters of the XNOR-popcount GEMM / GEMV.
struct Epilogue {
    uint32_t flags;          // BNN_EPI_* bits
    int32_t* D; int64_t ldD;
    const float* alpha;      // [N], or alpha[0] for all n with EPI_ALPHA_TENSOR
    float* Y; int64_t ldY;
    const float* R; int64_t ldR;
    const float* tau; const int8_t* dir;
    uint32_t* Op; int64_t ldOp;
    const float* bias;       // [N] with EPI_BIAS
    const uint32_t* Zp;      // ternary weights: nonzero plane (same ld as the sign plane Wp)
    const int32_t* nnz;      // ternary weights: nonzero count per weight row
    const float* beta;       // EPI_SIGN_PACK: per-column RSign shift (nullptr: 0)
};

enum : uint32_t { EPI_DOT = 1u, EPI_SCALE = 2u, EPI_RESIDUAL = 4u, EPI_THRESH = 8u,
                  EPI_ALPHA_TENSOR = 16u, EPI_BIAS = 32u, W_TERNARY = 64u, EPI_SIGN_PACK = 128u,
                  // set by the launchers only (never by a caller): touch the residual
                  // tile at the start of the K loop
                  EPI_PREFETCH_R = 1u << 30 };

// Epilogue of binary weights x INT8 activations.
// Compute units of the current device (256 if the query fails).
inline int num_cus() {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    return cus;
}

struct EpilogueI8 {
    uint32_t flags;          // EPI_DOT, EPI_SCALE, EPI_ALPHA_TENSOR
    int32_t* D; int64_t ldD;
    const float* alpha;      // [N], or alpha[0] with EPI_ALPHA_TENSOR
    const float* xscale;     // [M] or nullptr
    float* Y; int64_t ldY;
    const uint32_t* Zp;      // ternary weights (W_TERNARY): nonzero plane
    const int32_t* xsum;     // MFMA GEMM, binary weights: [M] row sums of q, or nullptr
};

hipError_t launch_pack_dense(const float* X, int64_t rows, int64_t K, int64_t ldX,
                             uint32_t* P, int64_t ldP, float* alpha, hipStream_t s);

// alpha[0] = fl32(sum |W| / (N K)), fp64 sums; work holds N doubles.
hipError_t launch_alpha_tensor(const float* W, int64_t N, int64_t K, int64_t ldW,
                               double* work, float* alpha, hipStream_t s);

// Ternary weights as sign + nonzero planes and nonzero counts (gamma != nullptr:
// RoundClip(w / gamma[0]); else the threshold delta).
hipError_t launch_pack_ternary(const float* W, int64_t N, int64_t K, int64_t ldW, const float* gamma,
                               float delta, uint32_t* S, uint32_t* Z, int64_t ld, int32_t* nnz,
                               hipStream_t s);

// Sign + pack with a per-column RSign shift: bit = !(x >= beta[k]).
hipError_t launch_pack_dense_rsign(const float* X, int64_t rows, int64_t K, int64_t ldX, const float* beta,
                                   uint32_t* P, int64_t ldP, hipStream_t s);

hipError_t launch_pack_im2col3x3(const float* X, int64_t B, int64_t H, int64_t W, int64_t C,
                                 uint32_t* P, int64_t ldP, hipStream_t s);

hipError_t launch_xnor_gemm(const uint32_t* Xp, int64_t ldX, const uint32_t* Wp, int64_t ldW,
                            int64_t M, int64_t N, int64_t K, const Epilogue& e, hipStream_t s);

// Implicit-im2col 3x3 binary convolution: Xp is the packed NHWC image
// [B*H*W, ldX] with C = 32 cw channel bits per pixel (cw in {2, 4, 8, 16}),
// Wp the packed OHWI weights [N, ldW], K = 9 C, M = B*H*W.
hipError_t launch_xnor_conv3x3(const uint32_t* Xp, int64_t ldX, const uint32_t* Wp, int64_t ldW,
                               int64_t M, int64_t N, int64_t H, int64_t W, int cw,
                               const Epilogue& e, hipStream_t s);

// Ternary weights (e.Zp, e.nnz) x binary activations with one weight row per
// lane; tern_gemm_t_eligible says whether it serves a ternary GEMM (else the
// ternary mode of launch_xnor_gemm).
bool tern_gemm_t_eligible();
hipError_t launch_tern_gemm_t(const uint32_t* Xp, int64_t ldX, const uint32_t* Sp, int64_t ldW,
                              int64_t M, int64_t N, int64_t K, const Epilogue& e, hipStream_t s);

// True when the streaming GEMV kernel serves this call (small M, no
// THRESH_PACK, row length within its register budget).
bool gemv_eligible(int64_t M, int64_t K, uint32_t flags);

hipError_t launch_xnor_gemv(const uint32_t* Xp, int64_t ldX, const uint32_t* Wp, int64_t ldW,
                            int64_t M, int64_t N, int64_t K, const Epilogue& e, hipStream_t s);

// Per-row absmax INT8 quantization (X != nullptr) or plain re-layout of int8
// rows (Xq_in != nullptr): writes any of Q (int8), bit planes + row sums, and
// the row scale.
hipError_t launch_act_i8(const float* X, int64_t ldX, const int8_t* Xq_in, int64_t ldXq_in,
                         int64_t M, int64_t K,
                         int8_t* Q, int64_t ldQ, uint32_t* Xb, int64_t ldXb, int32_t* xsum,
                         float* xscale, hipStream_t s);

// True when the bit-plane GEMV serves binary weights x INT8 activations.
// The XNOR GEMM on the fp4 matrix cores (exact +-1 products): D and/or Y = alpha * D.
hipError_t launch_xnor_gemm_fp4(const uint32_t* Xp, int64_t ldX, const uint32_t* Wp, int64_t ldW,
                                int64_t M, int64_t N, int64_t K, int32_t* D, int64_t ldD,
                                const float* alpha, bool alpha_tensor, float* Y, int64_t ldY, hipStream_t s);

// Binary weights x fp16 activations, one activation row: y = alpha * sum_k s x_k.
int64_t f16_gemv_max_k();
hipError_t launch_bwn_f16_gemv(const uint16_t* X, const uint32_t* Wp, int64_t ldW, int64_t N, int64_t K,
                               const float* alpha, bool alpha_tensor, float* Y, hipStream_t s);

bool i8_gemv_eligible(int64_t M, int64_t K);

hipError_t launch_bwn_i8_gemv(const uint32_t* Xb, int64_t ldXb, const int32_t* xsum,
                              const uint32_t* Wp, int64_t ldW,
                              int64_t M, int64_t N, int64_t K, const EpilogueI8& e, hipStream_t s);

hipError_t launch_bwn_i8_gemm(const int8_t* Xq, int64_t ldXq, const uint32_t* Wp, int64_t ldW,
                              int64_t M, int64_t N, int64_t K, const EpilogueI8& e, hipStream_t s);

hipError_t launch_dense_f32_sign_pack(const float* X, int64_t ldX, const float* W, int64_t ldW,
                                      int64_t M, int64_t N, int64_t K,
                                      uint32_t* Op, int64_t ldOp, hipStream_t s);

hipError_t launch_dense_binact_f32(const uint32_t* Xp, int64_t ldXp, const float* W, int64_t ldW,
                                   int64_t M, int64_t N, int64_t K,
                                   float* Y, int64_t ldY, hipStream_t s);

}  // namespace bnn
