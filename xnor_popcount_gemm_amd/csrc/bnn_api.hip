// C ABI of libbnn: argument validation and dispatch to the gfx950 kernels.
// Every check runs before anything is launched; a failed check returns a
// status and touches nothing.  The semantics of each entry point are
// documented (with their sources on the pages) in include/bnn.h.
#include <math.h>

#include <atomic>
#include <mutex>

#include "bnn.h"
#include "bnn_launch.hpp"

// Device scratch of bnn_weight_scale_tensor_noalloc: one fp64 partial sum per
// weight row.  Each GPU holds its own copy for the life of the process; host
// code reaches it only through the address hipGetSymbolAddress returns for
// that device (the array's name in host code is a host-side stand-in).
static __device__ __align__(256) double scratch[BNN_NOALLOC_MAX_ROWS];

namespace {

using bnn::Epilogue;

bool misaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }
bool misaligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) != 0; }

int64_t words_of(int64_t K) { return (K + 31) / 32; }

hipStream_t as_stream(bnn_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

bnn_status from_hip(hipError_t e) { return e == hipSuccess ? BNN_OK : BNN_ERR_HIP; }

// Common checks of a packed operand [rows, ld] holding K bits per row.
bnn_status check_packed(const uint32_t* p, int64_t K, int64_t ld) {
    if (!p) return BNN_ERR_NULL;
    if (ld < words_of(K)) return BNN_ERR_LD;
    if (misaligned16(p) || (ld % 4) != 0) return BNN_ERR_ALIGN;
    return BNN_OK;
}

bnn_status check_k(int64_t K) {
    return (K < 1 || K > BNN_MAX_K) ? BNN_ERR_SHAPE : BNN_OK;
}

// Shapes are kept within int32 index arithmetic inside the kernels.
bnn_status check_rows(int64_t rows) {
    return (rows < 0 || rows > ((int64_t)1 << 31) - 1) ? BNN_ERR_SHAPE : BNN_OK;
}

// conv_cw > 0: the activation operand is a packed NHWC image of conv_cw
// words per pixel (implicit im2col), not an im2col matrix of K bits per row.
bnn_status validate_fused(const bnn_fused_args* a, int64_t conv_cw = 0) {
    if (!a) return BNN_ERR_NULL;
    bnn_status st;
    if ((st = check_rows(a->M)) != BNN_OK) return st;
    if ((st = check_rows(a->N)) != BNN_OK) return st;
    if ((st = check_k(a->K)) != BNN_OK) return st;
    // the GEMM grid (256-row x 16-column tiles) must fit one launch dimension
    if (((a->M + 255) / 256) * ((a->N + 15) / 16) > ((int64_t)1 << 31) - 1) return BNN_ERR_SHAPE;
    const uint32_t f = a->epilogue;
    const uint32_t known = BNN_EPI_DOT_I32 | BNN_EPI_SCALE_F32 | BNN_EPI_RESIDUAL_F32 | BNN_EPI_THRESH_PACK |
                           BNN_EPI_ALPHA_TENSOR | BNN_EPI_BIAS_F32 | BNN_W_TERNARY | BNN_EPI_SIGN_PACK;
    if ((f & ~known) != 0) return BNN_ERR_UNSUPPORTED;
    if (!(f & (BNN_EPI_DOT_I32 | BNN_EPI_SCALE_F32 | BNN_EPI_THRESH_PACK))) return BNN_ERR_UNSUPPORTED;
    if ((f & (BNN_EPI_RESIDUAL_F32 | BNN_EPI_ALPHA_TENSOR | BNN_EPI_BIAS_F32 | BNN_EPI_SIGN_PACK)) &&
        !(f & BNN_EPI_SCALE_F32))
        return BNN_ERR_UNSUPPORTED;
    if ((f & BNN_EPI_SIGN_PACK) && (f & BNN_EPI_THRESH_PACK)) return BNN_ERR_UNSUPPORTED;   // one Op
    if (conv_cw > 0 && (f & BNN_W_TERNARY)) return BNN_ERR_UNSUPPORTED;
    if (f & BNN_EPI_BIAS_F32) {
        if (!a->bias) return BNN_ERR_NULL;
        if (misaligned4(a->bias)) return BNN_ERR_ALIGN;
    }
    if (f & BNN_W_TERNARY) {
        if ((st = check_packed(a->Zp, a->K, a->ldWp)) != BNN_OK) return st;
        if (!a->nnz) return BNN_ERR_NULL;
        if (misaligned4(a->nnz)) return BNN_ERR_ALIGN;
    }
    if (conv_cw > 0) {
        if ((st = check_packed(a->Xp, 32 * conv_cw, a->ldXp)) != BNN_OK) return st;
        if (a->M * a->ldXp > ((int64_t)1 << 31) - 1) return BNN_ERR_SHAPE;   // 32-bit pixel offsets
    } else {
        if ((st = check_packed(a->Xp, a->K, a->ldXp)) != BNN_OK) return st;
    }
    if ((st = check_packed(a->Wp, a->K, a->ldWp)) != BNN_OK) return st;
    if (f & BNN_EPI_SIGN_PACK) {
        if (!a->Op) return BNN_ERR_NULL;
        if (a->ldOp < words_of(a->N)) return BNN_ERR_LD;
        if (misaligned4(a->Op) || (a->beta && misaligned4(a->beta))) return BNN_ERR_ALIGN;
    }
    if (f & BNN_EPI_DOT_I32) {
        if (!a->D) return BNN_ERR_NULL;
        if (a->ldD < a->N) return BNN_ERR_LD;
        if (misaligned4(a->D)) return BNN_ERR_ALIGN;
    }
    if (f & BNN_EPI_SCALE_F32) {
        if (!a->Y || !a->alpha) return BNN_ERR_NULL;
        if (a->ldY < a->N) return BNN_ERR_LD;
        if (misaligned4(a->Y) || misaligned4(a->alpha)) return BNN_ERR_ALIGN;
    }
    if (f & BNN_EPI_RESIDUAL_F32) {
        if (!a->R) return BNN_ERR_NULL;
        if (a->ldR < a->N) return BNN_ERR_LD;
        if (misaligned4(a->R)) return BNN_ERR_ALIGN;
        if (a->R != a->Y && a->ldR == a->ldY) {
            // partial overlap of R and Y would make the result order-dependent
            const char* r0 = reinterpret_cast<const char*>(a->R);
            const char* y0 = reinterpret_cast<const char*>(a->Y);
            const int64_t span = (a->M > 0 ? (a->M - 1) * a->ldY + a->N : 0) * (int64_t)sizeof(float);
            if (span > 0 && r0 < y0 + span && y0 < r0 + span) return BNN_ERR_UNSUPPORTED;
        }
    }
    if (f & BNN_EPI_THRESH_PACK) {
        if (!a->tau || !a->dir || !a->Op) return BNN_ERR_NULL;
        if (a->ldOp < words_of(a->N)) return BNN_ERR_LD;
        if (misaligned4(a->Op) || misaligned4(a->tau)) return BNN_ERR_ALIGN;
    }
    return BNN_OK;
}

bnn_status run_fused(const bnn_fused_args* a, hipStream_t s) {
    if (a->M == 0 || a->N == 0) return BNN_OK;
    Epilogue e;
    e.flags = a->epilogue;
    e.D = a->D; e.ldD = a->ldD;
    e.alpha = a->alpha;
    e.Y = a->Y; e.ldY = a->ldY;
    e.R = a->R; e.ldR = a->ldR;
    e.tau = a->tau; e.dir = a->dir;
    e.Op = a->Op; e.ldOp = a->ldOp;
    e.bias = a->bias;
    e.Zp = a->Zp; e.nnz = a->nnz;
    e.beta = a->beta;
    if (bnn::gemv_eligible(a->M, a->K, e.flags))
        return from_hip(bnn::launch_xnor_gemv(a->Xp, a->ldXp, a->Wp, a->ldWp, a->M, a->N, a->K, e, s));
    if ((e.flags & bnn::W_TERNARY) && bnn::tern_gemm_t_eligible())
        return from_hip(bnn::launch_tern_gemm_t(a->Xp, a->ldXp, a->Wp, a->ldWp, a->M, a->N, a->K, e, s));
    return from_hip(bnn::launch_xnor_gemm(a->Xp, a->ldXp, a->Wp, a->ldWp, a->M, a->N, a->K, e, s));
}

bnn_status check_i8_rows(const int8_t* p, int64_t K, int64_t ld) {
    if (ld < K) return BNN_ERR_LD;
    if (misaligned16(p) || (ld % 16) != 0) return BNN_ERR_ALIGN;
    return BNN_OK;
}

bnn_status check_k_i8(int64_t K) {
    return (K < 1 || K > BNN_MAX_K_I8) ? BNN_ERR_SHAPE : BNN_OK;
}

// Which kernel serves a bnn_i8_args call: 1 = bit-plane GEMV, 2 = MFMA GEMM.
int i8_path(const bnn_i8_args* a) {
    const bool tern = (a->epilogue & BNN_W_TERNARY) != 0;
    if (a->Xb && (a->xsum || tern) && (a->M == 0 || bnn::i8_gemv_eligible(a->M, a->K))) return 1;
    if (a->Xq) return 2;
    return 0;
}

bnn_status validate_i8(const bnn_i8_args* a) {
    if (!a) return BNN_ERR_NULL;
    bnn_status st;
    if ((st = check_rows(a->M)) != BNN_OK) return st;
    if ((st = check_rows(a->N)) != BNN_OK) return st;
    if ((st = check_k_i8(a->K)) != BNN_OK) return st;
    if (((a->M + 127) / 128) * ((a->N + 127) / 128) > ((int64_t)1 << 31) - 1) return BNN_ERR_SHAPE;
    const uint32_t f = a->epilogue;
    const uint32_t known = BNN_EPI_DOT_I32 | BNN_EPI_SCALE_F32 | BNN_EPI_ALPHA_TENSOR | BNN_W_TERNARY;
    if ((f & ~known) != 0 || !(f & (BNN_EPI_DOT_I32 | BNN_EPI_SCALE_F32))) return BNN_ERR_UNSUPPORTED;
    if ((f & BNN_W_TERNARY) && (st = check_packed(a->Zp, a->K, a->ldWp)) != BNN_OK) return st;
    if ((f & BNN_EPI_ALPHA_TENSOR) && !(f & BNN_EPI_SCALE_F32)) return BNN_ERR_UNSUPPORTED;
    if ((st = check_packed(a->Wp, a->K, a->ldWp)) != BNN_OK) return st;
    const int path = i8_path(a);
    if (path == 0) return BNN_ERR_NULL;
    if (path == 1) {
        if ((st = check_packed(a->Xb, a->K, a->ldXb)) != BNN_OK) return st;
        if (a->xsum && misaligned4(a->xsum)) return BNN_ERR_ALIGN;
    } else {
        if ((st = check_i8_rows(a->Xq, a->K, a->ldXq)) != BNN_OK) return st;
        if (a->xsum && misaligned4(a->xsum)) return BNN_ERR_ALIGN;
        // the GEMM addresses activation rows and weight rows with 32-bit
        // byte offsets
        if (a->M * a->ldXq > ((int64_t)1 << 31) - 1) return BNN_ERR_SHAPE;
        if (a->N * a->ldWp >= ((int64_t)1 << 29)) return BNN_ERR_SHAPE;
    }
    if (a->xscale && misaligned4(a->xscale)) return BNN_ERR_ALIGN;
    if (f & BNN_EPI_DOT_I32) {
        if (!a->D) return BNN_ERR_NULL;
        if (a->ldD < a->N) return BNN_ERR_LD;
        if (misaligned4(a->D)) return BNN_ERR_ALIGN;
    }
    if (f & BNN_EPI_SCALE_F32) {
        if (!a->Y || !a->alpha) return BNN_ERR_NULL;
        if (a->ldY < a->N) return BNN_ERR_LD;
        if (misaligned4(a->Y) || misaligned4(a->alpha)) return BNN_ERR_ALIGN;
    }
    return BNN_OK;
}

// Shared checks of the two INT8 activation writers.
bnn_status check_act_i8_out(int64_t M, int64_t K, uint32_t* Xb, int64_t ldXb, int32_t* xsum) {
    bnn_status st;
    if ((st = check_rows(M)) != BNN_OK) return st;
    if ((st = check_k_i8(K)) != BNN_OK) return st;
    if (Xb) {
        if ((st = check_packed(Xb, K, ldXb)) != BNN_OK) return st;
        if (!xsum) return BNN_ERR_NULL;
    }
    if (xsum && misaligned4(xsum)) return BNN_ERR_ALIGN;
    return BNN_OK;
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

int64_t bnn_packed_words(int64_t K) { return K < 0 ? -1 : words_of(K); }

const char* bnn_status_string(bnn_status status) {
    switch (status) {
        case BNN_OK: return "BNN_OK";
        case BNN_ERR_NULL: return "BNN_ERR_NULL: a required pointer is NULL";
        case BNN_ERR_SHAPE: return "BNN_ERR_SHAPE: a size is negative or out of range";
        case BNN_ERR_LD: return "BNN_ERR_LD: a leading dimension is smaller than the row";
        case BNN_ERR_ALIGN: return "BNN_ERR_ALIGN: a packed operand is misaligned";
        case BNN_ERR_UNSUPPORTED: return "BNN_ERR_UNSUPPORTED: unsupported flags or geometry";
        case BNN_ERR_HIP: return "BNN_ERR_HIP: the HIP runtime reported a launch error";
    }
    return "unknown bnn_status";
}

bnn_status bnn_pack_weights(const float* W, int64_t N, int64_t K, int64_t ldW,
                            uint32_t* Wp, int64_t ldWp, float* alpha, bnn_stream_t stream)
{
    bnn_status st;
    if ((st = check_rows(N)) != BNN_OK) return st;
    if ((st = check_k(K)) != BNN_OK) return st;
    if (!W) return BNN_ERR_NULL;
    if (ldW < K) return BNN_ERR_LD;
    if (misaligned4(W)) return BNN_ERR_ALIGN;
    if ((st = check_packed(Wp, K, ldWp)) != BNN_OK) return st;
    if (alpha && misaligned4(alpha)) return BNN_ERR_ALIGN;
    if (N == 0) return BNN_OK;
    return from_hip(bnn::launch_pack_dense(W, N, K, ldW, Wp, ldWp, alpha, as_stream(stream)));
}

bnn_status bnn_pack_activations(const float* X, int64_t M, int64_t K, int64_t ldX,
                                const bnn_conv_geom* geom, uint32_t* Xp, int64_t ldXp,
                                bnn_stream_t stream)
{
    bnn_status st;
    if ((st = check_rows(M)) != BNN_OK) return st;
    if ((st = check_k(K)) != BNN_OK) return st;
    if (!X) return BNN_ERR_NULL;
    if (misaligned4(X)) return BNN_ERR_ALIGN;
    if ((st = check_packed(Xp, K, ldXp)) != BNN_OK) return st;
    if (geom) {
        if (geom->R != 3 || geom->S != 3 || geom->stride != 1 || geom->pad != 1) return BNN_ERR_UNSUPPORTED;
        if (geom->B < 0 || geom->H < 1 || geom->W < 1 || geom->C < 1) return BNN_ERR_SHAPE;
        if (geom->H > 65535 || geom->W > 65535) return BNN_ERR_SHAPE;
        if (geom->B * geom->H * geom->W != M || 9 * geom->C != K) return BNN_ERR_SHAPE;
        if (geom->B * geom->H * geom->W * geom->C > ((int64_t)1 << 40)) return BNN_ERR_SHAPE;
        if (M == 0) return BNN_OK;
        return from_hip(bnn::launch_pack_im2col3x3(X, geom->B, geom->H, geom->W, geom->C,
                                                   Xp, ldXp, as_stream(stream)));
    }
    if (ldX < K) return BNN_ERR_LD;
    if (M == 0) return BNN_OK;
    return from_hip(bnn::launch_pack_dense(X, M, K, ldX, Xp, ldXp, nullptr, as_stream(stream)));
}

bnn_status bnn_xnor_gemm(const uint32_t* Xp, int64_t ldXp, const uint32_t* Wp, int64_t ldWp,
                         int64_t M, int64_t N, int64_t K,
                         int32_t* D, int64_t ldD, const float* alpha, float* Y, int64_t ldY,
                         bnn_stream_t stream)
{
    if (!D && !Y) return BNN_ERR_NULL;
    bnn_fused_args a = {};
    a.Xp = Xp; a.ldXp = ldXp; a.Wp = Wp; a.ldWp = ldWp;
    a.M = M; a.N = N; a.K = K;
    a.epilogue = (D ? BNN_EPI_DOT_I32 : 0u) | (Y ? BNN_EPI_SCALE_F32 : 0u);
    a.D = D; a.ldD = ldD; a.alpha = alpha; a.Y = Y; a.ldY = ldY;
    const bnn_status st = validate_fused(&a);
    if (st != BNN_OK) return st;
    return run_fused(&a, as_stream(stream));
}

bnn_status bnn_xnor_gemm_mfma(const uint32_t* Xp, int64_t ldXp, const uint32_t* Wp, int64_t ldWp,
                              int64_t M, int64_t N, int64_t K,
                              int32_t* D, int64_t ldD, const float* alpha, float* Y, int64_t ldY,
                              bnn_stream_t stream)
{
    if (!D && !Y) return BNN_ERR_NULL;
    bnn_fused_args a = {};
    a.Xp = Xp; a.ldXp = ldXp; a.Wp = Wp; a.ldWp = ldWp;
    a.M = M; a.N = N; a.K = K;
    a.epilogue = (D ? BNN_EPI_DOT_I32 : 0u) | (Y ? BNN_EPI_SCALE_F32 : 0u);
    a.D = D; a.ldD = ldD; a.alpha = alpha; a.Y = Y; a.ldY = ldY;
    const bnn_status st = validate_fused(&a);
    if (st != BNN_OK) return st;
    if (M == 0 || N == 0) return BNN_OK;
    return from_hip(bnn::launch_xnor_gemm_fp4(Xp, ldXp, Wp, ldWp, M, N, K, D, ldD, alpha, false, Y, ldY,
                                              as_stream(stream)));
}

bnn_status bnn_linear_fused(const bnn_fused_args* args, bnn_stream_t stream)
{
    const bnn_status st = validate_fused(args);
    if (st != BNN_OK) return st;
    return run_fused(args, as_stream(stream));
}

bnn_status bnn_pack_activations_rsign(const float* X, int64_t M, int64_t K, int64_t ldX, const float* beta,
                                     uint32_t* Xp, int64_t ldXp, bnn_stream_t stream)
{
    bnn_status st;
    if ((st = check_rows(M)) != BNN_OK) return st;
    if ((st = check_k(K)) != BNN_OK) return st;
    if (!X || !beta) return BNN_ERR_NULL;
    if ((st = check_packed(Xp, K, ldXp)) != BNN_OK) return st;
    if (ldX < K) return BNN_ERR_LD;
    if (misaligned4(X) || misaligned4(beta)) return BNN_ERR_ALIGN;
    if (M == 0) return BNN_OK;
    return from_hip(bnn::launch_pack_dense_rsign(X, M, K, ldX, beta, Xp, ldXp, as_stream(stream)));
}

bnn_status bnn_conv3x3_fused(const bnn_fused_args* args, const bnn_conv_geom* geom, bnn_stream_t stream)
{
    if (!args || !geom) return BNN_ERR_NULL;
    if (geom->R != 3 || geom->S != 3 || geom->stride != 1 || geom->pad != 1) return BNN_ERR_UNSUPPORTED;
    if (geom->B < 0 || geom->H < 1 || geom->W < 1 || geom->C < 1) return BNN_ERR_SHAPE;
    const int64_t C = geom->C;
    if (C != 64 && C != 128 && C != 256 && C != 512) return BNN_ERR_UNSUPPORTED;
    if (args->M != geom->B * geom->H * geom->W || args->K != 9 * C) return BNN_ERR_SHAPE;
    const bnn_status st = validate_fused(args, C / 32);
    if (st != BNN_OK) return st;
    if (args->M == 0 || args->N == 0) return BNN_OK;
    Epilogue e;
    e.flags = args->epilogue;
    e.D = args->D; e.ldD = args->ldD;
    e.alpha = args->alpha;
    e.Y = args->Y; e.ldY = args->ldY;
    e.R = args->R; e.ldR = args->ldR;
    e.tau = args->tau; e.dir = args->dir;
    e.Op = args->Op; e.ldOp = args->ldOp;
    e.bias = args->bias;
    e.Zp = nullptr; e.nnz = nullptr;
    e.beta = args->beta;
    return from_hip(bnn::launch_xnor_conv3x3(args->Xp, args->ldXp, args->Wp, args->ldWp, args->M, args->N,
                                             geom->H, geom->W, (int)(C / 32), e, as_stream(stream)));
}

bnn_status bnn_pack_weights_ternary(const float* W, int64_t N, int64_t K, int64_t ldW,
                                    const float* gamma, float delta,
                                    uint32_t* Sp, uint32_t* Zp, int64_t ld, int32_t* nnz,
                                    bnn_stream_t stream)
{
    bnn_status st;
    if ((st = check_rows(N)) != BNN_OK) return st;
    if ((st = check_k(K)) != BNN_OK) return st;
    if (!W || !nnz) return BNN_ERR_NULL;
    if ((st = check_packed(Sp, K, ld)) != BNN_OK) return st;
    if ((st = check_packed(Zp, K, ld)) != BNN_OK) return st;
    if (ldW < K) return BNN_ERR_LD;
    if (misaligned4(W) || misaligned4(nnz) || (gamma && misaligned4(gamma))) return BNN_ERR_ALIGN;
    if (N == 0) return BNN_OK;
    return from_hip(bnn::launch_pack_ternary(W, N, K, ldW, gamma, delta, Sp, Zp, ld, nnz, as_stream(stream)));
}

bnn_status bnn_weight_scale_tensor(const float* W, int64_t N, int64_t K, int64_t ldW,
                                   double* work, float* alpha, bnn_stream_t stream)
{
    bnn_status st;
    if ((st = check_rows(N)) != BNN_OK) return st;
    if ((st = check_k(K)) != BNN_OK) return st;
    if (N < 1) return BNN_ERR_SHAPE;
    if (!W || !work || !alpha) return BNN_ERR_NULL;
    if (ldW < K) return BNN_ERR_LD;
    if (misaligned4(W) || misaligned4(alpha) || (reinterpret_cast<uintptr_t>(work) & 7u) != 0)
        return BNN_ERR_ALIGN;
    return from_hip(bnn::launch_alpha_tensor(W, N, K, ldW, work, alpha, as_stream(stream)));
}

namespace {

constexpr int kMaxDevices = 64;
std::atomic<double*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The scratch array's device address on the current device, looked up once
// per device (with that device current) and kept; nullptr on failure.
double* scratch_on_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    double* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
        void* addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
        p = static_cast<double*>(addr);
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

bnn_status bnn_weight_scale_tensor_noalloc(const float* W, int64_t N, int64_t K, int64_t ldW,
                                           float* alpha, bnn_stream_t stream)
{
    bnn_status st;
    if ((st = check_rows(N)) != BNN_OK) return st;
    if ((st = check_k(K)) != BNN_OK) return st;
    if (N < 1 || N > BNN_NOALLOC_MAX_ROWS) return BNN_ERR_SHAPE;
    if (!W || !alpha) return BNN_ERR_NULL;
    if (ldW < K) return BNN_ERR_LD;
    if (misaligned4(W) || misaligned4(alpha)) return BNN_ERR_ALIGN;
    double* work = scratch_on_current_device();
    if (!work) return BNN_ERR_HIP;
    // every row's partial sum is written before the second pass reads it, so
    // the scratch needs no clearing between calls
    return from_hip(bnn::launch_alpha_tensor(W, N, K, ldW, work, alpha, as_stream(stream)));
}

bnn_status bnn_quantize_act_i8(const float* X, int64_t M, int64_t K, int64_t ldX,
                               int8_t* Xq, int64_t ldXq,
                               uint32_t* Xb, int64_t ldXb, int32_t* xsum,
                               float* xscale, bnn_stream_t stream)
{
    bnn_status st;
    if ((st = check_act_i8_out(M, K, Xb, ldXb, xsum)) != BNN_OK) return st;
    if (!X || !xscale || (!Xq && !Xb)) return BNN_ERR_NULL;
    if (ldX < K) return BNN_ERR_LD;
    if (Xq && ldXq < K) return BNN_ERR_LD;
    if (misaligned4(X) || misaligned4(xscale)) return BNN_ERR_ALIGN;
    if (M == 0) return BNN_OK;
    return from_hip(bnn::launch_act_i8(X, ldX, nullptr, 0, M, K, Xq, ldXq, Xb, ldXb, xsum, xscale,
                                       as_stream(stream)));
}

bnn_status bnn_pack_act_i8(const int8_t* Xq, int64_t M, int64_t K, int64_t ldXq,
                           uint32_t* Xb, int64_t ldXb, int32_t* xsum, bnn_stream_t stream)
{
    bnn_status st;
    if (!Xq || !Xb) return BNN_ERR_NULL;
    if ((st = check_act_i8_out(M, K, Xb, ldXb, xsum)) != BNN_OK) return st;
    if (ldXq < K) return BNN_ERR_LD;
    if (M == 0) return BNN_OK;
    return from_hip(bnn::launch_act_i8(nullptr, 0, Xq, ldXq, M, K, nullptr, 0, Xb, ldXb, xsum, nullptr,
                                       as_stream(stream)));
}

bnn_status bnn_bwn_i8_linear(const bnn_i8_args* args, bnn_stream_t stream)
{
    const bnn_status st = validate_i8(args);
    if (st != BNN_OK) return st;
    if (args->M == 0 || args->N == 0) return BNN_OK;
    bnn::EpilogueI8 e;
    e.flags = args->epilogue;
    e.D = args->D; e.ldD = args->ldD;
    e.alpha = args->alpha;
    e.xscale = args->xscale;
    e.Y = args->Y; e.ldY = args->ldY;
    e.Zp = args->Zp;
    e.xsum = (args->epilogue & BNN_W_TERNARY) ? nullptr : args->xsum;
    hipStream_t s = as_stream(stream);
    if (i8_path(args) == 1)
        return from_hip(bnn::launch_bwn_i8_gemv(args->Xb, args->ldXb, args->xsum, args->Wp, args->ldWp,
                                                args->M, args->N, args->K, e, s));
    return from_hip(bnn::launch_bwn_i8_gemm(args->Xq, args->ldXq, args->Wp, args->ldWp,
                                            args->M, args->N, args->K, e, s));
}

bnn_status bnn_bwn_f16_gemv(const uint16_t* X, int64_t ldX, const uint32_t* Wp, int64_t ldWp,
                            int64_t M, int64_t N, int64_t K, uint32_t epilogue,
                            const float* alpha, float* Y, int64_t ldY, bnn_stream_t stream)
{
    bnn_status st;
    if ((st = check_rows(M)) != BNN_OK) return st;
    if ((st = check_rows(N)) != BNN_OK) return st;
    if (K < 1 || K > BNN_MAX_K_F16 || K > bnn::f16_gemv_max_k()) return BNN_ERR_SHAPE;
    if (epilogue & ~(uint32_t)(BNN_EPI_SCALE_F32 | BNN_EPI_ALPHA_TENSOR)) return BNN_ERR_UNSUPPORTED;
    if (!(epilogue & BNN_EPI_SCALE_F32)) return BNN_ERR_UNSUPPORTED;
    if ((st = check_packed(Wp, K, ldWp)) != BNN_OK) return st;
    if (!X || !alpha || !Y) return BNN_ERR_NULL;
    if (ldX < K || ldY < N) return BNN_ERR_LD;
    if (misaligned16(X) || ldX % 8 != 0 || misaligned4(alpha) || misaligned4(Y)) return BNN_ERR_ALIGN;
    if (M == 0 || N == 0) return BNN_OK;
    hipStream_t s = as_stream(stream);
    const bool at = (epilogue & BNN_EPI_ALPHA_TENSOR) != 0;
    for (int64_t m = 0; m < M; ++m) {
        const hipError_t e = bnn::launch_bwn_f16_gemv(X + m * ldX, Wp, ldWp, N, K, alpha, at, Y + m * ldY, s);
        if (e != hipSuccess) return BNN_ERR_HIP;
    }
    return BNN_OK;
}

bnn_status bnn_dense_f32_sign_pack(const float* X, int64_t ldX, const float* W, int64_t ldW,
                                   int64_t M, int64_t N, int64_t K,
                                   uint32_t* Op, int64_t ldOp, bnn_stream_t stream)
{
    bnn_status st;
    if ((st = check_rows(M)) != BNN_OK) return st;
    if ((st = check_rows(N)) != BNN_OK) return st;
    if ((st = check_k(K)) != BNN_OK) return st;
    if (!X || !W || !Op) return BNN_ERR_NULL;
    if (ldX < K || ldW < K || ldOp < words_of(N)) return BNN_ERR_LD;
    if (misaligned4(X) || misaligned4(W) || misaligned4(Op)) return BNN_ERR_ALIGN;
    if (M == 0) return BNN_OK;
    if (N == 0) return BNN_ERR_SHAPE;   // a packed output row needs at least one column
    return from_hip(bnn::launch_dense_f32_sign_pack(X, ldX, W, ldW, M, N, K, Op, ldOp, as_stream(stream)));
}

bnn_status bnn_dense_binact_f32(const uint32_t* Xp, int64_t ldXp, const float* W, int64_t ldW,
                                int64_t M, int64_t N, int64_t K,
                                float* Y, int64_t ldY, bnn_stream_t stream)
{
    bnn_status st;
    if ((st = check_rows(M)) != BNN_OK) return st;
    if ((st = check_rows(N)) != BNN_OK) return st;
    if ((st = check_k(K)) != BNN_OK) return st;
    if ((st = check_packed(Xp, K, ldXp)) != BNN_OK) return st;
    if (!W || !Y) return BNN_ERR_NULL;
    if (ldW < K || ldY < N) return BNN_ERR_LD;
    if (misaligned4(W) || misaligned4(Y)) return BNN_ERR_ALIGN;
    if (M == 0 || N == 0) return BNN_OK;
    return from_hip(bnn::launch_dense_binact_f32(Xp, ldXp, W, ldW, M, N, K, Y, ldY, as_stream(stream)));
}

}  // extern "C"
#pragma GCC visibility pop
