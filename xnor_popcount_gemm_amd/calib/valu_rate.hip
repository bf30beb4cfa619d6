// Issue-rate probes of the XOR-popcount instruction mix on gfx950, for the
// benchmark's roofline (measurement only: the product library libbnn.so does
// not contain or call this).  Each wave runs a register-only loop of one of
// three instruction streams, with its operands uniform (SGPR) and per-lane
// (VGPR) as in the GEMM's inner loop:
//   MIX : v_xor_b32 t, s, a ; s_nop 0 ; v_bcnt_u32_b32 c, t, c   (16 pairs)
//   XOR : 32 x v_xor_b32 t_i, s, a_i
//   BCNT: 32 x v_bcnt_u32_b32 c_j, a_i, c_j  (4 independent accumulators)
//   MIXV: MIX with the xor's uniform operand in a VGPR instead of an SGPR
// so the VALU lane-op rate of each stream is known exactly: 32 VALU wave
// instructions (2048 lane-ops) per loop iteration.  Wave 0 of workgroup 0
// also reads the shader clock counter (s_memtime) and the 100 MHz real-time
// counter (s_memrealtime) at its start and end, so the engine clock during
// the probe is measured.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

#define P1(A, S, C) "v_xor_b32 %[t], " S ", " A "\n\ts_nop 0\n\tv_bcnt_u32_b32 " C ", %[t], " C "\n\t"
#define P2(A, S) P1(A, S, "%[c0]") P1(A, "%[s1]", "%[c1]")
#define X1(T, S, A) "v_xor_b32 " T ", " S ", " A "\n\t"
#define X4(S) X1("%[t0]", S, "%[a0]") X1("%[t1]", S, "%[a1]") X1("%[t2]", S, "%[a2]") X1("%[t3]", S, "%[a3]")
#define B1(C, A) "v_bcnt_u32_b32 " C ", " A ", " C "\n\t"
#define B4(A) B1("%[c0]", A) B1("%[c1]", A) B1("%[c2]", A) B1("%[c3]", A)
#define V2(A, S) P1(A, S, "%[c0]") P1(A, "%[b1]", "%[c1]")

template <int MODE>
__global__ __launch_bounds__(256) void k_valu_probe(uint32_t* out, uint64_t* clk, int iters,
                                                    uint32_t s0, uint32_t s1, uint32_t s2, uint32_t s3)
{
    uint32_t a0 = threadIdx.x * 2654435761u, a1 = a0 ^ 0x9E3779B9u, a2 = a0 + 12345u, a3 = a0 * 3u;
    uint32_t c0 = 0, c1 = 0, c2 = 0, c3 = 0, t0 = 0, t1 = 0, t2 = 0, t3 = 0;
    uint32_t b0 = s0, b1 = s1, b2 = s2, b3 = s3;
    asm volatile("" : "+v"(b0), "+v"(b1), "+v"(b2), "+v"(b3));   // held in VGPRs
    const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
    uint64_t tm0 = 0, rt0 = 0;
    if (timer) { tm0 = clock64(); rt0 = wall_clock64(); }
    for (int i = 0; i < iters; ++i) {
        if constexpr (MODE == 0) {
            uint32_t t;
            asm volatile(P2("%[a0]", "%[s0]") P2("%[a1]", "%[s2]") P2("%[a2]", "%[s3]") P2("%[a3]", "%[s0]")
                         P2("%[a0]", "%[s2]") P2("%[a1]", "%[s3]") P2("%[a2]", "%[s0]") P2("%[a3]", "%[s2]")
                         : [c0] "+v"(c0), [c1] "+v"(c1), [t] "=&v"(t)
                         : [a0] "v"(a0), [a1] "v"(a1), [a2] "v"(a2), [a3] "v"(a3),
                           [s0] "s"(s0), [s1] "s"(s1), [s2] "s"(s2), [s3] "s"(s3));
        } else if constexpr (MODE == 1) {
            asm volatile(X4("%[s0]") X4("%[s1]") X4("%[s2]") X4("%[s3]") X4("%[s0]") X4("%[s1]") X4("%[s2]") X4("%[s3]")
                         : [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2), [t3] "=&v"(t3)
                         : [a0] "v"(a0), [a1] "v"(a1), [a2] "v"(a2), [a3] "v"(a3),
                           [s0] "s"(s0), [s1] "s"(s1), [s2] "s"(s2), [s3] "s"(s3));
            c0 ^= t0; c1 ^= t1; c2 ^= t2; c3 ^= t3;
        } else if constexpr (MODE == 2) {
            asm volatile(B4("%[a0]") B4("%[a1]") B4("%[a2]") B4("%[a3]") B4("%[a0]") B4("%[a1]") B4("%[a2]") B4("%[a3]")
                         : [c0] "+v"(c0), [c1] "+v"(c1), [c2] "+v"(c2), [c3] "+v"(c3)
                         : [a0] "v"(a0), [a1] "v"(a1), [a2] "v"(a2), [a3] "v"(a3));
        } else {
            // the uniform values in VGPRs (the same values as MIX's SGPRs)
            uint32_t t;
            asm volatile(V2("%[a0]", "%[b0]") V2("%[a1]", "%[b2]") V2("%[a2]", "%[b3]") V2("%[a3]", "%[b0]")
                         V2("%[a0]", "%[b2]") V2("%[a1]", "%[b3]") V2("%[a2]", "%[b0]") V2("%[a3]", "%[b2]")
                         : [c0] "+v"(c0), [c1] "+v"(c1), [t] "=&v"(t)
                         : [a0] "v"(a0), [a1] "v"(a1), [a2] "v"(a2), [a3] "v"(a3),
                           [b0] "v"(b0), [b1] "v"(b1), [b2] "v"(b2), [b3] "v"(b3));
        }
    }
    if (timer) {
        clk[0] = clock64() - tm0;
        clk[1] = wall_clock64() - rt0;
    }
    out[blockIdx.x * 256 + threadIdx.x] = c0 ^ c1 ^ c2 ^ c3;
}

}  // namespace

// Runs `mode` (0 MIX, 1 XOR, 2 BCNT, 3 MIXV) on blocks_per_cu 4-wave workgroups per
// CU (that many waves per SIMD), iters loop iterations each.  Writes the
// elapsed seconds of the timed launch, the shader-clock cycles and 100 MHz
// ticks seen by one wave, and the number of workgroups.  Returns 0 on success,
// else the HIP error code.  Allocates and frees its own buffers.
extern "C" __attribute__((visibility("default")))
int bnn_calib_valu(int mode, int blocks_per_cu, int iters, double* seconds, uint64_t* shader_cycles,
                   uint64_t* ref_ticks, int64_t* workgroups)
{
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return (int)e;
    const int blocks = cus * blocks_per_cu;
    uint32_t* out = nullptr;
    uint64_t* clk = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    if ((e = hipMalloc(&out, (size_t)blocks * 256 * sizeof(uint32_t))) != hipSuccess) return (int)e;
    if ((e = hipMalloc(&clk, 2 * sizeof(uint64_t))) != hipSuccess) { (void)hipFree(out); return (int)e; }
    e = hipEventCreate(&a);
    if (e == hipSuccess) e = hipEventCreate(&b);
    auto launch = [&](int n) {
        if (mode == 0) hipLaunchKernelGGL(k_valu_probe<0>, dim3(blocks), dim3(256), 0, 0, out, clk, n, 1u, 2u, 3u, 4u);
        else if (mode == 1) hipLaunchKernelGGL(k_valu_probe<1>, dim3(blocks), dim3(256), 0, 0, out, clk, n, 1u, 2u, 3u, 4u);
        else if (mode == 2) hipLaunchKernelGGL(k_valu_probe<2>, dim3(blocks), dim3(256), 0, 0, out, clk, n, 1u, 2u, 3u, 4u);
        else hipLaunchKernelGGL(k_valu_probe<3>, dim3(blocks), dim3(256), 0, 0, out, clk, n, 1u, 2u, 3u, 4u);
        return hipGetLastError();
    };
    if (e == hipSuccess) e = launch(iters / 4 + 1);                 // warm-up (clock ramp)
    if (e == hipSuccess) e = hipEventRecord(a, 0);
    if (e == hipSuccess) e = launch(iters);
    if (e == hipSuccess) e = hipEventRecord(b, 0);
    if (e == hipSuccess) e = hipEventSynchronize(b);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
    uint64_t hc[2] = {0, 0};
    if (e == hipSuccess) e = hipMemcpy(hc, clk, sizeof(hc), hipMemcpyDeviceToHost);
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
    (void)hipFree(out);
    (void)hipFree(clk);
    if (e != hipSuccess) return (int)e;
    *seconds = ms * 1e-3;
    *shader_cycles = hc[0];
    *ref_ticks = hc[1];
    *workgroups = blocks;
    return 0;
}
