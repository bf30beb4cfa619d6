// HBM read-stream probe for the benchmark's context figure (measurement
// only: the product library libbnn.so does not contain or call this).  A
// persistent grid reads a 2 GiB buffer once with 16-byte nontemporal loads:
// wave w takes 4 KiB chunks w, w + W, w + 2W, ... (W waves), so the chunks
// in flight at any moment are neighbours, 4 loads per lane in flight per
// chunk; each lane folds what it read into one word (xor) and stores it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_read_stream(const u32x4* __restrict__ src, int64_t chunks,
                                                     uint32_t* __restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * 256) >> 6;
    uint32_t acc = 0u;
    // a 4 KiB chunk is 256 16-byte granules: 4 per lane, lane-interleaved
    for (int64_t c = wave; c < chunks; c += nwaves) {
        const u32x4* p = src + c * 256 + lane;
        u32x4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __builtin_nontemporal_load(p + 64 * i);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    }
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 4 KiB) once per launch with blocks_per_cu
// 256-thread workgroups per CU; writes the best of `reps` timed launches
// (after one untimed) in seconds.  Returns 0 on success, else the HIP error
// code.  Allocates and frees its own buffers.
extern "C" __attribute__((visibility("default")))
int bnn_calib_read_stream(int64_t bytes, int blocks_per_cu, int reps, double* seconds)
{
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return (int)e;
    if (bytes <= 0 || bytes % 4096 != 0 || blocks_per_cu < 1 || reps < 1) return (int)hipErrorInvalidValue;
    const int blocks = cus * blocks_per_cu;
    void* buf = nullptr;
    uint32_t* out = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    if ((e = hipMalloc(&buf, (size_t)bytes)) != hipSuccess) return (int)e;
    if ((e = hipMalloc(&out, (size_t)blocks * 256 * sizeof(uint32_t))) != hipSuccess) { (void)hipFree(buf); return (int)e; }
    e = hipMemset(buf, 0x5A, (size_t)bytes);
    if (e == hipSuccess) e = hipEventCreate(&a);
    if (e == hipSuccess) e = hipEventCreate(&b);
    const int64_t chunks = bytes / 4096;
    double best = 1e30;
    for (int r = 0; r <= reps && e == hipSuccess; ++r) {
        e = hipEventRecord(a, 0);
        if (e == hipSuccess) {
            hipLaunchKernelGGL(k_read_stream, dim3(blocks), dim3(256), 0, 0,
                               reinterpret_cast<const u32x4*>(buf), chunks, out);
            e = hipGetLastError();
        }
        if (e == hipSuccess) e = hipEventRecord(b, 0);
        if (e == hipSuccess) e = hipEventSynchronize(b);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
        if (e == hipSuccess && r > 0 && ms * 1e-3 < best) best = ms * 1e-3;
    }
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
    (void)hipFree(out);
    (void)hipFree(buf);
    if (e != hipSuccess) return (int)e;
    *seconds = best;
    return 0;
}
