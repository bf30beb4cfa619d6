// Device-side helpers shared by the gfx950 kernels of libbnn.
//
// Encoding (page "First Principles: Why Binary Ops Can Be Exponentially
// Faster", section "1. Arithmetic: MAC -> XNOR + popcount"): bit value 0 is
// +1 and 1 is -1; element k of a row sits in word k/32 at bit k%32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bnn {

// A pointer into the constant address space: uniform loads through it become
// scalar (s_load_*) loads, so a weight row is broadcast to all 64 lanes from
// SGPRs instead of being replicated in VGPRs.
typedef const __attribute__((address_space(4))) uint32_t* cptr_u32;
typedef const __attribute__((address_space(4))) float* cptr_f32;
typedef const __attribute__((address_space(4))) int8_t* cptr_i8;

// Four 32-bit words (one 16-byte granule) as a vector.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// popcount(x) + acc as the single VALU op v_bcnt_u32_b32.  Written as asm so
// the compiler cannot re-associate a chain of accumulations into
// bcnt(x, 0) + v_add3 trees (one extra VALU op per two words).
__device__ __forceinline__ uint32_t popc_acc(uint32_t x, uint32_t acc) {
    uint32_t r;
    asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(acc));
    return r;
}

// Two accumulators over four words: c0 += sum_k popcount(x0[k] & w[k]),
// c1 += sum_k popcount(x1[k] & w[k]), with one s_nop 0 between each v_and and
// the bit count that reads it.  Measured on MI355X: a 32-bit VOP2 op (and,
// xor) issued right before or after a v_bcnt_u32_b32 of the same wave costs
// ~40% more issue time than with one nop between the two (independent or
// not); VOP2-only chains do not pay it.  The eight pairs form one asm block
// because the compiler separates consecutive asm blocks by a nop of its own.
__device__ __forceinline__ void and_popc_2x4(uint32_t& c0, uint32_t& c1, u32x4 x0, u32x4 x1, u32x4 w) {
    uint32_t t;
#define BNN_AP(X, W, C) "v_and_b32 %[t], " X ", " W "\n\ts_nop 0\n\tv_bcnt_u32_b32 " C ", %[t], " C "\n\t"
    asm(BNN_AP("%[a0]", "%[w0]", "%[c0]") BNN_AP("%[b0]", "%[w0]", "%[c1]")
        BNN_AP("%[a1]", "%[w1]", "%[c0]") BNN_AP("%[b1]", "%[w1]", "%[c1]")
        BNN_AP("%[a2]", "%[w2]", "%[c0]") BNN_AP("%[b2]", "%[w2]", "%[c1]")
        BNN_AP("%[a3]", "%[w3]", "%[c0]") BNN_AP("%[b3]", "%[w3]", "%[c1]")
        : [c0] "+v"(c0), [c1] "+v"(c1), [t] "=&v"(t)
        : [a0] "v"(x0.x), [a1] "v"(x0.y), [a2] "v"(x0.z), [a3] "v"(x0.w),
          [b0] "v"(x1.x), [b1] "v"(x1.y), [b2] "v"(x1.z), [b3] "v"(x1.w),
          [w0] "v"(w.x), [w1] "v"(w.y), [w2] "v"(w.z), [w3] "v"(w.w));
#undef BNN_AP
}

// Sign bit of an fp32 given by its bit pattern u, per the Notation of page
// "Extreme Quantization: Binary, Ternary & 1-bit LLMs": sign(x) = +1 for
// x >= 0, else -1; returned as the packed bit (0 for +1, 1 for -1).
// x >= 0 holds exactly for u in [0, 0x7F800000] (+0, positive finite incl.
// denormals, +inf) and u == 0x80000000 (-0.0); everything else (negative
// values, -inf, every NaN) is -1.  An integer test keeps the result
// independent of any denormal flushing mode of the float compare.
__device__ __forceinline__ uint32_t neg_bit(uint32_t u) {
    return (u > 0x7F800000u && u != 0x80000000u) ? 1u : 0u;
}

// OR of a 32-bit value over each aligned group of 8 consecutive lanes; the
// result is complete in the last lane of each group (lane % 8 == 7).  DPP
// row_shr with bound_ctrl reads 0 across a 16-lane row boundary, and the
// groups never straddle one.
__device__ __forceinline__ uint32_t or_reduce8_to_last(uint32_t v) {
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
    return v;
}

// Sum of a 32-bit value over each aligned group of 2^glog2 lanes (glog2 <=
// 6, wave-uniform); the total is complete in the last lane of each group.
// DPP row shifts accumulate inclusive sums inside 16-lane rows (bound_ctrl
// reads 0 before a row start; groups never straddle a row below 16 lanes);
// row_bcast15 / row_bcast31 carry row totals across rows for 32 / 64.
__device__ __forceinline__ uint32_t sum_reduce_to_last(uint32_t v, int glog2) {
    // branch-free: every step runs, steps beyond glog2 add 0
    uint32_t t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true); v += glog2 >= 1 ? t : 0u;  // row_shr:1
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true); v += glog2 >= 2 ? t : 0u;  // row_shr:2
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true); v += glog2 >= 3 ? t : 0u;  // row_shr:4
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true); v += glog2 >= 4 ? t : 0u;  // row_shr:8
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false); v += glog2 >= 5 ? t : 0u; // row_bcast:15 -> rows 1,3
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false); v += glog2 >= 6 ? t : 0u; // row_bcast:31 -> rows 2,3
    return v;
}

// The same group sum with the group size fixed at compile time: each step is
// one DPP add (the row shift folded into the add), nothing is selected.
template <int GLOG2>
__device__ __forceinline__ uint32_t sum_reduce_to_last_t(uint32_t v) {
    if (GLOG2 >= 1) v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);
    if (GLOG2 >= 2) v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);
    if (GLOG2 >= 3) v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);
    if (GLOG2 >= 4) v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);
    if (GLOG2 >= 5) v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);
    if (GLOG2 >= 6) v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
    return v;
}

}  // namespace bnn
