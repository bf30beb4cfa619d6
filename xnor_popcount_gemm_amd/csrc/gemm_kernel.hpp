// Kernel templates of the XNOR-popcount GEMM (dense rows and the implicit-im2col
// 3x3 convolution); included by gemm.hip and conv.hip, which instantiate them.
// XNOR-popcount GEMM for gfx950, with fused epilogues.
//
// Method (cited by page title and section / equation):
//  - <w,x> = N - 2 popcount(w_bit xor x_bit) with bit 0 = +1, bit 1 = -1 and
//    pad bits +1: "First Principles: Why Binary Ops Can Be Exponentially
//    Faster", section "1. Arithmetic: MAC -> XNOR + popcount"; the same
//    identity is eq. (6) of "Extreme Quantization: Binary, Ternary & 1-bit
//    LLMs" (section "XNOR-Net").
//  - y = alpha * (w_b^T x): "Extreme Quantization", eq. (1).
//  - batch-1 inference is bound by fetching the packed weights (about MN/8
//    bytes): "First Principles", sections "The cost of a neural network
//    step" and "Bandwidth math".
//  - BatchNorm followed by the next layer's sign: "Binary Neural Network
//    (BNN)" glossary, eq. (4) of "Extreme Quantization"; FP residual
//    shortcut: "State of the Art Survey", Bi-Real Net row.
//
// GEMM design (CDNA4, wave64, no MFMA -- the contraction is over bits):
//  - One lane owns one output row m; a wave owns 64 rows, a 256-thread
//    workgroup 256 rows x TN output columns.  Each lane keeps TN int32
//    popcount accumulators.
//  - The activation row is read K-chunk by K-chunk into VGPRs (KC words,
//    16-byte vector loads).  The TN weight rows of the tile are uniform
//    across the wave, so they are read with scalar loads (s_load_dwordx16)
//    into SGPRs and broadcast to all 64 lanes by the VALU's scalar operand:
//    each output word costs exactly v_xor_b32 (SGPR ^ VGPR) + v_bcnt_u32_b32
//    (popcount + accumulate), 2 VALU ops per 32 binary MACs, with no LDS
//    traffic and no barriers.  Scalar loads of the next column pair are
//    issued before the current pair's VALU ops (double-buffered SGPRs); one
//    vector load per lane and K-chunk brings the next chunk's weight lines
//    into L2 ahead of them.
//  - The xor and the bit count of each word are separated by one s_nop (see
//    xor_popc_2cols); the activation chunks alternate between two register
//    buffers, two chunks per loop iteration.
//  - Epilogue per lane: D = K - 2*acc, alpha scale, residual, or the folded
//    BatchNorm threshold with the output bits packed along n in registers
//    (TN/32 words per lane, no cross-lane traffic).


#pragma once

#include <stdlib.h>

#include "bnn_device.hpp"
#include "bnn_launch.hpp"

namespace bnn {
namespace {


typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load_granules(uint32_t* a, const uint32_t* __restrict__ src, int n4) {
#pragma unroll
    for (int q = 0; q < n4; ++q) {
        const uint4 v = *reinterpret_cast<const uint4*>(src + 4 * q);
        a[4 * q] = v.x; a[4 * q + 1] = v.y; a[4 * q + 2] = v.z; a[4 * q + 3] = v.w;
    }
}

// Two columns' accumulators c0, c1 over NW words: c0 += popcount(a[i] ^ u[i]),
// c1 += popcount(a[i] ^ v[i]) (u, v uniform, in SGPRs).  Each bit count is
// separated from the xor that produces its operand by one s_nop 0, and
// nothing else sits between the pairs.  Measured on MI355X (xor/bcnt
// streams, 4 waves per SIMD): a v_bcnt_u32_b32 right after the VALU op that
// writes its operand runs at ~63% of the mixed issue peak, with one nop in
// between at ~90%, and with a second nop after the bit count at ~70%.  One
// asm block covers NW words of both columns because the compiler puts a nop
// of its own between consecutive asm blocks.
#define BNN_XP(A, W, C) "v_xor_b32 %[t], " W ", " A "\n\ts_nop 0\n\tv_bcnt_u32_b32 " C ", %[t], " C "\n\t"
#define BNN_XP2(I) BNN_XP("%[a" #I "]", "%[u" #I "]", "%[c0]") BNN_XP("%[a" #I "]", "%[v" #I "]", "%[c1]")
#define BNN_XIN(I) [a##I] "v"(a[I]), [u##I] "s"(u[I]), [v##I] "s"(v[I])
template <int NW>
__device__ __forceinline__ void xor_popc_2cols(uint32_t& c0, uint32_t& c1, const uint32_t* a, const uint32_t* u,
                                               const uint32_t* v)
{
    uint32_t t;
    if constexpr (NW == 8) {
        asm(BNN_XP2(0) BNN_XP2(1) BNN_XP2(2) BNN_XP2(3) BNN_XP2(4) BNN_XP2(5) BNN_XP2(6) BNN_XP2(7)
            : [c0] "+v"(c0), [c1] "+v"(c1), [t] "=&v"(t)
            : BNN_XIN(0), BNN_XIN(1), BNN_XIN(2), BNN_XIN(3), BNN_XIN(4), BNN_XIN(5), BNN_XIN(6), BNN_XIN(7));
    } else if constexpr (NW == 4) {
        asm(BNN_XP2(0) BNN_XP2(1) BNN_XP2(2) BNN_XP2(3)
            : [c0] "+v"(c0), [c1] "+v"(c1), [t] "=&v"(t)
            : BNN_XIN(0), BNN_XIN(1), BNN_XIN(2), BNN_XIN(3));
    } else if constexpr (NW == 2) {
        asm(BNN_XP2(0) BNN_XP2(1)
            : [c0] "+v"(c0), [c1] "+v"(c1), [t] "=&v"(t)
            : BNN_XIN(0), BNN_XIN(1));
    } else {
        static_assert(NW == 1, "blocks of 8, 4, 2 or 1 words");
        asm(BNN_XP2(0)
            : [c0] "+v"(c0), [c1] "+v"(c1), [t] "=&v"(t)
            : BNN_XIN(0));
    }
}
#undef BNN_XIN
#undef BNN_XP2
#undef BNN_XP

// Scalar loads of the KCC words of CP consecutive weight rows starting at p
// (rows past the last live column re-read it).  MASK zeroes words >= nvalid.
template <int CP, int KCC, bool FULLN, bool MASK>
__device__ __forceinline__ void load_w(uint32_t (&w)[CP][KCC], cptr_u32 p, int64_t ldw, int j0, int nlast,
                                       int nvalid)
{
#pragma unroll
    for (int c = 0; c < CP; ++c) {
        const cptr_u32 q = FULLN ? p + c * ldw : p + (int64_t)min(j0 + c, nlast) * ldw;
#pragma unroll
        for (int kk = 0; kk < KCC; ++kk) w[c][kk] = (!MASK || kk < nvalid) ? q[kk] : 0u;
    }
}

// One K-chunk of KCC words for all TN columns.  The activation words a[] are
// already in VGPRs.  Weight rows are scalar-loaded CP columns per step into
// one of two SGPR sets: the loads of step s+1 are issued (and pinned there
// by a scheduling barrier) before the 2*CP*KCC VALU ops of step s, so each
// wait on the scalar counter (which must be lgkmcnt(0): scalar loads return
// out of order) comes a full step after its loads were issued.
// MASK: only the first nvalid words are live (the K tail).  FULLN: every
// column of the tile exists; otherwise columns past nlast re-read the last
// weight row (their results are discarded).
// TERN: ternary weights -- wbase rows are the sign plane, zbase rows (same
// stride) the nonzero plane, and a word contributes popcount((a ^ s) & z).
template <int TN, int KCC, int CP, bool FULLN, bool MASK, bool TERN>
__device__ __forceinline__ void xnor_chunk(uint32_t (&acc)[TN], const uint32_t (&a)[KCC],
                                           const uint32_t* __restrict__ wbase, const uint32_t* __restrict__ zbase,
                                           int k0, int nvalid, int64_t ldW, int nlast)
{
    int64_t ldw = ldW;
    asm volatile("" : "+s"(ldw));   // keep the TN row offsets out of the loop preheader
    const cptr_u32 p0 = (cptr_u32)(wbase + k0);
    const cptr_u32 z0 = (cptr_u32)((TERN ? zbase : wbase) + k0);
    uint32_t wc[CP][KCC], zc[CP][KCC];
    load_w<CP, KCC, FULLN, MASK>(wc, p0, ldw, 0, nlast, nvalid);
    if (TERN) load_w<CP, KCC, FULLN, MASK>(zc, z0, ldw, 0, nlast, nvalid);
#pragma unroll
    for (int j = 0; j < TN; j += CP) {
        // Consume the current set's scalar loads here (the counter wait lands
        // before the next loads are issued, not after them).
#pragma unroll
        for (int c = 0; c < CP; ++c)
#pragma unroll
            for (int kk = 0; kk < KCC; ++kk) {
                asm volatile("" : : "s"(wc[c][kk]));
                if (TERN) asm volatile("" : : "s"(zc[c][kk]));
            }
        uint32_t wn[CP][KCC], zn[CP][KCC];
        if (j + CP < TN) {
            load_w<CP, KCC, FULLN, MASK>(wn, p0 + (FULLN ? (int64_t)(j + CP) * ldw : 0), ldw, j + CP, nlast, nvalid);
            if (TERN)
                load_w<CP, KCC, FULLN, MASK>(zn, z0 + (FULLN ? (int64_t)(j + CP) * ldw : 0), ldw, j + CP, nlast, nvalid);
        }
        __builtin_amdgcn_sched_barrier(0);
        // word-outer, column-inner: CP independent accumulator chains interleave
        if constexpr (TERN) {
            // (a ^ s) & z compiles to v_mov + v_bitop3; with the bit count that
            // order already issues near the rate a nop-separated one reaches
#pragma unroll
            for (int kk = 0; kk < KCC; ++kk)
#pragma unroll
                for (int c = 0; c < CP; ++c)
                    acc[j + c] = popc_acc((a[kk] ^ wc[c][kk]) & zc[c][kk], acc[j + c]);
        } else {
            static_assert(CP == 2, "two columns per step");
            constexpr int NB = KCC % 8 == 0 ? 8 : KCC % 4 == 0 ? 4 : KCC % 2 == 0 ? 2 : 1;
#pragma unroll
            for (int k = 0; k < KCC; k += NB)
                xor_popc_2cols<NB>(acc[j], acc[j + 1], &a[k], &wc[0][k], &wc[1][k]);
        }
        if (j + CP < TN) {
#pragma unroll
            for (int c = 0; c < CP; ++c)
#pragma unroll
                for (int kk = 0; kk < KCC; ++kk) {
                    wc[c][kk] = wn[c][kk];
                    if (TERN) zc[c][kk] = zn[c][kk];
                }
        }
    }
}

// One dword per weight row of the tile at word offset k, loaded by the
// vector path: it brings the row's next cache line into L2 a whole chunk
// before the scalar loads ask for it, so a scalar-cache miss is served by L2
// instead of waiting on memory.  Lane l takes row l % TN (ternary: the
// nonzero plane on the second half of the lanes when TN <= 32); rows past
// the last live column take that column.
template <int TN, bool TERN>
__device__ __forceinline__ uint32_t touch_w(const uint32_t* __restrict__ wbase, const uint32_t* __restrict__ zbase,
                                            int64_t ldW, int k, int nlast)
{
    const int lane = threadIdx.x & 63;
    const int r = min(lane & (TN - 1), nlast);
    const uint32_t* base = (TERN && TN <= 32 && (lane & TN)) ? zbase : wbase;
    return base[(int64_t)r * ldW + k];
}

template <int TN, int KC, bool FULLN, bool TERN>
__device__ __forceinline__ void xnor_mainloop(uint32_t (&acc)[TN], const uint32_t* __restrict__ xrow,
                                              const uint32_t* __restrict__ wbase, const uint32_t* __restrict__ zbase,
                                              int Kw, int64_t ldW, int nlast)
{
    constexpr int CP = (TN >= 2) ? 2 : 1;
    const int kfull = (Kw / KC) * KC;
    // activation chunk double-buffered: the next chunk's vector loads are in
    // flight during this chunk's VALU work.  Two chunks per iteration with the
    // buffers' roles swapped, so no register copies between chunks.
    uint32_t a0[KC], a1[KC];
    uint32_t tw = 0u;
    if (kfull > 0) load_granules(a0, xrow, KC / 4);
    int k0 = 0;
    for (; k0 + 2 * KC <= kfull; k0 += 2 * KC) {
        // take delivery of a chunk (issued one chunk ago) before the next
        // chunk's loads go out, so no wait ever covers a fresh prefetch
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) asm volatile("" : : "v"(a0[kk]));
        asm volatile("" : : "v"(tw));
        load_granules(a1, xrow + k0 + KC, KC / 4);
        tw = touch_w<TN, TERN>(wbase, zbase, ldW, k0 + KC, nlast);
        xnor_chunk<TN, KC, CP, FULLN, false, TERN>(acc, a0, wbase, zbase, k0, KC, ldW, nlast);
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) asm volatile("" : : "v"(a1[kk]));
        asm volatile("" : : "v"(tw));
        if (k0 + 2 * KC < kfull) {
            load_granules(a0, xrow + k0 + 2 * KC, KC / 4);
            tw = touch_w<TN, TERN>(wbase, zbase, ldW, k0 + 2 * KC, nlast);
        }
        xnor_chunk<TN, KC, CP, FULLN, false, TERN>(acc, a1, wbase, zbase, k0 + KC, KC, ldW, nlast);
    }
    if (k0 < kfull) {                             // an odd last chunk, already in a0
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) asm volatile("" : : "v"(a0[kk]));
        xnor_chunk<TN, KC, CP, FULLN, false, TERN>(acc, a0, wbase, zbase, k0, KC, ldW, nlast);
    }
    // The K tail: one 8-word chunk when at least 8 words remain (16-word main
    // chunks), then 16-byte granules; only a granule that reaches past Kw is
    // masked (rows hold ld >= roundup(Kw, 4) words, so its loads stay inside).
    int kt = kfull;
    if (KC == 16 && Kw - kt >= 8) {
        uint32_t t8[8];
        load_granules(t8, xrow + kt, 2);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) asm volatile("" : : "v"(t8[kk]));
        xnor_chunk<TN, 8, CP, FULLN, false, TERN>(acc, t8, wbase, zbase, kt, 8, ldW, nlast);
        kt += 8;
    }
    for (; kt < Kw; kt += 4) {
        const int nvalid = min(4, Kw - kt);
        uint32_t t[4];
        load_granules(t, xrow + kt, 1);
        if (nvalid == 4) {
            xnor_chunk<TN, 4, CP, FULLN, false, TERN>(acc, t, wbase, zbase, kt, 4, ldW, nlast);
        } else {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) t[kk] = (kk < nvalid) ? t[kk] : 0u;
            xnor_chunk<TN, 4, CP, FULLN, true, TERN>(acc, t, wbase, zbase, kt, nvalid, ldW, nlast);
        }
    }
}

// Implicit im2col of a 3x3 / stride 1 / pad 1 binary convolution: the
// activation operand is the packed NHWC image (one row of CW = C/32 words
// per pixel, row stride ldc) and the virtual im2col row of output pixel p is
// the CW words of each of its 9 neighbours (tap t = 3 kh + kw; k = t C + c,
// the layout of the explicit im2col and of OHWI weights).  Taps outside the
// image are +1, i.e. zero words ("First Principles", section "1.
// Arithmetic": pad bits encode +1).  The neighbour of tap t sits at word
// offset base + (t/3 - 1) rowstep + (t%3 - 1) ldx (the last two terms are
// uniform, so only base and the in-image bit mask take vector registers).
// The 9 CW words run through KC-word chunks (TPC = KC/CW taps per chunk;
// the last 9 CW % KC words form a short tail chunk); the next chunk's
// neighbour loads are in flight during the current chunk's VALU work.
struct Taps {
    int base;        // word offset of the lane's own pixel
    uint32_t in;     // bit t: tap t lies inside the image
    int rowstep;     // words per image row (W ldx)
    int ldx;         // words per pixel
    __device__ __forceinline__ int off(int t) const { return base + (t / 3 - 1) * rowstep + (t % 3 - 1) * ldx; }
    __device__ __forceinline__ bool inside(int t) const { return (in >> t) & 1u; }
};
// Branch-free: a tap outside the image loads row 0 of the image, and
// conv_chunk_mask zeroes its words when the chunk is consumed (not at the
// load, which would wait for the data at once).  Every load is issued on
// every path, so the waits on the vector-memory counter stay exact (a branch
// around a load makes the compiler wait for all loads in flight).
template <int CW>
__device__ __forceinline__ void conv_chunk_load(uint32_t* a, const uint32_t* __restrict__ Xp,
                                                const Taps& tp, int t0, int ntaps)
{
#pragma unroll
    for (int t = 0; t < ntaps; ++t) {
        const uint32_t* __restrict__ src = Xp + (tp.inside(t0 + t) ? tp.off(t0 + t) : 0);
        if (CW >= 4) {
#pragma unroll
            for (int q = 0; q < CW / 4; ++q) {
                const uint4 v = *reinterpret_cast<const uint4*>(src + 4 * q);
                a[t * CW + 4 * q] = v.x; a[t * CW + 4 * q + 1] = v.y;
                a[t * CW + 4 * q + 2] = v.z; a[t * CW + 4 * q + 3] = v.w;
            }
        } else {
            const uint2 v = *reinterpret_cast<const uint2*>(src);
            a[t * CW] = v.x; a[t * CW + 1] = v.y;
        }
    }
}

template <int CW>
__device__ __forceinline__ void conv_chunk_mask(uint32_t* a, const Taps& tp, int t0, int ntaps)
{
#pragma unroll
    for (int t = 0; t < ntaps; ++t) {
        const bool in = tp.inside(t0 + t);
#pragma unroll
        for (int i = 0; i < CW; ++i) a[t * CW + i] = in ? a[t * CW + i] : 0u;
    }
}

// pfr: the lane's row of the residual tile, touched once per 128-byte line
// once the last chunk's data has arrived, so the tile streams in during the
// last chunk's VALU work with no wait placed on it before the epilogue; pf
// receives the loaded words (to be consumed).  Without a prefetch pfr is any
// valid word and cmask 0 (the same loads, all of that word): no branch, so
// the compiler's waits on the vector-memory counter stay exact.
template <int TN>
__device__ __forceinline__ void touch_residual(uint32_t& pf, const float* __restrict__ pfr, int cmask) {
#pragma unroll
    for (int c = 0; c < TN; c += 32) pf |= __float_as_uint(pfr[c & cmask]);
}

template <int TN, int CW, int KC, bool FULLN>
__device__ __forceinline__ void conv_mainloop(uint32_t (&acc)[TN], const uint32_t* __restrict__ Xp,
                                              const Taps& tp, const uint32_t* __restrict__ wbase,
                                              int64_t ldW, int nlast, uint32_t& pf, const float* __restrict__ pfr,
                                              int pfmask)
{
    constexpr int CP = (TN >= 2) ? 2 : 1;
    static_assert(KC % CW == 0, "whole taps per chunk");
    constexpr int TPC = KC / CW;                  // taps per chunk
    constexpr int NCH = 9 / TPC;                  // full chunks
    constexpr int TT = 9 - NCH * TPC;             // taps in the tail chunk
    uint32_t a[KC], an[KC];
    constexpr int TW = TT > 0 ? TT * CW : 1;
    uint32_t t[TW];
    // the tail taps are requested with the first chunk: no exposed load at the end
    if (TT > 0) conv_chunk_load<CW>(t, Xp, tp, NCH * TPC, TT);
    if (NCH > 0) conv_chunk_load<CW>(an, Xp, tp, 0, TPC);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) a[kk] = an[kk];
        conv_chunk_mask<CW>(a, tp, c * TPC, TPC);
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) asm volatile("" : : "v"(a[kk]));
        if (c + 1 < NCH) conv_chunk_load<CW>(an, Xp, tp, (c + 1) * TPC, TPC);
        else touch_residual<TN>(pf, pfr, pfmask);
        xnor_chunk<TN, KC, CP, FULLN, false, false>(acc, a, wbase, wbase, c * KC, KC, ldW, nlast);
    }
    if (TT > 0) {
        conv_chunk_mask<CW>(t, tp, NCH * TPC, TT);
        xnor_chunk<TN, TW, CP, FULLN, false, false>(acc, t, wbase, wbase, NCH * KC, TW, ldW, nlast);
    }
}

// Packed sign bits of a lane's TN outputs (bit j = column n0 + j), stored
// like the THRESH_PACK bits: WB = min(TN, 32) bits per store; the last
// column tile zeroes the rest of the row (pad bits and pad words).
template <int TN>
__device__ __forceinline__ void store_row_bits(const uint32_t (&wbits)[(TN + 31) / 32], uint32_t* __restrict__ orow,
                                               int n0, int ncols, int N, int64_t ldOp, bool last_tile)
{
    constexpr int WB = TN < 32 ? TN : 32;
#pragma unroll
    for (int q = 0; q < TN / WB; ++q) {
        const uint32_t word = WB == 32 ? wbits[q] : (wbits[0] >> (WB * q)) & ((1u << (WB & 31)) - 1u);
        const int nb = n0 + WB * q;
        if (nb < N) {
            if (WB == 32) orow[nb >> 5] = word;
            else if (WB == 16) reinterpret_cast<uint16_t*>(orow)[nb >> 4] = (uint16_t)word;
            else reinterpret_cast<uint8_t*>(orow)[nb >> 3] = (uint8_t)word;
        }
    }
    if (last_tile) {
        uint8_t* ob = reinterpret_cast<uint8_t*>(orow);
        const int64_t first = (int64_t)(n0 + WB * ((ncols + WB - 1) / WB)) / 8;   // after the last store
        const int64_t wfirst = (first + 3) / 4;
        for (int64_t b = first; b < wfirst * 4 && b < ldOp * 4; ++b) ob[b] = 0u;
        for (int64_t w = wfirst; w < ldOp; ++w) orow[w] = 0u;
    }
}

__device__ __forceinline__ bool aligned16(const void* p) {
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// Epilogue through LDS for outputs that are HBM-heavy relative to their
// K loop (small K, e.g. the conv blocks).  Each lane owns one row, so a
// direct store instruction would touch 64 rows at once.  Instead the wave
// stages CH columns of its 64 x TN tile in LDS (row stride CH+1 words: the
// writes are bank-conflict free) and reads them back transposed: in each
// pass, CH/4 consecutive lanes cover one row's CH columns as 16-byte pieces,
// so every store (and residual load) instruction covers 64*16/(CH*4) whole
// row segments of CH*4 bytes.  Only full, 16-byte aligned tiles use it; LDS
// is private to the wave (no workgroup barrier).
// D of column j of a tile: K - 2 acc for binary weights, nnz[n] - 2 acc for
// ternary ones (nnz is uniform across the wave: a scalar load).
template <bool TERN>
__device__ __forceinline__ int32_t dval(uint32_t acc, int K, const Epilogue& e, int n) {
    const int32_t base = TERN ? (int32_t)((cptr_u32)(const uint32_t*)e.nnz)[n] : K;
    return base - 2 * (int32_t)acc;
}

// The staging shape: CH columns per pass (32 = one 128-byte line per row
// segment; measured on MI355X, 64-byte segments run the conv GEMMs 25-50%
// slower) and RH rows at a time (all 64: staging the rows in two halves of
// 32 to halve the LDS footprint measured 10% slower at 16384^3 and 12-29%
// on the conv GEMMs).
// (Staging D as int16 pairs, half the LDS, measured no faster on MI355X:
// 57.9 -> 60.0 us on the 14x14x256 conv GEMM, 94.5 -> 97.5 us on 56x56x64.)
template <int TN>
struct Stage {
    static constexpr int CH = TN < 32 ? TN : 32;
    static constexpr int RH = 64;
    static constexpr int RW = CH + 1;             // words per staged row (odd: no bank conflicts)
    static constexpr int words = RH * RW;
};

template <int TN, bool TERN>
__device__ __forceinline__ void epilogue_lds(const uint32_t (&acc)[TN], uint32_t* __restrict__ lds,
                                             int wrow0, int M, int n0, int K, const Epilogue& e)
{
    constexpr int CH = Stage<TN>::CH;
    constexpr int RH = Stage<TN>::RH;
    constexpr int RW = Stage<TN>::RW;
    constexpr int G4 = CH / 4;
    constexpr int RPP = 64 / G4;                  // rows per read pass
    constexpr int GLOG = G4 == 8 ? 3 : G4 == 4 ? 2 : G4 == 2 ? 1 : 0;
    const int lane = threadIdx.x & 63;
    // In a read pass lane l covers row q * RPP + l / G4 of the staged rows and
    // column group cg = l % G4, so a lane's alpha, bias and beta pieces are the
    // same in every pass: loaded once per column group.  The residual pieces
    // of all passes of a half are requested before any is used, so their
    // latencies overlap instead of adding up.
    const int cg = lane & (G4 - 1);
#pragma unroll
    for (int c0 = 0; c0 < TN; c0 += CH) {
        const int nc = n0 + c0 + 4 * cg;
        float4 av = make_float4(0.0f, 0.0f, 0.0f, 0.0f), bv = av, tv = av;
        if (e.flags & EPI_SCALE) {
            if (e.flags & EPI_ALPHA_TENSOR) { const float a = e.alpha[0]; av = make_float4(a, a, a, a); }
            else av = *reinterpret_cast<const float4*>(e.alpha + nc);
        }
        if (e.flags & EPI_BIAS) bv = *reinterpret_cast<const float4*>(e.bias + nc);
        if ((e.flags & EPI_SIGN_PACK) && e.beta)
            tv = make_float4(e.beta[nc], e.beta[nc + 1], e.beta[nc + 2], e.beta[nc + 3]);
#pragma unroll
        for (int h = 0; h < 64 / RH; ++h) {
            if (lane / RH == h) {
#pragma unroll
                for (int j = 0; j < CH; ++j)
                    lds[(lane % RH) * RW + j] = (uint32_t)dval<TERN>(acc[c0 + j], K, e, n0 + c0 + j);
            }
            // the accumulators are dead from here: keep the residual loads
            // below so the two sets are never live together
            __builtin_amdgcn_sched_barrier(0);
            constexpr int NP = RH / RPP;          // read passes per half
            f32x4 rv[NP];
            if (e.flags & EPI_RESIDUAL) {
#pragma unroll
                for (int q = 0; q < NP; ++q) {
                    const int m = min(wrow0 + h * RH + q * RPP + lane / G4, M - 1);
                    rv[q] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(e.R + (int64_t)m * e.ldR + nc));
                }
            } else {
#pragma unroll
                for (int q = 0; q < NP; ++q) rv[q] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int q = 0; q < NP; ++q) {
                const int r = q * RPP + lane / G4;
                int32_t d[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) d[i] = (int32_t)lds[r * RW + 4 * cg + i];
                const int m = wrow0 + h * RH + r;
                if (m < M) {
                    const int n = nc;
                    if (e.flags & EPI_DOT)
                        *reinterpret_cast<int4*>(e.D + (int64_t)m * e.ldD + n) = make_int4(d[0], d[1], d[2], d[3]);
                    if (e.flags & EPI_SCALE) {
                        const float4 a = av;
                        f32x4 y = {a.x * (float)d[0], a.y * (float)d[1], a.z * (float)d[2], a.w * (float)d[3]};
                        if (e.flags & EPI_BIAS) {
                            const float4 b = bv;
                            y = y + (f32x4){b.x, b.y, b.z, b.w};
                        }
                        if (e.flags & EPI_RESIDUAL) y = y + rv[q];
                        __builtin_nontemporal_store(y, reinterpret_cast<f32x4*>(e.Y + (int64_t)m * e.ldY + n));
                        if (e.flags & EPI_SIGN_PACK) {
                            // sign(y - beta_n) as bits (0 = +1), OR-ed over the G4 lanes of
                            // the row segment; the last lane stores the CH bits
                            const float4 bt = tv;
                            const uint32_t nib = (y[0] >= bt.x ? 0u : 1u) | ((y[1] >= bt.y ? 0u : 1u) << 1) |
                                                 ((y[2] >= bt.z ? 0u : 1u) << 2) | ((y[3] >= bt.w ? 0u : 1u) << 3);
                            uint32_t bits = nib << (4 * cg);
                            if (GLOG >= 1) bits |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)bits, 0x111, 0xF, 0xF, true);
                            if (GLOG >= 2) bits |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)bits, 0x112, 0xF, 0xF, true);
                            if (GLOG >= 3) bits |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)bits, 0x114, 0xF, 0xF, true);
                            if (cg == G4 - 1) {
                                const int nb = n0 + c0;
                                uint32_t* orow = e.Op + (int64_t)m * e.ldOp;
                                if (CH == 32) orow[nb >> 5] = bits;
                                else if (CH == 16) reinterpret_cast<uint16_t*>(orow)[nb >> 4] = (uint16_t)bits;
                                else reinterpret_cast<uint8_t*>(orow)[nb >> 3] = (uint8_t)bits;
                            }
                        }
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// Epilogue modes: EPI_DIRECT stores each lane's row from registers;
// EPI_STAGED stages the tile through LDS (whole row segments per store).
enum : int { EPI_DIRECT = 0, EPI_STAGED = 1 };

// Whether a tile can take the staged epilogue: full tile, no THRESH_PACK,
// 16-byte aligned outputs and operands.
__device__ __forceinline__ bool staged_ok(const Epilogue& e, bool full) {
    return full && !(e.flags & EPI_THRESH) &&
           (!(e.flags & EPI_DOT) || (aligned16(e.D) && e.ldD % 4 == 0)) &&
           (!(e.flags & EPI_SCALE) || (aligned16(e.Y) && e.ldY % 4 == 0 &&
                                       ((e.flags & EPI_ALPHA_TENSOR) || aligned16(e.alpha)))) &&
           (!(e.flags & EPI_BIAS) || aligned16(e.bias)) &&
           (!(e.flags & EPI_RESIDUAL) || (aligned16(e.R) && e.ldR % 4 == 0));
}

// CW > 0: implicit-im2col 3x3 convolution over the packed NHWC image Xp
// (CW words per pixel, row stride ldX, image convH x convW); K = 9 * 32 CW.
// Resident waves per SIMD the register allocation must allow (512 VGPRs per
// lane and SIMD: 3 waves at <= 168 registers, 5 at <= 96, 8 at <= 64).  Left
// to itself the compiler gave the 64-wide staged tile 170 registers (2 waves,
// 12% slower at 16384^3 than at 3).
template <int TN>
struct MinWaves { static constexpr int value = TN >= 64 ? 3 : TN == 32 ? 5 : 8; };

template <int TN, int KC, int EPI, int WAVES, bool TERN, int CW, int MW = MinWaves<TN>::value>
__global__ __launch_bounds__(WAVES * 64, MW) void k_xnor_gemm(
    const uint32_t* __restrict__ Xp, int64_t ldX, const uint32_t* __restrict__ Wp, int64_t ldW,
    int M, int N, int K, int tiles_n, Epilogue e, int convH, int convW)
{
    constexpr bool EPI_LDS = EPI != EPI_DIRECT;
    constexpr int kLdsWords = Stage<TN>::words;
    __shared__ uint32_t lds_epi[EPI_LDS ? WAVES * kLdsWords : 1];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int tn = blockIdx.x % tiles_n;
    const int tm = blockIdx.x / tiles_n;
    const int wrow0 = tm * (WAVES * 64) + wave * 64;
    if (wrow0 >= M) return;                       // whole wave past the last row
    const int m = wrow0 + lane;
    const int n0 = tn * TN;
    const int Kw = (K + 31) >> 5;
    const int nlast = N - 1 - n0;                 // last live column of this tile
    const uint32_t* __restrict__ xrow = Xp + (int64_t)min(m, M - 1) * ldX;
    const uint32_t* __restrict__ wbase = Wp + (int64_t)n0 * ldW;
    const uint32_t* __restrict__ zbase = TERN ? e.Zp + (int64_t)n0 * ldW : wbase;

    const int ncols = min(TN, N - n0);
    const bool full = (ncols == TN);
    const bool staged = EPI_LDS && staged_ok(e, full);

    // Residual prefetch (the conv loop): the lane's row of the residual tile
    uint32_t pf = 0u;
    const bool pfon = staged && (e.flags & EPI_PREFETCH_R) && (e.flags & EPI_RESIDUAL);
    const float* __restrict__ pfr = pfon ? e.R + (int64_t)min(m, M - 1) * e.ldR + n0
                                         : reinterpret_cast<const float*>(Xp);
    const int pfmask = pfon ? -1 : 0;

    uint32_t acc[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[j] = 0u;
    if (CW > 0) {
        // the taps of this lane's output pixel (m = (b H + oh) W + ow)
        const int mc = min(m, M - 1);
        const int ow = mc % convW, oh = (mc / convW) % convH;
        Taps tp;
        tp.base = mc * (int)ldX;
        tp.rowstep = convW * (int)ldX;
        tp.ldx = (int)ldX;
        tp.in = 0u;
#pragma unroll
        for (int t = 0; t < 9; ++t) {
            const int dh = t / 3 - 1, dw = t % 3 - 1;
            const bool inside = oh + dh >= 0 && oh + dh < convH && ow + dw >= 0 && ow + dw < convW;
            tp.in |= (inside ? 1u : 0u) << t;
        }
        if (n0 + TN <= N) conv_mainloop<TN, (CW > 0 ? CW : 2), KC, true>(acc, Xp, tp, wbase, ldW, nlast, pf, pfr, pfmask);
        else              conv_mainloop<TN, (CW > 0 ? CW : 2), KC, false>(acc, Xp, tp, wbase, ldW, nlast, pf, pfr, pfmask);
    } else {
        if (n0 + TN <= N) xnor_mainloop<TN, KC, true, TERN>(acc, xrow, wbase, zbase, Kw, ldW, nlast);
        else              xnor_mainloop<TN, KC, false, TERN>(acc, xrow, wbase, zbase, Kw, ldW, nlast);
    }

    asm volatile("" : : "v"(pf));
    if (staged) {
        epilogue_lds<TN, TERN>(acc, lds_epi + wave * kLdsWords, wrow0, M, n0, K, e);
        if ((e.flags & EPI_SIGN_PACK) && tn == tiles_n - 1 && m < M) {
            // the stores above covered the row's bits up to n0 + TN (a whole
            // number of bytes); zero what follows up to ldOp words
            uint32_t* orow = e.Op + (int64_t)m * e.ldOp;
            uint8_t* ob = reinterpret_cast<uint8_t*>(orow);
            const int64_t first = (int64_t)(n0 + TN) / 8;
            const int64_t wfirst = (first + 3) / 4;
            for (int64_t b = first; b < wfirst * 4 && b < e.ldOp * 4; ++b) ob[b] = 0u;
            for (int64_t w = wfirst; w < e.ldOp; ++w) orow[w] = 0u;
        }
        return;
    }
    if (m >= M) return;
    // Epilogue in groups of 4 columns to keep live ranges short (16-byte
    // stores when the row segment is aligned and complete).
    const bool vecD = full && aligned16(e.D) && (e.ldD % 4 == 0);
    const bool vecY = full && aligned16(e.Y) && (e.ldY % 4 == 0);
    const bool vecR = full && aligned16(e.R) && (e.ldR % 4 == 0);
    int32_t* drow = e.D + (int64_t)m * e.ldD + n0;
    float* yrow = e.Y + (int64_t)m * e.ldY + n0;
    const float* rrow = e.R + (int64_t)m * e.ldR + n0;
    // per-tensor alpha: every column reads alpha[0]
    const int astr = (e.flags & EPI_ALPHA_TENSOR) ? 0 : 1;
    cptr_f32 al = (cptr_f32)(e.alpha + n0 * astr);
    cptr_f32 bi = (cptr_f32)(e.bias + n0);
    uint32_t sbits[(TN + 31) / 32];               // SIGN_PACK: bit j = sign of column n0 + j
#pragma unroll
    for (int w = 0; w < (TN + 31) / 32; ++w) sbits[w] = 0u;
#pragma unroll
    for (int q = 0; q < TN / 4; ++q) {
        int32_t d[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = dval<TERN>(acc[4 * q + i], K, e, n0 + min(4 * q + i, ncols - 1));
        if (e.flags & EPI_DOT) {
            if (vecD) *reinterpret_cast<int4*>(drow + 4 * q) = make_int4(d[0], d[1], d[2], d[3]);
            else {
#pragma unroll
                for (int i = 0; i < 4; ++i) if (4 * q + i < ncols) drow[4 * q + i] = d[i];
            }
        }
        if (e.flags & EPI_SCALE) {
            float y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = al[min(4 * q + i, ncols - 1) * astr] * (float)d[i];
            if (e.flags & EPI_BIAS) {
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = y[i] + bi[min(4 * q + i, ncols - 1)];
            }
            if (e.flags & EPI_RESIDUAL) {
                if (vecR) {
                    const float4 rv = *reinterpret_cast<const float4*>(rrow + 4 * q);
                    y[0] = y[0] + rv.x; y[1] = y[1] + rv.y; y[2] = y[2] + rv.z; y[3] = y[3] + rv.w;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) if (4 * q + i < ncols) y[i] = y[i] + rrow[4 * q + i];
                }
            }
            if (vecY) *reinterpret_cast<float4*>(yrow + 4 * q) = make_float4(y[0], y[1], y[2], y[3]);
            else {
#pragma unroll
                for (int i = 0; i < 4; ++i) if (4 * q + i < ncols) yrow[4 * q + i] = y[i];
            }
            if (e.flags & EPI_SIGN_PACK) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = 4 * q + i;
                    const float bt = e.beta ? e.beta[n0 + min(j, ncols - 1)] : 0.0f;
                    if (j < ncols && !(y[i] >= bt)) sbits[j >> 5] |= 1u << (j & 31);
                }
            }
        }
    }
    if (e.flags & EPI_SIGN_PACK)
        store_row_bits<TN>(sbits, e.Op + (int64_t)m * e.ldOp, n0, ncols, N, e.ldOp, tn == tiles_n - 1);
    if (e.flags & EPI_THRESH) {
        // Output bits of this lane's row, packed along n: bit (n % 32) of word
        // n / 32.  A tile owns TN/8 whole bytes of the row (n0 is a multiple
        // of TN), so tiles never share a byte.
        cptr_f32 tau = (cptr_f32)(e.tau + n0);
        const int8_t* dir = e.dir + n0;
        uint32_t* orow = e.Op + (int64_t)m * e.ldOp;
        constexpr int WB = TN < 32 ? TN : 32;          // bits per store
#pragma unroll
        for (int q = 0; q < TN / WB; ++q) {
            uint32_t word = 0u;
#pragma unroll
            for (int b = 0; b < WB; ++b) {
                const int j = WB * q + b;
                const int jj = min(j, ncols - 1);
                const float v = (float)((int32_t)dir[jj] * dval<TERN>(acc[j], K, e, n0 + jj));
                const uint32_t bit = (j < ncols && !(v >= tau[jj])) ? 1u : 0u;
                word |= bit << b;
            }
            const int nb = n0 + WB * q;                // first column of this store
            if (nb < N) {
                if (WB == 32) orow[nb >> 5] = word;
                else if (WB == 16) reinterpret_cast<uint16_t*>(orow)[nb >> 4] = (uint16_t)word;
                else reinterpret_cast<uint8_t*>(orow)[nb >> 3] = (uint8_t)word;
            }
        }
        if (tn == tiles_n - 1) {
            // zero the rest of the row: bytes after this tile (pad bits of the
            // last word, if the tile is narrower than a word) and the pad words
            uint8_t* ob = reinterpret_cast<uint8_t*>(orow);
            const int64_t first = (int64_t)(n0 + WB * ((ncols + WB - 1) / WB)) / 8;   // after the last store
            const int64_t wfirst = (first + 3) / 4;
            for (int64_t b = first; b < wfirst * 4 && b < e.ldOp * 4; ++b) ob[b] = 0u;
            for (int64_t w = wfirst; w < e.ldOp; ++w) orow[w] = 0u;
        }
    }
}

int tile_cols_from_env() {
    const char* v = getenv("BNN_GEMM_TN");
    if (!v) return 0;
    const int t = atoi(v);
    return (t == 8 || t == 16 || t == 32 || t == 64) ? t : 0;
}

// Tuning override of the epilogue mode (results never change): "direct" or
// "staged"; -1 when unset.
int epilogue_from_env() {
    const char* v = getenv("BNN_GEMM_EPI");
    if (!v) return -1;
    if (v[0] == 'd') return EPI_DIRECT;
    if (v[0] == 's') return EPI_STAGED;
    return -1;
}

// The epilogue of a launch: staged through LDS for D and Y outputs (whole
// row segments per store), direct for THRESH_PACK (its bits leave from
// registers).
int pick_epilogue(const Epilogue& e) {
    if (!(e.flags & (EPI_DOT | EPI_SCALE)) || (e.flags & EPI_THRESH)) return EPI_DIRECT;
    const int ov = epilogue_from_env();
    return ov >= 0 ? ov : EPI_STAGED;
}

// Column tile: 64-wide tiles (the most reuse of each activation chunk) once
// the launch has >= 6 rounds of 8 waves per SIMD; otherwise 32-wide (16 or 8
// only when N itself is that narrow).  Measured on MI355X with the staged
// epilogue: 32-wide tiles beat 16-wide ones on the 14x14x256 and 56x56x64
// conv GEMMs and on the 1024 x 4096 x 4096 threshold layer.
int pick_tile_cols(int64_t M, int64_t N) {
    const int t = tile_cols_from_env();
    if (t) return t;
    const int64_t row_waves = (M + 63) / 64;
    const int64_t rounds_wave = (int64_t)num_cus() * 4 * 8;
    if (row_waves * ((N + 63) / 64) >= 6 * rounds_wave) return 64;
    if (N > 16) return 32;
    return N <= 8 ? 8 : 16;
}

}  // namespace

}  // namespace bnn
