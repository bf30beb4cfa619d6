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
// each lane expands the 16 weight bits of its B fragment to 16 bytes right
// before the MFMA (a multiply spreads a nibble into bytes).  Given the row
// sums xsum[m] = sum_k q[m,k], the bytes are the bits themselves (0 / 1)
// and D = xsum - 2 sum_k q w; otherwise an XOR makes them +1 / -1 (0x01 /
// 0xFF, no borrows between bytes).
//
// On this chip a SIMD does not issue VALU work while its matrix core runs an
// MFMA (measured: the times add), so the expansion cost counts in full.  It
// is spent per weight column and amortised over the rows that share the
// expanded fragment; each wave therefore spans all 256 rows of the
// workgroup tile: 16 x 2 fragments, 32 MFMAs per 64-wide k-step against 2
// weight-fragment expansions.  (Wider wave tiles would halve the LDS reads
// of A per MFMA but need 256 accumulator registers; as AGPRs that cost as
// many register moves as they saved.)
//
// Fragment layout used for both operands: lane l holds row (A) or column (B)
// l % 16 and the 16 consecutive k of group l / 16 within the 64-wide step.
// A and B use the same k assignment, so each output is the full sum over k.
// The int32 result of lane l, register r is row 4*(l/16) + r, column l % 16.
//
// Tiling: a 512-thread workgroup (8 waves) computes 256 activation rows x
// 256 weight rows; wave w takes all rows and columns 32 w .. +31.  The k
// range is walked in stages of 128 (two MFMA k-steps) with one barrier per
// stage.  The workgroup's A tile (256 rows x 128 bytes per stage) goes
// straight from global memory into a 2-deep ring of LDS buffers (buffer
// loads to LDS, issued one stage ahead of their use: a 4-deep ring of these
// 32 KiB stages leaves no LDS for the ternary weights' second plane, and
// with binary weights it ran out of registers); 16-byte piece j of A row r sits
// at slot j ^ (r % 8) of the row's eight slots, so every 8 consecutive
// lanes of a fragment read (8 rows of one k-group) fall on 8 distinct
// 4-bank groups of a 32-bank window: 16-byte LDS reads are served 8 lanes
// at a time (a pattern distinct only across 16 lanes measured half the
// throughput).  The weight bits move in chunks of 4 stages (64 bytes per
// weight row, whole 64-byte L2 requests; a request per row and k-step
// would carry 8 useful bytes) into a double-buffered LDS chunk.  With the A
// tile shared by 256 weight rows, the L2 request rate (the limit of a
// 256 x 128 tile) stays below one per clock and channel.
#include <type_traits>

#include "bnn_device.hpp"
#include "bnn_launch.hpp"

namespace bnn {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kBM = 256, kBN = 256, kKS = 64;  // workgroup tile: activation rows x weight rows x MFMA k-step
constexpr int kSub = 2, kST = kSub * kKS;       // k-steps per stage, k per stage
constexpr int kWN = kBN / kWaves;               // wave tile: all kBM rows x kWN columns
constexpr int kFM = kBM / 16, kFN = kWN / 16;   // 16 x 16 fragments per wave tile
constexpr int kCS = 4;          // stages per weight chunk
constexpr int kCW = kCS * kST / 32;             // words per weight row in a chunk (16: 64 bytes)

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

// 16 weight bits to 16 bytes holding the bits themselves (0 or 1).
__device__ __forceinline__ v4i expand_bits01(uint32_t bits16) {
    v4i r;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        r[q] = (int)((((bits16 >> (4 * q)) & 0xFu) * 0x00204081u) & 0x01010101u);
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

constexpr int kAPieces = kBM * kST / 16 / kThreads;      // 16-byte A pieces per lane per stage
constexpr int kBPieces = kBN * kCW * 4 / 16 / kThreads;  // 16-byte weight pieces per lane per chunk
static_assert(kAPieces == 4 && kBPieces == 2 && kFN == 2 && kSub == 2, "the staging below assumes these");

// s_waitcnt immediate that waits for at most n outstanding vector-memory
// operations (vmcnt in bits 3:0 and 15:14) and not on the other counters.
constexpr unsigned waitcnt_vm(int n) {
    return (unsigned)(n & 0xF) | ((unsigned)((n >> 4) & 3) << 14) | (0x7u << 4) | (0xFu << 8);
}

// Workgroup barrier without the release/acquire fence of __syncthreads():
// that fence also waits for every direct-to-LDS load in flight, which would
// drain the prefetch ring each step.  The caller first waits for the loads
// the next step reads (its own, by vmcnt; the barrier then covers the
// other waves'), and the LDS reads of the finished step have all returned
// (the MFMAs consumed them).  The clobber keeps the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void barrier_keep_loads() { asm volatile("s_barrier" ::: "memory"); }

typedef __attribute__((address_space(3))) void* lptr_t;

// Buffer resource over [base, base + bytes) for raw (stride 0) dword loads.
// The tiles move with buffer loads to LDS rather than global_load_lds: the
// latter is a FLAT instruction, and with one in flight the compiler no
// longer counts LDS reads in order, so it waits for all of them at the
// first use.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

template <int I> using Ic = std::integral_constant<int, I>;

// TERN: Wp is the sign plane, e.Zp the nonzero plane of ternary weights.
// XS: binary weights with the activation row sums e.xsum given.
template <bool TERN, bool XS>
__global__ __launch_bounds__(kThreads, 1) void k_bwn_i8_gemm(
    const int8_t* __restrict__ Xq, int64_t ldX, const uint32_t* __restrict__ Wp, int64_t ldW,
    int M, int N, int K, int tiles_n, EpilogueI8 e)
{
    static_assert(!(TERN && XS), "row sums serve binary weights only");
    constexpr int kPL = TERN ? 2 : 1;                // weight planes
    constexpr int kNB = 2;                           // A ring depth
    // Separate LDS objects, each reached through a compile-time index, so
    // the compiler can tell a load into one buffer from a read of another
    // and does not wait for the prefetch before the current stage's reads.
    __shared__ __attribute__((aligned(16))) int8_t lds_a0[kBM * kST], lds_a1[kBM * kST];
    // weight chunks (two buffers): sign (or binary) plane and, ternary, the
    // nonzero plane
    __shared__ __attribute__((aligned(16))) uint32_t lds_b0[kBN * kCW], lds_b1[kBN * kCW];
    __shared__ __attribute__((aligned(16))) uint32_t lds_z0[TERN ? kBN * kCW : 4], lds_z1[TERN ? kBN * kCW : 4];
    static_assert(kNB == 2, "the A ring is lds_a0 / lds_a1");
    auto abuf = [&](auto I) -> int8_t* {
        if constexpr (decltype(I)::value % kNB == 0) return lds_a0;
        else return lds_a1;
    };
    auto bbuf = [&](auto I) -> uint32_t* {
        if constexpr ((decltype(I)::value & 1) == 0) return lds_b0;
        else return lds_b1;
    };
    auto zbuf = [&](auto I) -> uint32_t* {
        if constexpr ((decltype(I)::value & 1) == 0) return lds_z0;
        else return lds_z1;
    };
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;

    // Tile order.  Workgroups go to the 8 XCDs round-robin by id; renumber
    // so that each XCD owns a contiguous range of tiles, and walk that range
    // in groups of kGroupM activation-row tiles per weight-row tile, so the
    // workgroups resident on one XCD share their A rows and weight rows in
    // that XCD's L2.
    int tile = blockIdx.x;
    const int ntiles = gridDim.x;
    if (ntiles % 8 == 0) tile = (tile % 8) * (ntiles / 8) + tile / 8;
    constexpr int kGroupM = 8;
    const int tiles_m = ntiles / tiles_n;
    const int grp = tile / (kGroupM * tiles_n);
    const int gm0 = grp * kGroupM;
    const int gsz = min(tiles_m - gm0, kGroupM);
    const int in_grp = tile - grp * kGroupM * tiles_n;
    const int tm = gm0 + in_grp % gsz, tn = in_grp / gsz;
    const int m_blk = tm * kBM, n_blk = tn * kBN;

    // A staging.  Instruction i of wave w fills tile rows 8 (kAPieces w + i)
    // .. +7 (1 KiB of LDS): lane l takes row r = 8 (kAPieces w + i) + l / 8,
    // LDS slot l % 8, and loads the piece j stored there, j = slot ^ (r % 8)
    // = (l % 8) ^ (l / 8).  Stages inside K load straight into LDS (a 16-byte
    // buffer load to LDS writes lane l's 16 bytes at the instruction's LDS
    // base + 16 l); the stage holding the end of the row goes through
    // registers, masked past K.
    const __amdgpu_buffer_rsrc_t arsrc = buffer_rsrc(Xq, M * (int)ldX);          // M * ldX < 2^31
    int aoff[kAPieces];                            // byte offset of row r
#pragma unroll
    for (int i = 0; i < kAPieces; ++i)
        aoff[i] = min(m_blk + 8 * (kAPieces * wave + i) + (lane >> 3), M - 1) * (int)ldX;
    const int apiece = ((lane & 7) ^ (lane >> 3)) << 4;   // byte offset of piece j in the row
    // Weight staging.  A chunk holds words kCW c .. +kCW-1 of each weight
    // row of the tile; column c's 64 bytes take LDS slots 4 c .. 4 c + 3
    // (16 bytes each) and its 16-byte piece p sits in slot 4 c + ((p + c / 4)
    // % 4), so the 16 columns of a fragment read fall on 16 distinct 4-bank
    // groups.  Instruction j of wave w fills slots 4 (128 j + 16 w) .. +63:
    // lane l takes column 128 j + 16 w + l / 4 and piece ((l % 4) - l / 16)
    // % 4.  A piece that starts at or past the row stride (only beyond K)
    // reads the row's last piece instead: its bits meet zero activations or
    // stages that are not computed.
    const int ldw = (int)ldW;
    const __amdgpu_buffer_rsrc_t brsrc = buffer_rsrc(Wp, N * ldw * 4);           // N * ldW < 2^29
    const __amdgpu_buffer_rsrc_t zrsrc = buffer_rsrc(TERN ? e.Zp : Wp, N * ldw * 4);
    int boff[kBPieces];                            // word offset of the lane's weight row
    const int bpiece = ((lane & 3) - (lane >> 4)) & 3;
#pragma unroll
    for (int j = 0; j < kBPieces; ++j) boff[j] = min(n_blk + 128 * j + 16 * wave + (lane >> 2), N - 1) * ldw;
    auto issue_a = [&](auto I, int k0, bool direct) {
        int8_t* la = abuf(I);
        if (direct) {
#pragma unroll
            for (int i = 0; i < kAPieces; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (lptr_t)(la + (kAPieces * wave + i) * 1024), 16,
                                                         aoff[i] + k0 + apiece, 0, 0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < kAPieces; ++i) {
                const v4i v = load_a<true>(Xq + aoff[i], k0 + apiece, K);
                *reinterpret_cast<v4i*>(la + (kAPieces * wave + i) * 1024 + 16 * lane) = v;
            }
        }
    };
    auto issue_b = [&](auto I, int chunk) {
        uint32_t* lb = bbuf(I);
        uint32_t* lz = zbuf(I);
        const int w0 = min(kCW * chunk + 4 * bpiece, ldw - 4);
#pragma unroll
        for (int j = 0; j < kBPieces; ++j) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(brsrc, (lptr_t)(lb + 16 * (128 * j + 16 * wave)), 16,
                                                     (boff[j] + w0) * 4, 0, 0, 0);
            if (TERN)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(zrsrc, (lptr_t)(lz + 16 * (128 * j + 16 * wave)), 16,
                                                         (boff[j] + w0) * 4, 0, 0, 0);
        }
    };
    // fragment reads: A row 16 f + r16, k-group g of sub-step u at byte
    // abase[u] + 2048 f ((16 f + r16) % 8 = r16 % 8); weight word 2 t + g / 2
    // of chunk k-step t = 2 (stage % 4) + u of column wave kWN + 16 q + r16:
    // piece stage % 4, word 2 u + g / 2 of it
    int abase[kSub];
#pragma unroll
    for (int u = 0; u < kSub; ++u) abase[u] = r16 * kST + (((4 * u + g) ^ (r16 & 7)) << 4);
    const int bcol0 = wave * kWN + r16;            // + 16 q
    const int bcr = (r16 >> 2) & 3;                // (column / 4) % 4, the same for both q
    // combined ternary word of lane group g: Z bits low, (S & Z) bits high
    auto tern_word = [](uint32_t sw, uint32_t zw, int gg) {
        const int sh = 16 * (gg & 1);
        return ((zw >> sh) & 0xFFFFu) | (((sw & zw) >> sh) << 16);
    };

    v4i acc[kFM][kFN];
#pragma unroll
    for (int f = 0; f < kFM; ++f)
#pragma unroll
        for (int q = 0; q < kFN; ++q) acc[f][q] = (v4i){0, 0, 0, 0};

    const int stages = (K + kST - 1) / kST;
    const int full_stages = K / kST;
    const int chunks = (stages + kCS - 1) / kCS;
    constexpr int kA = kAPieces;                   // vector-memory instructions per direct A stage
    constexpr int kB = kBPieces * kPL;             // ... per weight chunk

    // The weight words of the next stage are read at the end of the current
    // one (its chunk is in LDS by then) and those of its first k-step
    // expanded, so a stage starts with its MFMAs as soon as the first A
    // fragment arrives; the second k-step's words are expanded between the
    // MFMAs of the two k-steps (into the same registers).
    v4i bx[kFN];
    uint32_t sw1[kFN], zw1[kFN];
    auto expand = [&](int q, uint32_t sw, uint32_t zw) {
        if (TERN) bx[q] = expand_ternary(tern_word(sw, zw, g));
        else if (XS) bx[q] = expand_bits01(sw >> (16 * (g & 1)));
        else bx[q] = expand_signs(sw >> (16 * (g & 1)));
    };
    auto load_bx = [&](auto P) {                  // P: stage % 8
        constexpr int st = decltype(P)::value;
        const uint32_t* lb = bbuf(Ic<st / kCS>{});
        const uint32_t* lz = zbuf(Ic<st / kCS>{});
        const int bw = 4 * (((st % kCS) + bcr) & 3) + (g >> 1);
#pragma unroll
        for (int q = 0; q < kFN; ++q) {
            const int wi = (bcol0 + 16 * q) * kCW + bw;
            const uint32_t sw0 = lb[wi];
            const uint32_t zw0 = TERN ? lz[wi] : 0u;
            sw1[q] = lb[wi + 2];
            zw1[q] = TERN ? lz[wi + 2] : 0u;
            expand(q, sw0, zw0);
        }
    };
    // stage s reads A buffer s % 3; LDS reads run ahead of their use: the
    // first kH A fragments are issued first, and each later one as soon as
    // the MFMAs of the fragment whose registers it takes have been issued
    // (across the two k-steps of the stage).
    auto compute = [&](auto IA) {
        const int8_t* la = abuf(IA);
        constexpr int kH = TERN ? kFM / 4 : kFM / 2;
        constexpr int kF = kSub * kFM;             // fragments per stage
        v4i a[kH];
#pragma unroll
        for (int f = 0; f < kH; ++f) a[f] = *reinterpret_cast<const v4i*>(la + abase[0] + 2048 * f);
#pragma unroll
        for (int x = 0; x < kF; ++x) {
            const int f = x % kFM;
            if (x == kFM) {
#pragma unroll
                for (int q = 0; q < kFN; ++q) expand(q, sw1[q], zw1[q]);
            }
#pragma unroll
            for (int q = 0; q < kFN; ++q)
                acc[f][q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[x % kH], bx[q], acc[f][q], 0, 0, 0);
            if (x + kH < kF) {
                const int un = (x + kH) / kFM, fn = (x + kH) % kFM;
                a[x % kH] = *reinterpret_cast<const v4i*>(la + abase[un] + 2048 * fn);
            }
        }
        // keep that order (DS reads, then MFMA / DS pairs with the second
        // k-step's expansion between the k-steps, then MFMAs)
        __builtin_amdgcn_sched_group_barrier(0x100, kH, 0);
#pragma unroll
        for (int x = 0; x < kF - kH; ++x) {
            if (x == kFM) __builtin_amdgcn_sched_group_barrier(0x002, 1000, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, kFN, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kH * kFN, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    // Prologue: weight chunks 0 and 1 and A stage 0, all complete before the
    // first stage.
    issue_b(Ic<0>{}, 0);
    issue_b(Ic<1>{}, 1);
    issue_a(Ic<0>{}, 0, 0 < full_stages);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    load_bx(Ic<0>{});

    // Stage s issues A stage s + kNB - 1 (into the buffer read during stage
    // s - 1), computes, prepares the next stage's weight fragments and, at
    // the end of the last stage of chunk c - 1 (s = 4 c - 1), issues chunk
    // c + 1 (into the buffer of chunk c - 1, last read at the end of stage
    // s - 1).  In the steady state all of it lies inside K, so every load is
    // direct and the loads issued after those of stage s + 1 are known: A of
    // stages s + 2 .. s + kNB - 1 and the chunks issued at the ends of stages
    // s + 2 - kNB .. s.  A chunk is then complete (and, after the barrier,
    // visible) at least one stage before its first read.
    auto chunk_issues = [](int lo, int hi) {     // stages t in [lo, hi] with t % 4 == 3 (lo >= -3)
        int n = 0;
        for (int t = lo; t <= hi; ++t) n += ((t + 8) % kCS) == kCS - 1;
        return n;
    };
    auto fast_stage = [&](int s, auto P) {
        constexpr int ph = decltype(P)::value;      // s % 8
        issue_a(Ic<(ph + kNB - 1) % kNB>{}, (s + kNB - 1) * kST, true);
        __builtin_amdgcn_sched_barrier(0);           // the prefetch goes out before the stage's LDS reads
        compute(Ic<ph % kNB>{});
        load_bx(Ic<(ph + 1) % 8>{});
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ph % kCS == kCS - 1) issue_b(Ic<(ph / kCS + 2) & 1>{}, s / kCS + 2);
        constexpr int after = (kNB - 2) * kA + kB * chunk_issues(ph + 2 - kNB, ph);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(after));
        barrier_keep_loads();
    };
    static_assert((4 - 2) * kAPieces + kBPieces * 2 <= 63, "vmcnt holds at most 63");
    // General stage (the tail, where loads may be masked or missing): the
    // same order with every issue checked, and a full wait.
    auto stage = [&](int s, auto P) {
        constexpr int ph = decltype(P)::value;
        const int t_issue = s + kNB - 1;
        if (t_issue < stages)
            issue_a(Ic<(ph + kNB - 1) % kNB>{}, t_issue * kST, t_issue < full_stages);
        compute(Ic<ph % kNB>{});
        if (s + 1 < stages) load_bx(Ic<(ph + 1) % 8>{});
        if (ph % kCS == kCS - 1 && s / kCS + 2 < chunks) issue_b(Ic<(ph / kCS + 2) & 1>{}, s / kCS + 2);
        __builtin_amdgcn_s_waitcnt(0);               // every load of this lane, then the workgroup's
        __syncthreads();
    };
    auto run8 = [&](int s0, auto body) {
        body(s0 + 0, Ic<0>{}); body(s0 + 1, Ic<1>{}); body(s0 + 2, Ic<2>{}); body(s0 + 3, Ic<3>{});
        body(s0 + 4, Ic<4>{}); body(s0 + 5, Ic<5>{}); body(s0 + 6, Ic<6>{}); body(s0 + 7, Ic<7>{});
    };
    int s = 0;
    // eight stages are fast while their A issues (up to stage s + 6 + kNB)
    // lie in K
    for (; s + 8 + kNB - 1 <= full_stages; s += 8) run8(s, fast_stage);
    for (; s < stages; s += 8)
        run8(s, [&](int ss, auto P) { if (ss < stages) stage(ss, P); });

    // Epilogue.  Full tiles with 16-byte aligned output rows go through LDS
    // (the A buffers are free now): in 8 passes of 2 fragment rows, each
    // wave parks its 32 x kWN int32 block in its own 8 KiB quarter of an A
    // buffer (column c of row r at word r * 36 + c: the stride of 36 words
    // puts the 4 lane groups of a fragment, rows 4 apart, on disjoint
    // 16-bank groups) and reads it back as 16-byte row pieces, so every store
    // instruction writes 8 whole 128-byte row segments.  Other tiles store
    // element by element.
    const bool full = m_blk + kBM <= M && n_blk + kBN <= N &&
                      (!(e.flags & EPI_DOT) || ((reinterpret_cast<uintptr_t>(e.D) & 15u) == 0 && e.ldD % 4 == 0)) &&
                      (!(e.flags & EPI_SCALE) || ((reinterpret_cast<uintptr_t>(e.Y) & 15u) == 0 && e.ldY % 4 == 0));
    if (full) {
        constexpr int kPS = 36;                    // parked row stride in words
        static_assert(32 * kPS * 4 <= kBM * kST / 4, "a wave's parked block fits a quarter of an A buffer");
        int8_t* pb = (wave >> 2) == 0 ? lds_a0 : lds_a1;
        int32_t* park = reinterpret_cast<int32_t*>(pb + (wave & 3) * (kBM * kST / 4));
        const int pc = 4 * (lane & 7);             // read-back: 4 columns of row 8 p + lane / 8
        const int n = n_blk + wave * kWN + pc;
        float an[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (e.flags & EPI_SCALE) {
#pragma unroll
            for (int c = 0; c < 4; ++c) an[c] = e.alpha[(e.flags & EPI_ALPHA_TENSOR) ? 0 : n + c];
        }
#pragma unroll
        for (int pass = 0; pass < kFM / 2; ++pass) {
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int q = 0; q < kFN; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        park[(16 * f + 4 * g + r) * kPS + 16 * q + r16] = acc[2 * pass + f][q][r];
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int row = 8 * p + (lane >> 3);
                v4i d = *reinterpret_cast<const v4i*>(&park[row * kPS + pc]);
                const int64_t m = m_blk + 32 * pass + row;
                if (XS) {
                    const int32_t xs = e.xsum[m];
                    d[0] = xs - 2 * d[0]; d[1] = xs - 2 * d[1]; d[2] = xs - 2 * d[2]; d[3] = xs - 2 * d[3];
                }
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
    for (int q = 0; q < kFN; ++q) {
        const int n = n_blk + wave * kWN + 16 * q + r16;
        if (n >= N) continue;
        float an = 0.0f;
        if (e.flags & EPI_SCALE) an = e.alpha[(e.flags & EPI_ALPHA_TENSOR) ? 0 : n];
#pragma unroll
        for (int f = 0; f < kFM; ++f)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m_blk + 16 * f + 4 * g + r;
                if (m >= M) continue;
                int32_t d = acc[f][q][r];
                if (XS) d = e.xsum[m] - 2 * d;     // D = xsum - 2 sum q w
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
        hipLaunchKernelGGL((k_bwn_i8_gemm<true, false>), grid, block, 0, s, Xq, ldXq, Wp, ldW, (int)M, (int)N, (int)K, tiles_n, e);
    else if (e.xsum)
        hipLaunchKernelGGL((k_bwn_i8_gemm<false, true>), grid, block, 0, s, Xq, ldXq, Wp, ldW, (int)M, (int)N, (int)K, tiles_n, e);
    else
        hipLaunchKernelGGL((k_bwn_i8_gemm<false, false>), grid, block, 0, s, Xq, ldXq, Wp, ldW, (int)M, (int)N, (int)K, tiles_n, e);
    return hipGetLastError();
}

}  // namespace bnn
