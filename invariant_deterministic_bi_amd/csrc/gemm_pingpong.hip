// Batch-invariant bf16 GEMM, 256 x BN tiles (BN = 256, 192 or 128), eight
// wavefronts in a ping-pong schedule.  Below BN = 256 each wavefront owns a
// 128 x BN/4 block and issues BN/64 B loads per memory phase instead of
// four; everything else below is written for BN = 256.
//
// The two wavefronts that share a SIMD (w and w + 4) belong to different
// groups: group 0 (wavefronts 0..3) owns output rows 0..127 of the tile and
// group 1 rows 128..255, each wavefront a 128 x 64 block.  A K step of 64
// columns has two phases, separated by barriers.  In each phase one group
// runs its 64 MFMAs of the step back to back on fragments already in
// registers, while the other group reads its fragments for its next compute
// phase from LDS and issues its share of the LDS-DMA loads for later steps.
// Each SIMD therefore always has one wavefront feeding the matrix core and
// one doing everything else.
//
// LDS (160 KB): A rows 0..127 in a 2-deep ring of 64-column stages, A rows
// 128..255 in another, and B (256 rows) in a 3-deep ring.  With stage s read
// by group 0 in phase b of step s - 1 and by group 1 in phase a of step s,
// the loads of stage s are issued as follows (each issuing wavefront: 8 DMA
// instructions per memory phase, 1 KB each):
//   A rows 0..127   by group 1, phase a of step s - 2
//   A rows 128..255 by group 0, phase b of step s - 2
//   B rows 0..127   by group 0, phase b of step s - 3
//   B rows 128..255 by group 1, phase a of step s - 2
// so every wavefront, at the end of its memory phase, waits until only that
// phase's 8 loads are in flight: the loads of its previous memory phase are
// the ones the other group reads next.
//
// Bits: an output element's chain is the tiled kernel's (same MFMA, 32-K
// chunks in ascending order from +0, 2 * ceil(K / 64) of them, one bf16 RNE);
// which wavefront, phase or tile order computes it does not enter.

#include "gemm_kernel.h"

namespace bi {
namespace pingpong {

using namespace gemm_detail;

constexpr int kBM = 256, kNT = 512;
constexpr int kHalf = 128 * kRowBytes;    // one 64-column stage of 128 rows: 16 KB
constexpr int kOffA0 = 0, kOffA1 = 2 * kHalf, kOffB = 4 * kHalf;

// What depends on the tile width BN (256 or 192 columns).
template <int BN>
struct Shape {
    static constexpr int FN = BN / 64;            // 16-column blocks per wavefront
    static constexpr int BW = BN / 8;             // B rows per wavefront per memory phase
    static constexpr int BL = BW / 8;             // B DMA instructions per memory phase
    static constexpr int LOADS = 4 + BL;          // DMA instructions per memory phase
    static constexpr int BStage = BN * kRowBytes;
    static constexpr int Lds = 4 * kHalf + 3 * BStage;  // 160 KB at BN = 256, 136 KB at 192
    static constexpr int CStride = BN * 2 + 16;   // padded bf16 output row in LDS
    static_assert(BN == 256 || BN == 192 || BN == 128, "tile widths of the ping-pong schedule");
    static_assert(kBM * CStride <= Lds, "the output tile is staged in the ring space");
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int OFF>
__device__ __forceinline__ u32x4 rd128(uint32_t addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF) : "memory");
    return v;
}

// Per-lane constants of an 8-row DMA instruction into a 128-byte-per-row
// staged tile: lane -> row rl = lane >> 3 of the 8, physical chunk lane & 7,
// which holds logical chunk swz(row, lane & 7).  swz reads row bits 1..3;
// bit 3 comes from the 8-row group (v = (row0 >> 3) & 1), bits 1..2 from rl.
struct DmaLane {
    int off[2];  // rl * ld * 2 + logical chunk * 16, for v = 0, 1
    int kc[2];   // logical chunk * 8 (its first K column), for v = 0, 1
    int rl;
    __device__ __forceinline__ void init(int lane, int64_t ld) {
        rl = lane >> 3;
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const int c = swz(rl + 8 * v, lane & 7);
            off[v] = (int)(rl * ld * 2) + c * 16;
            kc[v] = c * 8;
        }
    }
};

// Rows row0 .. row0+7 (row0 % 8 == 0, V = its bit 3) of K stage k0.
template <int V>
__device__ __forceinline__ void dma8(const i32x4 &rs, char *tile, const DmaLane &dl, int row0, int k0,
                                     int K, int rows_valid, int64_t ld, bool live) {
    int voff = dl.off[V] + (int)(row0 * ld * 2) + k0 * 2;
    if (!(live && row0 + 8 <= rows_valid && k0 + kBK <= K)) {  // some lanes out of range
        const bool ok = live && row0 + dl.rl < rows_valid && k0 + dl.kc[V] < K;
        voff = ok ? voff : (int)0x80000000;
    }
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane(rs.x);
    r.y = __builtin_amdgcn_readfirstlane(rs.y);
    r.z = __builtin_amdgcn_readfirstlane(rs.z);
    r.w = __builtin_amdgcn_readfirstlane(rs.w);
    bi_raw_buffer_load_lds(r, (__attribute__((address_space(3))) uint32_t *)(tile + row0 * kRowBytes), 16, voff,
                           0, 0, 0);
}

template <int BN>
__global__ __launch_bounds__(kNT, 1) void pingpong_kernel(GemmArgs p) {
    using S = Shape<BN>;
    constexpr int FN = S::FN;
    __shared__ __attribute__((aligned(1024))) char lds[S::Lds];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = wave >> 2, j = wave & 3;  // group, column strip
    const int nk = (p.K + 63) >> 6;  // 64-column stages (two 32-wide chunks each)
    const int G = gridDim.x;
    const bool spread = (G % 8) == 0;
    const int slot = spread ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    const uint32_t lds0 = lds_addr(lds);

    for (int base = 0; base < p.num_tiles; base += G) {
        const int L = base + slot;
        if (L >= p.num_tiles) break;
        int bh, tm, tn;
        tile_coords(L, p.tiles_m, p.tiles_n, bh, tm, tn);
        const int m0 = tm * kBM, n0 = tn * BN;
        const uint16_t *Ab = static_cast<const uint16_t *>(p.A) + (int64_t)m0 * p.lda;
        const uint16_t *Bb = static_cast<const uint16_t *>(p.B) + (int64_t)n0 * p.ldb;
        const int rows_a = min(kBM, p.M - m0), rows_b = min(BN, p.N - n0);
        const i32x4 ra = make_rsrc(Ab, (uint32_t)(((int64_t)(rows_a - 1) * p.lda + p.K) * 2));
        const i32x4 rb = make_rsrc(Bb, (uint32_t)(((int64_t)(rows_b - 1) * p.ldb + p.K) * 2));
        DmaLane dla, dlb;
        dla.init(lane, p.lda);
        dlb.init(lane, p.ldb);

        // This wavefront's 8 loads of one memory phase.  Group 1 (phase a of
        // step t): A rows 0..127 of stage t + 2 and B rows 128..255 of stage
        // t + 2.  Group 0 (phase b of step t): A rows 128..255 of stage t + 2
        // and B rows 0..127 of stage t + 3.  Each wavefront takes 32 rows of
        // each.  Stages past the last issue zero-filling loads into the slot
        // they would use, which nobody reads.
        // B rows rb0, rb0 + 8, ... of one stage: BL instructions.  Bit 3 of
        // an 8-row group's first row selects the DMA lane offsets; rb0 is
        // b_row0 + BW * j, so at BW = 24 it alternates with j's parity.
        auto dma_b = [&](char *b_tile, int rb0, int k0, bool live) {
            if constexpr (S::BL == 4) {
                dma8<0>(rb, b_tile, dlb, rb0, k0, p.K, rows_b, p.ldb, live);
                dma8<1>(rb, b_tile, dlb, rb0 + 8, k0, p.K, rows_b, p.ldb, live);
                dma8<0>(rb, b_tile, dlb, rb0 + 16, k0, p.K, rows_b, p.ldb, live);
                dma8<1>(rb, b_tile, dlb, rb0 + 24, k0, p.K, rows_b, p.ldb, live);
            } else if constexpr (S::BL == 2) {
                dma8<0>(rb, b_tile, dlb, rb0, k0, p.K, rows_b, p.ldb, live);
                dma8<1>(rb, b_tile, dlb, rb0 + 8, k0, p.K, rows_b, p.ldb, live);
            } else if (j & 1) {
                dma8<1>(rb, b_tile, dlb, rb0, k0, p.K, rows_b, p.ldb, live);
                dma8<0>(rb, b_tile, dlb, rb0 + 8, k0, p.K, rows_b, p.ldb, live);
                dma8<1>(rb, b_tile, dlb, rb0 + 16, k0, p.K, rows_b, p.ldb, live);
            } else {
                dma8<0>(rb, b_tile, dlb, rb0, k0, p.K, rows_b, p.ldb, live);
                dma8<1>(rb, b_tile, dlb, rb0 + 8, k0, p.K, rows_b, p.ldb, live);
                dma8<0>(rb, b_tile, dlb, rb0 + 16, k0, p.K, rows_b, p.ldb, live);
            }
        };
        auto issue = [&](int t) {
            const int sa = t + 2, sbb = g ? t + 2 : t + 3;
            const int a_row0 = g ? 0 : 128;   // tile row of the A half this group loads
            const int b_row0 = g ? BN / 2 : 0;
            // the A half buffer holds its 128 rows as rows 0..127
            char *a_tile = lds + (g ? kOffA0 : kOffA1) + (sa & 1) * kHalf - a_row0 * kRowBytes;
            char *b_tile = lds + kOffB + (sbb % 3) * S::BStage;
            const int ra0 = a_row0 + 32 * j, rb0 = b_row0 + S::BW * j;
            dma8<0>(ra, a_tile, dla, ra0, sa * kBK, p.K, rows_a, p.lda, sa < nk);
            dma8<1>(ra, a_tile, dla, ra0 + 8, sa * kBK, p.K, rows_a, p.lda, sa < nk);
            dma8<0>(ra, a_tile, dla, ra0 + 16, sa * kBK, p.K, rows_a, p.lda, sa < nk);
            dma8<1>(ra, a_tile, dla, ra0 + 24, sa * kBK, p.K, rows_a, p.lda, sa < nk);
            dma_b(b_tile, rb0, sbb * kBK, sbb < nk);
        };

        // This wavefront's fragments of one stage: fa[K step][16-row block],
        // fb[K step][16-column block].
        u32x4 fa[2][8], fb[2][4];  // fb[..][FN..3] unused below BN = 256
        f32x4 acc[8][FN];
#pragma unroll
        for (int fm = 0; fm < 8; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

        // Fragment reads of stage s.  Rows 16 apart share swz (it reads a
        // row's low four bits), so one address per operand and K step serves
        // all its blocks, the block offset going in the instruction.
        const int r16 = lane & 15;
        const uint32_t a_lane = lds0 + (g ? kOffA1 : kOffA0) + r16 * kRowBytes;
        const uint32_t b_lane = lds0 + kOffB + ((BN / 4) * j + r16) * kRowBytes;
        const uint32_t sw0 = swz(r16, lane >> 4) * 16, sw1 = swz(r16, 4 + (lane >> 4)) * 16;
#define BI_PP_READ(s)                                                                          \
    do {                                                                                       \
        const uint32_t a0 = a_lane + ((s) & 1) * kHalf + sw0, a1 = a_lane + ((s) & 1) * kHalf + sw1; \
        const uint32_t b0 = b_lane + ((s) % 3) * S::BStage + sw0, b1 = b_lane + ((s) % 3) * S::BStage + sw1; \
        fa[0][0] = rd128<0 * 2048>(a0); fa[0][1] = rd128<1 * 2048>(a0);                      \
        fa[0][2] = rd128<2 * 2048>(a0); fa[0][3] = rd128<3 * 2048>(a0);                      \
        fa[0][4] = rd128<4 * 2048>(a0); fa[0][5] = rd128<5 * 2048>(a0);                      \
        fa[0][6] = rd128<6 * 2048>(a0); fa[0][7] = rd128<7 * 2048>(a0);                      \
        fb[0][0] = rd128<0 * 2048>(b0); fb[0][1] = rd128<1 * 2048>(b0);                      \
        if constexpr (FN >= 3) fb[0][2] = rd128<2 * 2048>(b0);                               \
        if constexpr (FN == 4) fb[0][3] = rd128<3 * 2048>(b0);                               \
        fa[1][0] = rd128<0 * 2048>(a1); fa[1][1] = rd128<1 * 2048>(a1);                      \
        fa[1][2] = rd128<2 * 2048>(a1); fa[1][3] = rd128<3 * 2048>(a1);                      \
        fa[1][4] = rd128<4 * 2048>(a1); fa[1][5] = rd128<5 * 2048>(a1);                      \
        fa[1][6] = rd128<6 * 2048>(a1); fa[1][7] = rd128<7 * 2048>(a1);                      \
        fb[1][0] = rd128<0 * 2048>(b1); fb[1][1] = rd128<1 * 2048>(b1);                      \
        if constexpr (FN >= 3) fb[1][2] = rd128<2 * 2048>(b1);                               \
        if constexpr (FN == 4) fb[1][3] = rd128<3 * 2048>(b1);                               \
    } while (0)
// The reads are complete, and the compiler may not use their registers
// before this point.
#define BI_PP_SETTLE()                                                                         \
    do {                                                                                       \
        asm volatile("s_waitcnt lgkmcnt(0)"                                                   \
                     : "+v"(fa[0][0]), "+v"(fa[0][1]), "+v"(fa[0][2]), "+v"(fa[0][3]),         \
                       "+v"(fa[0][4]), "+v"(fa[0][5]), "+v"(fa[0][6]), "+v"(fa[0][7])::"memory"); \
        asm volatile(""                                                                        \
                     : "+v"(fa[1][0]), "+v"(fa[1][1]), "+v"(fa[1][2]), "+v"(fa[1][3]),         \
                       "+v"(fa[1][4]), "+v"(fa[1][5]), "+v"(fa[1][6]), "+v"(fa[1][7])::"memory"); \
        asm volatile("" : "+v"(fb[0][0]), "+v"(fb[0][1]), "+v"(fb[1][0]), "+v"(fb[1][1])::"memory"); \
        if constexpr (FN >= 3) asm volatile("" : "+v"(fb[0][2]), "+v"(fb[1][2])::"memory");    \
        if constexpr (FN == 4) asm volatile("" : "+v"(fb[0][3]), "+v"(fb[1][3])::"memory");    \
    } while (0)
#define BI_PP_COMPUTE()                                                                        \
    do {                                                                                       \
        _Pragma("unroll") for (int ks = 0; ks < 2; ++ks)                                       \
        _Pragma("unroll") for (int fm = 0; fm < 8; ++fm)                                       \
        _Pragma("unroll") for (int fn = 0; fn < FN; ++fn)                                      \
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                             \
                __builtin_bit_cast(bf16x8, fa[ks][fm]), __builtin_bit_cast(bf16x8, fb[ks][fn]), \
                acc[fm][fn], 0, 0, 0);                                                         \
    } while (0)

        // Prologue: the memory phases of steps -3 .. -1 (stages 0, 1 and the
        // first half of B(2)); group 0's step -3 loads only B(0)'s first half
        // (its A1(-1) half is a stage that does not exist).  Then everything
        // lands, and group 0 reads its fragments of stage 0.
        if (g == 0) dma_b(lds + kOffB, S::BW * j, 0, nk > 0);
        issue(-2);
        issue(-1);
        wait_vmcnt<0>();
        lds_barrier();
        // One loop body serves both groups, group 1 running half a step
        // behind: each iteration is [compute stage t] barrier [read stage t + 1,
        // issue loads] barrier.  Group 0's compute is phase a of step t, its
        // memory work phase b; group 1 starts with the memory work of phase a
        // of step 0, so its compute is phase b of step t and its memory work
        // phase a of step t + 1 -- and it issues the loads of step t + 1.  The
        // barriers pair up: group 0 ends with one more.  A read of stage nk
        // reads a slot nobody uses (harmless, in bounds).
        if (g == 0) {
            BI_PP_READ(0);
            BI_PP_SETTLE();
        }
        lds_barrier();
        if (g == 1) {
            BI_PP_READ(0);
            issue(0);
            BI_PP_SETTLE();
            wait_vmcnt<S::LOADS>();
            lds_barrier();
        }
        // sched_barrier(0) keeps the compiler from moving MFMAs (which touch
        // no memory) across the phase barriers.
        for (int t = 0; t < nk; ++t) {
            __builtin_amdgcn_sched_barrier(0);
            BI_PP_COMPUTE();
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            BI_PP_READ(t + 1);
            issue(t + g);
            BI_PP_SETTLE();
            wait_vmcnt<S::LOADS>();
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        if (g == 0) lds_barrier();
#undef BI_PP_READ
#undef BI_PP_SETTLE
#undef BI_PP_COMPUTE

        // Epilogue: every load has landed (the zero-filling ones included),
        // then fp32 -> bf16 RNE into a padded LDS tile and 16-byte row chunks
        // to global memory.
        wait_vmcnt<0>();
        lds_barrier();
        char *ct = lds;
#pragma unroll
        for (int fm = 0; fm < 8; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int col = (BN / 4) * j + fn * 16 + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 128 * g + fm * 16 + (lane >> 4) * 4 + i;
                    *reinterpret_cast<uint16_t *>(ct + row * S::CStride + col * 2) =
                        (uint16_t)f32_to_bf16_rne(acc[fm][fn][i]);
                }
            }
        __syncthreads();
        constexpr int CPR = BN / 8;
        uint16_t *Yb = static_cast<uint16_t *>(p.Y);
        for (int q = tid; q < rows_a * CPR; q += kNT) {
            const int row = q / CPR, c8 = q % CPR;
            const int col = n0 + c8 * 8;
            const uint4 v = *reinterpret_cast<const uint4 *>(ct + row * S::CStride + c8 * 16);
            uint16_t *dst = Yb + (int64_t)(m0 + row) * p.ldy + col;
            if (col + 8 <= p.N && (((uintptr_t)dst) & 15) == 0) {
                *reinterpret_cast<uint4 *>(dst) = v;
            } else {
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (col + e < p.N) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
            }
        }
        __syncthreads();  // the LDS is reused by the next tile's prologue
    }
}

// ---------------------------------------------------------------------------
// The NVFP4 weight (bf16 A, raw NVFP4 B: codes [N, K/2], E4M3 scales [N,
// K/16], K % 64 == 0) in the same ping-pong schedule, 256 x 256 tiles.
//
// B reaches LDS raw: per 64-column stage, 256 rows of 32 code bytes and 4
// scale bytes (9 KB, against 32 KB of bf16), by LDS DMA.  In its memory
// phase each wavefront reads the raw bytes of its own 64 columns and decodes
// them straight into its B fragment registers (the exact decode of the tiled
// kernel: FP4 pair convert with a unit scale, one fp32 multiply by the E4M3
// scale, top halves), beside the other group's MFMAs.  The decoded fragment
// holds the same bf16 values the tiled kernel reads from its decoded LDS
// tile, so every output element's chain -- and its bits -- are the same.
//
// The small B stage frees LDS for deeper prefetch: with W memory phases in
// flight per wavefront, stage s of
//   A rows 0..127   is issued by group 1 in phase a of step s - 1 - W,
//   A rows 128..255 by group 0 in phase b of step s - 1 - W,
//   B rows 0..127   by group 0 in phase b of step s - 2 - W,
//   B rows 128..255 by group 1 in phase a of step s - 1 - W,
// and each wavefront, at the end of a memory phase, waits until only its
// last W phases' loads are in flight.  The A half rings hold W + 1 stages,
// the raw B ring W + 2 (a slot is reissued only after both groups read it).
// ---------------------------------------------------------------------------
template <int W>
struct Nv4Shape {
    static constexpr int BN = 256, FN = 4;
    static constexpr int RA = W + 1, RB = W + 2;  // ring depths
    static constexpr int CodeBytes = BN * 32, RawStage = BN * 36;
    static constexpr int OffB = 2 * RA * kHalf;   // after the two A half rings
    static constexpr int Pipe = OffB + RB * RawStage;
    static constexpr int CStride = BN * 2 + 16;
    static constexpr int CBytes = kBM * CStride;
    static constexpr int Lds = Pipe > CBytes ? Pipe : CBytes;
    static_assert(Lds <= 160 * 1024, "LDS budget of gfx950");
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int OFF0, int OFF1>
__device__ __forceinline__ u32x2 rd2x32(uint32_t addr) {
    u32x2 v;
    asm volatile("ds_read2_b32 %0, %1 offset0:%2 offset1:%3" : "=v"(v) : "v"(addr), "n"(OFF0), "n"(OFF1) : "memory");
    return v;
}
template <int OFF>
__device__ __forceinline__ uint32_t rd32(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF) : "memory");
    return v;
}

template <int W>
__global__ __launch_bounds__(kNT, 1) void pingpong_nvfp4_kernel(GemmArgs p) {
    using S = Nv4Shape<W>;
    constexpr int BN = S::BN, FN = S::FN;
    __shared__ __attribute__((aligned(1024))) char lds[S::Lds];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = wave >> 2, j = wave & 3;  // group, column strip
    const int nk = p.K >> 6;  // 64-column stages (K % 64 == 0)
    const int cpr = p.K >> 1, spr = p.K >> 4;  // code / scale bytes per weight row
    const int G = gridDim.x;
    const bool spread = (G % 8) == 0;
    const int slot = spread ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    const uint32_t lds0 = lds_addr(lds);
    // this wavefront's loads per memory phase: 4 A instructions, 1 code
    // instruction (32 rows), and for j < 2 one scale instruction (64 rows)
    const bool scale_wave = j < 2;

    for (int base = 0; base < p.num_tiles; base += G) {
        const int L = base + slot;
        if (L >= p.num_tiles) break;
        int bh, tm, tn;
        tile_coords(L, p.tiles_m, p.tiles_n, bh, tm, tn);
        const int m0 = tm * kBM, n0 = tn * BN;
        const uint16_t *Ab = static_cast<const uint16_t *>(p.A) + (int64_t)m0 * p.lda;
        const uint8_t *Cb = static_cast<const uint8_t *>(p.B) + (int64_t)n0 * cpr;
        const uint8_t *Sb = static_cast<const uint8_t *>(p.B_scales) + (int64_t)n0 * spr;
        const int rows_a = min(kBM, p.M - m0), rows_b = min(BN, p.N - n0);
        const i32x4 ra = make_rsrc(Ab, (uint32_t)(((int64_t)(rows_a - 1) * p.lda + p.K) * 2));
        const i32x4 rc = make_rsrc(Cb, (uint32_t)(rows_b * cpr));
        const i32x4 rs = make_rsrc(Sb, (uint32_t)(rows_b * spr));
        DmaLane dla;
        dla.init(lane, p.lda);
        // raw B DMA lanes: group g fills rows 128 g .. 128 g + 127 of a stage
        const int crow = 128 * g + 32 * j + (lane >> 1);        // code row of this lane
        const int code_off = crow < rows_b ? crow * cpr + (lane & 1) * 16 : (int)0x80000000;
        const int srow = 128 * g + 64 * j + lane;               // scale row (j < 2)
        const int scale_off = srow < rows_b ? srow * spr : (int)0x80000000;

        auto dma_raw = [&](int s, bool live) {
            char *st = lds + S::OffB + (s % S::RB) * S::RawStage;
            i32x4 r;
            r.x = __builtin_amdgcn_readfirstlane(rc.x);
            r.y = __builtin_amdgcn_readfirstlane(rc.y);
            r.z = __builtin_amdgcn_readfirstlane(rc.z);
            r.w = __builtin_amdgcn_readfirstlane(rc.w);
            const int vc = (live && code_off >= 0) ? code_off + s * 32 : (int)0x80000000;
            bi_raw_buffer_load_lds(r, (__attribute__((address_space(3))) uint32_t *)(st + (128 * g + 32 * j) * 32),
                                   16, vc, 0, 0, 0);
            if (scale_wave) {
                i32x4 q;
                q.x = __builtin_amdgcn_readfirstlane(rs.x);
                q.y = __builtin_amdgcn_readfirstlane(rs.y);
                q.z = __builtin_amdgcn_readfirstlane(rs.z);
                q.w = __builtin_amdgcn_readfirstlane(rs.w);
                const int vs = (live && scale_off >= 0) ? scale_off + s * 4 : (int)0x80000000;
                bi_raw_buffer_load_lds(
                    q, (__attribute__((address_space(3))) uint32_t *)(st + S::CodeBytes + (128 * g + 64 * j) * 4), 4,
                    vs, 0, 0, 0);
            }
        };
        // The loads of one memory phase: group 1 in phase a of step u, group
        // 0 in phase b of step u.
        auto issue = [&](int u) {
            const int sa = u + 1 + W, sbb = g ? u + 1 + W : u + 2 + W;
            const int a_row0 = g ? 0 : 128;   // tile row of the A half this group loads
            char *a_tile = lds + (g ? 0 : S::RA * kHalf) + (sa % S::RA) * kHalf - a_row0 * kRowBytes;
            const int ra0 = a_row0 + 32 * j;
            dma8<0>(ra, a_tile, dla, ra0, sa * kBK, p.K, rows_a, p.lda, sa < nk);
            dma8<1>(ra, a_tile, dla, ra0 + 8, sa * kBK, p.K, rows_a, p.lda, sa < nk);
            dma8<0>(ra, a_tile, dla, ra0 + 16, sa * kBK, p.K, rows_a, p.lda, sa < nk);
            dma8<1>(ra, a_tile, dla, ra0 + 24, sa * kBK, p.K, rows_a, p.lda, sa < nk);
            dma_raw(sbb, sbb < nk);
        };
        auto wait_phases = [&]() {  // only the last W memory phases' loads in flight
            if (scale_wave) wait_vmcnt<6 * W>();
            else wait_vmcnt<5 * W>();
        };

        u32x4 fa[2][8];
        f32x4 acc[8][FN];
#pragma unroll
        for (int fm = 0; fm < 8; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

        const int r16 = lane & 15;
        const uint32_t a_lane = lds0 + (g ? S::RA * kHalf : 0) + r16 * kRowBytes;
        const uint32_t sw0 = swz(r16, lane >> 4) * 16, sw1 = swz(r16, 4 + (lane >> 4)) * 16;
        // raw B of this lane: code dwords of chunks (lane >> 4) and 4 + (lane >> 4)
        // of column 64 j + 16 fn + r16, and that column's scale dword
        const uint32_t c_lane = lds0 + S::OffB + (64 * j + r16) * 32 + (lane >> 4) * 4;
        const uint32_t s_lane = lds0 + S::OffB + S::CodeBytes + (64 * j + r16) * 4;
        const int sshift = (lane >> 5) * 8;  // the scale byte of K chunk 0 (chunk 1: two bytes up)
        u32x2 cw[4];
        uint32_t sv[4];
        u32x4 bc0, bc1;  // the B fragments of the 16-column block being multiplied
        // Memory phase: the raw B bytes and A's fragments of stage s.
#define BI_P4_READ(s)                                                                          \
    do {                                                                                       \
        const uint32_t cb = c_lane + ((s) % S::RB) * S::RawStage;                              \
        const uint32_t sb = s_lane + ((s) % S::RB) * S::RawStage;                              \
        cw[0] = rd2x32<0, 4>(cb); cw[1] = rd2x32<0, 4>(cb + 512);                              \
        cw[2] = rd2x32<0, 4>(cb + 1024); cw[3] = rd2x32<0, 4>(cb + 1536);                      \
        sv[0] = rd32<0>(sb); sv[1] = rd32<64>(sb); sv[2] = rd32<128>(sb); sv[3] = rd32<192>(sb); \
        const uint32_t a0 = a_lane + ((s) % S::RA) * kHalf + sw0, a1 = a_lane + ((s) % S::RA) * kHalf + sw1; \
        fa[0][0] = rd128<0 * 2048>(a0); fa[0][1] = rd128<1 * 2048>(a0);                      \
        fa[0][2] = rd128<2 * 2048>(a0); fa[0][3] = rd128<3 * 2048>(a0);                      \
        fa[0][4] = rd128<4 * 2048>(a0); fa[0][5] = rd128<5 * 2048>(a0);                      \
        fa[0][6] = rd128<6 * 2048>(a0); fa[0][7] = rd128<7 * 2048>(a0);                      \
        fa[1][0] = rd128<0 * 2048>(a1); fa[1][1] = rd128<1 * 2048>(a1);                      \
        fa[1][2] = rd128<2 * 2048>(a1); fa[1][3] = rd128<3 * 2048>(a1);                      \
        fa[1][4] = rd128<4 * 2048>(a1); fa[1][5] = rd128<5 * 2048>(a1);                      \
        fa[1][6] = rd128<6 * 2048>(a1); fa[1][7] = rd128<7 * 2048>(a1);                      \
    } while (0)
#define BI_P4_SETTLE()                                                                         \
    do {                                                                                       \
        asm volatile("s_waitcnt lgkmcnt(0)"                                                   \
                     : "+v"(fa[0][0]), "+v"(fa[0][1]), "+v"(fa[0][2]), "+v"(fa[0][3]),         \
                       "+v"(fa[0][4]), "+v"(fa[0][5]), "+v"(fa[0][6]), "+v"(fa[0][7])::"memory"); \
        asm volatile(""                                                                        \
                     : "+v"(fa[1][0]), "+v"(fa[1][1]), "+v"(fa[1][2]), "+v"(fa[1][3]),         \
                       "+v"(fa[1][4]), "+v"(fa[1][5]), "+v"(fa[1][6]), "+v"(fa[1][7])::"memory"); \
        asm volatile("" : "+v"(cw[0]), "+v"(cw[1]), "+v"(cw[2]), "+v"(cw[3]), "+v"(sv[0]), "+v"(sv[1]), \
                     "+v"(sv[2]), "+v"(sv[3])::"memory");                                      \
    } while (0)
// B fragments of 16-column block fn from the raw bytes (K chunks 0 and 1).
#define BI_P4_DECODE(fn, b0, b1)                                                               \
    do {                                                                                       \
        const uint32_t sh = sv[fn] >> sshift;                                                  \
        const uint4 d0 = decode8(cw[fn].x, e4m3_value<0>(sh));                                 \
        const uint4 d1 = decode8(cw[fn].y, e4m3_value<2>(sh));                                 \
        b0 = u32x4{d0.x, d0.y, d0.z, d0.w};                                                    \
        b1 = u32x4{d1.x, d1.y, d1.z, d1.w};                                                    \
    } while (0)
// Compute phase: block 0's fragments were decoded at the end of the memory
// phase; block fn + 1's are decoded while block fn's 16 MFMAs run (the
// group barriers interleave one MFMA with two VALU instructions).  Every
// accumulator still sees K chunk 0, then chunk 1.
#define BI_P4_COMPUTE()                                                                        \
    do {                                                                                       \
        _Pragma("unroll") for (int fn = 0; fn < FN; ++fn) {                                    \
            u32x4 n0, n1;                                                                      \
            if (fn + 1 < FN) BI_P4_DECODE(fn + 1, n0, n1);                                     \
            _Pragma("unroll") for (int fm = 0; fm < 8; ++fm)                                   \
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                         \
                    __builtin_bit_cast(bf16x8, fa[0][fm]), __builtin_bit_cast(bf16x8, bc0), acc[fm][fn], 0, 0, 0); \
            _Pragma("unroll") for (int fm = 0; fm < 8; ++fm)                                   \
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                         \
                    __builtin_bit_cast(bf16x8, fa[1][fm]), __builtin_bit_cast(bf16x8, bc1), acc[fm][fn], 0, 0, 0); \
            if (fn + 1 < FN) {                                                                 \
                bc0 = n0;                                                                      \
                bc1 = n1;                                                                      \
            }                                                                                  \
        }                                                                                      \
        _Pragma("unroll") for (int i = 0; i < 48; ++i) {                                       \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                 \
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);                                 \
        }                                                                                      \
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);                                    \
    } while (0)

        // Prologue: B rows 0..127 of stage 0 (group 0), then the memory
        // phases of steps -1-W .. -1; everything lands; group 0 reads stage 0.
        if (g == 0) dma_raw(0, nk > 0);
#pragma unroll
        for (int u = -1 - W; u < 0; ++u) issue(u);
        wait_vmcnt<0>();
        lds_barrier();
        if (g == 0) {
            BI_P4_READ(0);
            BI_P4_SETTLE();
            BI_P4_DECODE(0, bc0, bc1);
        }
        lds_barrier();
        if (g == 1) {
            BI_P4_READ(0);
            issue(0);
            BI_P4_SETTLE();
            BI_P4_DECODE(0, bc0, bc1);
            wait_phases();
            lds_barrier();
        }
        for (int t = 0; t < nk; ++t) {
            __builtin_amdgcn_sched_barrier(0);
            BI_P4_COMPUTE();
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            BI_P4_READ(t + 1);
            issue(t + g);
            BI_P4_SETTLE();
            BI_P4_DECODE(0, bc0, bc1);
            wait_phases();
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        if (g == 0) lds_barrier();
#undef BI_P4_READ
#undef BI_P4_SETTLE
#undef BI_P4_DECODE
#undef BI_P4_COMPUTE

        // Epilogue: every load has landed; fp32 x alpha -> bf16 RNE into a
        // padded LDS tile, then 16-byte row chunks to global memory.
        wait_vmcnt<0>();
        lds_barrier();
        char *ct = lds;
#pragma unroll
        for (int fm = 0; fm < 8; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int col = 64 * j + fn * 16 + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 128 * g + fm * 16 + (lane >> 4) * 4 + i;
                    *reinterpret_cast<uint16_t *>(ct + row * S::CStride + col * 2) =
                        (uint16_t)f32_to_bf16_rne(acc[fm][fn][i] * p.alpha);
                }
            }
        __syncthreads();
        constexpr int CPR = BN / 8;
        uint16_t *Yb = static_cast<uint16_t *>(p.Y);
        for (int q = tid; q < rows_a * CPR; q += kNT) {
            const int row = q / CPR, c8 = q % CPR;
            const int col = n0 + c8 * 8;
            const uint4 v = *reinterpret_cast<const uint4 *>(ct + row * S::CStride + c8 * 16);
            uint16_t *dst = Yb + (int64_t)(m0 + row) * p.ldy + col;
            if (col + 8 <= p.N && (((uintptr_t)dst) & 15) == 0) {
                *reinterpret_cast<uint4 *>(dst) = v;
            } else {
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (col + e < p.N) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
            }
        }
        __syncthreads();  // the LDS is reused by the next tile's prologue
    }
}

}  // namespace pingpong

hipError_t launch_pingpong_nvfp4(const GemmArgs &a, int grid, int depth, hipStream_t s) {
    if (a.batch != 1 || grid < 1 || a.group_off || a.K % 64 != 0) return hipErrorInvalidValue;
    if ((depth > 0 ? depth : kPingPongNvfp4Depth) == 1)
        hipLaunchKernelGGL(pingpong::pingpong_nvfp4_kernel<1>, dim3(grid), dim3(pingpong::kNT), 0, s, a);
    else
        hipLaunchKernelGGL(pingpong::pingpong_nvfp4_kernel<2>, dim3(grid), dim3(pingpong::kNT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pingpong(const GemmArgs &a, int bn, int grid, hipStream_t s) {
    if (a.batch != 1 || grid < 1 || a.group_off) return hipErrorInvalidValue;
    if (bn == 256)
        hipLaunchKernelGGL(pingpong::pingpong_kernel<256>, dim3(grid), dim3(pingpong::kNT), 0, s, a);
    else if (bn == 192)
        hipLaunchKernelGGL(pingpong::pingpong_kernel<192>, dim3(grid), dim3(pingpong::kNT), 0, s, a);
    else if (bn == 128)
        hipLaunchKernelGGL(pingpong::pingpong_kernel<128>, dim3(grid), dim3(pingpong::kNT), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace bi
