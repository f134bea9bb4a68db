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
// scale bytes (9 KB, against 32 KB of bf16), by LDS DMA.  The two groups
// take different shares of the memory work, so that the decode arithmetic
// never runs beside the other group's decode:
//   * group 0, in its memory phase (phase b of step s - 1), reads A rows
//     0..127 and the raw B of stage s, decodes the B fragments of its
//     wavefront's 64 columns straight into registers (the exact decode of
//     the tiled kernel: FP4 pair convert with a unit scale, one fp32
//     multiply by the E4M3 scale, top halves) and writes them to a decoded
//     B buffer in LDS;
//   * group 1, in its memory phase (phase a of step s), reads A rows
//     128..255 and the decoded B fragments of its wavefront's columns (the
//     same 64 columns), and issues every LDS-DMA load: A rows 0..127, A
//     rows 128..255 and the raw B of stage s + 2, in phase a of step s.
// Each compute phase is then 64 MFMAs on fragments in registers.  Group 1
// waits, at the end of a memory phase, until only that phase's loads are in
// flight; stage s's loads (issued in phase a of step s - 2) have landed by
// the end of phase a of step s - 1, before group 0 reads them in phase b of
// step s - 1.  Rings: A rows 0..127 two stages, A rows 128..255 three (group
// 1 reads stage s and reissues its slot in the same phase), raw B two, the
// decoded B one (written in phase b of step s - 1, read in phase a of s).
// The decoded fragments hold the same bf16 values the tiled kernel reads
// from its decoded LDS tile, so every output element's chain -- and its
// bits -- are the same.
// ---------------------------------------------------------------------------
struct Nv4Shape {
    static constexpr int BN = 256, FN = 4;
    static constexpr int RA0 = 2, RA1 = 3, RR = 2;  // ring depths
    static constexpr int CodeBytes = BN * 32, RawStage = BN * 36;
    static constexpr int OffA1 = RA0 * kHalf;
    static constexpr int OffRaw = OffA1 + RA1 * kHalf;
    static constexpr int OffDec = OffRaw + RR * RawStage;
    static constexpr int DecBytes = BN * kRowBytes;   // 32 KB: 8 KB per column strip
    static constexpr int Pipe = OffDec + DecBytes;
    static constexpr int CStride = BN * 2 + 16;
    static constexpr int CBytes = kBM * CStride;
    static constexpr int Lds = Pipe > CBytes ? Pipe : CBytes;
    static constexpr int LOADS = 11;  // group 1's DMA instructions per memory phase, per wavefront
    static_assert(Lds <= 160 * 1024, "LDS budget of gfx950");
};

template <int OFF>
__device__ __forceinline__ uint32_t rd32(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF) : "memory");
    return v;
}
template <int OFF>
__device__ __forceinline__ void wr128(uint32_t addr, const u32x4 &v) {
    asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(addr), "v"(v), "n"(OFF) : "memory");
}

__global__ __launch_bounds__(kNT, 1) void pingpong_nvfp4_kernel(GemmArgs p) {
    using S = Nv4Shape;
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
        // Raw B DMA lanes (group 1 wavefront j: code rows 64 j .. 64 j + 63 in
        // two instructions of 32 rows, scale rows 64 j .. 64 j + 63 in one).
        // A row's 32 code bytes are two 16-byte halves (K chunks 0 and 1 of
        // the stage); rows whose bit 3 is set store them swapped, so that the
        // fragment reads of rows r and r + 8 fall in different LDS banks.
        const int crow = 64 * j + (lane >> 1);                   // code row of instruction 0
        const int chalf = (lane & 1) ^ ((crow >> 3) & 1);        // the half this lane fetches
        const int code_off0 = crow < rows_b ? crow * cpr + chalf * 16 : (int)0x80000000;
        const int code_off1 = crow + 32 < rows_b ? (crow + 32) * cpr + chalf * 16 : (int)0x80000000;
        const int srow = 64 * j + lane;
        const int scale_off = srow < rows_b ? srow * spr : (int)0x80000000;

        // Group 1's loads of one memory phase (phase a of step u): stage u + 2
        // of A rows 0..127, A rows 128..255 and raw B.  Stages past the last
        // issue zero-filling loads into the slot they would use.
        auto issue = [&](int u) {
            const int st = u + 2;
            const bool live = st < nk;
            char *a0 = lds + (st % S::RA0) * kHalf;
            char *a1 = lds + S::OffA1 + (st % S::RA1) * kHalf - 128 * kRowBytes;
            const int r0 = 32 * j, r1 = 128 + 32 * j;
            dma8<0>(ra, a0, dla, r0, st * kBK, p.K, rows_a, p.lda, live);
            dma8<1>(ra, a0, dla, r0 + 8, st * kBK, p.K, rows_a, p.lda, live);
            dma8<0>(ra, a0, dla, r0 + 16, st * kBK, p.K, rows_a, p.lda, live);
            dma8<1>(ra, a0, dla, r0 + 24, st * kBK, p.K, rows_a, p.lda, live);
            dma8<0>(ra, a1, dla, r1, st * kBK, p.K, rows_a, p.lda, live);
            dma8<1>(ra, a1, dla, r1 + 8, st * kBK, p.K, rows_a, p.lda, live);
            dma8<0>(ra, a1, dla, r1 + 16, st * kBK, p.K, rows_a, p.lda, live);
            dma8<1>(ra, a1, dla, r1 + 24, st * kBK, p.K, rows_a, p.lda, live);
            char *raw = lds + S::OffRaw + (st % S::RR) * S::RawStage;
            i32x4 r;
            r.x = __builtin_amdgcn_readfirstlane(rc.x);
            r.y = __builtin_amdgcn_readfirstlane(rc.y);
            r.z = __builtin_amdgcn_readfirstlane(rc.z);
            r.w = __builtin_amdgcn_readfirstlane(rc.w);
            const int vc0 = (live && code_off0 >= 0) ? code_off0 + st * 32 : (int)0x80000000;
            const int vc1 = (live && code_off1 >= 0) ? code_off1 + st * 32 : (int)0x80000000;
            bi_raw_buffer_load_lds(r, (__attribute__((address_space(3))) uint32_t *)(raw + 64 * j * 32), 16, vc0, 0,
                                   0, 0);
            bi_raw_buffer_load_lds(r, (__attribute__((address_space(3))) uint32_t *)(raw + (64 * j + 32) * 32), 16,
                                   vc1, 0, 0, 0);
            i32x4 q;
            q.x = __builtin_amdgcn_readfirstlane(rs.x);
            q.y = __builtin_amdgcn_readfirstlane(rs.y);
            q.z = __builtin_amdgcn_readfirstlane(rs.z);
            q.w = __builtin_amdgcn_readfirstlane(rs.w);
            const int vs = (live && scale_off >= 0) ? scale_off + st * 4 : (int)0x80000000;
            bi_raw_buffer_load_lds(q, (__attribute__((address_space(3))) uint32_t *)(raw + S::CodeBytes + 64 * j * 4),
                                   4, vs, 0, 0, 0);
        };

        u32x4 fa[2][8], fb[2][4];
        f32x4 acc[8][FN];
#pragma unroll
        for (int fm = 0; fm < 8; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

        const int r16 = lane & 15;
        const uint32_t sw0 = swz(r16, lane >> 4) * 16, sw1 = swz(r16, 4 + (lane >> 4)) * 16;
        // group 0 reads A rows 0..127 from the 2-deep ring, group 1 rows
        // 128..255 from the 3-deep one
        const uint32_t a_lane = lds0 + (g ? S::OffA1 : 0) + r16 * kRowBytes;
        // raw B (group 0): the code dword of 8-element group (lane >> 4) in
        // K chunk 0 and in K chunk 1 of column 64 j + 16 fn + r16, each in the
        // half the swizzle put it in, and that column's scale dword
        const uint32_t c_lane0 = lds0 + S::OffRaw + (64 * j + r16) * 32 + ((r16 >> 3) & 1) * 16 + (lane >> 4) * 4;
        const uint32_t c_lane1 = c_lane0 ^ 16u;
        const uint32_t s_lane = lds0 + S::OffRaw + S::CodeBytes + (64 * j + r16) * 4;
        const int sshift = (lane >> 5) * 8;  // the scale byte of K chunk 0 (chunk 1: two bytes up)
        // decoded B: wavefront strip j's fragments, fragment (ks, fn) of lane l
        // at ((ks * 4 + fn) * 64 + l) * 16
        const uint32_t d_lane = lds0 + S::OffDec + j * 8192 + lane * 16;

#define BI_P4_READ_A(s)                                                                        \
    do {                                                                                       \
        const uint32_t ab = a_lane + (g ? ((s) % S::RA1) : ((s) % S::RA0)) * kHalf;            \
        const uint32_t a0 = ab + sw0, a1 = ab + sw1;                                           \
        fa[0][0] = rd128<0 * 2048>(a0); fa[0][1] = rd128<1 * 2048>(a0);                      \
        fa[0][2] = rd128<2 * 2048>(a0); fa[0][3] = rd128<3 * 2048>(a0);                      \
        fa[0][4] = rd128<4 * 2048>(a0); fa[0][5] = rd128<5 * 2048>(a0);                      \
        fa[0][6] = rd128<6 * 2048>(a0); fa[0][7] = rd128<7 * 2048>(a0);                      \
        fa[1][0] = rd128<0 * 2048>(a1); fa[1][1] = rd128<1 * 2048>(a1);                      \
        fa[1][2] = rd128<2 * 2048>(a1); fa[1][3] = rd128<3 * 2048>(a1);                      \
        fa[1][4] = rd128<4 * 2048>(a1); fa[1][5] = rd128<5 * 2048>(a1);                      \
        fa[1][6] = rd128<6 * 2048>(a1); fa[1][7] = rd128<7 * 2048>(a1);                      \
    } while (0)
#define BI_P4_SETTLE_A()                                                                       \
    do {                                                                                       \
        asm volatile("s_waitcnt lgkmcnt(0)"                                                   \
                     : "+v"(fa[0][0]), "+v"(fa[0][1]), "+v"(fa[0][2]), "+v"(fa[0][3]),         \
                       "+v"(fa[0][4]), "+v"(fa[0][5]), "+v"(fa[0][6]), "+v"(fa[0][7])::"memory"); \
        asm volatile(""                                                                        \
                     : "+v"(fa[1][0]), "+v"(fa[1][1]), "+v"(fa[1][2]), "+v"(fa[1][3]),         \
                       "+v"(fa[1][4]), "+v"(fa[1][5]), "+v"(fa[1][6]), "+v"(fa[1][7])::"memory"); \
    } while (0)
#define BI_P4_SETTLE_B()                                                                       \
    do {                                                                                       \
        asm volatile("" : "+v"(fb[0][0]), "+v"(fb[0][1]), "+v"(fb[0][2]), "+v"(fb[0][3])::"memory"); \
        asm volatile("" : "+v"(fb[1][0]), "+v"(fb[1][1]), "+v"(fb[1][2]), "+v"(fb[1][3])::"memory"); \
    } while (0)
        // Group 0's memory phase for stage s: raw B first (its decode starts
        // as soon as it lands), then A; decode; hand the fragments to group 1.
        auto mem0 = [&](int s) {
            const uint32_t cb0 = c_lane0 + (s % S::RR) * S::RawStage;
            const uint32_t cb1 = c_lane1 + (s % S::RR) * S::RawStage;
            const uint32_t sb = s_lane + (s % S::RR) * S::RawStage;
            uint32_t c0[4], c1[4], sv[4];
            c0[0] = rd32<0>(cb0); c1[0] = rd32<0>(cb1);
            c0[1] = rd32<512>(cb0); c1[1] = rd32<512>(cb1);
            c0[2] = rd32<1024>(cb0); c1[2] = rd32<1024>(cb1);
            c0[3] = rd32<1536>(cb0); c1[3] = rd32<1536>(cb1);
            sv[0] = rd32<0>(sb); sv[1] = rd32<64>(sb); sv[2] = rd32<128>(sb); sv[3] = rd32<192>(sb);
            BI_P4_READ_A(s);
            // the 12 raw reads are the oldest of the 28 in flight
            asm volatile("s_waitcnt lgkmcnt(15)"
                         : "+v"(c0[0]), "+v"(c0[1]), "+v"(c0[2]), "+v"(c0[3]), "+v"(c1[0]), "+v"(c1[1]),
                           "+v"(c1[2]), "+v"(c1[3]), "+v"(sv[0]), "+v"(sv[1]), "+v"(sv[2]), "+v"(sv[3])::"memory");
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const uint32_t sh = sv[fn] >> sshift;
                const uint4 d0 = decode8(c0[fn], e4m3_value<0>(sh));
                const uint4 d1 = decode8(c1[fn], e4m3_value<2>(sh));
                fb[0][fn] = u32x4{d0.x, d0.y, d0.z, d0.w};
                fb[1][fn] = u32x4{d1.x, d1.y, d1.z, d1.w};
            }
            wr128<0 * 1024>(d_lane, fb[0][0]); wr128<1 * 1024>(d_lane, fb[0][1]);
            wr128<2 * 1024>(d_lane, fb[0][2]); wr128<3 * 1024>(d_lane, fb[0][3]);
            wr128<4 * 1024>(d_lane, fb[1][0]); wr128<5 * 1024>(d_lane, fb[1][1]);
            wr128<6 * 1024>(d_lane, fb[1][2]); wr128<7 * 1024>(d_lane, fb[1][3]);
            BI_P4_SETTLE_A();
            BI_P4_SETTLE_B();
        };
        // Group 1's memory phase for stage s: A and the decoded B, then the
        // loads of stage s + 2.
        auto mem1 = [&](int s, int u) {
            BI_P4_READ_A(s);
            fb[0][0] = rd128<0 * 1024>(d_lane); fb[0][1] = rd128<1 * 1024>(d_lane);
            fb[0][2] = rd128<2 * 1024>(d_lane); fb[0][3] = rd128<3 * 1024>(d_lane);
            fb[1][0] = rd128<4 * 1024>(d_lane); fb[1][1] = rd128<5 * 1024>(d_lane);
            fb[1][2] = rd128<6 * 1024>(d_lane); fb[1][3] = rd128<7 * 1024>(d_lane);
            issue(u);
            BI_P4_SETTLE_A();
            BI_P4_SETTLE_B();
            wait_vmcnt<S::LOADS>();
        };
#define BI_P4_COMPUTE()                                                                        \
    do {                                                                                       \
        _Pragma("unroll") for (int ks = 0; ks < 2; ++ks)                                       \
        _Pragma("unroll") for (int fm = 0; fm < 8; ++fm)                                       \
        _Pragma("unroll") for (int fn = 0; fn < FN; ++fn)                                      \
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                             \
                __builtin_bit_cast(bf16x8, fa[ks][fm]), __builtin_bit_cast(bf16x8, fb[ks][fn]), \
                acc[fm][fn], 0, 0, 0);                                                         \
    } while (0)

        // Prologue: group 1 issues stages 0 and 1; everything lands; group 0
        // reads and decodes stage 0 (handing it to group 1); group 1 reads
        // stage 0 and issues stage 2.
        if (g == 1) {
            issue(-2);
            issue(-1);
        }
        wait_vmcnt<0>();
        lds_barrier();
        if (g == 0) mem0(0);
        lds_barrier();
        if (g == 1) {
            mem1(0, 0);
            lds_barrier();
        }
        // One loop body serves both groups, group 1 half a step behind: each
        // iteration is [compute stage t] barrier [memory phase for stage
        // t + 1] barrier.
        for (int t = 0; t < nk; ++t) {
            __builtin_amdgcn_sched_barrier(0);
            BI_P4_COMPUTE();
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            if (g == 0)
                mem0(t + 1);
            else
                mem1(t + 1, t + 1);
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        if (g == 0) lds_barrier();
#undef BI_P4_READ_A
#undef BI_P4_SETTLE_A
#undef BI_P4_SETTLE_B
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

hipError_t launch_pingpong_nvfp4(const GemmArgs &a, int grid, hipStream_t s) {
    if (a.batch != 1 || grid < 1 || a.group_off || a.K % 64 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pingpong::pingpong_nvfp4_kernel, dim3(grid), dim3(pingpong::kNT), 0, s, a);
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
