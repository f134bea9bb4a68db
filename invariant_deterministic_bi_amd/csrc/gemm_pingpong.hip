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
                __builtin_bit_cast(bf16x8, fb[ks][fn]), __builtin_bit_cast(bf16x8, fa[ks][fm]), \
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

        // Epilogue.  The MFMA takes the weight fragment first, so each
        // accumulator block is transposed: lane l of block (fm, fn) holds
        // output row 16 fm + (l & 15) of its group and the four consecutive
        // columns 16 fn + 4 (l >> 4) .. + 3.  (Operand order changes no bit:
        // each element is the same sum of the same exact products in the same
        // K order.)  They are rounded (RNE) to four bf16 and written to a
        // padded LDS tile as one 8-byte write -- with a 528-byte row stride
        // the 32 lanes of a half-wavefront hit all 64 banks once -- then
        // 16-byte row chunks go to global memory.  First every load has landed
        // (the zero-filling ones included).
        wait_vmcnt<0>();
        lds_barrier();
        char *ct = lds;
#pragma unroll
        for (int fm = 0; fm < 8; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int row = 128 * g + fm * 16 + (lane & 15);
                const int col = (BN / 4) * j + fn * 16 + (lane >> 4) * 4;
                const uint32_t e0 = f32_to_bf16_rne(acc[fm][fn][0]), e1 = f32_to_bf16_rne(acc[fm][fn][1]);
                const uint32_t e2 = f32_to_bf16_rne(acc[fm][fn][2]), e3 = f32_to_bf16_rne(acc[fm][fn][3]);
                *reinterpret_cast<uint2 *>(ct + row * S::CStride + col * 2) = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
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
        // the LDS is reused by the next tile's prologue: its reads are done
        // (the global stores may still be in flight; a __syncthreads() would
        // wait for them too)
        lds_barrier();
    }
}

// ---------------------------------------------------------------------------
// The NVFP4 weight (bf16 A, raw NVFP4 B: codes [N, K/2], E4M3 scales [N,
// K/16], K % 64 == 0) in the same ping-pong schedule, 256 x 256 tiles.
//
// B reaches LDS raw: per 64-column stage, 256 rows of 32 code bytes and 4
// scale bytes (9 KB, against 32 KB of bf16), by LDS DMA.  Each B stage is
// decoded once, half by each group, in their memory phases: a SIMD issues
// VALU work at about half rate for a lone wavefront, so the decode of a
// whole stage by one group would outlast the other group's 64 MFMAs.  The
// decode is the tiled kernel's exact one (FP4 pair convert with a unit
// scale, one fp32 multiply by the E4M3 scale, top halves).
//   * group 0, in its memory phase for stage s (phase b of step s - 1),
//     reads A rows 0..127, the decoded K chunk 1 of stage s and the raw
//     K chunk 0 of stage s; it decodes chunk 0 of its wavefront's 64
//     columns straight into registers and writes it to the decoded B
//     buffer, and issues the LDS-DMA loads of A rows 128..255 of stage s + 2;
//   * group 1, in its memory phase for stage s (phase a of step s), reads A
//     rows 128..255 and both decoded chunks of stage s, decodes K chunk 1 of
//     stage s + 1 from its raw bytes into the decoded B buffer (after its
//     reads of stage s's chunk 1 from the same slots: one wavefront's LDS
//     operations execute in order), and issues the LDS-DMA loads of A rows
//     0..127 and the raw B of stage s + 3 (after its A reads are done: A
//     stage s + 3 takes stage s's slot).
// Wavefront j of either group works on columns 64 j .. 64 j + 63, so a
// decoded fragment goes from one wavefront to its partner on the other
// group.  Each compute phase is 64 MFMAs on fragments in registers.  Each
// wavefront waits, at the start of its memory phase, until only its
// previous memory phase's loads are in flight: group 1's loads of stage
// s + 1 (issued two memory phases earlier) have then landed, for its own
// decode of raw chunk 1 of stage s + 1 and, after the barrier, for group
// 0's reads of stage s + 1; group 0's A rows 128..255 of stage s + 1 have
// landed before group 1 reads them in the next phase.  Every load so has
// about two phase pairs to land.  Rings: A rows 0..127, A rows 128..255
// and raw B three stages each, the decoded B one per K chunk.  The decoded fragments hold the same bf16 values the tiled
// kernel reads from its decoded LDS tile, so every output element's chain
// -- and its bits -- are the same.
// ---------------------------------------------------------------------------
struct Nv4Shape {
    static constexpr int BN = 256, FN = 4;
    static constexpr int RA0 = 3, RA1 = 3, RR = 3;  // ring depths
    static constexpr int CodeBytes = BN * 32, RawStage = BN * 36;
    static constexpr int OffA1 = RA0 * kHalf;
    static constexpr int OffRaw = OffA1 + RA1 * kHalf;
    static constexpr int OffDec = OffRaw + RR * RawStage;
    static constexpr int DecBytes = BN * kRowBytes;   // 32 KB: 8 KB per column strip
    static constexpr int Pipe = OffDec + DecBytes;
    static constexpr int CStride = BN * 2 + 16;
    static constexpr int CBytes = kBM * CStride;
    static constexpr int Lds = Pipe > CBytes ? Pipe : CBytes;
    static constexpr int LOADS0 = 4;  // DMA instructions per memory phase, per wavefront: group 0
    static constexpr int LOADS1 = 7;  // and group 1
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

        // LDS-DMA loads.  Each lane's offset within a stage is fixed per
        // tile (the DmaLane and raw-lane offsets above); the stage's offset
        // goes in the scalar offset, so an instruction costs no vector
        // arithmetic.  A stage past the last gets a scalar offset that puts
        // every lane beyond its buffer, so its loads fill zeros.  Rows past M
        // (or N) lie beyond their buffer too -- A's range ends with row M - 1,
        // and a raw lane past N carries an offset of 2^31 -- and K % 64 == 0,
        // so no other check is needed.  (Offsets stay below 2^32: A lanes
        // are below 2^26, and raw buffers end below 2^29 < 2^30.)
        const i32x4 ra_s = {__builtin_amdgcn_readfirstlane(ra.x), __builtin_amdgcn_readfirstlane(ra.y),
                            __builtin_amdgcn_readfirstlane(ra.z), __builtin_amdgcn_readfirstlane(ra.w)};
        const i32x4 rc_s = {__builtin_amdgcn_readfirstlane(rc.x), __builtin_amdgcn_readfirstlane(rc.y),
                            __builtin_amdgcn_readfirstlane(rc.z), __builtin_amdgcn_readfirstlane(rc.w)};
        const i32x4 rs_s = {__builtin_amdgcn_readfirstlane(rs.x), __builtin_amdgcn_readfirstlane(rs.y),
                            __builtin_amdgcn_readfirstlane(rs.z), __builtin_amdgcn_readfirstlane(rs.w)};
        typedef __attribute__((address_space(3))) uint32_t lds_u32;
        // 8 rows (row0 % 8 == 0) of A stage st into the 128-row tile `tile`
        // (row0 relative to the tile's first row r_base)
        auto dma_a = [&](char *tile, int r_base, int row0, int st) {
            const int soff = st < nk ? (int)((r_base + row0) * p.lda * 2) + st * (kBK * 2) : (int)0x80000000;
            const int voff = ((row0 >> 3) & 1) ? dla.off[1] : dla.off[0];
            bi_raw_buffer_load_lds(ra_s, (lds_u32 *)(tile + row0 * kRowBytes), 16, voff, soff, 0, 0);
        };
        // A rows 0..127 of stage st (group 1: rows 32 j .. 32 j + 31)
        auto issue_a0 = [&](int st) {
            char *a0 = lds + (st % S::RA0) * kHalf;
            dma_a(a0, 0, 32 * j, st);
            dma_a(a0, 0, 32 * j + 8, st);
            dma_a(a0, 0, 32 * j + 16, st);
            dma_a(a0, 0, 32 * j + 24, st);
        };
        // A rows 128..255 of stage st (group 0: rows 128 + 32 j .. + 31)
        auto issue_a1 = [&](int st) {
            char *a1 = lds + S::OffA1 + (st % S::RA1) * kHalf;
            dma_a(a1, 128, 32 * j, st);
            dma_a(a1, 128, 32 * j + 8, st);
            dma_a(a1, 128, 32 * j + 16, st);
            dma_a(a1, 128, 32 * j + 24, st);
        };
        // raw B of stage st (group 1: code rows 64 j .. 64 j + 63 in two
        // instructions of 32 rows, their scale rows in one)
        auto issue_raw = [&](int st) {
            const bool live = st < nk;
            char *raw = lds + S::OffRaw + (st % S::RR) * S::RawStage;
            const int sc = live ? st * 32 : 0x40000000, ss = live ? st * 4 : 0x40000000;
            bi_raw_buffer_load_lds(rc_s, (lds_u32 *)(raw + 64 * j * 32), 16, code_off0, sc, 0, 0);
            bi_raw_buffer_load_lds(rc_s, (lds_u32 *)(raw + (64 * j + 32) * 32), 16, code_off1, sc, 0, 0);
            bi_raw_buffer_load_lds(rs_s, (lds_u32 *)(raw + S::CodeBytes + 64 * j * 4), 4, scale_off, ss, 0, 0);
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

#define BI_P4_READ_A_KS(s, ks)                                                                 \
    do {                                                                                       \
        const uint32_t ab = a_lane + (g ? ((s) % S::RA1) : ((s) % S::RA0)) * kHalf;            \
        const uint32_t ak = ab + ((ks) ? sw1 : sw0);                                           \
        fa[ks][0] = rd128<0 * 2048>(ak); fa[ks][1] = rd128<1 * 2048>(ak);                    \
        fa[ks][2] = rd128<2 * 2048>(ak); fa[ks][3] = rd128<3 * 2048>(ak);                    \
        fa[ks][4] = rd128<4 * 2048>(ak); fa[ks][5] = rd128<5 * 2048>(ak);                    \
        fa[ks][6] = rd128<6 * 2048>(ak); fa[ks][7] = rd128<7 * 2048>(ak);                    \
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
        // Raw K chunk CH of stage s for this lane: the code dword of its
        // 8-element group in each of its four columns, and their scale
        // dwords; and their decode into four fragments.
        auto read_raw = [&](int s, uint32_t (&c)[4], uint32_t (&sv)[4], auto ch_tag) {
            constexpr int CH = decltype(ch_tag)::value;
            const uint32_t cb = (CH ? c_lane1 : c_lane0) + (s % S::RR) * S::RawStage;
            const uint32_t sb = s_lane + (s % S::RR) * S::RawStage;
            c[0] = rd32<0>(cb); c[1] = rd32<512>(cb); c[2] = rd32<1024>(cb); c[3] = rd32<1536>(cb);
            sv[0] = rd32<0>(sb); sv[1] = rd32<64>(sb); sv[2] = rd32<128>(sb); sv[3] = rd32<192>(sb);
        };
        auto decode_chunk = [&](const uint32_t (&c)[4], const uint32_t (&sv)[4], u32x4 (&out)[4], auto ch_tag) {
            constexpr int CH = decltype(ch_tag)::value;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const uint32_t sh = sv[fn] >> sshift;
                const uint4 d = decode8(c[fn], e4m3_value<2 * CH>(sh));
                out[fn] = u32x4{d.x, d.y, d.z, d.w};
            }
        };
        using Ch0 = std::integral_constant<int, 0>;
        using Ch1 = std::integral_constant<int, 1>;
        // Group 0's memory phase for stage s: raw chunk 0 and the decoded
        // chunk 1; decode chunk 0 into registers and hand it to group 1; then
        // A.  (A is read after the decode so that the decode's temporaries
        // and the A fragments are never live together.)
        auto mem0 = [&](int s) {
            wait_vmcnt<S::LOADS0>();
            uint32_t c[4], sv[4];
            read_raw(s, c, sv, Ch0{});
            fb[1][0] = rd128<4 * 1024>(d_lane); fb[1][1] = rd128<5 * 1024>(d_lane);
            fb[1][2] = rd128<6 * 1024>(d_lane); fb[1][3] = rd128<7 * 1024>(d_lane);
            BI_P4_READ_A_KS(s, 0);
            // the 8 raw reads are the oldest of the 20 in flight
            asm volatile("s_waitcnt lgkmcnt(12)"
                         : "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]), "+v"(sv[0]), "+v"(sv[1]),
                           "+v"(sv[2]), "+v"(sv[3])::"memory");
            decode_chunk(c, sv, fb[0], Ch0{});
            wr128<0 * 1024>(d_lane, fb[0][0]); wr128<1 * 1024>(d_lane, fb[0][1]);
            wr128<2 * 1024>(d_lane, fb[0][2]); wr128<3 * 1024>(d_lane, fb[0][3]);
            BI_P4_READ_A_KS(s, 1);
            issue_a1(s + 2);
            BI_P4_SETTLE_A();
            BI_P4_SETTLE_B();
        };
        // Group 1's memory phase for stage s: wait for the loads of stage
        // s + 1 (issued two memory phases ago); both decoded chunks of stage
        // s and the raw chunk 1 of stage s + 1, decoded into the buffer; A;
        // then, once its A reads are done (A stage s + 3 reuses their slot),
        // the loads of step u.
        auto mem1 = [&](int s, int u) {
            wait_vmcnt<S::LOADS1>();
            uint32_t c[4], sv[4];
            read_raw(s + 1, c, sv, Ch1{});
            fb[0][0] = rd128<0 * 1024>(d_lane); fb[0][1] = rd128<1 * 1024>(d_lane);
            fb[0][2] = rd128<2 * 1024>(d_lane); fb[0][3] = rd128<3 * 1024>(d_lane);
            fb[1][0] = rd128<4 * 1024>(d_lane); fb[1][1] = rd128<5 * 1024>(d_lane);
            fb[1][2] = rd128<6 * 1024>(d_lane); fb[1][3] = rd128<7 * 1024>(d_lane);
            BI_P4_READ_A_KS(s, 0);
            // the 8 raw reads are the oldest of the 24 in flight
            asm volatile("s_waitcnt lgkmcnt(15)"
                         : "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]), "+v"(sv[0]), "+v"(sv[1]),
                           "+v"(sv[2]), "+v"(sv[3])::"memory");
            u32x4 nd[4];
            decode_chunk(c, sv, nd, Ch1{});
            wr128<4 * 1024>(d_lane, nd[0]); wr128<5 * 1024>(d_lane, nd[1]);
            wr128<6 * 1024>(d_lane, nd[2]); wr128<7 * 1024>(d_lane, nd[3]);
            BI_P4_READ_A_KS(s, 1);
            BI_P4_SETTLE_A();
            BI_P4_SETTLE_B();
            issue_a0(u + 3);
            issue_raw(u + 3);
        };
        // Group 1 alone, before the first step: chunk 1 of stage 0.
        auto dec1_first = [&]() {
            uint32_t c[4], sv[4];
            read_raw(0, c, sv, Ch1{});
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]), "+v"(sv[0]), "+v"(sv[1]),
                           "+v"(sv[2]), "+v"(sv[3])::"memory");
            u32x4 nd[4];
            decode_chunk(c, sv, nd, Ch1{});
            wr128<4 * 1024>(d_lane, nd[0]); wr128<5 * 1024>(d_lane, nd[1]);
            wr128<6 * 1024>(d_lane, nd[2]); wr128<7 * 1024>(d_lane, nd[3]);
        };
#define BI_P4_COMPUTE()                                                                        \
    do {                                                                                       \
        _Pragma("unroll") for (int ks = 0; ks < 2; ++ks)                                       \
        _Pragma("unroll") for (int fm = 0; fm < 8; ++fm)                                       \
        _Pragma("unroll") for (int fn = 0; fn < FN; ++fn)                                      \
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                             \
                __builtin_bit_cast(bf16x8, fb[ks][fn]), __builtin_bit_cast(bf16x8, fa[ks][fm]), \
                acc[fm][fn], 0, 0, 0);                                                         \
    } while (0)

        // Prologue: group 1 issues stages 0..2; everything lands; group 1
        // decodes chunk 1 of stage 0; group 0 reads stage 0 and decodes its
        // chunk 0; group 1 reads stage 0, decodes chunk 1 of stage 1 and
        // issues stage 3.
        if (g == 1) {
#pragma unroll
            for (int st = 0; st < 3; ++st) {
                issue_a0(st);
                issue_raw(st);
            }
            issue_a1(0);
            issue_a1(1);
        }
        wait_vmcnt<0>();
        lds_barrier();
        if (g == 1) dec1_first();
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
#undef BI_P4_READ_A_KS
#undef BI_P4_SETTLE_A
#undef BI_P4_SETTLE_B
#undef BI_P4_COMPUTE

        // Epilogue: every load has landed; fp32 x alpha -> bf16 RNE into a
        // padded LDS tile, then 16-byte row chunks to global memory.  The
        // accumulator blocks are transposed, as in the bf16 kernel (the MFMA
        // takes the weight fragment first): lane l of block (fm, fn) holds
        // row 16 fm + (l & 15) of its group and the four consecutive columns
        // 16 fn + 4 (l >> 4) .. + 3, written as one 8-byte LDS store.
        wait_vmcnt<0>();
        lds_barrier();
        char *ct = lds;
#pragma unroll
        for (int fm = 0; fm < 8; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int row = 128 * g + fm * 16 + (lane & 15);
                const int col = 64 * j + fn * 16 + (lane >> 4) * 4;
                const uint32_t e0 = f32_to_bf16_rne(acc[fm][fn][0] * p.alpha);
                const uint32_t e1 = f32_to_bf16_rne(acc[fm][fn][1] * p.alpha);
                const uint32_t e2 = f32_to_bf16_rne(acc[fm][fn][2] * p.alpha);
                const uint32_t e3 = f32_to_bf16_rne(acc[fm][fn][3] * p.alpha);
                *reinterpret_cast<uint2 *>(ct + row * S::CStride + col * 2) = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
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
        // the LDS is reused by the next tile's prologue: its reads are done
        // (the global stores may still be in flight; a __syncthreads() would
        // wait for them too)
        lds_barrier();
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
