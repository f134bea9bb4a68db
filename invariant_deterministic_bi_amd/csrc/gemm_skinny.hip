// Skinny GEMM path for M <= 16 (bf16 A; bf16 or raw NVFP4 weight): every
// valid output row fits one 16-row MFMA block, so the weight is the whole
// traffic.  Each work item is one MFMA block of the output, NB = 16 or 8
// columns wide (8 when N/16 would leave fewer than two items per compute
// unit).  One 64-thread workgroup streams the item's weight rows and the A
// rows through its own small LDS ring (runs of 256 bytes per row per slot,
// consecutive slots continuing the row) and runs the block's MFMA chain.
// Workgroups share nothing, so there is no barrier, and about eight fit on a
// compute unit, which overlaps their LDS, decode and MFMA latencies.
//
// Bits: an output element is acc <- MFMA_16x16x32_bf16(a, b, acc) over the
// 32-wide K chunks in ascending order from +0 -- the same instruction, chunk
// count (2 * ceil(K / 64), as in the tiled kernel) and operand values as the
// tiled mainloop -- then (x alpha for NVFP4) one bf16 RNE.  Which wavefront
// and lane hold the element does not enter, so rows agree bit for bit with
// the tiled kernel at any M; the invariance tests compare the two.

#include "gemm_kernel.h"

namespace bi {
namespace skinny {

using namespace gemm_detail;

constexpr int kKC = 128;          // K columns per ring slot (four MFMA chunks)
constexpr int kRowB = kKC * 2;    // bf16 bytes of one row per slot
constexpr int kTrash = 1024;      // landing area of out-of-range slot loads
constexpr int kLdsBudget = 20 * 1024;  // per workgroup: about eight per compute unit

// 256-byte rows (16 chunks): chunk c of row r sits at c ^ f(r), f from row
// bits 0..3 into chunk bits 2,3 / 0 / 1.  A fragment read (rows 0..15, chunks
// 4c..4c+3 by lane group) then touches 16 distinct 16-byte bank groups in
// every 16-lane LDS service set (lanes 8j..8j+7 with 8j+32..8j+39, or 16
// consecutive lanes).
__device__ __forceinline__ int swr(int r, int c) {
    return c ^ (((r & 3) << 2) | ((r >> 2) & 1) | (((r >> 3) & 1) << 1));
}
// 64-byte NVFP4 code rows (4 chunks): 32-bit reads of 16 rows x 4 dwords hit
// 64 distinct banks.
__device__ __forceinline__ int swc(int r, int c) { return c ^ ((r >> 2) & 3); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// MA: A rows loaded (4, 8 or 16 >= M); NB: weight rows (output columns) per
// work item (8 or 16).
template <int MA, int BMODE, int NB>
struct SCfg {
    static constexpr bool RAW = BMODE == OPND_NVFP4_RAW;
    static constexpr int A_BYTES = MA * kRowB;
    static constexpr int CODE_BYTES = 16 * (kKC / 2);           // 16 rows reserved
    static constexpr int SCALE_BYTES = 256;                     // 16 rows x 8 B + landing pad
    static constexpr int B_BYTES = RAW ? CODE_BYTES + SCALE_BYTES : NB * kRowB;
    static constexpr int SLOT = A_BYTES + B_BYTES;
    static constexpr int IA = MA / 4;                   // A loads per slot (four rows each)
    static constexpr int IB = RAW ? 2 : NB / 4;         // B loads per slot
    static constexpr int T = IA + IB;
    static constexpr int S_VM = 62 / T + 2;
    static constexpr int S_LDS = (kLdsBudget - kTrash) / SLOT;
    static constexpr int S1 = S_VM < S_LDS ? S_VM : S_LDS;
    static constexpr int S2 = S1 > 16 ? 16 : S1;
    static constexpr int S = S2 < 3 ? 3 : S2;
    static constexpr int LDS = S * SLOT + kTrash;
    static_assert((S - 2) * T < 64, "vmcnt range");
};

__device__ __forceinline__ i32x4 uniform(const i32x4 &x) {
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane(x.x);
    r.y = __builtin_amdgcn_readfirstlane(x.y);
    r.z = __builtin_amdgcn_readfirstlane(x.z);
    r.w = __builtin_amdgcn_readfirstlane(x.w);
    return r;
}

__device__ __forceinline__ void dma16(const i32x4 &rs, char *dst, int voff) {
    bi_raw_buffer_load_lds(uniform(rs), (__attribute__((address_space(3))) uint32_t *)dst, 16, voff,
                           0, 0, 0);
}
__device__ __forceinline__ void dma4(const i32x4 &rs, char *dst, int voff) {
    bi_raw_buffer_load_lds(uniform(rs), (__attribute__((address_space(3))) uint32_t *)dst, 4, voff,
                           0, 0, 0);
}

__device__ __forceinline__ u32x4 rd128(uint32_t addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
__device__ __forceinline__ uint32_t rd32(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
__device__ __forceinline__ uint32_t rd8(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_u8 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}

template <int MA, int BMODE, int NB>
__global__ __launch_bounds__(64) void skinny_kernel(GemmArgs p) {
    using C = SCfg<MA, BMODE, NB>;
    constexpr int S = C::S, T = C::T, SLOT = C::SLOT;
    constexpr bool RAW = C::RAW;
    __shared__ __attribute__((aligned(16))) char lds[C::LDS];
    char *trash = lds + S * SLOT;
    const int lane = threadIdx.x;
    const int nk = 2 * ((p.K + kBK - 1) / kBK);  // 32-wide chunks, as in the tiled kernel
    const int nslots = (nk + 3) / 4;
    const int items = (p.N + NB - 1) / NB;

    // A rows 0..M-1 (M <= MA), shared by every work item
    const i32x4 ra = make_rsrc(p.A, (uint32_t)(((int64_t)(p.M - 1) * p.lda + p.K) * 2));
    const int q_row = lane >> 4;   // + 4j for load j of a 256-byte-row operand
    const int q_chunk = lane & 15; // physical chunk this lane fills

    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int n0 = item * NB;
        const int rows_b = min(NB, p.N - n0);
        i32x4 rb, rsc;
        if constexpr (RAW) {
            rb = make_rsrc(static_cast<const uint8_t *>(p.B) + (int64_t)n0 * (p.K >> 1),
                           (uint32_t)(rows_b * (p.K >> 1)));
            rsc = make_rsrc(static_cast<const uint8_t *>(p.B_scales) + (int64_t)n0 * (p.K >> 4),
                            (uint32_t)(rows_b * (p.K >> 4)));
        } else {
            rb = make_rsrc(static_cast<const uint16_t *>(p.B) + (int64_t)n0 * p.ldb,
                           (uint32_t)(((int64_t)(rows_b - 1) * p.ldb + p.K) * 2));
            rsc = rb;
        }

        // all loads of slot s (out-of-range slots land in the trash area and
        // keep the per-slot load count exact)
        auto issue = [&](int s) {
            const bool live = s < nslots;
            char *base = lds + (s % S) * SLOT;
            const int k0 = s * kKC;
#pragma unroll
            for (int j = 0; j < C::IA; ++j) {
                const int r = 4 * j + q_row;
                const int k = k0 + swr(r, q_chunk) * 8;
                const bool ok = live && r < p.M && k < p.K;
                dma16(ra, live ? base + j * 1024 : trash,
                      ok ? (int)((int64_t)r * p.lda * 2 + k * 2) : (int)0x80000000);
            }
            char *bb = base + C::A_BYTES;
            if constexpr (RAW) {
                {   // codes: lane -> row lane >> 2, 16-byte chunk lane & 3
                    const int r = lane >> 2;
                    const int byte = (k0 >> 1) + swc(r, lane & 3) * 16;
                    const bool ok = live && r < rows_b && byte < (p.K >> 1);
                    dma16(rb, live ? bb : trash, ok ? r * (p.K >> 1) + byte : (int)0x80000000);
                }
                {   // scales: lanes 0..31 -> row lane >> 1, dword lane & 1
                    const int r = lane >> 1;
                    const int sbyte = (k0 >> 4) + (lane & 1) * 4;
                    const bool ok = live && lane < 32 && r < rows_b && sbyte < (p.K >> 4);
                    dma4(rsc, live ? bb + C::CODE_BYTES : trash,
                         ok ? r * (p.K >> 4) + sbyte : (int)0x80000000);
                }
            } else {
#pragma unroll
                for (int j = 0; j < C::IB; ++j) {
                    const int r = 4 * j + q_row;
                    const int k = k0 + swr(r, q_chunk) * 8;
                    const bool ok = live && r < rows_b && k < p.K;
                    dma16(rb, live ? bb + j * 1024 : trash,
                          ok ? (int)((int64_t)r * p.ldb * 2 + k * 2) : (int)0x80000000);
                }
            }
        };

        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < S - 1; ++s) issue(s);

        const int r = lane & 15, sub = lane >> 4;
        const int ar = r < MA ? r : 0;        // A rows past MA are never loaded: reuse row 0
        const int br = RAW ? r : (r < NB ? r : r - NB);  // weight rows past NB: reuse a loaded row
        for (int kt = 0; kt < nslots; ++kt) {
            wait_vmcnt<(S - 2) * T>();
            const uint32_t sa = lds_addr(lds + (kt % S) * SLOT);
            const uint32_t sb = sa + C::A_BYTES;
            u32x4 af[4], bfr[4];
            uint32_t cw[4], sc[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                af[c] = rd128(sa + ar * kRowB + swr(ar, 4 * c + sub) * 16);
                if constexpr (RAW) {
                    cw[c] = rd32(sb + r * (kKC / 2) + swc(r, c) * 16 + 4 * sub);
                    sc[c] = rd8(sb + C::CODE_BYTES + r * (kKC / 16) + 2 * c + (sub >> 1));
                } else {
                    bfr[c] = rd128(sb + br * kRowB + swr(br, 4 * c + sub) * 16);
                }
            }
            // the reads are complete before their registers are used and
            // before this slot's ring position is refilled
            if constexpr (RAW)
                asm volatile("s_waitcnt lgkmcnt(0)"
                             : "+v"(af[0]), "+v"(af[1]), "+v"(af[2]), "+v"(af[3]), "+v"(cw[0]),
                               "+v"(cw[1]), "+v"(cw[2]), "+v"(cw[3]), "+v"(sc[0]), "+v"(sc[1]),
                               "+v"(sc[2]), "+v"(sc[3])::"memory");
            else
                asm volatile("s_waitcnt lgkmcnt(0)"
                             : "+v"(af[0]), "+v"(af[1]), "+v"(af[2]), "+v"(af[3]), "+v"(bfr[0]),
                               "+v"(bfr[1]), "+v"(bfr[2]), "+v"(bfr[3])::"memory");
            issue(kt + S - 1);
            if constexpr (RAW) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint4 d = decode8(cw[c], e4m3_value(sc[c]));
                    bfr[c] = u32x4{d.x, d.y, d.z, d.w};
                }
            }
            if (kt * 4 + 4 <= nk) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[c]),
                                                                  __builtin_bit_cast(bf16x8, bfr[c]),
                                                                  acc, 0, 0, 0);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (kt * 4 + c < nk)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, af[c]), __builtin_bit_cast(bf16x8, bfr[c]),
                            acc, 0, 0, 0);
            }
        }

        // lane holds rows 4*sub .. 4*sub+3 of column n0 + (lane & 15)
        const int col = n0 + r;
        if (r < NB && col < p.N) {
            uint16_t *Y = static_cast<uint16_t *>(p.Y);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * sub + i;
                float v = acc[i];
                if constexpr (RAW) v = v * p.alpha;
                if (row < p.M) Y[(int64_t)row * p.ldy + col] = (uint16_t)f32_to_bf16_rne(v);
            }
        }
    }
    wait_vmcnt<0>();  // trailing out-of-range loads land before the workgroup ends
}

template <int MA, int BMODE, int NB>
hipError_t launch_ma(const GemmArgs &a, int grid, hipStream_t s) {
    hipLaunchKernelGGL((skinny_kernel<MA, BMODE, NB>), dim3(grid), dim3(64), 0, s, a);
    return hipGetLastError();
}

template <int BMODE, int NB>
hipError_t launch_mode(const GemmArgs &a, int ma, int grid, hipStream_t s) {
    switch (ma) {
        case 4: return launch_ma<4, BMODE, NB>(a, grid, s);
        case 8: return launch_ma<8, BMODE, NB>(a, grid, s);
        case 16: return launch_ma<16, BMODE, NB>(a, grid, s);
    }
    return hipErrorInvalidValue;
}

template <int BMODE, int NB>
int lds_of(int M) {
    return M <= 4 ? SCfg<4, BMODE, NB>::LDS : M <= 8 ? SCfg<8, BMODE, NB>::LDS : SCfg<16, BMODE, NB>::LDS;
}

}  // namespace skinny

int skinny_lds_bytes(int b_mode, int M, int nb) {
    const bool raw = b_mode == OPND_NVFP4_RAW;
    if (nb == 8) return raw ? skinny::lds_of<OPND_NVFP4_RAW, 8>(M) : skinny::lds_of<OPND_BF16_ROWS, 8>(M);
    return raw ? skinny::lds_of<OPND_NVFP4_RAW, 16>(M) : skinny::lds_of<OPND_BF16_ROWS, 16>(M);
}

hipError_t launch_skinny(int b_mode, int nb, int ma, const GemmArgs &a, int grid, hipStream_t s) {
    if (a.M < 1 || a.M > ma || ma > 16 || (nb != 8 && nb != 16)) return hipErrorInvalidValue;
    if (b_mode == OPND_BF16_ROWS)
        return nb == 8 ? skinny::launch_mode<OPND_BF16_ROWS, 8>(a, ma, grid, s)
                       : skinny::launch_mode<OPND_BF16_ROWS, 16>(a, ma, grid, s);
    if (b_mode == OPND_NVFP4_RAW)
        return nb == 8 ? skinny::launch_mode<OPND_NVFP4_RAW, 8>(a, ma, grid, s)
                       : skinny::launch_mode<OPND_NVFP4_RAW, 16>(a, ma, grid, s);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Direct path for a bf16 weight at M <= 16.  At this size the weight is the
// whole HBM traffic and each weight byte is used once, so it skips LDS: every
// lane loads its MFMA fragments straight into registers (16 bytes per lane,
// one 1 KB instruction per 32-wide K chunk of a 16-column item) through a
// rolling window of D chunk pairs in flight per wavefront.  One 64-thread
// workgroup streams items b, b + grid, ...; the window runs on across item
// boundaries.  A rows are loaded the same way.  For M <= 8 one A instruction
// covers two chunks (rows 0..7 of chunk c in lanes 0..7 of each 16-lane row,
// rows 0..7 of chunk c + 1 in lanes 8..15), and a DPP rotation by eight lanes
// brings the second chunk into place; lanes 8..15 then carry A rows 8..15,
// which only feed output rows beyond M.
//
// The hardware orders nothing here but the loads themselves: they are
// compiler-visible, so the compiler places each vmcnt wait before the first
// use of a loaded register.
//
// Bits: an output element's chain is the tiled kernel's (same MFMA, 32-K
// chunks in ascending order from +0, 2 * ceil(K / 64) of them with a zero
// trailing chunk when K % 64 == 32, one bf16 RNE), so rows are bitwise those
// of the tiled kernel at any M.
// ---------------------------------------------------------------------------
namespace direct {

using namespace gemm_detail;

constexpr int kMark = (int)0x80000000;  // buffer offset that reads zero

__device__ __forceinline__ i32x4 ror8(const i32x4 &v) {  // lane i <- lane i ^ 8 within 16
    i32x4 o;
    o.x = __builtin_amdgcn_mov_dpp(v.x, 0x128, 0xF, 0xF, false);
    o.y = __builtin_amdgcn_mov_dpp(v.y, 0x128, 0xF, 0xF, false);
    o.z = __builtin_amdgcn_mov_dpp(v.z, 0x128, 0xF, 0xF, false);
    o.w = __builtin_amdgcn_mov_dpp(v.w, 0x128, 0xF, 0xF, false);
    return o;
}

// AP: A packed two chunks per instruction (M <= 8).  D: chunk pairs in flight
// (a divisor of the pair count ceil(K / 64), chosen by the host).  RB: 16-row
// blocks of A (M <= 16 * RB); each block has its own accumulator and runs the
// same chain, one MFMA per chunk, against the same weight fragments.
template <int AP, int D, int RB = 1>
__global__ __launch_bounds__(64) void direct_kernel(GemmArgs p) {
    static_assert(RB == 1 || !AP, "two-chunk A packing is for M <= 8");
    constexpr int AL = AP ? 1 : 2 * RB;  // A loads per pair; the weight takes two
    const int lane = threadIdx.x;
    const int r = lane & 15, sub = lane >> 4;
    const int items = (p.N + 15) >> 4;
    const int np = (p.K + 63) >> 6;  // chunk pairs: 2 * ceil(K / 64) chunks
    const int my_items = (items - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const i32x4 ra = make_rsrc(p.A, (uint32_t)(((int64_t)(p.M - 1) * p.lda + p.K) * 2));
    // byte offset of a lane's 16 bytes within pair 0, and its first K column;
    // load j is row block j / 2, chunk j % 2 (unpacked)
    int a_lane[AL], a_kl[AL];
#pragma unroll
    for (int j = 0; j < AL; ++j) {
        const int row = AP ? (r & 7) : r + 16 * (j >> 1), ch = AP ? (r >> 3) : (j & 1);
        a_lane[j] = row < p.M ? (int)(row * p.lda * 2) + 64 * ch + 16 * sub : kMark;
        a_kl[j] = 32 * ch + 8 * sub;
    }
    const int kfull = p.K >> 6;  // pairs whose 64 columns all lie below K

    int is_item = 0, is_p = 0;   // next pair to load
    i32x4 rb;
    int w_lane[2];
    auto set_item = [&]() {
        const int n0 = ((int)blockIdx.x + is_item * (int)gridDim.x) * 16;
        const int rows_b = is_item < my_items ? min(16, p.N - n0) : 0;
        rb = make_rsrc(static_cast<const uint16_t *>(p.B) + (int64_t)(rows_b > 0 ? n0 : 0) * p.ldb,
                       rows_b > 0 ? (uint32_t)(((int64_t)(rows_b - 1) * p.ldb + p.K) * 2) : 0u);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            w_lane[j] = r < rows_b ? (int)(r * p.ldb * 2) + 64 * j + 16 * sub : kMark;
    };
    set_item();
    // loads of the next pair (past the last item: zero-reading offsets, no traffic)
    auto issue = [&](i32x4 *av, i32x4 *wv) {
        const int koff = is_p * 128;
        const bool tail = is_p >= kfull;
#pragma unroll
        for (int j = 0; j < AL; ++j) {
            int o = a_lane[j] + koff;
            if (tail && 64 * is_p + a_kl[j] >= p.K) o = kMark;
            av[j] = bi_raw_buffer_load_b128(ra, o, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            int o = w_lane[j] + koff;
            if (tail && 64 * is_p + 32 * j + 8 * sub >= p.K) o = kMark;
            wv[j] = bi_raw_buffer_load_b128(rb, o, 0, 0);
        }
        if (++is_p == np) {
            is_p = 0;
            ++is_item;
            set_item();
        }
    };

    i32x4 as[D][AL], ws[D][2];
#pragma unroll
    for (int d = 0; d < D; ++d) issue(as[d], ws[d]);
    uint16_t *Y = static_cast<uint16_t *>(p.Y);
    for (int t = 0; t < my_items; ++t) {
        f32x4 acc[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int pb = 0; pb < np; pb += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
#pragma unroll
                for (int b = 0; b < RB; ++b) {
                    const i32x4 a0 = as[d][AP ? 0 : 2 * b];
                    const i32x4 a1 = AP ? ror8(as[d][0]) : as[d][2 * b + 1];
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0),
                                                                     __builtin_bit_cast(bf16x8, ws[d][0]), acc[b], 0, 0, 0);
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1),
                                                                     __builtin_bit_cast(bf16x8, ws[d][1]), acc[b], 0, 0, 0);
                }
                issue(as[d], ws[d]);
            }
        }
        // lane holds rows 16*b + 4*sub .. +3 of column n0 + r
        const int col = ((int)blockIdx.x + t * (int)gridDim.x) * 16 + r;
        if (col < p.N) {
#pragma unroll
            for (int b = 0; b < RB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * b + 4 * sub + i;
                    if (row < p.M) Y[(int64_t)row * p.ldy + col] = (uint16_t)f32_to_bf16_rne(acc[b][i]);
                }
        }
    }
}

template <int AP>
hipError_t launch_ap(const GemmArgs &a, int d, int grid, hipStream_t s) {
    switch (d) {
        case 16: hipLaunchKernelGGL((direct_kernel<AP, 16>), dim3(grid), dim3(64), 0, s, a); break;
        case 8: hipLaunchKernelGGL((direct_kernel<AP, 8>), dim3(grid), dim3(64), 0, s, a); break;
        case 4: hipLaunchKernelGGL((direct_kernel<AP, 4>), dim3(grid), dim3(64), 0, s, a); break;
        case 2: hipLaunchKernelGGL((direct_kernel<AP, 2>), dim3(grid), dim3(64), 0, s, a); break;
        case 1: hipLaunchKernelGGL((direct_kernel<AP, 1>), dim3(grid), dim3(64), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// RB row blocks (M <= 16 * RB), unpacked A; the register budget caps D at
// 16 / RB chunk pairs (A takes 8 * RB registers per pair).
template <int RB>
hipError_t launch_rb(const GemmArgs &a, int d, int grid, hipStream_t s) {
    constexpr int DMAX = 16 / RB;
    if (d > DMAX) return hipErrorInvalidValue;
    switch (d) {
        case 8: if constexpr (DMAX >= 8) hipLaunchKernelGGL((direct_kernel<0, 8, RB>), dim3(grid), dim3(64), 0, s, a); break;
        case 4: if constexpr (DMAX >= 4) hipLaunchKernelGGL((direct_kernel<0, 4, RB>), dim3(grid), dim3(64), 0, s, a); break;
        case 2: hipLaunchKernelGGL((direct_kernel<0, 2, RB>), dim3(grid), dim3(64), 0, s, a); break;
        case 1: hipLaunchKernelGGL((direct_kernel<0, 1, RB>), dim3(grid), dim3(64), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// NVFP4 weight, the same direct scheme.  The unit is a group of four 32-wide
// chunks (128 K columns; K % 128 == 0).  Per group a lane loads 16 code bytes
// (row r, chunk 4q + sub: the instruction covers 16 rows x 64 bytes) and the
// row's 8 scale bytes.  The lane that holds chunk 4q + j's codes for row r is
// (r, j), while the MFMA wants code dword s of that chunk in lane (r, s): a
// 4 x 4 transpose across the four 16-lane rows, done with two 32-lane and two
// 16-lane swaps.  Each lane then decodes its eight elements into the bf16
// fragment as in the tiled kernel (FP4 pair convert, exact fp32 scale
// multiply, top halves), so the MFMA operands are the same bf16 values.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void transpose4(uint32_t &x0, uint32_t &x1, uint32_t &x2, uint32_t &x3) {
    // rows = 16-lane groups, registers = dwords: x_j row s <- x_s row j
    auto a = __builtin_amdgcn_permlane32_swap(x0, x2, false, false);
    auto b = __builtin_amdgcn_permlane32_swap(x1, x3, false, false);
    auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    x0 = c[0];
    x1 = c[1];
    x2 = d[0];
    x3 = d[1];
}

// AP: A packed two chunks per load (M <= 8).  D: groups in flight (a divisor
// of K / 128, chosen by the host).  RB: 16-row blocks of A (M <= 16 * RB);
// each decoded weight fragment feeds every block's chain.
template <int AP, int D, int RB = 1>
__global__ __launch_bounds__(64) void direct_nvfp4_kernel(GemmArgs p) {
    static_assert(RB == 1 || !AP, "two-chunk A packing is for M <= 8");
    constexpr int AL = AP ? 2 : 4 * RB;  // A loads per group: load j is block j / 4, chunk j % 4
    const int lane = threadIdx.x;
    const int r = lane & 15, sub = lane >> 4;
    const int items = (p.N + 15) >> 4;
    const int ng = p.K >> 7;
    const int cpr = p.K >> 1, spr = p.K >> 4;  // code / scale bytes per weight row
    const int my_items = (items - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const i32x4 ra = make_rsrc(p.A, (uint32_t)(((int64_t)(p.M - 1) * p.lda + p.K) * 2));
    int a_lane[AL];
#pragma unroll
    for (int j = 0; j < AL; ++j) {
        const int row = AP ? (r & 7) : r + 16 * (j >> 2), ch = AP ? 2 * j + (r >> 3) : (j & 3);
        a_lane[j] = row < p.M ? (int)(row * p.lda * 2) + 64 * ch + 16 * sub : kMark;
    }
    const int sshift = 8 * (sub >> 1);  // this lane's byte within each scale byte pair

    int is_item = 0, is_g = 0;
    i32x4 rc, rs;
    int c_lane = kMark, s_lane = kMark;
    auto set_item = [&]() {
        const int n0 = ((int)blockIdx.x + is_item * (int)gridDim.x) * 16;
        const int rows_b = is_item < my_items ? min(16, p.N - n0) : 0;
        const int64_t b0 = rows_b > 0 ? n0 : 0;
        rc = make_rsrc(static_cast<const uint8_t *>(p.B) + b0 * cpr, rows_b > 0 ? (uint32_t)(rows_b * cpr) : 0u);
        rs = make_rsrc(static_cast<const uint8_t *>(p.B_scales) + b0 * spr,
                       rows_b > 0 ? (uint32_t)(rows_b * spr) : 0u);
        c_lane = r < rows_b ? r * cpr + 16 * sub : kMark;
        s_lane = r < rows_b ? r * spr : kMark;
    };
    set_item();
    auto issue = [&](i32x4 *av, i32x4 &cv, i32x2 &sv) {
#pragma unroll
        for (int j = 0; j < AL; ++j) av[j] = bi_raw_buffer_load_b128(ra, a_lane[j] + 256 * is_g, 0, 0);
        cv = bi_raw_buffer_load_b128(rc, c_lane + 64 * is_g, 0, 0);
        sv = bi_raw_buffer_load_b64(rs, s_lane + 8 * is_g, 0, 0);
        if (++is_g == ng) {
            is_g = 0;
            ++is_item;
            set_item();
        }
    };

    i32x4 as[D][AL], cs[D];
    i32x2 ss[D];
#pragma unroll
    for (int d = 0; d < D; ++d) issue(as[d], cs[d], ss[d]);
    uint16_t *Y = static_cast<uint16_t *>(p.Y);
    for (int t = 0; t < my_items; ++t) {
        f32x4 acc[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int gb = 0; gb < ng; gb += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                uint32_t y[4] = {(uint32_t)cs[d].x, (uint32_t)cs[d].y, (uint32_t)cs[d].z, (uint32_t)cs[d].w};
                transpose4(y[0], y[1], y[2], y[3]);
                // chunk j's scale: byte 2j + (sub >> 1) of the group's 8 scale bytes
                const uint32_t s01 = (uint32_t)ss[d].x >> sshift, s23 = (uint32_t)ss[d].y >> sshift;
                const float sc[4] = {e4m3_value<0>(s01), e4m3_value<2>(s01), e4m3_value<0>(s23),
                                     e4m3_value<2>(s23)};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint4 w = decode8(y[j], sc[j]);
                    const i32x4 wv = {(int)w.x, (int)w.y, (int)w.z, (int)w.w};
#pragma unroll
                    for (int b = 0; b < RB; ++b) {
                        const i32x4 a = AP ? ((j & 1) ? ror8(as[d][j >> 1]) : as[d][j >> 1]) : as[d][4 * b + j];
                        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                                         __builtin_bit_cast(bf16x8, wv), acc[b], 0, 0, 0);
                    }
                }
                issue(as[d], cs[d], ss[d]);
            }
        }
        const int col = ((int)blockIdx.x + t * (int)gridDim.x) * 16 + r;
        if (col < p.N) {
#pragma unroll
            for (int b = 0; b < RB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * b + 4 * sub + i;
                    if (row < p.M) Y[(int64_t)row * p.ldy + col] = (uint16_t)f32_to_bf16_rne(acc[b][i] * p.alpha);
                }
        }
    }
}

template <int RB>
hipError_t launch_nvfp4_rb(const GemmArgs &a, int d, int grid, hipStream_t s) {
    switch (d) {
        case 4: hipLaunchKernelGGL((direct_nvfp4_kernel<0, 4, RB>), dim3(grid), dim3(64), 0, s, a); break;
        case 2: hipLaunchKernelGGL((direct_nvfp4_kernel<0, 2, RB>), dim3(grid), dim3(64), 0, s, a); break;
        case 1: hipLaunchKernelGGL((direct_nvfp4_kernel<0, 1, RB>), dim3(grid), dim3(64), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int AP>
hipError_t launch_nvfp4_ap(const GemmArgs &a, int d, int grid, hipStream_t s) {
    switch (d) {
        case 8: hipLaunchKernelGGL((direct_nvfp4_kernel<AP, 8>), dim3(grid), dim3(64), 0, s, a); break;
        case 4: hipLaunchKernelGGL((direct_nvfp4_kernel<AP, 4>), dim3(grid), dim3(64), 0, s, a); break;
        case 2: hipLaunchKernelGGL((direct_nvfp4_kernel<AP, 2>), dim3(grid), dim3(64), 0, s, a); break;
        case 1: hipLaunchKernelGGL((direct_nvfp4_kernel<AP, 1>), dim3(grid), dim3(64), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Direct path with A in LDS.  The workgroup (1 to 8 wavefronts, each streaming
// its own items) first copies A rows 0..M-1 into LDS by DMA, overlapping the
// first weight prefetch, and every chunk's A fragment is then one LDS read:
// the only global loads in the loop are the weight's (one 1 KB load per bf16
// chunk; one code and one scale load per four NVFP4 chunks).  Used when the
// padded A fits kALds bytes.  Row stride: whole 1 KB DMA blocks plus 16 bytes,
// so the up to 16 rows of a fragment read fall in distinct bank groups.
// ---------------------------------------------------------------------------
constexpr int kALds = 144 * 1024;  // one workgroup (up to eight wavefronts) per compute unit

__device__ __forceinline__ int a_stride(int K) { return ((K * 2 + 1023) >> 10) * 1024 + 16; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 rd_a(uint32_t addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return __builtin_bit_cast(i32x4, v);
}
template <int N, int U>
__device__ __forceinline__ void wait_a(i32x4 (&a)[U]) {
    static_assert(N >= 0 && N < 16, "lgkmcnt field is 4 bits");
    if constexpr (U == 2)
        asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a[0]), "+v"(a[1]) : "n"(N) : "memory");
    else
        asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]) : "n"(N) : "memory");
}

// FP4: NVFP4 weight, four-chunk units; else bf16, chunk pairs.  D: units in
// flight (even; a divisor of the unit count, chosen by the host).
// NB: output columns per item; 8 (bf16 only) loads a pair as one 8-row x
// 128-byte instruction: rows 0..7 of chunk c in lanes 0..7 of each 16-lane
// row, of chunk c + 1 in lanes 8..15, and a DPP rotation by eight lanes gives
// chunk c + 1 its place; lanes 8..15 then carry columns that are not stored.
// AFP4 (with FP4): A is NVFP4 too (codes [M, K/2], scales [M, K/16], lda in
// elements); its rows are decoded exactly to bf16 on the way into LDS -- the
// same values the tiled kernel's NVFP4 A staging stores -- and the rest is
// the bf16-A kernel.
template <bool FP4, int NB, int D, bool AFP4 = false>
__global__ __launch_bounds__(512) void direct_alds_kernel(GemmArgs p) {
    static_assert(!AFP4 || FP4, "an NVFP4 A goes with an NVFP4 weight");
    constexpr int U = FP4 ? 4 : 2;      // chunks per unit
    constexpr int LPU = NB == 8 ? 1 : 2; // global loads per unit
    static_assert(NB == 16 || (NB == 8 && !FP4), "8-column items are bf16 only");
    static_assert(D % 2 == 0, "A fragments alternate between two register sets");
    __shared__ __attribute__((aligned(1024))) char lds[kALds];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nwv = (int)(blockDim.x >> 6);
    const int r = lane & 15, sub = lane >> 4;
    const int items = (p.N + NB - 1) / NB;
    const int nu = FP4 ? (p.K >> 7) : ((p.K + 63) >> 6);
    const int slot = (int)blockIdx.x * nwv + w, slots = (int)gridDim.x * nwv;
    const int my_items = slot < items ? (items - slot + slots - 1) / slots : 0;
    const int stride = a_stride(p.K);

    // 1. A rows by LDS DMA, 1 KB blocks shared out over the wavefronts; an
    // NVFP4 A in 32-element units (16 code bytes, two scale bytes), decoded
    // and written by every thread
    if constexpr (AFP4) {
        const uint8_t *pc = static_cast<const uint8_t *>(p.A);
        const uint8_t *ps = static_cast<const uint8_t *>(p.A_scales);
        const int upr = p.K >> 5;
        for (int q = (int)threadIdx.x; q < p.M * upr; q += (int)blockDim.x) {
            const int row = q / upr, u = q - row * upr;
            const uint4 c = *reinterpret_cast<const uint4 *>(pc + (int64_t)row * (p.lda >> 1) + u * 16);
            const uint32_t sv = *reinterpret_cast<const uint16_t *>(ps + (int64_t)row * (p.lda >> 4) + u * 2);
            const float s0 = e4m3_value(sv & 0xFFu), s1 = e4m3_value(sv >> 8);
            char *dst = lds + row * stride + u * 64;
            lds_write_b128(dst, decode8(c.x, s0));
            lds_write_b128(dst + 16, decode8(c.y, s0));
            lds_write_b128(dst + 32, decode8(c.z, s1));
            lds_write_b128(dst + 48, decode8(c.w, s1));
        }
    } else {
        const i32x4 ra = make_rsrc(p.A, (uint32_t)(((int64_t)(p.M - 1) * p.lda + p.K) * 2));
        const int bpr = (p.K * 2 + 1023) >> 10;
        for (int b = w; b < p.M * bpr; b += nwv) {
            const int row = b / bpr, part = b - row * bpr;
            const int k = part * 512 + lane * 8;
            bi_raw_buffer_load_lds(ra, (__attribute__((address_space(3))) uint32_t *)(lds + row * stride + part * 1024),
                                   16, k < p.K ? (int)(row * p.lda * 2 + k * 2) : kMark, 0, 0, 0);
        }
    }

    asm volatile("" ::: "memory");  // the weight loads below stay younger than the A copies

    // 2. weight window (compiler-visible loads)
    int is_item = 0, is_u = 0;
    i32x4 rb, rs;
    int w_lane = kMark, s_lane = kMark;
    const int cpr = p.K >> 1, spr = p.K >> 4;
    auto set_item = [&]() {
        const int n0 = (slot + is_item * slots) * NB;
        const int rows_b = is_item < my_items ? min(NB, p.N - n0) : 0;
        const int64_t b0 = rows_b > 0 ? n0 : 0;
        if constexpr (FP4) {
            rb = make_rsrc(static_cast<const uint8_t *>(p.B) + b0 * cpr, rows_b > 0 ? (uint32_t)(rows_b * cpr) : 0u);
            rs = make_rsrc(static_cast<const uint8_t *>(p.B_scales) + b0 * spr,
                           rows_b > 0 ? (uint32_t)(rows_b * spr) : 0u);
            w_lane = r < rows_b ? r * cpr + 16 * sub : kMark;
            s_lane = r < rows_b ? r * spr : kMark;
        } else {
            rb = make_rsrc(static_cast<const uint16_t *>(p.B) + b0 * p.ldb,
                           rows_b > 0 ? (uint32_t)(((int64_t)(rows_b - 1) * p.ldb + p.K) * 2) : 0u);
            const int row = NB == 8 ? (r & 7) : r;
            w_lane = row < rows_b ? (int)(row * p.ldb * 2) + (NB == 8 ? 64 * (r >> 3) : 0) + 16 * sub : kMark;
        }
    };
    set_item();
    const int kfull = p.K >> 6;  // bf16 pairs whose 64 columns all lie below K
    auto issue = [&](i32x4 &x0, i32x4 &x1) {
        if constexpr (FP4) {
            x0 = bi_raw_buffer_load_b128(rb, w_lane + 64 * is_u, 0, 0);
            const i32x2 s = bi_raw_buffer_load_b64(rs, s_lane + 8 * is_u, 0, 0);
            x1 = i32x4{s.x, s.y, 0, 0};
        } else if constexpr (NB == 8) {
            int o = w_lane + 128 * is_u;
            if (is_u >= kfull && 64 * is_u + 32 * (r >> 3) + 8 * sub >= p.K) o = kMark;
            // non-temporal: faster here (qkv 6144x4096 at M = 1 ... 16 by 12%,
            // down 4096x12288 at M = 1 by 10%), slower on the other streams
            x0 = bi_raw_buffer_load_b128(rb, o, 0, 2);
        } else {
            int o0 = w_lane + 128 * is_u, o1 = o0 + 64;
            if (is_u >= kfull) {
                if (64 * is_u + 8 * sub >= p.K) o0 = kMark;
                if (64 * is_u + 32 + 8 * sub >= p.K) o1 = kMark;
            }
            x0 = bi_raw_buffer_load_b128(rb, o0, 0, 0);
            x1 = bi_raw_buffer_load_b128(rb, o1, 0, 0);
        }
        if (++is_u == nu) {
            is_u = 0;
            ++is_item;
            set_item();
        }
    };
    i32x4 ws0[D], ws1[D];
#pragma unroll
    for (int d = 0; d < D; ++d) issue(ws0[d], ws1[d]);

    // 3. this wavefront's A blocks are older than its D * LPU weight loads
    wait_vmcnt<D * LPU>();
    lds_barrier();

    // 4. the items; A fragments read one unit ahead
    const uint32_t a_base = lds_addr(lds) + (uint32_t)(min(r, p.M - 1) * stride) + 16 * sub;
    i32x4 af[2][U];
#pragma unroll
    for (int j = 0; j < U; ++j) af[0][j] = rd_a(a_base + 64 * j);
    const int sshift = 8 * (sub >> 1);
    uint16_t *Y = static_cast<uint16_t *>(p.Y);
    for (int t = 0; t < my_items; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int ub = 0; ub < nu; ub += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int un = (ub + d + 1 == nu) ? 0 : ub + d + 1;  // next unit (next item's first)
#pragma unroll
                for (int j = 0; j < U; ++j) af[(d + 1) & 1][j] = rd_a(a_base + 64 * (un * U + j));
                wait_a<U, U>(af[d & 1]);
                if constexpr (FP4) {
                    uint32_t y[4] = {(uint32_t)ws0[d].x, (uint32_t)ws0[d].y, (uint32_t)ws0[d].z, (uint32_t)ws0[d].w};
                    transpose4(y[0], y[1], y[2], y[3]);
                    const uint32_t s01 = (uint32_t)ws1[d].x >> sshift, s23 = (uint32_t)ws1[d].y >> sshift;
                    const float sc[4] = {e4m3_value<0>(s01), e4m3_value<2>(s01), e4m3_value<0>(s23),
                                         e4m3_value<2>(s23)};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint4 q = decode8(y[j], sc[j]);
                        const i32x4 wv = {(int)q.x, (int)q.y, (int)q.z, (int)q.w};
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[d & 1][j]),
                                                                      __builtin_bit_cast(bf16x8, wv), acc, 0, 0, 0);
                    }
                } else {
                    const i32x4 w1 = NB == 8 ? ror8(ws0[d]) : ws1[d];
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[d & 1][0]),
                                                                  __builtin_bit_cast(bf16x8, ws0[d]), acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[d & 1][1]),
                                                                  __builtin_bit_cast(bf16x8, w1), acc, 0, 0, 0);
                }
                issue(ws0[d], ws1[d]);
            }
        }
        const int col = (slot + t * slots) * NB + r;
        if (r < NB && col < p.N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * sub + i;
                float v = acc[i];
                if constexpr (FP4) v = v * p.alpha;
                if (row < p.M) Y[(int64_t)row * p.ldy + col] = (uint16_t)f32_to_bf16_rne(v);
            }
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

template <bool FP4, int NB, bool AFP4 = false>
hipError_t launch_alds(const GemmArgs &a, int d, int grid, int nwv, hipStream_t s) {
    const dim3 b(64 * nwv);
    switch (d) {
        case 32:
            if constexpr (NB == 8) {
                hipLaunchKernelGGL((direct_alds_kernel<FP4, NB, 32>), dim3(grid), b, 0, s, a);
                break;
            }
            return hipErrorInvalidValue;
        case 16: hipLaunchKernelGGL((direct_alds_kernel<FP4, NB, 16, AFP4>), dim3(grid), b, 0, s, a); break;
        case 8: hipLaunchKernelGGL((direct_alds_kernel<FP4, NB, 8, AFP4>), dim3(grid), b, 0, s, a); break;
        case 4: hipLaunchKernelGGL((direct_alds_kernel<FP4, NB, 4, AFP4>), dim3(grid), b, 0, s, a); break;
        case 2: hipLaunchKernelGGL((direct_alds_kernel<FP4, NB, 2, AFP4>), dim3(grid), b, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Direct path for 16 < M <= 64 with A staged in LDS in K chunks.  A of up to
// 16 RB rows no longer fits the LDS whole, so it goes in chunks of
// CK = 2048 / RB columns (64 KB), two buffers: chunk c + 1 is copied by LDS
// DMA while chunk c is read.  Each wavefront streams one 16-column item of
// the weight through its register window (as the A-in-LDS kernel does) over
// the whole K range, and each weight fragment feeds the RB row blocks'
// chains; the wavefronts of a workgroup share the A chunks.  One barrier per
// chunk.  The per-element chain is the tiled kernel's: one MFMA per 32-wide
// K chunk, ascending from +0.  FP4: NVFP4 weight (four-chunk units, K %
// 128 == 0); else bf16 (chunk pairs).  D: units in flight, a divisor of the
// units per A chunk.  Needs K % CK == 0 (checked by the host).
// AFP4 (with FP4): A is NVFP4 rows (codes [M, K/2], scales [M, K/16], lda
// in elements, lda % 32 == 0), decoded exactly to bf16 as each chunk is
// staged -- the values the tiled kernel's NVFP4 A staging stores.  Chunk
// c + 1's first loads go out at the start of chunk c and are decoded and
// written at its end, before the barrier.
// ---------------------------------------------------------------------------
// Waits until at most N LDS reads are outstanding; the NF fragment
// registers are operands of the wait, so none of them is used before it.
template <int N, int NF>
__device__ __forceinline__ void wait_frags(i32x4 *a) {
    static_assert(N >= 0 && N < 16, "lgkmcnt field is 4 bits");
    if constexpr (NF == 4)
        asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]) : "n"(N) : "memory");
    else if constexpr (NF == 8)
        asm volatile("s_waitcnt lgkmcnt(%8)"
                     : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7])
                     : "n"(N)
                     : "memory");
    else {
        static_assert(NF == 16, "4, 8 or 16 fragments");
        asm volatile("s_waitcnt lgkmcnt(%16)"
                     : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7]),
                       "+v"(a[8]), "+v"(a[9]), "+v"(a[10]), "+v"(a[11]), "+v"(a[12]), "+v"(a[13]), "+v"(a[14]),
                       "+v"(a[15])
                     : "n"(N)
                     : "memory");
    }
}

template <int RB>
struct AChunk {
    static constexpr int CK = 2048 / RB;          // K columns per staged chunk
    static constexpr int ROWS = 16 * RB;
    static constexpr int AS = CK * 2 + 16;        // padded LDS row stride (bank spread)
    static constexpr int BUF = ROWS * AS;
    static constexpr int BPR = CK * 2 / 1024;     // 1 KB DMA blocks per row and chunk (0: a 512-byte row)
    static_assert(RB == 2 || RB == 4 || RB == 8, "two, four or eight row blocks");
    static_assert(2 * BUF <= 160 * 1024, "two chunk buffers fit the LDS");
};

template <bool FP4, int RB, int D, bool AFP4 = false>
__global__ __launch_bounds__(512) void direct_achunk_kernel(GemmArgs p) {
    static_assert(!AFP4 || FP4, "an NVFP4 A goes with an NVFP4 weight");
    using AC = AChunk<RB>;
    constexpr int U = FP4 ? 4 : 2;                 // 32-wide chunks per unit
    constexpr int UPC = AC::CK / (32 * U);         // units per A chunk
    constexpr int LPU = 2;                         // weight loads per unit
    static_assert(UPC % D == 0, "the window steps within a chunk");
    static_assert(FP4 || D % 2 == 0, "bf16: units alternate between two fragment sets");
    static_assert(UPC * LPU < 64, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) char lds[2 * AC::BUF];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nwv = (int)(blockDim.x >> 6);
    const int r = lane & 15, sub = lane >> 4;
    const int items = (p.N + 15) >> 4;
    const int nch = p.K / AC::CK;
    const int nu = nch * UPC;                      // units per item
    const i32x4 ra = make_rsrc(p.A, (uint32_t)(((int64_t)(p.M - 1) * p.lda + p.K) * 2));
    const int cpr = p.K >> 1, spr = p.K >> 4;
    const int sshift = 8 * (sub >> 1);
    uint16_t *Y = static_cast<uint16_t *>(p.Y);
    const uint32_t lds0 = lds_addr(lds);

    // A chunk c into buffer c & 1: rows 0..M-1, 1 KB blocks shared out over
    // the wavefronts (rows beyond M are never read: fragment reads clamp)
    auto stage = [&](int c) {
        if constexpr (AFP4) return;
        char *buf = lds + (c & 1) * AC::BUF;
        if constexpr (AC::BPR == 0) {
            // 512-byte rows: one row per instruction, lanes 0..31
            for (int row = w; row < p.M; row += nwv) {
                const int k = c * AC::CK + (lane & 31) * 8;
                if (lane < 32)
                    bi_raw_buffer_load_lds(ra, (__attribute__((address_space(3))) uint32_t *)(buf + row * AC::AS), 16,
                                           (int)(row * p.lda * 2) + k * 2, 0, 0, 0);
            }
            return;
        }
        for (int b = w; b < p.M * AC::BPR; b += nwv) {
            const int row = b / AC::BPR, part = b - row * AC::BPR;
            const int k = c * AC::CK + part * 512 + lane * 8;
            bi_raw_buffer_load_lds(ra, (__attribute__((address_space(3))) uint32_t *)(buf + row * AC::AS + part * 1024),
                                   16, (int)(row * p.lda * 2) + k * 2, 0, 0, 0);
        }
    };
    // NVFP4 A: chunk c in 32-element units (16 code bytes, two scale bytes),
    // AG per thread per group; group g's loads, then its decode and writes
    constexpr int AG = RB == 8 ? 2 : 4;            // (eight row blocks: registers are short)
    constexpr int UPR = AC::CK / 32;               // units per row and chunk
    const int a4_units = AFP4 ? p.M * UPR : 0;
    const int a4_groups = (a4_units + AG * (int)blockDim.x - 1) / (AG * (int)blockDim.x);
    uint4 qa[AG];
    uint32_t qs[AG];
    auto a4_load = [&](int c, int g) {
        if constexpr (AFP4) {
            const uint8_t *pc = static_cast<const uint8_t *>(p.A);
            const uint8_t *ps = static_cast<const uint8_t *>(p.A_scales);
#pragma unroll
            for (int i = 0; i < AG; ++i) {
                const int q = (g * AG + i) * (int)blockDim.x + (int)threadIdx.x;
                if (q < a4_units) {
                    const int row = q / UPR, u = c * UPR + (q - row * UPR);
                    qa[i] = *reinterpret_cast<const uint4 *>(pc + (int64_t)row * (p.lda >> 1) + u * 16);
                    qs[i] = *reinterpret_cast<const uint16_t *>(ps + (int64_t)row * (p.lda >> 4) + u * 2);
                }
            }
        }
    };
    auto a4_write = [&](int c, int g) {
        if constexpr (AFP4) {
#pragma unroll
            for (int i = 0; i < AG; ++i) {
                const int q = (g * AG + i) * (int)blockDim.x + (int)threadIdx.x;
                if (q < a4_units) {
                    const int row = q / UPR, u = q - row * UPR;
                    const float s0 = e4m3_value(qs[i] & 0xFFu), s1 = e4m3_value(qs[i] >> 8);
                    char *dst = lds + (c & 1) * AC::BUF + row * AC::AS + u * 64;
                    lds_write_b128(dst, decode8(qa[i].x, s0));
                    lds_write_b128(dst + 16, decode8(qa[i].y, s0));
                    lds_write_b128(dst + 32, decode8(qa[i].z, s1));
                    lds_write_b128(dst + 48, decode8(qa[i].w, s1));
                }
            }
        }
    };

    for (int round = 0; (int)blockIdx.x * nwv + round * (int)gridDim.x * nwv < items; ++round) {
        const int item = (int)blockIdx.x * nwv + w + round * (int)gridDim.x * nwv;
        const int n0 = item * 16;
        const int rows_b = item < items ? min(16, p.N - n0) : 0;
        const int64_t b0 = rows_b > 0 ? n0 : 0;
        i32x4 rb, rs;
        int w_lane, s_lane = kMark;
        if constexpr (FP4) {
            rb = make_rsrc(static_cast<const uint8_t *>(p.B) + b0 * cpr, rows_b > 0 ? (uint32_t)(rows_b * cpr) : 0u);
            rs = make_rsrc(static_cast<const uint8_t *>(p.B_scales) + b0 * spr,
                           rows_b > 0 ? (uint32_t)(rows_b * spr) : 0u);
            w_lane = r < rows_b ? r * cpr + 16 * sub : kMark;
            s_lane = r < rows_b ? r * spr : kMark;
        } else {
            rb = make_rsrc(static_cast<const uint16_t *>(p.B) + b0 * p.ldb,
                           rows_b > 0 ? (uint32_t)(((int64_t)(rows_b - 1) * p.ldb + p.K) * 2) : 0u);
            rs = rb;
            w_lane = r < rows_b ? (int)(r * p.ldb * 2) + 16 * sub : kMark;
        }
        // unit u of this wavefront's item into (x0, x1); units past the last
        // read zeros (a wavefront past the last item reads only zeros)
        auto issue = [&](int u, i32x4 &x0, i32x4 &x1) {
            const bool live = u < nu;
            if constexpr (FP4) {
                x0 = bi_raw_buffer_load_b128(rb, live ? w_lane + 64 * u : kMark, 0, 0);
                const i32x2 sv = bi_raw_buffer_load_b64(rs, live ? s_lane + 8 * u : kMark, 0, 0);
                x1 = i32x4{sv.x, sv.y, 0, 0};
            } else {
                x0 = bi_raw_buffer_load_b128(rb, live ? w_lane + 128 * u : kMark, 0, 0);
                x1 = bi_raw_buffer_load_b128(rb, live ? w_lane + 128 * u + 64 : kMark, 0, 0);
            }
        };

        // chunk 0, then the weight window; chunk 0's copies are older than
        // the window's D * LPU loads
        stage(0);
        for (int g = 0; g < a4_groups; ++g) {
            a4_load(0, g);
            a4_write(0, g);
        }
        asm volatile("" ::: "memory");
        i32x4 ws0[D], ws1[D];
#pragma unroll
        for (int d = 0; d < D; ++d) issue(d, ws0[d], ws1[d]);
        wait_vmcnt<D * LPU>();
        lds_barrier();

        f32x4 acc[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        // this lane's A row in each block, clamped to a staged row
        uint32_t a_row[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) a_row[b] = (uint32_t)(min(16 * b + r, p.M - 1) * AC::AS) + 16 * sub;
        for (int c = 0; c < nch; ++c) {
            // the next chunk's copies go out before this chunk's weight loads,
            // so waiting for all but those UPC * LPU loads covers them
            if (c + 1 < nch) {
                stage(c + 1);
                if (a4_groups > 0) a4_load(c + 1, 0);
            }
            asm volatile("" ::: "memory");
            const uint32_t cb = lds0 + (uint32_t)((c & 1) * AC::BUF);
            // bf16 with at most eight fragments per unit: the A fragments of
            // unit 0 (set 0); each unit then reads the next unit's into the
            // other set before its own MFMAs (sixteen would overrun the LDS
            // counter, so eight row blocks read each unit's own)
            constexpr bool PF = !FP4 && RB * U <= 8;
            // NVFP4 with eight row blocks: two halves of four blocks, each
            // read, waited for and multiplied in turn (registers are short)
            constexpr int H = FP4 && RB * U > 16 ? 2 : 1;
            constexpr int RBH = RB / H;
            i32x4 af[PF ? 2 : 1][RBH * U];
            if constexpr (PF) {
#pragma unroll
                for (int b = 0; b < RB; ++b)
#pragma unroll
                    for (int j = 0; j < U; ++j) af[0][b * U + j] = rd_a(cb + a_row[b] + 64 * j);
            }
            for (int ub = 0; ub < UPC; ub += D) {
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    const int ul = ub + d;                 // unit within the chunk
                    constexpr int NF = RBH * U;
                    i32x4 wv[U];
                    i32x4 *a = af[PF ? (d & 1) : 0];
                    if constexpr (FP4) {
#pragma unroll
                        for (int h = 0; h < H; ++h) {
                            // fragment reads first: the decode covers their latency
#pragma unroll
                            for (int b = 0; b < RBH; ++b)
#pragma unroll
                                for (int j = 0; j < U; ++j)
                                    a[b * U + j] = rd_a(cb + a_row[h * RBH + b] + 64 * (ul * U + j));
                            if (h == 0) {
                                uint32_t y[4] = {(uint32_t)ws0[d].x, (uint32_t)ws0[d].y, (uint32_t)ws0[d].z,
                                                 (uint32_t)ws0[d].w};
                                transpose4(y[0], y[1], y[2], y[3]);
                                const uint32_t s01 = (uint32_t)ws1[d].x >> sshift, s23 = (uint32_t)ws1[d].y >> sshift;
                                const float sc[4] = {e4m3_value<0>(s01), e4m3_value<2>(s01), e4m3_value<0>(s23),
                                                     e4m3_value<2>(s23)};
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    const uint4 q = decode8(y[j], sc[j]);
                                    wv[j] = i32x4{(int)q.x, (int)q.y, (int)q.z, (int)q.w};
                                }
                            }
                            wait_frags<0, NF>(a);
#pragma unroll
                            for (int j = 0; j < U; ++j)
#pragma unroll
                                for (int b = 0; b < RBH; ++b)
                                    acc[h * RBH + b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                        __builtin_bit_cast(bf16x8, a[b * U + j]), __builtin_bit_cast(bf16x8, wv[j]),
                                        acc[h * RBH + b], 0, 0, 0);
                        }
                    } else if constexpr (!PF) {
                        wv[0] = ws0[d];
                        wv[1] = ws1[d];
#pragma unroll
                        for (int b = 0; b < RB; ++b)
#pragma unroll
                            for (int j = 0; j < U; ++j) a[b * U + j] = rd_a(cb + a_row[b] + 64 * (ul * U + j));
                        wait_frags<0, NF>(a);
                    } else {
                        wv[0] = ws0[d];
                        wv[1] = ws1[d];
                        if (ul + 1 < UPC) {
                            i32x4 *an = af[(d + 1) & 1];
#pragma unroll
                            for (int b = 0; b < RB; ++b)
#pragma unroll
                                for (int j = 0; j < U; ++j)
                                    an[b * U + j] = rd_a(cb + a_row[b] + 64 * ((ul + 1) * U + j));
                            wait_frags<NF, NF>(a);
                        } else {
                            wait_frags<0, NF>(a);
                        }
                    }
                    if constexpr (!FP4) {
#pragma unroll
                        for (int j = 0; j < U; ++j)
#pragma unroll
                            for (int b = 0; b < RB; ++b)
                                acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8, a[b * U + j]), __builtin_bit_cast(bf16x8, wv[j]),
                                    acc[b], 0, 0, 0);
                    }
                    issue(c * UPC + ul + D, ws0[d], ws1[d]);
                }
            }
            // NVFP4 A: chunk c + 1 decoded into the other buffer (read last in
            // chunk c - 1, before the previous barrier)
            if (AFP4 && c + 1 < nch) {
                a4_write(c + 1, 0);
                for (int g = 1; g < a4_groups; ++g) {
                    a4_load(c + 1, g);
                    a4_write(c + 1, g);
                }
            }
            // chunk c + 1 has landed (its copies are older than this chunk's
            // UPC * LPU weight loads; its LDS writes end at the barrier), and
            // every wavefront is done with chunk c, whose buffer chunk c + 2
            // reuses
            wait_vmcnt<UPC * LPU>();
            lds_barrier();
        }
        const int col = n0 + r;
        if (r < rows_b) {
#pragma unroll
            for (int b = 0; b < RB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * b + 4 * sub + i;
                    float v = acc[b][i];
                    if constexpr (FP4) v = v * p.alpha;
                    if (row < p.M) Y[(int64_t)row * p.ldy + col] = (uint16_t)f32_to_bf16_rne(v);
                }
        }
        wait_vmcnt<0>();  // the window's trailing zero loads land before the next round
        lds_barrier();
    }
}

template <bool FP4, int RB, bool AFP4 = false>
hipError_t launch_achunk_rb(const GemmArgs &a, int d, int grid, int nwv, hipStream_t s) {
    constexpr int UPC = AChunk<RB>::CK / (32 * (FP4 ? 4 : 2));
    const dim3 b(64 * nwv);
    switch (d) {
        case 8: if constexpr (UPC % 8 == 0) { hipLaunchKernelGGL((direct_achunk_kernel<FP4, RB, 8, AFP4>), dim3(grid), b, 0, s, a); break; } return hipErrorInvalidValue;
        case 4: if constexpr (UPC % 4 == 0) { hipLaunchKernelGGL((direct_achunk_kernel<FP4, RB, 4, AFP4>), dim3(grid), b, 0, s, a); break; } return hipErrorInvalidValue;
        case 2: hipLaunchKernelGGL((direct_achunk_kernel<FP4, RB, 2, AFP4>), dim3(grid), b, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace direct

// A power of two <= dmax dividing `units`: `depth` if given, else `dflt`.
static int pick_depth(int units, int depth, int dflt, int dmax) {
    int d = depth > 0 ? depth : dflt;
    d = d > dmax ? dmax : d;
    while (d & (d - 1)) d &= d - 1;
    while (units % d) d >>= 1;
    return d;
}

bool direct_alds_fits(int M, int K) {
    const int stride = ((K * 2 + 1023) / 1024) * 1024 + 16;
    return (int64_t)M * stride <= direct::kALds;
}

// A in LDS: units of 2 (bf16) or 4 (NVFP4) chunks; D even, dividing the unit count.
bool direct_alds_ok(int M, int K, bool fp4) {
    const int nu = fp4 ? K / 128 : (K + 63) / 64;
    return M >= 1 && M <= 16 && direct_alds_fits(M, K) && (fp4 ? K % 128 == 0 : true) && nu % 2 == 0;
}

hipError_t launch_direct_alds(const GemmArgs &a, bool fp4, bool afp4, int nb, int waves, int cus, int depth,
                              hipStream_t s) {
    if (waves < 1 || cus < 1 || !direct_alds_ok(a.M, a.K, fp4) || (nb != 8 && nb != 16) || (fp4 && nb != 16) ||
        (afp4 && (!fp4 || a.lda % 32 != 0 || !a.A_scales)))
        return hipErrorInvalidValue;
    const int nu = fp4 ? a.K / 128 : (a.K + 63) / 64;
    // at most one workgroup per compute unit (the A copy takes most of LDS)
    int nwv = (waves + cus - 1) / cus;
    nwv = nwv < 1 ? 1 : nwv > 8 ? 8 : nwv;
    // NVFP4 units in flight: 8, or 4 when two wavefronts share a SIMD (their
    // decode interleaves, and fewer registers per wavefront are live)
    const int d = pick_depth(nu, depth == 1 ? 2 : depth,
                             fp4 ? (nwv > 4 ? 4 : 8) : (nb == 16 || a.K >= 8192) ? 16 : 8, nb == 8 ? 32 : 16);
    if (d < 2) return hipErrorInvalidValue;  // the unit count is even (direct_alds_ok)
    const int grid = (waves + nwv - 1) / nwv;
    if (afp4) return direct::launch_alds<true, 16, true>(a, d, grid, nwv, s);
    if (fp4) return direct::launch_alds<true, 16>(a, d, grid, nwv, s);
    return nb == 8 ? direct::launch_alds<false, 8>(a, d, grid, nwv, s)
                   : direct::launch_alds<false, 16>(a, d, grid, nwv, s);
}

// K-chunked A in LDS (16 < M <= 64): rb = 2 or 4 row blocks, K % (2048 / rb)
// == 0 (and K % 128 == 0 for an NVFP4 weight); `waves` streaming wavefronts,
// one 16-column item each per round.  afp4 (with fp4): A is NVFP4 rows
// (lda % 32 == 0, A_scales set).
bool direct_achunk_ok(int M, int K, int rb, bool fp4) {
    if (rb != 2 && rb != 4 && rb != 8) return false;
    const int ck = 2048 / rb;
    return M > 16 * (rb / 2) && M <= 16 * rb && K % ck == 0 && (!fp4 || K % 128 == 0);
}

hipError_t launch_direct_achunk(const GemmArgs &a, bool fp4, bool afp4, int rb, int waves, int cus, int depth,
                                hipStream_t s) {
    if (waves < 1 || cus < 1 || a.M < 1 || a.M > 16 * rb || (rb != 2 && rb != 4 && rb != 8) || a.K % (2048 / rb) != 0 ||
        (fp4 && a.K % 128 != 0) || (afp4 && (!fp4 || a.lda % 32 != 0 || !a.A_scales)))
        return hipErrorInvalidValue;
    // one workgroup per compute unit (two 64 KB chunk buffers), up to eight
    // wavefronts; an NVFP4 A takes at least four (its decode is shared by
    // the workgroup's wavefronts, so fewer workgroups with more wavefronts
    // beat one wavefront each)
    int nwv = (waves + cus - 1) / cus;
    nwv = nwv < 1 ? 1 : nwv > 8 ? 8 : nwv;
    if (afp4 && nwv < 4) nwv = waves < 4 ? waves : 4;
    const int grid = (waves + nwv - 1) / nwv;
    const int upc = (2048 / rb) / (32 * (fp4 ? 4 : 2));
    // depth 1 is taken as 2: two units are the least the window holds
    int d = depth > 1 ? depth : depth == 1 ? 2 : fp4 ? 4 : 8;
    d = d > 8 ? 8 : d;
    while (d & (d - 1)) d &= d - 1;
    while (d > 2 && upc % d) d >>= 1;
    if (d < 2 || upc % d) return hipErrorInvalidValue;
    if (afp4) return rb == 2   ? direct::launch_achunk_rb<true, 2, true>(a, d, grid, nwv, s)
                     : rb == 4 ? direct::launch_achunk_rb<true, 4, true>(a, d, grid, nwv, s)
                               : direct::launch_achunk_rb<true, 8, true>(a, d, grid, nwv, s);
    if (fp4) return rb == 2   ? direct::launch_achunk_rb<true, 2>(a, d, grid, nwv, s)
                    : rb == 4 ? direct::launch_achunk_rb<true, 4>(a, d, grid, nwv, s)
                              : direct::launch_achunk_rb<true, 8>(a, d, grid, nwv, s);
    return rb == 2   ? direct::launch_achunk_rb<false, 2>(a, d, grid, nwv, s)
           : rb == 4 ? direct::launch_achunk_rb<false, 4>(a, d, grid, nwv, s)
                     : direct::launch_achunk_rb<false, 8>(a, d, grid, nwv, s);
}

hipError_t launch_direct_nvfp4(const GemmArgs &a, int rb, int ap, int grid, int depth, hipStream_t s) {
    if (a.M < 1 || a.M > 16 * rb || grid < 1 || a.K % 128 != 0 || (ap && (rb != 1 || a.M > 8)))
        return hipErrorInvalidValue;
    switch (rb) {
        case 4: return direct::launch_nvfp4_rb<4>(a, pick_depth(a.K / 128, depth, 2, 2), grid, s);
        case 2: return direct::launch_nvfp4_rb<2>(a, pick_depth(a.K / 128, depth, 4, 4), grid, s);
        case 1: {
            const int d = pick_depth(a.K / 128, depth, 8, 8);
            return ap ? direct::launch_nvfp4_ap<1>(a, d, grid, s) : direct::launch_nvfp4_ap<0>(a, d, grid, s);
        }
    }
    return hipErrorInvalidValue;
}

hipError_t launch_direct(const GemmArgs &a, int rb, int ap, int grid, int depth, hipStream_t s) {
    if (a.M < 1 || a.M > 16 * rb || grid < 1 || (ap && (rb != 1 || a.M > 8))) return hipErrorInvalidValue;
    switch (rb) {
        case 8: return direct::launch_rb<8>(a, pick_depth((a.K + 63) / 64, depth, 2, 2), grid, s);
        case 4: return direct::launch_rb<4>(a, pick_depth((a.K + 63) / 64, depth, 4, 4), grid, s);
        case 2: return direct::launch_rb<2>(a, pick_depth((a.K + 63) / 64, depth, 8, 8), grid, s);
        case 1: {
            const int d = pick_depth((a.K + 63) / 64, depth, a.K >= 8192 ? 16 : 8, 16);
            return ap ? direct::launch_ap<1>(a, d, grid, s) : direct::launch_ap<0>(a, d, grid, s);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace bi
