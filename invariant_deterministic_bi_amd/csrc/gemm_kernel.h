// Batch-invariant GEMM mainloop for gfx950 (kernel template; instantiated
// once per operand mode in gemm_<mode>.hip): dense bf16 GEMM, BMM and the
// NVFP4 weight GEMM share one kernel template.
//
// Invariance argument (what makes output row i independent of M and of the
// other rows):
//   * every output element is owned by exactly one wavefront lane for the
//     whole K range -- one workgroup per tile, no split-K, no atomics;
//   * its value is the chain acc = MFMA_16x16x32_bf16(a_k, b_k, acc) over
//     32-wide K chunks in ascending order, starting from +0, followed by one
//     bf16 round-to-nearest-even (and, for NVFP4, one fp32 multiply by alpha
//     just before it);
//   * operand rows beyond M (or N) and K columns beyond K are zero-filled in
//     LDS (out-of-range buffer loads return zero) and never read from memory;
//     MFMA blocks whose 16 rows are all beyond M are skipped.  Neither touches
//     a valid row's chain;
//   * the tile shape comes from (N, K) only; M sets the tile count; the
//     persistent grid size and the tile-to-workgroup order only decide which
//     workgroup runs which tile.
//
// Data movement: bf16 operands stored [rows, K] go from HBM straight into LDS
// (buffer_load ... lds, 16 bytes per lane) into rings of SA (A) and SB (B)
// buffers, SA-1 and SB-1 K-steps ahead of the MFMAs; operands that need a
// transform on the way (the [K, N] BMM operand, NVFP4 codes) go through
// registers and are stored one step ahead.  The
// output tile is staged through LDS so that every global store is a full
// 16-byte chunk of a row.
//
// Prior art: the vLLM PR #39912 summary page (section "implementation
// breakdown") pins a persistent tile scheduler and one default config for the
// batch-invariant NVFP4 GEMM on NVIDIA parts; the same principle is kept, the
// tiling here is this file's own for 64-wide wavefronts, LDS DMA and bf16
// MFMA on gfx950.

#pragma once

#include "bi_internal.h"

#include <type_traits>

typedef int bi_i32x4 __attribute__((ext_vector_type(4)));

// LLVM intrinsic: per-lane buffer load of `size` bytes written to LDS at
// M0-base + lane * size; an offset outside the buffer's range writes zeros.
__device__ void bi_raw_buffer_load_lds(bi_i32x4 rsrc,
                                       __attribute__((address_space(3))) uint32_t *lds, int size,
                                       int voffset, int soffset, int offset,
                                       int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");
// LLVM intrinsic: per-lane buffer load of 16 bytes into registers; an offset
// outside the buffer's range reads zeros.
__device__ bi_i32x4 bi_raw_buffer_load_b128(bi_i32x4 rsrc, int voffset, int soffset,
                                            int aux) __asm("llvm.amdgcn.raw.buffer.load.v4i32");
typedef int bi_i32x2 __attribute__((ext_vector_type(2)));
__device__ bi_i32x2 bi_raw_buffer_load_b64(bi_i32x4 rsrc, int voffset, int soffset,
                                           int aux) __asm("llvm.amdgcn.raw.buffer.load.v2i32");

namespace bi {
namespace gemm_detail {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef bi_i32x4 i32x4;
typedef bi_i32x2 i32x2;

constexpr int kBK = 64;  // K columns per LDS stage (two 32-wide MFMA steps)
constexpr int kRowBytes = kBK * 2;  // one staged operand row: eight 16-byte chunks

// Buffer resource for a byte range starting at `base` (gfx9 data format word).
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t num_bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
    r.z = __builtin_amdgcn_readfirstlane((int)num_bytes);
    r.w = 0x00020000;
    return r;
}

// LDS layout of a staged operand tile: row r (an M row of A or an N column
// of B) holds kBK bf16 = eight 16-byte chunks; logical chunk c of row r lives
// in physical slot r*8 + swz(r, c), swz(r, c) = c ^ f(r) with f built from
// bits 1..3 of r.  A 16-byte LDS read on gfx950 serves lanes 8j..8j+7
// together with lanes 8j+32..8j+39 (four cycles per instruction when those
// 16 lanes touch 16 distinct 16-byte bank groups); an MFMA fragment read puts
// rows 0..7 (or 8..15) of a block at chunks c and c+2 in such a lane set, and
// f makes those 16 slots distinct (it also keeps lanes 16j..16j+15 distinct).
// f depends on r's low four bits only, so fragment blocks 16 rows apart differ
// by a constant byte offset (an instruction immediate).  swz(r, .) is an
// involution.
__device__ __forceinline__ int swz(int r, int c) {
    return c ^ (((r >> 1) & 1) | (r & 4) | ((r >> 2) & 2));
}

// LDS accesses that overlap in-flight LDS-DMA prefetch.  The compiler cannot
// tell which LDS bytes an LDS DMA writes, so before any LDS access it can see
// it waits for every outstanding one (vmcnt(0)), which would drain the whole
// prefetch ring each K step.  These accesses are written as inline asm, which
// it does not track; every buffer they touch is ordered by the explicit vmcnt
// waits and barriers of the mainloop instead, and each read waits for its own
// result (lgkmcnt) before returning.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) char *)p;
}
__device__ __forceinline__ uint2 lds_read_b64_u8(const void *p8, const void *pb, uint32_t &byte) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    u32x2 v;
    // early-clobber outputs: the first read's result must not share a
    // register with the second read's address
    asm volatile("ds_read_u8 %1, %3\n\tds_read_b64 %0, %2\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v), "=&v"(byte)
                 : "v"(lds_addr(p8)), "v"(lds_addr(pb))
                 : "memory");
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void lds_write_b16(void *p, uint32_t v) {  // low half of v
    asm volatile("ds_write_b16 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_write_b16_hi(void *p, uint32_t v) {  // high half of v
    asm volatile("ds_write_b16_d16_hi %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_write_b128(void *p, const uint4 &v) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = {v.x, v.y, v.z, v.w};
    asm volatile("ds_write_b128 %0, %1" : : "v"(lds_addr(p)), "v"(w) : "memory");
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// FP8 E4M3 (fn) byte (sign bit 7, exponent bits 6..3 with bias 7, mantissa
// bits 2..0; exponent 0 is subnormal m/8 * 2^-6; S.1111.111 is NaN) as an
// fp32 value, by gfx950's FP8 convert, which implements exactly this format
// (checked against the definition for all 256 bytes).  BYTE selects the byte
// of the dword.
template <int BYTE = 0>
__device__ __forceinline__ float e4m3_value(uint32_t w) {
    return __builtin_amdgcn_cvt_f32_fp8((int)w, BYTE);
}

// Eight NVFP4 elements (one code dword, element 2j in the low nibble of byte
// j) sharing one E4M3 scale -> one 16-byte chunk of bf16, using gfx950's
// FP4 -> fp32 pair convert.  That instruction applies only the power-of-two
// part of its scale operand, so it is given 1.0 and yields the exact e2m1
// values; one fp32 multiply by the scale is then exact (e2m1 * e4m3 has at
// most 6 significant bits and lies in [2^-10, 2688], normal in fp32 and
// bf16), and the top halves of the products are the exact bf16s -- for every
// code and every finite scale byte, in two VALU ops per element.
template <int BYTE>
__device__ __forceinline__ uint32_t decode_pair(uint32_t cw, float s) {
    const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, BYTE);
    return __builtin_amdgcn_perm(__float_as_uint(v.y * s), __float_as_uint(v.x * s), 0x07060302u);
}

__device__ __forceinline__ uint4 decode8(uint32_t cw, float s) {
    return make_uint4(decode_pair<0>(cw, s), decode_pair<1>(cw, s), decode_pair<2>(cw, s),
                      decode_pair<3>(cw, s));
}

// ---------------------------------------------------------------------------
// Direct (LDS-DMA) operand: bf16 [rows, K], K contiguous.  NWI wavefronts
// issue its loads; issuing wavefront w fills rows [w*ROWS/NWI, (w+1)*ROWS/NWI)
// of the tile, eight rows per instruction.
// ---------------------------------------------------------------------------
template <int ROWS, int NWI>
struct DirectOperand {
    static constexpr int RPW = ROWS / NWI;  // rows per issuing wavefront
    static constexpr int INSTR = RPW / 8;   // LDS-DMA instructions per wavefront per stage
    static_assert(RPW % 8 == 0, "each issuing wavefront must own a multiple of 8 rows");

    i32x4 rsrc;
    int row0_off;   // byte offset of this lane's row for instruction 0
    int rows_left;  // valid rows from this lane's row for instruction 0 on
    int step_off;   // byte offset between consecutive instructions (8 rows)

    // base: the tile's first row; rows_valid rows exist; ld in elements.
    __device__ __forceinline__ void setup(const uint16_t *base, int rows_valid, int64_t ld, int K,
                                          int w, int lane) {
        const uint32_t bytes = rows_valid > 0 ? (uint32_t)(((int64_t)(rows_valid - 1) * ld + K) * 2) : 0u;
        rsrc = make_rsrc(base, bytes);
        const int row = w * RPW + (lane >> 3);
        row0_off = (int)(row * ld * 2);
        rows_left = rows_valid - row;
        step_off = (int)(8 * ld * 2);
    }

    // Issue the loads of K-step `k0` into the LDS tile at `lds_tile`.  A
    // step with live == false issues the same instructions with every lane
    // out of range: they write zeros and keep the vmcnt bookkeeping exact.
    __device__ __forceinline__ void issue(char *lds_tile, int k0, int K, int w, int lane,
                                          bool live) const {
#pragma unroll
        for (int j = 0; j < INSTR; ++j) {
            const int row = w * RPW + j * 8 + (lane >> 3);
            const int c = swz(row, lane & 7);           // logical chunk landing in slot lane&7
            const int gk = k0 + c * 8;
            const bool ok = live && j * 8 < rows_left && gk < K;
            const int voff = ok ? row0_off + j * step_off + gk * 2 : (int)0x80000000;
            char *dst = lds_tile + (w * RPW + j * 8) * kRowBytes;
            i32x4 r;  // the descriptor must be scalar: restate its uniformity here
            r.x = __builtin_amdgcn_readfirstlane(rsrc.x);
            r.y = __builtin_amdgcn_readfirstlane(rsrc.y);
            r.z = __builtin_amdgcn_readfirstlane(rsrc.z);
            r.w = __builtin_amdgcn_readfirstlane(rsrc.w);
            bi_raw_buffer_load_lds(r, (__attribute__((address_space(3))) uint32_t *)dst, 16, voff,
                                   0, 0, 0);
        }
    }
};

// ---------------------------------------------------------------------------
// NVFP4 operand through a raw LDS ring: the code bytes ([rows, K/2]) and the
// scale bytes ([rows, K/16]) of a 64-column K step go from HBM into LDS by
// DMA -- codes as 16-byte chunks (32 rows per instruction), scales as dwords
// (64 rows per instruction, issued by the first issuing wavefront only) --
// and are decoded into the bf16 tile layout by all threads one step before
// the MFMAs read them.  Needs K % 64 == 0 (dword-aligned scale rows).
// ---------------------------------------------------------------------------
template <int ROWS, int NWI>
struct RawNvfp4Operand {
    static constexpr int RPW = ROWS / NWI;            // rows per issuing wavefront
    static constexpr int CODE_INSTR = RPW / 32;       // code instructions per wavefront per stage
    static constexpr int SCALE_INSTR = ROWS / 64;     // scale instructions (wavefront 0 only)
    static constexpr int CODES = ROWS * 32;           // code bytes per stage
    static constexpr int STAGE = ROWS * 36;           // + scale bytes
    static_assert(RPW % 32 == 0 && ROWS % 64 == 0, "raw NVFP4 ring needs 32 rows per wavefront");

    i32x4 rc, rs;          // code and scale descriptors for the tile's rows
    int code_off;          // byte offset of this lane's code chunk for instruction 0
    int scale_off;         // byte offset of this lane's scale dword for instruction 0
    int rows_left_c, rows_left_s;
    int code_row_step;     // bytes between code rows 32 apart
    int scale_row_step;    // bytes between scale rows 64 apart

    __device__ __forceinline__ void setup(const uint8_t *codes, const uint8_t *scales, int rows_valid,
                                          int K, int w, int lane) {
        const int cpr = K >> 1, spr = K >> 4;  // code / scale bytes per row
        rc = make_rsrc(codes, rows_valid > 0 ? (uint32_t)(rows_valid * cpr) : 0u);
        rs = make_rsrc(scales, rows_valid > 0 ? (uint32_t)(rows_valid * spr) : 0u);
        const int crow = w * RPW + (lane >> 1);
        code_off = crow * cpr + (lane & 1) * 16;
        rows_left_c = rows_valid - crow;
        scale_off = lane * spr;
        rows_left_s = rows_valid - lane;
        code_row_step = 32 * cpr;
        scale_row_step = 64 * spr;
    }

    // Loads of K step k0 into the raw stage at `raw`; live == false issues the
    // same instructions with every lane out of range (zero-filling no-ops).
    __device__ __forceinline__ void issue(char *raw, int k0, int w, int lane, bool live) const {
        i32x4 r;
        r.x = __builtin_amdgcn_readfirstlane(rc.x);
        r.y = __builtin_amdgcn_readfirstlane(rc.y);
        r.z = __builtin_amdgcn_readfirstlane(rc.z);
        r.w = __builtin_amdgcn_readfirstlane(rc.w);
#pragma unroll
        for (int j = 0; j < CODE_INSTR; ++j) {
            const bool ok = live && j * 32 < rows_left_c;
            const int voff = ok ? code_off + j * code_row_step + (k0 >> 1) : (int)0x80000000;
            char *dst = raw + (w * RPW + j * 32) * 32;
            bi_raw_buffer_load_lds(r, (__attribute__((address_space(3))) uint32_t *)dst, 16, voff, 0, 0, 0);
        }
        if (w == 0) {
            i32x4 q;
            q.x = __builtin_amdgcn_readfirstlane(rs.x);
            q.y = __builtin_amdgcn_readfirstlane(rs.y);
            q.z = __builtin_amdgcn_readfirstlane(rs.z);
            q.w = __builtin_amdgcn_readfirstlane(rs.w);
#pragma unroll
            for (int j = 0; j < SCALE_INSTR; ++j) {
                const bool ok = live && j * 64 < rows_left_s;
                const int voff = ok ? scale_off + j * scale_row_step + (k0 >> 4) : (int)0x80000000;
                char *dst = raw + CODES + j * 64 * 4;
                bi_raw_buffer_load_lds(q, (__attribute__((address_space(3))) uint32_t *)dst, 4, voff, 0, 0, 0);
            }
        }
    }

    // Decode the raw stage into the bf16 tile (all NT threads, one 16-element
    // scale block per thread and pass).
    template <int NT>
    __device__ __forceinline__ static void decode(const char *raw, char *tile, int tid) {
        constexpr int UNITS = ROWS * 4;  // 16 elements each
        uint4 *dst = reinterpret_cast<uint4 *>(tile);
#pragma unroll
        for (int i = 0; i < (UNITS + NT - 1) / NT; ++i) {
            const int u = tid + i * NT;
            if (UNITS % NT == 0 || u < UNITS) {
                const int row = u >> 2, q = u & 3;
                uint32_t sbyte;
                const uint2 c = lds_read_b64_u8(raw + row * 32 + q * 8, raw + CODES + row * 4 + q, sbyte);
                const float s = e4m3_value(sbyte);
                lds_write_b128(dst + row * 8 + swz(row, q * 2), decode8(c.x, s));
                lds_write_b128(dst + row * 8 + swz(row, q * 2 + 1), decode8(c.y, s));
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Register-staged operands: global -> registers (load), registers -> LDS
// (store).  NT threads cooperate.
// ---------------------------------------------------------------------------
template <int ROWS, int MODE, int NT>
struct Staged;

// bf16 [rows, K] and raw-ring NVFP4 operands go to LDS by DMA; nothing is
// staged in registers.
template <int ROWS, int NT>
struct Staged<ROWS, OPND_BF16_ROWS, NT> {
    __device__ __forceinline__ void load(const void *, const void *, int64_t, int, int, int, int,
                                         int) {}
    __device__ __forceinline__ void store(char *, int) const {}
};
template <int ROWS, int NT>
struct Staged<ROWS, OPND_NVFP4_RAW, NT> : Staged<ROWS, OPND_BF16_ROWS, NT> {};

// bf16 [K, cols], cols contiguous (the BMM right operand).  Each 16-byte
// global chunk holds 8 consecutive columns at one k; it is transposed into the
// row-per-column LDS layout with 2-byte stores.
template <int ROWS, int NT>
struct Staged<ROWS, OPND_BF16_KN, NT> {
    static constexpr int CPR = ROWS / 8;  // chunks per k row of the tile
    static constexpr int TOTAL = kBK * CPR;
    static constexpr int PER = (TOTAL + NT - 1) / NT;
    uint4 r[PER];

    __device__ __forceinline__ void load(const void *base, const void *, int64_t ld, int col0,
                                         int ncols, int k0, int K, int tid) {
        const uint16_t *p = static_cast<const uint16_t *>(base);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = tid + i * NT;
            if (TOTAL % NT == 0 || q < TOTAL) {
                const int kk = q / CPR, n8 = q % CPR;
                const int gk = k0 + kk, gn = col0 + n8 * 8;
                if (gk < K && gn < ncols)
                    r[i] = *reinterpret_cast<const uint4 *>(p + (int64_t)gk * ld + gn);
                else
                    r[i] = make_uint4(0, 0, 0, 0);
            }
        }
    }
    __device__ __forceinline__ void store(char *lds_tile, int tid) const {
        uint16_t *l16 = reinterpret_cast<uint16_t *>(lds_tile);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = tid + i * NT;
            if (TOTAL % NT == 0 || q < TOTAL) {
                const int kk = q / CPR, n8 = q % CPR;
                const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int n = n8 * 8 + j;
                    uint16_t *dst = l16 + (n * 8 + swz(n, kk >> 3)) * 8 + (kk & 7);
                    if (j & 1) lds_write_b16_hi(dst, w[j >> 1]);
                    else lds_write_b16(dst, w[j >> 1]);
                }
            }
        }
    }
};

// NVFP4 [rows, K/2] codes + [rows, K/16] scales; ld is the row stride in
// elements (codes stride ld/2 bytes, scales stride ld/16 bytes).  One unit is
// 32 elements: 16 code bytes and 2 scale bytes, decoded to bf16 at LDS-store
// time.
template <int ROWS, int NT>
struct Staged<ROWS, OPND_NVFP4_ROWS, NT> {
    static constexpr int TOTAL = ROWS * (kBK / 32);
    static constexpr int PER = (TOTAL + NT - 1) / NT;
    uint4 r[PER];
    uint32_t s[PER];

    __device__ __forceinline__ void load(const void *base, const void *scales, int64_t ld,
                                         int row0, int nrows, int k0, int K, int tid) {
        const uint8_t *pc = static_cast<const uint8_t *>(base);
        const uint8_t *ps = static_cast<const uint8_t *>(scales);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = tid + i * NT;
            if (TOTAL % NT == 0 || q < TOTAL) {
                const int row = q >> 1, h = q & 1;
                const int gr = row0 + row, gk = k0 + h * 32;
                if (gr < nrows && gk < K) {
                    r[i] = *reinterpret_cast<const uint4 *>(pc + (int64_t)gr * (ld >> 1) + (gk >> 1));
                    s[i] = *reinterpret_cast<const uint16_t *>(ps + (int64_t)gr * (ld >> 4) + (gk >> 4));
                } else {
                    r[i] = make_uint4(0, 0, 0, 0);
                    s[i] = 0;
                }
            }
        }
    }
    __device__ __forceinline__ void store(char *lds_tile, int tid) const {
        uint4 *lds = reinterpret_cast<uint4 *>(lds_tile);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = tid + i * NT;
            if (TOTAL % NT == 0 || q < TOTAL) {
                const int row = q >> 1, h = q & 1;
                const float s0 = e4m3_value(s[i] & 0xFFu), s1 = e4m3_value((s[i] >> 8) & 0xFFu);
                lds_write_b128(lds + row * 8 + swz(row, h * 4 + 0), decode8(r[i].x, s0));
                lds_write_b128(lds + row * 8 + swz(row, h * 4 + 1), decode8(r[i].y, s0));
                lds_write_b128(lds + row * 8 + swz(row, h * 4 + 2), decode8(r[i].z, s1));
                lds_write_b128(lds + row * 8 + swz(row, h * 4 + 3), decode8(r[i].w, s1));
            }
        }
    }
};

template <int MODE>
__device__ __forceinline__ int64_t elem_bytes_x2() {
    // twice the bytes per element, so NVFP4 (half a byte) stays integral
    return (MODE == OPND_NVFP4_ROWS || MODE == OPND_NVFP4_RAW) ? 1 : 4;
}

// Wait until at most N vector-memory operations of this wavefront are
// outstanding (they retire in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------------------
// Tile order.  A workgroup's linear slot L (after spreading consecutive slots
// over the 8 XCDs so each XCD gets a contiguous run) is mapped to (head, tm,
// tn) in groups of GM tile-rows: consecutive slots walk down GM M-tiles, then
// step to the next N-tile, so the workgroups resident on one XCD share both
// A rows and B columns in its L2.
// ---------------------------------------------------------------------------
constexpr int kGroupM = 4;

__device__ __forceinline__ void tile_coords(int L, int tiles_m, int tiles_n, int &bh, int &tm,
                                            int &tn) {
    const int per_head = tiles_m * tiles_n;
    bh = L / per_head;
    const int l = L - bh * per_head;
    const int in_group = kGroupM * tiles_n;
    const int g = l / in_group;
    const int first = g * kGroupM;
    const int gsz = min(tiles_m - first, kGroupM);
    const int r = l - g * in_group;
    tm = first + r % gsz;
    tn = r / gsz;
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN, int SA, int SB, int AMODE, int BMODE>
struct Cfg {
    static constexpr int NW = WGM * WGN, NT = NW * 64;
    static constexpr int WTM = BM / WGM, WTN = BN / WGN;
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    static constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes;
    static constexpr int B_RING = SA * A_BYTES;  // B ring follows the A ring
    static constexpr int C_STRIDE = BN * 2 + 16;  // padded bf16 output row in LDS
    static constexpr int C_BYTES = BM * C_STRIDE;
    static constexpr bool A_DIRECT = AMODE == OPND_BF16_ROWS;
    static constexpr bool B_DIRECT = BMODE == OPND_BF16_ROWS;
    static constexpr bool B_RAW = BMODE == OPND_NVFP4_RAW;
    // B_RAW: a bf16 B double buffer plus a raw ring of SB stages
    static constexpr int RAW_STAGE = BN * 36;
    static constexpr int PIPE_BYTES =
        SA * A_BYTES + (B_RAW ? 2 * B_BYTES + SB * RAW_STAGE : SB * B_BYTES);
    static constexpr int LDS_BYTES = PIPE_BYTES > C_BYTES ? PIPE_BYTES : C_BYTES;
    static_assert(FM >= 1 && FN >= 1, "wave tile must hold at least one 16x16 block");
    static_assert(SA >= 2 && SB >= SA, "ring depths");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of gfx950");

    // When both operands are loaded by LDS DMA, the first half of the
    // wavefronts issues all A loads and the second half all B loads.  A
    // wavefront's vmcnt then counts only its own operand's loads, which
    // retire in issue order, so waiting for A(kt) never waits for the deeper
    // B prefetch.  Otherwise every wavefront issues its share of A.
    static constexpr bool SPLIT = A_DIRECT && (B_DIRECT || B_RAW);
    static constexpr int NWA = SPLIT ? NW / 2 : NW;
    static constexpr int NWB = SPLIT ? NW - NW / 2 : NW;
    static constexpr int LA = A_DIRECT ? BM / NWA / 8 : 0;  // instructions per A wavefront per stage
    static constexpr int LB = B_DIRECT ? BN / NWB / 8 : 0;  // per B wavefront per stage
    static constexpr int LR = B_RAW ? BN / NWB / 32 : 0;    // raw code instructions per B wavefront
    static constexpr int LR0 = B_RAW ? BN / 64 : 0;         // + raw scale instructions (B wavefront 0)
    // Iteration kt issues A(kt+SA-1) (A wavefronts) and B(kt+SB-1) (B
    // wavefronts), out-of-range steps included (as zero-filling no-ops), so
    // before stage kt is read an A wavefront has issued exactly (SA-2)*LA
    // loads after A(kt) and a B wavefront (SB-2)*LB after B(kt).
    static constexpr int WAIT_A = (SA - 2) * LA;
    static constexpr int WAIT_B = (SB - 2) * LB;
};

// LDS barrier for the mainloop: this wavefront's LDS reads and writes are
// complete, then all wavefronts meet.  Unlike __syncthreads() it does not
// drain outstanding global loads (the LDS-DMA prefetch of later stages keeps
// flying); the vmcnt wait before it covers the stage about to be read.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One tile.  NL = number of leading 16-row MFMA blocks of this wavefront's
// sub-tile that hold a valid row (FM for a full tile, fewer at the M edge, 0
// for a wavefront whose rows all lie beyond M).  Blocks fm >= NL are neither
// read nor multiplied; every block fm < NL runs the same chain of MFMAs in
// the same order whatever NL is, so a row's bits do not depend on it.  All
// wavefronts run the same sequence of loads and barriers.
template <int BM, int BN, int WGM, int WGN, int SA, int SB, int AMODE, int BMODE, int NL, bool COMPACT>
__device__ __forceinline__ void run_tile(const GemmArgs &p, char *lds, int m0, int n0,
                                         const char *Ab, const char *Bb, uint16_t *Yb) {
    using C = Cfg<BM, BN, WGM, WGN, SA, SB, AMODE, BMODE>;
    constexpr int NT = C::NT, FN = C::FN, WTM = C::WTM, WTN = C::WTN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
    const int wm = wave / WGN, wn = wave % WGN;
    const int nk = (p.K + kBK - 1) / kBK;

    // COMPACT (a tile whose valid rows all lie in its first 16): rows beyond
    // M are neither loaded nor multiplied, so the LDS is re-laid out as rings
    // of SBX stages: 16 A rows and (for a bf16 B) a full B stage each, as many
    // as the workgroup's LDS holds (at most 16).  A is issued by wavefront 0.
    // A and B are then prefetched deep enough to stream the weight at the
    // per-CU rate; the K order and every MFMA of the valid rows are unchanged.
    constexpr bool CA = COMPACT && C::A_DIRECT;
    constexpr bool BDMA = C::B_DIRECT || C::B_RAW;        // B arrives by LDS DMA
    constexpr int A16 = 16 * kRowBytes;
    constexpr int FREE = C::B_RAW ? C::LDS_BYTES - 2 * C::B_BYTES : C::LDS_BYTES;
    constexpr int PER_STAGE = A16 + (C::B_RAW ? C::RAW_STAGE : C::B_BYTES);
    constexpr int DC_RAW = BDMA ? FREE / PER_STAGE : SB;
    constexpr int DC = DC_RAW > 16 ? 16 : (DC_RAW < SB ? SB : DC_RAW);
    constexpr int SBX = (CA && BDMA) ? DC : SB;             // B ring depth (raw ring for B_RAW)
    constexpr int SAX = CA ? SBX : SA;                      // A ring depth
    constexpr int A_ROWS = CA ? 16 : BM;                    // rows per A stage
    // LDS: [A ring][B ring: SBX bf16 stages, or 2 for B_RAW][raw ring: SBX stages]
    constexpr int B_RING_X = SAX * A_ROWS * kRowBytes;
    constexpr int RAW_RING_X = B_RING_X + 2 * C::B_BYTES;
    static_assert(!C::B_RAW || RAW_RING_X + SBX * C::RAW_STAGE <= C::LDS_BYTES, "raw ring must fit");
    static_assert(!CA || C::B_RAW || B_RING_X + SBX * C::B_BYTES <= C::LDS_BYTES, "compact rings must fit");
    using RawOp = RawNvfp4Operand<(C::B_RAW ? BN : 64), (C::B_RAW ? C::NWB : 2)>;
    DirectOperand<A_ROWS, CA ? 1 : C::NWA> da;
    DirectOperand<BN, C::NWB> db;
    RawOp dr;
    Staged<BM, AMODE, NT> sa;
    Staged<BN, BMODE, NT> sb;
    // wave-uniform roles
    const bool a_wave = C::A_DIRECT && (CA ? wave == 0 : (!C::SPLIT || wave < C::NWA));
    const bool b_wave = BDMA && (!C::SPLIT || wave >= C::NWA);
    const int bw = C::SPLIT ? wave - C::NWA : wave;
    constexpr int LAX = CA ? 2 : C::LA;            // A instructions per A wavefront per stage
    constexpr int WAIT_AX = (SAX - 2) * LAX;
    // set up the descriptors on every wavefront (unconditionally, so the
    // compiler keeps them uniform); each wavefront issues only its role's loads
    if constexpr (C::A_DIRECT)
        da.setup(reinterpret_cast<const uint16_t *>(Ab) + (int64_t)m0 * p.lda, min(A_ROWS, p.M - m0),
                 p.lda, p.K, CA ? 0 : (C::SPLIT ? wave % C::NWA : wave), lane);
    if constexpr (C::B_DIRECT)
        db.setup(reinterpret_cast<const uint16_t *>(Bb) + (int64_t)n0 * p.ldb, min(BN, p.N - n0),
                 p.ldb, p.K, C::SPLIT ? bw % C::NWB : bw, lane);
    if constexpr (C::B_RAW)
        dr.setup(reinterpret_cast<const uint8_t *>(Bb) + (int64_t)n0 * (p.K >> 1),
                 static_cast<const uint8_t *>(p.B_scales) + (int64_t)n0 * (p.K >> 4), min(BN, p.N - n0),
                 p.K, C::SPLIT ? bw % C::NWB : bw, lane);

    f32x4 acc[NL > 0 ? NL : 1][FN];
#pragma unroll
    for (int fm = 0; fm < NL; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto a_buf = [&](int s) -> char * { return lds + (s % SAX) * (A_ROWS * kRowBytes); };
    auto b_buf = [&](int s) -> char * {
        return lds + B_RING_X + (C::B_RAW ? (s & 1) : (s % SBX)) * C::B_BYTES;
    };
    auto raw_buf = [&](int s) -> char * { return lds + RAW_RING_X + (s % SBX) * C::RAW_STAGE; };
    // iteration j of the issue schedule (j < 0: prologue): A(j+SAX-1),
    // B(j+SBX-1), raw(j+SBX) -- a raw stage is decoded one iteration before
    // its MFMAs, so it is fetched one iteration earlier.
    // When B wavefronts have a deeper ring than A (full tiles, split
    // issue), they issue their B loads after their first K step's MFMAs:
    // the A wavefronts' loads then go to the vector memory unit alone at the
    // top of the step while the B wavefronts run MFMAs, and the other way
    // round half a step later, so each SIMD always has one wavefront on MFMAs.
    constexpr bool LATE_B = !COMPACT && C::SPLIT && C::B_DIRECT && SBX > SAX;
    auto issue_b = [&](int j) {
        if constexpr (C::B_DIRECT) {
            const int s = j + SBX - 1;
            if (b_wave && s >= 0) db.issue(b_buf(s), s * kBK, p.K, bw, lane, s < nk);
        }
    };
    auto issue = [&](int j, bool with_b = true) {
        if constexpr (C::A_DIRECT) {
            const int s = j + SAX - 1;
            if (a_wave && s >= 0) da.issue(a_buf(s), s * kBK, p.K, CA ? 0 : wave, lane, s < nk);
        }
        if (with_b) issue_b(j);
        if constexpr (C::B_RAW) {
            const int s = j + SBX;
            if (b_wave && s >= 0) dr.issue(raw_buf(s), s * kBK, bw, lane, s < nk);
        }
    };
    // raw-ring wait of a B wavefront: its loads after raw(s) number exactly
    // `after` schedule iterations' worth
    auto wait_raw = [&](auto after_tag) {
        constexpr int AFTER = decltype(after_tag)::value;
        if (bw == 0) wait_vmcnt<AFTER * (C::LR + C::LR0)>();
        else wait_vmcnt<AFTER * C::LR>();
    };

    // prologue: register-staged stage 0, then schedule iterations up to -1
    if constexpr (!C::A_DIRECT) {
        sa.load(Ab, p.A_scales, p.lda, m0, p.M, 0, p.K, tid);
        sa.store(a_buf(0), tid);
    }
    if constexpr (!C::B_DIRECT && !C::B_RAW) {
        sb.load(Bb, p.B_scales, p.ldb, n0, p.N, 0, p.K, tid);
        sb.store(b_buf(0), tid);
    }
    constexpr int LEAD = C::B_RAW ? (SBX > SAX - 1 ? SBX : SAX - 1) : (SBX > SAX ? SBX - 1 : SAX - 1);
    for (int j = -LEAD; j < 0; ++j) issue(j);
    if constexpr (C::B_RAW) {
        // raw(0) was issued in iteration -SBX: SBX-1 iterations follow it
        if (b_wave) wait_raw(std::integral_constant<int, SBX - 1>{});
        lds_barrier();
        RawOp::template decode<NT>(raw_buf(0), b_buf(0), tid);
    }

    for (int kt = 0; kt < nk; ++kt) {
        if constexpr (C::A_DIRECT)
            if (a_wave) wait_vmcnt<WAIT_AX>();
        if constexpr (C::B_DIRECT)
            if (b_wave && !a_wave) wait_vmcnt<(SBX - 2) * C::LB>();
        if constexpr (C::B_RAW)
            // raw(kt+1), decoded in this iteration, was issued SBX-2 iterations
            // before the last one
            if (b_wave && !a_wave) wait_raw(std::integral_constant<int, SBX - 2>{});
        lds_barrier();
        // register-staged loads for kt+1 first, then this iteration's direct
        // loads, so that waiting on the former never waits on the latter
        const bool more = kt + 1 < nk;
        if constexpr (!C::A_DIRECT) if (more) sa.load(Ab, p.A_scales, p.lda, m0, p.M, (kt + 1) * kBK, p.K, tid);
        if constexpr (!C::B_DIRECT && !C::B_RAW) if (more) sb.load(Bb, p.B_scales, p.ldb, n0, p.N, (kt + 1) * kBK, p.K, tid);
        issue(kt, !LATE_B);
        bool b_issued = !LATE_B;
        // The next stage's decode: with eight wavefronts the two sharing a
        // SIMD (w and w+4) take opposite orders -- w decodes before its MFMAs,
        // w+4 after them -- so one's decode arithmetic runs beside the other's
        // MFMAs and never holds registers while fragments are live.
        const bool decode_first = C::NW < 8 || wave < C::NW / 2;
        if constexpr (C::B_RAW)
            if (more && decode_first) RawOp::template decode<NT>(raw_buf(kt + 1), b_buf(kt + 1), tid);

        if constexpr (NL > 0) {
            const uint4 *la = reinterpret_cast<const uint4 *>(a_buf(kt));
            const uint4 *lb = reinterpret_cast<const uint4 *>(b_buf(kt));
            constexpr int KS = kBK / 32;
            // With four wavefronts (one per SIMD), small wave tiles read every
            // fragment of the stage first (they return in order) and then run
            // the MFMAs, which wait only for the fragments they consume.  With
            // eight wavefronts the SIMD's second wavefront hides the read
            // latency, and a 128x128 wave tile would need 128 fragment
            // registers, so those read one 32-wide K step at a time.  Either
            // way each accumulator sees the same MFMA sequence.
            constexpr bool ALL_FIRST = NL * FN < 64 && C::NW < 8;
            bf16x8 bfrag[ALL_FIRST ? KS : 1][FN], afrag[ALL_FIRST ? KS : 1][NL > 0 ? NL : 1];
            auto read_frags = [&](int ks, int slot) {
                const int c = ks * 4 + (lane >> 4);
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    const int col = wn * WTN + fn * 16 + (lane & 15);
                    bfrag[slot][fn] = __builtin_bit_cast(bf16x8, lb[col * 8 + swz(col, c)]);
                }
#pragma unroll
                for (int fm = 0; fm < NL; ++fm) {
                    const int row = wm * WTM + fm * 16 + (lane & 15);
                    afrag[slot][fm] = __builtin_bit_cast(bf16x8, la[row * 8 + swz(row, c)]);
                }
            };
            auto mfmas = [&](int slot) {
#pragma unroll
                for (int fm = 0; fm < NL; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            afrag[slot][fm], bfrag[slot][fn], acc[fm][fn], 0, 0, 0);
            };
            if constexpr (ALL_FIRST) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) read_frags(ks, ks);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) mfmas(ks);
                __builtin_amdgcn_sched_barrier(0);
            } else {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    read_frags(ks, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    mfmas(0);
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (LATE_B)
                        if (ks == 0) {
                            issue_b(kt);
                            b_issued = true;
                        }
                }
            }
        }
        // every B wavefront issues exactly one B stage per iteration
        if constexpr (LATE_B)
            if (!b_issued) issue_b(kt);
        if constexpr (C::B_RAW)
            if (more && !decode_first) RawOp::template decode<NT>(raw_buf(kt + 1), b_buf(kt + 1), tid);
        if (more) {
            if constexpr (!C::A_DIRECT) sa.store(a_buf(kt + 1), tid);
            if constexpr (!C::B_DIRECT && !C::B_RAW) sb.store(b_buf(kt + 1), tid);
        }
    }

    // Epilogue: fp32 -> (alpha) -> bf16 RNE into a padded LDS tile, then
    // full 16-byte row chunks to global memory.
    __syncthreads();
#pragma unroll
    for (int fm = 0; fm < NL; ++fm) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int col = wn * WTN + fn * 16 + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wm * WTM + fm * 16 + (lane >> 4) * 4 + i;
                float v = acc[fm][fn][i];
                if constexpr (BMODE == OPND_NVFP4_ROWS || BMODE == OPND_NVFP4_RAW) v = v * p.alpha;
                *reinterpret_cast<uint16_t *>(lds + row * C::C_STRIDE + col * 2) =
                    (uint16_t)f32_to_bf16_rne(v);
            }
        }
    }
    __syncthreads();
    constexpr int CPR = BN / 8;  // 16-byte chunks per output row
    const int rows_valid = min(BM, p.M - m0);
    for (int q = tid; q < rows_valid * CPR; q += NT) {
        const int row = q / CPR, c8 = q % CPR;
        const int col = n0 + c8 * 8;
        const uint4 v = *reinterpret_cast<const uint4 *>(lds + row * C::C_STRIDE + c8 * 16);
        uint16_t *dst = Yb + (int64_t)(m0 + row) * p.ldy + col;
        if (col + 8 <= p.N && (((uintptr_t)dst) & 15) == 0) {
            *reinterpret_cast<uint4 *>(dst) = v;
        } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (col + j < p.N) dst[j] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
        }
    }
    // the LDS is reused by the next tile's prologue: its reads are done
    // (the global stores may still be in flight; a __syncthreads() would
    // wait for them too)
    lds_barrier();
}

template <int BM, int BN, int WGM, int WGN, int SA, int SB, int AMODE, int BMODE>
__global__ __launch_bounds__(WGM *WGN * 64, 1) void gemm_kernel(GemmArgs p) {
    using C = Cfg<BM, BN, WGM, WGN, SA, SB, AMODE, BMODE>;
    constexpr int FM = C::FM, WTM = C::WTM;
    __shared__ __attribute__((aligned(16))) char lds[C::LDS_BYTES];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WGN;
    const int G = gridDim.x;
    const bool spread = (G % 8) == 0;
    const int slot = spread ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;

    // Grouped mode: tiles are enumerated compactly, expert by expert, each
    // expert holding ceil(rows / BM) * tiles_n of them; L only grows, so the
    // walk over the experts' row ranges is resumed, not restarted (scalar,
    // wave-uniform).  num_tiles is the host's bound (ceil(T / BM) + E) *
    // tiles_n; a workgroup stops at the first L past the real total.
    int g_e = 0;
    int64_t g_pref = 0, g_o0 = 0, g_o1 = 0;
    auto g_range = [&](int e) {
        int64_t o0 = p.group_off[e], o1 = p.group_off[e + 1];
        o0 = o0 < 0 ? 0 : (o0 > p.total_rows ? p.total_rows : o0);
        o1 = o1 < o0 ? o0 : (o1 > p.total_rows ? p.total_rows : o1);
        g_o0 = o0;
        g_o1 = o1;
    };
    if (p.group_off) g_range(0);

    for (int base = 0; base < p.num_tiles; base += G) {
        const int L = base + slot;
        if (L >= p.num_tiles) break;
        int bh, tm, tn;
        GemmArgs q = p;
        const char *Ab, *Bb;
        uint16_t *Yb;
        if (p.group_off) {
            for (;;) {
                const int64_t nt = ((g_o1 - g_o0 + BM - 1) / BM) * p.tiles_n;
                if (L < g_pref + nt) break;
                g_pref += nt;
                if (++g_e >= p.batch) break;
                g_range(g_e);
            }
            if (g_e >= p.batch) break;
            const int l = static_cast<int>(L - g_pref);
            bh = g_e;
            tm = l / p.tiles_n;
            tn = l - tm * p.tiles_n;
            q.M = static_cast<int>(g_o1 - g_o0);
            Ab = static_cast<const char *>(p.A) + g_o0 * p.lda * elem_bytes_x2<AMODE>() / 2;
            Bb = static_cast<const char *>(p.B) + bh * p.sB * elem_bytes_x2<BMODE>() / 2;
            Yb = static_cast<uint16_t *>(p.Y) + g_o0 * p.ldy;
        } else {
            tile_coords(L, p.tiles_m, p.tiles_n, bh, tm, tn);
            Ab = static_cast<const char *>(p.A) + bh * p.sA * elem_bytes_x2<AMODE>() / 2;
            Bb = static_cast<const char *>(p.B) + bh * p.sB * elem_bytes_x2<BMODE>() / 2;
            Yb = static_cast<uint16_t *>(p.Y) + bh * p.sY;
        }
        const int m0 = tm * BM, n0 = tn * BN;

        // live 16-row blocks of this wavefront's sub-tile, rounded up to the
        // next instantiated count (wave-uniform)
        const int rows_left = q.M - m0 - wm * WTM;
        const int nlive = rows_left <= 0 ? 0 : min(FM, (rows_left + 15) / 16);
        // Compact tiles (valid rows all in the first 16) re-lay the LDS for
        // deep weight prefetch.  The raw-NVFP4 256-column instance skips it:
        // its deep raw ring does not fit the register file beside the full
        // path, and M <= 16 calls take the skinny kernel anyway.  Such tiles
        // run the full path with one live block (same bits).
        if (q.M - m0 <= 16 && !(BMODE == OPND_NVFP4_RAW && BN >= 256)) {
            // every valid row of the tile is in wavefront row 0's first block
            if (wm == 0)
                run_tile<BM, BN, WGM, WGN, SA, SB, AMODE, BMODE, 1, true>(q, lds, m0, n0, Ab, Bb, Yb);
            else
                run_tile<BM, BN, WGM, WGN, SA, SB, AMODE, BMODE, 0, true>(q, lds, m0, n0, Ab, Bb, Yb);
        } else if (nlive == 0)
            run_tile<BM, BN, WGM, WGN, SA, SB, AMODE, BMODE, 0, false>(q, lds, m0, n0, Ab, Bb, Yb);
        else if (nlive == 1 || FM == 1)
            run_tile<BM, BN, WGM, WGN, SA, SB, AMODE, BMODE, 1, false>(q, lds, m0, n0, Ab, Bb, Yb);
        else if (nlive <= 2 || FM == 2)
            run_tile<BM, BN, WGM, WGN, SA, SB, AMODE, BMODE, (FM < 2 ? FM : 2), false>(q, lds, m0, n0, Ab, Bb, Yb);
        else if (nlive <= 4 || FM <= 4)
            run_tile<BM, BN, WGM, WGN, SA, SB, AMODE, BMODE, (FM < 4 ? FM : 4), false>(q, lds, m0, n0, Ab, Bb, Yb);
        else
            run_tile<BM, BN, WGM, WGN, SA, SB, AMODE, BMODE, FM, false>(q, lds, m0, n0, Ab, Bb, Yb);
    }
}

template <int BM, int BN, int WGM, int WGN, int SA, int SB, int AM, int BMD>
hipError_t launch_one(const GemmArgs &a, int grid, hipStream_t s) {
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WGM, WGN, SA, SB, AM, BMD>), dim3(grid),
                       dim3(WGM * WGN * 64), 0, s, a);
    return hipGetLastError();
}

template <int AM, int BMD, int V>
hipError_t launch_variant(const GemmArgs &a, int grid, hipStream_t s) {
    constexpr TileShape t = kTileShapes[V];
    // register-staged B (NVFP4 codes, the [K, N] BMM operand) is stored one
    // step ahead, so its ring needs only as many buffers as A's.  A raw NVFP4
    // ring needs 32 rows per B wavefront; other shapes take the staged path
    // (same bits).
    constexpr int nwb = (AM == OPND_BF16_ROWS) ? t.wgm * t.wgn - t.wgm * t.wgn / 2 : t.wgm * t.wgn;
    constexpr bool raw_ok = (t.bn / nwb) % 32 == 0 && t.bn % 64 == 0;
    constexpr int bmd = (BMD == OPND_NVFP4_RAW && !raw_ok) ? OPND_NVFP4_ROWS : BMD;
    constexpr int sb = (bmd == OPND_BF16_ROWS || bmd == OPND_NVFP4_RAW) ? t.sb : t.sa;
    return launch_one<t.bm, t.bn, t.wgm, t.wgn, t.sa, sb, AM, bmd>(a, grid, s);
}

template <int AM, int BMD>
hipError_t launch_modes(const GemmRecipe &r, const GemmArgs &a, int grid, hipStream_t s) {
    static_assert(kNumTileShapes == 19, "one case per compiled tile shape");
    switch (r.variant) {
        case 0: return launch_variant<AM, BMD, 0>(a, grid, s);
        case 1: return launch_variant<AM, BMD, 1>(a, grid, s);
        case 2: return launch_variant<AM, BMD, 2>(a, grid, s);
        case 3: return launch_variant<AM, BMD, 3>(a, grid, s);
        case 4: return launch_variant<AM, BMD, 4>(a, grid, s);
        case 5: return launch_variant<AM, BMD, 5>(a, grid, s);
        case 6: return launch_variant<AM, BMD, 6>(a, grid, s);
        case 7: return launch_variant<AM, BMD, 7>(a, grid, s);
        case 8: return launch_variant<AM, BMD, 8>(a, grid, s);
        case 9: return launch_variant<AM, BMD, 9>(a, grid, s);
        case 10: return launch_variant<AM, BMD, 10>(a, grid, s);
        case 11: return launch_variant<AM, BMD, 11>(a, grid, s);
        case 12: return launch_variant<AM, BMD, 12>(a, grid, s);
        case kPingPongVariant: return launch_variant<AM, BMD, 12>(a, grid, s);  // same shape, classic schedule
        case 14: return launch_variant<AM, BMD, 14>(a, grid, s);
        case 15: return launch_variant<AM, BMD, 15>(a, grid, s);
        case 16: return launch_variant<AM, BMD, 16>(a, grid, s);
        case kPingPong192Variant: return launch_variant<AM, BMD, 16>(a, grid, s);  // same shape, classic schedule
        case kPingPong128Variant: return launch_variant<AM, BMD, 9>(a, grid, s);   // same shape, classic schedule
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gemm_detail
}  // namespace bi
