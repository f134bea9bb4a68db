// Batch-invariant GEMM mainloop for gfx950: dense bf16 GEMM, BMM and the
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
//   * rows beyond M are zero-filled in LDS and never read from memory; their
//     MFMA blocks are skipped when a whole 16-row block is out of range.
//     Neither touches a valid row's chain;
//   * the tile shape comes from (N, K) only; M sets the tile count; the
//     persistent grid size only decides which workgroup runs which tile.
//
// Prior art: the vLLM PR #39912 summary page (section "implementation
// breakdown") pins a persistent tile scheduler and one default config for the
// batch-invariant NVFP4 GEMM on NVIDIA parts; the same principle is kept, the
// tiling is this file's own for 64-wide wavefronts and bf16 MFMA.

#include "bi_internal.h"

namespace bi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 wavefronts, arranged 2 x 2 over the tile
constexpr int kBK = 64;        // K columns per LDS stage (two 32-wide MFMA steps)

// LDS layout of a staged operand tile: row r (an M row of A or an N column
// of B) holds kBK bf16 = eight 16-byte chunks; chunk c of row r lives in
// slot r*8 + swz(r, c).  The XOR spreads the 16 rows that one MFMA fragment
// read touches over distinct bank groups.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// FP4 E2M1 code (sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0)
// as an fp32 bit pattern.
__device__ __forceinline__ uint32_t e2m1_bits(uint32_t c) {
    const uint32_t mag = c & 7u, e = mag >> 1, m = mag & 1u;
    const uint32_t b = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3F000000u : 0u);
    return b | ((c & 8u) << 28);
}

// FP8 E4M3 (fn) byte (sign bit 7, exponent bits 6..3 with bias 7, mantissa
// bits 2..0; exponent 0 is subnormal m/8 * 2^-6) as an fp32 value.
__device__ __forceinline__ float e4m3_value(uint32_t s) {
    const uint32_t e = (s >> 3) & 15u, m = s & 7u;
    const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
    return (s & 0x80u) ? -v : v;
}

// 32 NVFP4 elements (16 code bytes, low nibble first) with their two scales
// -> four 16-byte chunks of bf16.  e2m1 * e4m3 has at most 6 significant bits
// and lies in [2^-10, 2688], so the fp32 product is exact and its top half is
// the exact bf16.
__device__ __forceinline__ void decode32(const uint4 &codes, uint32_t sc, uint4 out[4]) {
    const float s0 = e4m3_value(sc & 0xFFu), s1 = e4m3_value((sc >> 8) & 0xFFu);
    const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float s = j < 2 ? s0 : s1;
        uint32_t o[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t byte = (cw[j] >> (8 * b)) & 0xFFu;
            const uint32_t lo = __float_as_uint(__uint_as_float(e2m1_bits(byte & 15u)) * s) >> 16;
            const uint32_t hi = __float_as_uint(__uint_as_float(e2m1_bits(byte >> 4)) * s) >> 16;
            o[b] = lo | (hi << 16);
        }
        out[j] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// ---------------------------------------------------------------------------
// Operand stagers: global -> registers (load), registers -> LDS (store).
// ROWS is the tile extent along M (for A) or N (for B).
// ---------------------------------------------------------------------------
template <int ROWS, int MODE>
struct Stager;

// bf16 [rows, K], K contiguous.
template <int ROWS>
struct Stager<ROWS, OPND_BF16_ROWS> {
    static constexpr int TOTAL = ROWS * (kBK / 8);
    static constexpr int PER = (TOTAL + kThreads - 1) / kThreads;
    uint4 r[PER];

    __device__ __forceinline__ void load(const void *base, const void *, int64_t ld, int row0,
                                         int nrows, int k0, int K, int tid) {
        const uint16_t *p = static_cast<const uint16_t *>(base);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = tid + i * kThreads;
            if (TOTAL % kThreads == 0 || q < TOTAL) {
                const int row = q >> 3, c = q & 7;
                const int gr = row0 + row, gk = k0 + c * 8;
                if (gr < nrows && gk < K)
                    r[i] = *reinterpret_cast<const uint4 *>(p + (int64_t)gr * ld + gk);
                else
                    r[i] = make_uint4(0, 0, 0, 0);
            }
        }
    }
    __device__ __forceinline__ void store(uint4 *lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = tid + i * kThreads;
            if (TOTAL % kThreads == 0 || q < TOTAL) {
                const int row = q >> 3, c = q & 7;
                lds[row * 8 + swz(row, c)] = r[i];
            }
        }
    }
};

// bf16 [K, cols], cols contiguous (the BMM right operand).  Each 16-byte
// global chunk holds 8 consecutive columns at one k; it is transposed into the
// row-per-column LDS layout with 2-byte stores.
template <int ROWS>
struct Stager<ROWS, OPND_BF16_KN> {
    static constexpr int CPR = ROWS / 8;  // chunks per k row of the tile
    static constexpr int TOTAL = kBK * CPR;
    static constexpr int PER = (TOTAL + kThreads - 1) / kThreads;
    uint4 r[PER];

    __device__ __forceinline__ void load(const void *base, const void *, int64_t ld, int col0,
                                         int ncols, int k0, int K, int tid) {
        const uint16_t *p = static_cast<const uint16_t *>(base);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = tid + i * kThreads;
            if (TOTAL % kThreads == 0 || q < TOTAL) {
                const int kk = q / CPR, n8 = q % CPR;
                const int gk = k0 + kk, gn = col0 + n8 * 8;
                if (gk < K && gn < ncols)
                    r[i] = *reinterpret_cast<const uint4 *>(p + (int64_t)gk * ld + gn);
                else
                    r[i] = make_uint4(0, 0, 0, 0);
            }
        }
    }
    __device__ __forceinline__ void store(uint4 *lds, int tid) const {
        uint16_t *l16 = reinterpret_cast<uint16_t *>(lds);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = tid + i * kThreads;
            if (TOTAL % kThreads == 0 || q < TOTAL) {
                const int kk = q / CPR, n8 = q % CPR;
                const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int n = n8 * 8 + j;
                    const uint16_t v = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
                    l16[(n * 8 + swz(n, kk >> 3)) * 8 + (kk & 7)] = v;
                }
            }
        }
    }
};

// NVFP4 [rows, K/2] codes + [rows, K/16] scales; ld is the row stride in
// elements (codes stride ld/2 bytes, scales stride ld/16 bytes).  One unit is
// 32 elements: 16 code bytes and 2 scale bytes, decoded to bf16 at LDS-store
// time.
template <int ROWS>
struct Stager<ROWS, OPND_NVFP4_ROWS> {
    static constexpr int TOTAL = ROWS * (kBK / 32);
    static constexpr int PER = (TOTAL + kThreads - 1) / kThreads;
    uint4 r[PER];
    uint32_t s[PER];

    __device__ __forceinline__ void load(const void *base, const void *scales, int64_t ld,
                                         int row0, int nrows, int k0, int K, int tid) {
        const uint8_t *pc = static_cast<const uint8_t *>(base);
        const uint8_t *ps = static_cast<const uint8_t *>(scales);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = tid + i * kThreads;
            if (TOTAL % kThreads == 0 || q < TOTAL) {
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
    __device__ __forceinline__ void store(uint4 *lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = tid + i * kThreads;
            if (TOTAL % kThreads == 0 || q < TOTAL) {
                const int row = q >> 1, h = q & 1;
                uint4 out[4];
                decode32(r[i], s[i], out);
#pragma unroll
                for (int j = 0; j < 4; ++j) lds[row * 8 + swz(row, h * 4 + j)] = out[j];
            }
        }
    }
};

template <int MODE>
__device__ __forceinline__ int64_t elem_bytes_x2() {
    // twice the bytes per element, so NVFP4 (half a byte) stays integral
    return MODE == OPND_NVFP4_ROWS ? 1 : 4;
}

// ---------------------------------------------------------------------------
// The kernel.  Tile (bh, tm, tn) covers rows tm*BM.. of head bh and output
// columns tn*BN..; tiles are enumerated with tn fastest.
// ---------------------------------------------------------------------------
template <int BM, int BN, int AMODE, int BMODE>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(GemmArgs p) {
    constexpr int WTM = BM / 2, WTN = BN / 2;  // per-wavefront sub-tile
    constexpr int FM = WTM / 16, FN = WTN / 16;
    __shared__ uint4 lds[2][(BM + BN) * 8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int nk = (p.K + kBK - 1) / kBK;

    Stager<BM, AMODE> sa;
    Stager<BN, BMODE> sb;

    for (int t = blockIdx.x; t < p.num_tiles; t += gridDim.x) {
        const int tn = t % p.tiles_n;
        const int rest = t / p.tiles_n;
        const int tm = rest % p.tiles_m;
        const int bh = rest / p.tiles_m;
        const int m0 = tm * BM, n0 = tn * BN;

        const char *Ab = static_cast<const char *>(p.A) + bh * p.sA * elem_bytes_x2<AMODE>() / 2;
        const char *Bb = static_cast<const char *>(p.B) + bh * p.sB * elem_bytes_x2<BMODE>() / 2;
        uint16_t *Yb = static_cast<uint16_t *>(p.Y) + bh * p.sY;

        // wave-uniform: does this wavefront's fm-th 16-row block hold a valid row?
        bool live[FM];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) live[fm] = (m0 + wm * WTM + fm * 16) < p.M;

        f32x4 acc[FM][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

        sa.load(Ab, p.A_scales, p.lda, m0, p.M, 0, p.K, tid);
        sb.load(Bb, p.B_scales, p.ldb, n0, p.N, 0, p.K, tid);
        sa.store(lds[0], tid);
        sb.store(lds[0] + BM * 8, tid);
        __syncthreads();

        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) {
                sa.load(Ab, p.A_scales, p.lda, m0, p.M, (kt + 1) * kBK, p.K, tid);
                sb.load(Bb, p.B_scales, p.ldb, n0, p.N, (kt + 1) * kBK, p.K, tid);
            }
            const uint4 *la = lds[cur];
            const uint4 *lb = lds[cur] + BM * 8;
#pragma unroll
            for (int ks = 0; ks < kBK / 32; ++ks) {
                const int c = ks * 4 + (lane >> 4);
                bf16x8 bfrag[FN];
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    const int col = wn * WTN + fn * 16 + (lane & 15);
                    bfrag[fn] = __builtin_bit_cast(bf16x8, lb[col * 8 + swz(col, c)]);
                }
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    if (!live[fm]) continue;
                    const int row = wm * WTM + fm * 16 + (lane & 15);
                    const bf16x8 afrag = __builtin_bit_cast(bf16x8, la[row * 8 + swz(row, c)]);
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag, bfrag[fn],
                                                                              acc[fm][fn], 0, 0, 0);
                }
            }
            if (kt + 1 < nk) {
                sa.store(lds[cur ^ 1], tid);
                sb.store(lds[cur ^ 1] + BM * 8, tid);
            }
            __syncthreads();
        }

        // Epilogue: lane holds rows 4*(lane/16)+i, column lane%16 of each block.
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            if (!live[fm]) continue;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int col = n0 + wn * WTN + fn * 16 + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = m0 + wm * WTM + fm * 16 + (lane >> 4) * 4 + i;
                    if (row < p.M && col < p.N) {
                        float v = acc[fm][fn][i];
                        if constexpr (BMODE == OPND_NVFP4_ROWS) v = v * p.alpha;
                        Yb[(int64_t)row * p.ldy + col] = (uint16_t)f32_to_bf16_rne(v);
                    }
                }
            }
        }
    }
}

template <int BM, int BN, int AM, int BMD>
hipError_t launch_one(const GemmArgs &a, int grid, hipStream_t s) {
    hipLaunchKernelGGL((gemm_kernel<BM, BN, AM, BMD>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int AM, int BMD>
hipError_t launch_modes(const GemmRecipe &r, const GemmArgs &a, int grid, hipStream_t s) {
    switch (r.variant) {
        case 0: return launch_one<128, 128, AM, BMD>(a, grid, s);
        case 1: return launch_one<128, 64, AM, BMD>(a, grid, s);
        case 2: return launch_one<64, 64, AM, BMD>(a, grid, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemm(int a_mode, int b_mode, const GemmRecipe &r, const GemmArgs &args,
                       int grid, hipStream_t stream) {
    if (a_mode == OPND_BF16_ROWS && b_mode == OPND_BF16_ROWS)
        return launch_modes<OPND_BF16_ROWS, OPND_BF16_ROWS>(r, args, grid, stream);
    if (a_mode == OPND_BF16_ROWS && b_mode == OPND_BF16_KN)
        return launch_modes<OPND_BF16_ROWS, OPND_BF16_KN>(r, args, grid, stream);
    if (a_mode == OPND_BF16_ROWS && b_mode == OPND_NVFP4_ROWS)
        return launch_modes<OPND_BF16_ROWS, OPND_NVFP4_ROWS>(r, args, grid, stream);
    if (a_mode == OPND_NVFP4_ROWS && b_mode == OPND_NVFP4_ROWS)
        return launch_modes<OPND_NVFP4_ROWS, OPND_NVFP4_ROWS>(r, args, grid, stream);
    return hipErrorInvalidValue;
}

}  // namespace bi
