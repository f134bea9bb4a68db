// Batch-invariant BMM for a short reduction (K = 64, 128 or 256): per head
// h, Y[h] = A[h] . B[h] with A [M, K], B [K, N] (N contiguous), bf16 in,
// fp32 accumulation, bf16 out.  The MLA-absorbed shape of the vLLM batch
// invariance tracking issue ("BMM optimization" item) is K = 128, N = 512.
//
// With K this short the operands are tiny next to the output (at M = 1024
// the output is 8x the bytes of A and B together), so the kernel is built to
// keep output stores and operand loads overlapping:
//   - a work unit is (head, 128-column block); its workgroup transposes that
//     B block into LDS once ([n][k], k contiguous) and keeps it;
//   - it then streams 64-row tiles of A through the block: the next tile's
//     A rows are loaded into registers before the current tile's products
//     are computed and stored, so the stores are issued after those loads
//     and waiting for the loads never waits for the stores (vector memory
//     operations retire in issue order);
//   - about 65 KB of LDS at K = 128 leaves room for two workgroups per
//     compute unit, so one unit's stores drain while another computes.
//
// Bits: each output element is the chain of the tiled kernel -- the same
// 16x16x32 bf16 MFMA with fp32 accumulation over 32-wide K chunks in
// ascending order from 0, every lane feeding the same k values in the same
// register positions -- then one bf16 round to nearest even.  Which unit,
// tile or row position computes an element does not enter, so the result is
// bitwise that of every tiled variant and independent of M, of the heads in
// the call and of the grid.

#include "gemm_kernel.h"

namespace bi {
namespace bmm {

using gemm_detail::f32_to_bf16_rne;
using gemm_detail::bf16x8;
using gemm_detail::f32x4;

constexpr int kBN = 128;  // columns per unit
constexpr int kBM = 64;   // rows per streamed A tile
constexpr int kFM = kBM / 16;  // 16-row MFMA blocks per tile
constexpr int kNT = 256;  // four wavefronts, 32 columns each
constexpr int kCStride = kBN * 2 + 16;  // padded bf16 output row in LDS

template <int K>
struct Layout {
    static constexpr int KC = K / 32;                   // MFMA K chunks
    static constexpr int CPR = K / 8;                   // 16-byte chunks per LDS row
    static constexpr int ROWB = K * 2;                  // bytes per LDS row
    static constexpr int SWM = (CPR < 16 ? CPR : 16) - 1;  // chunk swizzle mask
    static constexpr int B_OFF = 0;
    static constexpr int A_OFF = kBN * ROWB;
    static constexpr int C_OFF = A_OFF + kBM * ROWB;
    static constexpr int BYTES = C_OFF + kBM * kCStride;
    static constexpr int A_PER = kBM * CPR / kNT;       // A chunks per thread per tile
    static constexpr int PAIRS = (kBN / 8) * (K / 8);   // 8 x 8 blocks of the B block
    static constexpr int PPT = (PAIRS + kNT - 1) / kNT; // blocks per thread
    static_assert(kBM * CPR % kNT == 0, "A tile chunks split evenly over the threads");
    static_assert(BYTES <= 160 * 1024, "LDS budget of gfx950");
};

// LDS byte offset of 16-byte chunk c of row r of the A tile (rows of ROWB
// bytes); the chunk index is XORed with the row's low bits so that the 16
// rows a fragment read touches fall on different banks.
template <int K>
__device__ __forceinline__ int swz_off(int r, int c) {
    using L = Layout<K>;
    return r * L::ROWB + ((c ^ (r & L::SWM)) << 4);
}

// The same for a row n of the transposed B block, XORed with (n ^ (n >> 3)):
// distinct for the 16 consecutive rows a fragment read touches and for the
// 16 rows 8 apart that one store instruction of the transpose writes.
template <int K>
__device__ __forceinline__ int swz_b(int n, int c) {
    using L = Layout<K>;
    return n * L::ROWB + ((c ^ ((n ^ (n >> 3)) & L::SWM)) << 4);
}

template <int K>
__global__ __launch_bounds__(kNT, (K <= 128 ? 2 : 1)) void bmm_kernel(GemmArgs p) {
    using L = Layout<K>;
    __shared__ __attribute__((aligned(16))) char lds[L::BYTES];
    char *Bt = lds + L::B_OFF;
    char *At = lds + L::A_OFF;
    char *Ct = lds + L::C_OFF;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nblk = (p.N + kBN - 1) / kBN;
    const int units = p.batch * nblk;
    const int mtiles = (p.M + kBM - 1) / kBM;
    const int G = gridDim.x;
    // workgroups on one XCD (blockIdx % 8) take consecutive units, so the
    // column blocks of one head share that XCD's L2 for A
    const bool spread = (G % 8) == 0;
    const int slot = spread ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;

    for (int u = slot; u < units; u += G) {
        const int h = u / nblk, n0 = (u - h * nblk) * kBN;
        const uint16_t *Ah = static_cast<const uint16_t *>(p.A) + (int64_t)h * p.sA;
        const uint16_t *Bh = static_cast<const uint16_t *>(p.B) + (int64_t)h * p.sB;
        uint16_t *Yh = static_cast<uint16_t *>(p.Y) + (int64_t)h * p.sY;

        __syncthreads();  // the previous unit's readers of Bt, At and Ct are done
        // B block: K rows of 128 columns -> Bt[n][k].  A (column chunk c, k
        // group g) pair is an 8 x 8 block: 8 columns (N % 8 == 0, so all in or
        // all out) of rows 8g .. 8g+7.  Its 8 loads are issued first, then it
        // is transposed in registers and written as 8 rows of 16 bytes.
        {
            uint4 bv[L::PPT][8];
#pragma unroll
            for (int t = 0; t < L::PPT; ++t) {
                const int pr = tid + t * kNT;
                const int c = pr % (kBN / 8), g = pr / (kBN / 8);
                const int n = n0 + c * 8;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    bv[t][i] = (pr < L::PAIRS && n < p.N)
                                   ? *reinterpret_cast<const uint4 *>(Bh + (int64_t)(8 * g + i) * p.ldb + n)
                                   : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < L::PPT; ++t) {
                const int pr = tid + t * kNT;
                if (pr < L::PAIRS) {
                    const int c = pr % (kBN / 8), g = pr / (kBN / 8);
                    uint32_t w[8][4];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        w[i][0] = bv[t][i].x; w[i][1] = bv[t][i].y;
                        w[i][2] = bv[t][i].z; w[i][3] = bv[t][i].w;
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        // column c*8+j: element j of each row, k ascending
                        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                        const int wd = j >> 1;
                        uint4 o;
                        o.x = __builtin_amdgcn_perm(w[1][wd], w[0][wd], sel);
                        o.y = __builtin_amdgcn_perm(w[3][wd], w[2][wd], sel);
                        o.z = __builtin_amdgcn_perm(w[5][wd], w[4][wd], sel);
                        o.w = __builtin_amdgcn_perm(w[7][wd], w[6][wd], sel);
                        *reinterpret_cast<uint4 *>(Bt + swz_b<K>(c * 8 + j, g)) = o;
                    }
                }
            }
        }

        // A tile loads into registers (rows beyond M read as zero)
        uint4 ar[L::A_PER];
        auto load_a = [&](int m0) {
#pragma unroll
            for (int i = 0; i < L::A_PER; ++i) {
                const int q = tid + i * kNT;
                const int r = q / L::CPR, c = q % L::CPR;
                ar[i] = (m0 + r < p.M)
                            ? *reinterpret_cast<const uint4 *>(Ah + (int64_t)(m0 + r) * p.lda + c * 8)
                            : make_uint4(0, 0, 0, 0);
            }
        };
        load_a(0);

        for (int mt = 0; mt < mtiles; ++mt) {
            const int m0 = mt * kBM;
            // the previous tile's fragment reads and output-tile reads are done
            // (the barrier after its output tile was written, and this one)
#pragma unroll
            for (int i = 0; i < L::A_PER; ++i) {
                const int q = tid + i * kNT;
                const int r = q / L::CPR, c = q % L::CPR;
                *reinterpret_cast<uint4 *>(At + swz_off<K>(r, c)) = ar[i];
            }
            __syncthreads();
            if (mt + 1 < mtiles) load_a(m0 + kBM);  // in flight during this tile

            // kBM x 128 products: wavefront w owns columns 32w .. 32w+31,
            // kFM 16-row blocks by two 16-column blocks
            f32x4 acc[kFM][2];
#pragma unroll
            for (int fm = 0; fm < kFM; ++fm)
#pragma unroll
                for (int fn = 0; fn < 2; ++fn) acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int r16 = lane & 15, kq = lane >> 4;
#pragma unroll
            for (int kc = 0; kc < L::KC; ++kc) {
                uint4 fa[kFM], fb[2];
#pragma unroll
                for (int fm = 0; fm < kFM; ++fm)
                    fa[fm] = *reinterpret_cast<const uint4 *>(At + swz_off<K>(fm * 16 + r16, kc * 4 + kq));
#pragma unroll
                for (int fn = 0; fn < 2; ++fn)
                    fb[fn] = *reinterpret_cast<const uint4 *>(
                        Bt + swz_b<K>(wave * 32 + fn * 16 + r16, kc * 4 + kq));
#pragma unroll
                for (int fm = 0; fm < kFM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < 2; ++fn)
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, fa[fm]), __builtin_bit_cast(bf16x8, fb[fn]),
                            acc[fm][fn], 0, 0, 0);
            }

            // output tile: fp32 -> bf16 RNE into LDS, then 16-byte row chunks
#pragma unroll
            for (int fm = 0; fm < kFM; ++fm)
#pragma unroll
                for (int fn = 0; fn < 2; ++fn) {
                    const int col = wave * 32 + fn * 16 + r16;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = fm * 16 + kq * 4 + i;
                        *reinterpret_cast<uint16_t *>(Ct + row * kCStride + col * 2) =
                            (uint16_t)f32_to_bf16_rne(acc[fm][fn][i]);
                    }
                }
            __syncthreads();
            constexpr int CPRO = kBN / 8;  // output chunks per row
#pragma unroll
            for (int i = 0; i < kBM * CPRO / kNT; ++i) {
                const int q = tid + i * kNT;
                const int row = q / CPRO, c8 = q % CPRO;
                const int col = n0 + c8 * 8;
                if (m0 + row < p.M && col < p.N)
                    *reinterpret_cast<uint4 *>(Yh + (int64_t)(m0 + row) * p.ldy + col) =
                        *reinterpret_cast<const uint4 *>(Ct + row * kCStride + c8 * 16);
            }
        }
    }
}

}  // namespace bmm

bool bmm_short_k_ok(int K) { return K == 64 || K == 128 || K == 256; }

int bmm_short_k_lds_bytes(int K) {
    switch (K) {
        case 64: return bmm::Layout<64>::BYTES;
        case 128: return bmm::Layout<128>::BYTES;
        case 256: return bmm::Layout<256>::BYTES;
    }
    return 0;
}

hipError_t launch_bmm_short_k(const GemmArgs &a, int grid, hipStream_t s) {
    if (grid < 1 || a.N % 8 != 0) return hipErrorInvalidValue;
    switch (a.K) {
        case 64: hipLaunchKernelGGL(bmm::bmm_kernel<64>, dim3(grid), dim3(bmm::kNT), 0, s, a); break;
        case 128: hipLaunchKernelGGL(bmm::bmm_kernel<128>, dim3(grid), dim3(bmm::kNT), 0, s, a); break;
        case 256: hipLaunchKernelGGL(bmm::bmm_kernel<256>, dim3(grid), dim3(bmm::kNT), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace bi
