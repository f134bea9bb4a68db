// Batch-invariant decode attention over a latent (MLA-absorbed) KV cache.
// The vLLM batch-invariance tracking issue lists the MLA attention backends
// among the operators batch-invariant mode must cover, and the vLLM-Ascend
// guide requires deterministic attention kernels.  Request b holds L_b
// cached latent rows kv_t (Dqk components; the first Dv are the value).
// Every (request, head) result is computed in an order fixed by L_b, Dqk
// and Dv alone -- never by the other requests, the batch size, the head
// count, the grid, the launch or the schedule.  Two kernels, chosen by
// (Dqk, Dv) only:
//
// MFMA kernel (Dqk <= 32*KC, Dv <= 128*VB for a compiled (KC, VB)): a
// request's tokens form chunks of kMlaChunk.  Within chunk c the 32-token
// blocks are taken in ascending order, with one running max m, weight sum l
// and fp32 value accumulator O per head of a group of 16:
//   S^T = K . Q^T        16x16x32 bf16 MFMA, tokens as rows, heads as
//                        columns; Dqk in two parts (32-wide chunks 0 ..
//                        KC/2 - 1 and KC/2 .. KC - 1), each an ascending
//                        MFMA chain from zero, added part 0 + part 1; times
//                        scale;
//   m' = max(m, block max);  alpha = exp2((m - m') * log2 e);
//   p_t = exp2((s_t - m') * log2 e)  (hardware exp2; 0 past L_b);
//   l = alpha * l + the lane's p_t in a fixed order (a head's four lane
//                        sums added in a fixed butterfly at the chunk's end);
//   O^T = alpha * O^T + V^T . P_hi^T + V^T . P_lo^T, where P_hi = bf16(p)
//                        and P_lo = bf16(p - P_hi) (the pair carries p to
//                        about 2^-18 relative), V^T transposed in registers.
// That gives the chunk's (m_c, l_c, O_c).  The chunks are folded in
// ascending order (fold_head, fold_elem) and o = bf16_rne(O / l).  Either
// one workgroup per (request, head group) walks all chunks and folds them
// in registers, or, given a workspace, one workgroup per chunk writes
// (m_c, l_c, O_c) and mla_fold_kernel folds them: the same operations, so
// the same bits.  A workgroup has four computing wavefronts (wavefront w
// takes score part w >> 1 of token half w & 1 and value dims 128 w ..) and
// four copying wavefronts that stream the blocks into a ring of LDS buffers
// by LDS DMA, two barriers per block.

// VALU kernel (other shapes): one workgroup per (request, head); one thread
// per token computes the score as an fp32 fma chain over d ascending, the
// weights are exp2((s_t - max s) * log2 e), their sum a fixed butterfly, and
// wave w accumulates p_t * v_t over tokens w, w+4, ... as fp32 fma chains,
// merged ((u0 + u1) + u2) + u3 and divided by the sum.

#include <atomic>

#include "bi_internal.h"
#include "gemm_kernel.h"  // buffer-resource loads (zeros past the range, no branch)

namespace bi {
namespace {

constexpr int kNT = 256;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint32_t to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two floats rounded to bf16 (nearest even), packed low then high: the
// hardware conversion.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// LDS: q widened to fp32, one score/weight per token, the four waves' value
// partials.  LT = the most tokens a request may hold.
template <int LT>
struct MlaLds {
    float q[kMlaMaxDqk];
    float p[LT];
    float u[4][kMlaMaxDv];
    float red[4];
};

template <int LT>
__global__ __launch_bounds__(kNT) void mla_valu_kernel(MlaArgs a) {
    __shared__ __attribute__((aligned(16))) MlaLds<LT> s;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int Dqk = a.Dqk, Dv = a.Dv, nc = Dqk >> 3, ng = Dv >> 3;
    const int64_t units = (int64_t)a.B * a.H;
    for (int64_t bh = blockIdx.x; bh < units; bh += gridDim.x) {
        const int b = (int)(bh / a.H);
        int L = a.lens[b];
        L = L < 0 ? 0 : (L > a.Lmax ? a.Lmax : L);
        const uint16_t *q = static_cast<const uint16_t *>(a.q) + bh * Dqk;
        const uint16_t *kv = static_cast<const uint16_t *>(a.kv) + (int64_t)b * a.Lmax * Dqk;
        uint16_t *o = static_cast<uint16_t *>(a.out) + bh * Dv;

        __syncthreads();  // the previous unit's readers of s are done
        for (int d = tid; d < Dqk; d += kNT) s.q[d] = __uint_as_float((uint32_t)q[d] << 16);
        __syncthreads();

        // scores
        float mx = -INFINITY;
        for (int t = tid; t < L; t += kNT) {
            const uint4 *k = reinterpret_cast<const uint4 *>(kv + (int64_t)t * Dqk);
            float dot = 0.f;
            for (int c = 0; c < nc; ++c) {
                const uint4 v = k[c];
                const float *qq = s.q + 8 * c;
                dot = __builtin_fmaf(qq[0], lo_bf16(v.x), dot);
                dot = __builtin_fmaf(qq[1], hi_bf16(v.x), dot);
                dot = __builtin_fmaf(qq[2], lo_bf16(v.y), dot);
                dot = __builtin_fmaf(qq[3], hi_bf16(v.y), dot);
                dot = __builtin_fmaf(qq[4], lo_bf16(v.z), dot);
                dot = __builtin_fmaf(qq[5], hi_bf16(v.z), dot);
                dot = __builtin_fmaf(qq[6], lo_bf16(v.w), dot);
                dot = __builtin_fmaf(qq[7], hi_bf16(v.w), dot);
            }
            const float sc = dot * a.scale;
            s.p[t] = sc;
            mx = fmaxf(mx, sc);
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d, 64));
        if (lane == 0) s.red[w] = mx;
        __syncthreads();
        const float m = fmaxf(fmaxf(s.red[0], s.red[1]), fmaxf(s.red[2], s.red[3]));
        __syncthreads();  // every thread has read s.red

        // weights and their sum (each thread rewrites only its own tokens)
        float ls = 0.f;
        for (int t = tid; t < L; t += kNT) {
            const float e = __builtin_amdgcn_exp2f((s.p[t] - m) * kLog2e);
            s.p[t] = e;
            ls += e;
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) ls += __shfl_xor(ls, d, 64);
        if (lane == 0) s.red[w] = ls;
        __syncthreads();  // s.red and every weight are written
        const float l = ((s.red[0] + s.red[1]) + s.red[2]) + s.red[3];

        // weighted values: wave w takes tokens w, w+4, ...; lane owns 8 columns
        for (int g = lane; g < ng; g += 64) {
            float u[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int t = w; t < L; t += 4) {
                const uint4 v = *reinterpret_cast<const uint4 *>(kv + (int64_t)t * Dqk + 8 * g);
                const float pt = s.p[t];
                u[0] = __builtin_fmaf(pt, lo_bf16(v.x), u[0]);
                u[1] = __builtin_fmaf(pt, hi_bf16(v.x), u[1]);
                u[2] = __builtin_fmaf(pt, lo_bf16(v.y), u[2]);
                u[3] = __builtin_fmaf(pt, hi_bf16(v.y), u[3]);
                u[4] = __builtin_fmaf(pt, lo_bf16(v.z), u[4]);
                u[5] = __builtin_fmaf(pt, hi_bf16(v.z), u[5]);
                u[6] = __builtin_fmaf(pt, lo_bf16(v.w), u[6]);
                u[7] = __builtin_fmaf(pt, hi_bf16(v.w), u[7]);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) s.u[w][8 * g + j] = u[j];
        }
        __syncthreads();
        for (int g = tid; g < ng; g += kNT) {
            uint32_t r[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float y[2];
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int c = 8 * g + 2 * j + k;
                    const float uc = ((s.u[0][c] + s.u[1][c]) + s.u[2][c]) + s.u[3][c];
                    y[k] = L > 0 ? uc / l : 0.f;
                }
                r[j] = to_bf16_rne(y[0]) | (to_bf16_rne(y[1]) << 16);
            }
            *reinterpret_cast<uint4 *>(o + 8 * g) = make_uint4(r[0], r[1], r[2], r[3]);
        }
    }
}


typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kNW = 4;                    // computing wavefronts per workgroup (MFMA kernel)
constexpr int kNCopy = 4;                 // copying wavefronts per workgroup (MFMA kernel)

constexpr int kOutOfRange = 0x7FFFFFF0;  // a buffer offset past every range: loads read zeros
constexpr int kReadOnce = 2;  // cache policy of the cache-row copies: non-temporal (each row is read once)

__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Fold of chunk c's (m_c, l_c, O_c) into the running (M, Lsum, Osum), the
// same operations in the one-workgroup path and in the fold kernel.
__device__ __forceinline__ void fold_head(int c, float m_c, float l_c, float &M, float &Ls, float &fa, float &fb) {
    if (c == 0) {
        M = m_c; Ls = l_c; fa = 0.f; fb = 1.f;
        return;
    }
    const float Mn = fmaxf(M, m_c);
    fa = __builtin_amdgcn_exp2f((M - Mn) * kLog2e);
    fb = __builtin_amdgcn_exp2f((m_c - Mn) * kLog2e);
    Ls = __builtin_fmaf(l_c, fb, Ls * fa);
    M = Mn;
}
__device__ __forceinline__ float fold_elem(int c, float o_c, float os, float fa, float fb) {
    return c == 0 ? o_c : __builtin_fmaf(o_c, fb, os * fa);
}

// LDS geometry of the MFMA kernel for KC: a staged 32-token block is 32 rows
// of 4 KC 16-byte chunks (Dqk padded to 32 KC; zeros past Dqk), unpadded,
// with chunk c of row r at slot c ^ (r & 7) of the row, so that the 16 rows
// a fragment read touches spread over the banks.  The block is one
// contiguous range of the cache, copied as 2 KC 1 KB LDS-DMA pieces.
template <int KC>
struct MlaStage {
    static constexpr int CPR = 4 * KC;            // 16-byte chunks per row
    static constexpr int ROWB = 16 * CPR;         // bytes per row
    static constexpr int BUF = 32 * ROWB;         // one 32-token block
    static constexpr int PIECES = BUF / 1024;     // LDS-DMA instructions per block
    static constexpr int NBUF = 4;                // ring of blocks: three in flight
    static constexpr int PW = PIECES / kNCopy;    // pieces per copying wavefront and block
    static constexpr int PA = PW / 2 + 1;         // of them issued while the scores run
    static constexpr int KH = KC / 2;             // score chunks per computing wavefront
    static_assert(CPR % 8 == 0 && BUF % 1024 == 0 && PIECES % kNCopy == 0 && KC % 2 == 0,
                  "whole swizzle groups, pieces and score halves");
};
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16v(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}
__device__ __forceinline__ u32x4_t lds16(const char *p) { return *reinterpret_cast<const u32x4_t *>(p); }
// Wait until at most n (0, 1 or 2) blocks of PER LDS-DMA instructions each
// are still in flight from this wavefront.
template <int PER>
__device__ __forceinline__ void wait_blocks(int n) {
    if (n >= 2) gemm_detail::wait_vmcnt<2 * PER>();
    else if (n == 1) gemm_detail::wait_vmcnt<PER>();
    else gemm_detail::wait_vmcnt<0>();
}
constexpr int kScoreAhead = 4;  // score fragments in flight
// The largest x over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane
// groups of one MFMA column), by lane swaps between the 16- and 32-lane
// halves (max is exact and symmetric, so the order does not matter).
__device__ __forceinline__ float max_lane_groups(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int KC, int VB>
__global__ __launch_bounds__((kNW + kNCopy) * 64, 1) void mla_mfma_kernel(MlaArgs a) {
    using S = MlaStage<KC>;
    constexpr int NB = S::NBUF, PW = S::PW, PA = S::PA;
    constexpr int NT = (kNW + kNCopy) * 64;
    constexpr int VBW = (VB + kNW - 1) / kNW;  // value blocks per computing wavefront
    static_assert(2 * PW < 64, "two blocks in flight fit the vmcnt field");
    static_assert(VB * 128 * 17 * 4 <= NB * S::BUF, "the output tile fits in the ring");
    __shared__ __attribute__((aligned(1024))) char kvs[NB * S::BUF];
    // partial scores: [part p][half h] at ss[2 p + h], part p over the score
    // chunks p KH .. p KH + KH - 1
    __shared__ __attribute__((aligned(16))) f32x4_t ss[4][64];
    // a chunk's O^T (or the final fold), [dim][head] padded, in the ring: it
    // is written only once every copy into the ring has landed and been read
    float(*ob)[17] = reinterpret_cast<float(*)[17]>(kvs);
    __shared__ float Lr[16];  // the heads' weight sums, for the output
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool copier = w >= kNW;  // wavefronts kNW.. copy, the others compute
    const int dw = w - kNW;
    const int r16 = lane & 15, g = lane >> 4;
    const int Dqk = a.Dqk, Dv = a.Dv, H = a.H;
    const int HG = (H + 15) >> 4;
    // Per-lane fragment offsets.  Score reads (row 16 h + r16 of a block,
    // chunk 4 cc + g): slot (4 cc + g) ^ (r16 & 7) is byte 64 cc + koff[cc &
    // 1] of the row.  Value reads (row 16 (k >> 2) + 4 g +
    // m, m = k & 3; chunk 16 vb + r16, wrapped into a shorter row): byte
    // voff[m] + 16 ROWB (k >> 2) + 256 vb of the block.
    const int r7 = r16 & 7, kb2 = (r7 >> 2) & 1, kg = 16 * ((g ^ r7) & 3);
    const int koff[2] = {kg + 64 * kb2, kg - 64 * kb2};
    const int rr = (S::CPR < 16 ? r16 & 7 : r16) ^ (4 * (g & 1));
    int voff[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) voff[m] = (4 * g + m) * S::ROWB + 16 * (rr ^ m);
    // A key is a request (or a request's chunk); its head groups read the same
    // cache rows.  Units are ordered so that a key's head groups get the same
    // unit index mod 8 -- the same XCD, and so one L2, when the grid is a
    // multiple of 8 (workgroups are dealt to the XCDs round-robin).
    const int ncu = a.ws ? a.nchunk : 1;  // chunks per request in the key
    const int64_t keys = (int64_t)a.B * ncu;
    const int64_t units = mla_mfma_units(keys, HG);
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        const int64_t grp = u / (8 * HG);
        const int r = (int)(u - grp * 8 * HG);
        const int64_t key = grp * 8 + (r & 7);
        if (key >= keys) continue;  // padding of the last group of 8 keys (uniform per workgroup)
        const int hg = r >> 3;
        // (chunks key: chunk key / B of request key % B, so that the first
        // chunks, the longest, come first)
        const int b = (int)(a.ws ? key % a.B : key), h0 = hg * 16;
        int L = a.lens[b];
        L = L < 0 ? 0 : (L > a.Lmax ? a.Lmax : L);
        const int nc = (L + kMlaChunk - 1) / kMlaChunk;
        const int c0 = a.ws ? (int)(key / a.B) : 0, c1 = a.ws ? c0 + 1 : nc;
        if (c0 >= nc && a.ws) continue;  // a chunk past the request's end (uniform per workgroup)
        const uint16_t *kvb = static_cast<const uint16_t *>(a.kv) + (int64_t)b * a.Lmax * Dqk;
        const uint16_t *qb = static_cast<const uint16_t *>(a.q) + ((int64_t)b * H + h0) * Dqk;

        __syncthreads();  // the previous unit's readers of the LDS are done
        // the score B fragments of computing wavefront w: head r16, dims
        // 32 cc + 8 g .. + 7 for its chunks cc = (w >> 1) KH + i (zeros past
        // Dqk or H); their loads overlap the first copies
        u32x4_t qreg[S::KH];
        if (!copier) {
#pragma unroll
            for (int i = 0; i < S::KH; ++i) {
                const int d = 32 * ((w >> 1) * S::KH + i) + 8 * g;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (h0 + r16 < H && d < Dqk) v = *reinterpret_cast<const uint4 *>(qb + (int64_t)r16 * Dqk + d);
                qreg[i] = u32x4_t{v.x, v.y, v.z, v.w};
            }
        }

        const int nblk = (L + 31) >> 5;
        // the request's L cached rows; rows at or past L read as zeros
        gemm_detail::i32x4 rkv = gemm_detail::make_rsrc(kvb, (uint32_t)L * (uint32_t)Dqk * 2u);
        rkv.x = __builtin_amdgcn_readfirstlane(rkv.x);
        rkv.y = __builtin_amdgcn_readfirstlane(rkv.y);
        rkv.z = __builtin_amdgcn_readfirstlane(rkv.z);
        rkv.w = __builtin_amdgcn_readfirstlane(rkv.w);
        // pieces dw + kNCopy j, J0 <= j < J1, of block kb into buffer bi by
        // LDS DMA (copying wavefronts): lane l of piece i lands at position
        // 64 i + l of the block, row p / CPR, slot p % CPR, and reads its
        // chunk's bytes
        auto stage = [&](auto j0c, auto j1c, int kb, int bi) {
            constexpr int J0 = decltype(j0c)::value, J1 = decltype(j1c)::value;
            char *dst = kvs + bi * S::BUF + 1024 * dw;
            // recomputed per call (kept out of the loop-invariant registers)
            int p0 = 64 * dw + lane;
            asm volatile("" : "+v"(p0));
            const int tb = kb * 32 * Dqk * 2;
#pragma unroll
            for (int j = J0; j < J1; ++j) {
                const int pos = p0 + 64 * kNCopy * j;
                const int row = pos / S::CPR, slot = pos - row * S::CPR;
                const int c = slot ^ (row & 7);
                const int off = tb + row * Dqk * 2 + 16 * c;
                bi_raw_buffer_load_lds(rkv, (__attribute__((address_space(3))) uint32_t *)(dst + 1024 * kNCopy * j), 16,
                                       16 * c < Dqk * 2 ? off : kOutOfRange, 0, 0, kReadOnce);
            }
        };
        using C0 = std::integral_constant<int, 0>;
        using CA = std::integral_constant<int, PA>;
        using CW = std::integral_constant<int, PW>;

        // this wavefront's running fold over chunks (one-workgroup path):
        // O in os_r, the head's (M, L) in Mh, Lh (every computing lane of a
        // head holds the same values)
        f32x4_t os_r[VBW][8];
        float Mh = 0.f, Lh = 0.f;
        // the unit's blocks kbu0 .. kbu_end - 1 (its chunks' blocks in order)
        // stream through the ring without a break: block kb in buffer
        // (kb - kbu0) % NB
        const int kbu0 = c0 * (kMlaChunk / 32), kbu_end = min(nblk, c1 * (kMlaChunk / 32));
        if (kbu_end > kbu0) {
            // the first two blocks, then the wait for the first; the rest of
            // the ring fills in the first block's two phases (an earlier
            // unit's stores are out of the count first)
            if (copier) {
                gemm_detail::wait_vmcnt<0>();
                stage(C0{}, CW{}, kbu0, 0);
                if (kbu0 + 1 < kbu_end) {
                    stage(C0{}, CW{}, kbu0 + 1, 1);
                    wait_blocks<PW>(1);
                } else {
                    wait_blocks<PW>(0);
                }
            }
            gemm_detail::lds_barrier();  // block kbu0 is in LDS
        }
        // the blocks in ascending order, two barriers each (the copying and
        // the computing wavefronts run loops of their own with the same
        // barriers): computing wavefront w takes part w >> 1 of the scores
        // of half w & 1, and value blocks w, w + kNW, ...; the copying
        // wavefronts copy block kb + NB - 1 in two parts, one beside the
        // scores, one beside the values
        if (copier) {
            static_assert(NB == 4, "the first block's phases fill the ring");
            for (int kb = kbu0; kb < kbu_end; ++kb) {
                const int bn = (kb - kbu0 + NB - 1) % NB;
                const bool more = kb + NB - 1 < kbu_end;
                if (kb == kbu0) {
                    if (kbu0 + 2 < kbu_end) stage(C0{}, CW{}, kbu0 + 2, 2);
                } else if (more) {
                    stage(C0{}, CA{}, kb + NB - 1, bn);
                }
                gemm_detail::lds_barrier();
                // the rest; then block kb + 1 has landed (the blocks after it
                // may still be in flight)
                if (kb == kbu0) {
                    if (more) stage(C0{}, CW{}, kb + NB - 1, bn);
                } else if (more) {
                    stage(CA{}, CW{}, kb + NB - 1, bn);
                }
                wait_blocks<PW>(max(0, min(kbu_end - 1, kb + NB - 1) - (kb + 1)));
                gemm_detail::lds_barrier();
            }
        } else {
            for (int c = c0; c < c1; ++c) {
                f32x4_t o[VBW][8];
#pragma unroll
                for (int vi = 0; vi < VBW; ++vi)
#pragma unroll
                    for (int j = 0; j < 8; ++j) o[vi][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                float m_run = -INFINITY, l_part = 0.f;
                const int kb0 = c * (kMlaChunk / 32), kb_end = min(nblk, (c + 1) * (kMlaChunk / 32));
                for (int kb = kb0; kb < kb_end; ++kb) {
                    const char *kbase = kvs + ((kb - kbu0) % NB) * S::BUF;
                    const int t0 = kb * 32;
                    // this wavefront's first value block: lane (r16, g) reads
                    // tokens 16 (k >> 2) + 4 g + (k & 3), chunk 16 vb + r16
                    // (wrapped into the row where the block has fewer chunks:
                    // rows past Dv)
                    u32x4_t vv[8];
                    if (w < VB) {
#pragma unroll
                        for (int k = 0; k < 8; ++k) vv[k] = lds16(kbase + voff[k & 3] + 16 * S::ROWB * (k >> 2) + 256 * w);
                    }
                    {
                        // part w >> 1 of S^T half w & 1: lane (token r16 of the
                        // half, group g), chunks c0s .. c0s + KH - 1 ascending;
                        // the K fragment of a chunk read kScoreAhead - 1 ahead
                        f32x4_t sacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
                        const char *krow = kbase + (16 * (w & 1) + r16) * S::ROWB;
                        const int c0s = (w >> 1) * S::KH;
                        u32x4_t kf[kScoreAhead];
#pragma unroll
                        for (int i = 0; i < kScoreAhead - 1 && i < S::KH; ++i)
                            kf[i] = lds16(krow + koff[(c0s + i) & 1] + 64 * (c0s + i));
#pragma unroll
                        for (int i = 0; i < S::KH; ++i) {
                            const int in = i + kScoreAhead - 1;
                            if (in < S::KH) kf[in % kScoreAhead] = lds16(krow + koff[(c0s + in) & 1] + 64 * (c0s + in));
                            __builtin_amdgcn_sched_barrier(0);  // keeps the reads this far ahead
                            sacc = mfma16v(kf[i % kScoreAhead], qreg[i], sacc);
                        }
                        ss[w][lane] = sacc;
                    }
                    gemm_detail::lds_barrier();  // the partial scores are in LDS
                    // half h: part 0 + part 1; tokens at or past L weigh 0
                    const f32x4_t sraw[2] = {ss[0][lane] + ss[2][lane], ss[1][lane] + ss[3][lane]};
                    float sv[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) sv[k] = sraw[k >> 2][k & 3] * a.scale;
                    if (t0 + 32 > L) {
#pragma unroll
                        for (int k = 0; k < 8; ++k)
                            if (t0 + 16 * (k >> 2) + 4 * g + (k & 3) >= L) sv[k] = -INFINITY;
                    }
                    float bm = sv[0];
#pragma unroll
                    for (int k = 1; k < 8; ++k) bm = fmaxf(bm, sv[k]);
                    bm = max_lane_groups(bm);
                    const float m_new = fmaxf(m_run, bm);  // finite: token t0 < L is in the block
                    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * kLog2e);
                    m_run = m_new;
                    float pv[8];
                    l_part *= alpha;
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        pv[k] = __builtin_amdgcn_exp2f((sv[k] - m_new) * kLog2e);
                        l_part += pv[k];
                    }
                    // P_hi = bf16(p), P_lo = bf16(p - P_hi), round to nearest even
                    uint32_t hi[4], lo[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        hi[q] = bf16_pair(pv[2 * q], pv[2 * q + 1]);
                        lo[q] = bf16_pair(pv[2 * q] - __uint_as_float(hi[q] << 16),
                                          pv[2 * q + 1] - __uint_as_float(hi[q] & 0xFFFF0000u));
                    }
                    const uint4 phi = make_uint4(hi[0], hi[1], hi[2], hi[3]);
                    const uint4 plo = make_uint4(lo[0], lo[1], lo[2], lo[3]);
                    // values (dims past Dv compute rows that are never stored)
#pragma unroll
                    for (int vi = 0; vi < VBW; ++vi) {
                        const int vb = w + kNW * vi;
                        if (vb >= VB) break;
                        // (a factor of 1 in every lane, the common case once
                        // the maximum settles, leaves O as it is)
                        if (__any(alpha != 1.f)) {
#pragma unroll
                            for (int j = 0; j < 8; ++j) o[vi][j] *= alpha;
                        }
                        if (vi > 0) {
#pragma unroll
                            for (int k = 0; k < 8; ++k) vv[k] = lds16(kbase + voff[k & 3] + 16 * S::ROWB * (k >> 2) + 256 * vb);
                        }
                        uint32_t wcur[8][4];
#pragma unroll
                        for (int k = 0; k < 8; ++k) {
                            wcur[k][0] = vv[k].x; wcur[k][1] = vv[k].y; wcur[k][2] = vv[k].z; wcur[k][3] = vv[k].w;
                        }
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            // V^T row (dim 128 vb + 8 r16 + j) over the 8 tokens, in the order of pv
                            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                            const int wd = j >> 1;
                            const uint4 av = make_uint4(__builtin_amdgcn_perm(wcur[1][wd], wcur[0][wd], sel),
                                                        __builtin_amdgcn_perm(wcur[3][wd], wcur[2][wd], sel),
                                                        __builtin_amdgcn_perm(wcur[5][wd], wcur[4][wd], sel),
                                                        __builtin_amdgcn_perm(wcur[7][wd], wcur[6][wd], sel));
                            o[vi][j] = mfma16(av, phi, o[vi][j]);
                            o[vi][j] = mfma16(av, plo, o[vi][j]);
                        }
                    }
                    // every wavefront is done with this block's buffer (which
                    // block kb + NB reuses) and with the scores; block kb + 1
                    // has landed
                    gemm_detail::lds_barrier();
                }

                // the chunk's (m_c, l_c, O_c): every computing wavefront holds
                // the same m and l, its O^T rows are its value blocks' dims
                float lw = l_part;
                lw += __shfl_xor(lw, 16, 64);
                lw += __shfl_xor(lw, 32, 64);
                if (a.ws) {
                    // this chunk's partial m[16], l[16], O[16][Dv], from the
                    // registers: lane (r16, g) holds head r16's dims 128 vb +
                    // 32 g + 8 i + j at o[vi][j][i]
                    float *pw = a.ws + (((int64_t)b * HG + hg) * ncu + c) * (32 + 16 * (int64_t)Dv);
                    if (w == 0 && g == 0) {
                        pw[r16] = m_run;
                        pw[16 + r16] = lw;
                    }
#pragma unroll
                    for (int vi = 0; vi < VBW; ++vi) {
                        const int vb = w + kNW * vi;
                        if (vb >= VB) break;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int d = 128 * vb + 32 * g + 8 * i;
                            if (d >= Dv) continue;
                            float4 *dst = reinterpret_cast<float4 *>(pw + 32 + (int64_t)r16 * Dv + d);
                            dst[0] = make_float4(o[vi][0][i], o[vi][1][i], o[vi][2][i], o[vi][3][i]);
                            dst[1] = make_float4(o[vi][4][i], o[vi][5][i], o[vi][6][i], o[vi][7][i]);
                        }
                    }
                } else {
                    // the fold, in the lanes
                    float fa, fb;
                    fold_head(c, m_run, lw, Mh, Lh, fa, fb);
#pragma unroll
                    for (int vi = 0; vi < VBW; ++vi)
#pragma unroll
                        for (int j = 0; j < 8; ++j)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                os_r[vi][j][i] = fold_elem(c, o[vi][j][i], os_r[vi][j][i], fa, fb);
                }
            }
        }
        if (a.ws) continue;
        // the fold into ob, then out[b][h0 + h][8c .. 8c + 7]
        if (L > 0) {
            if (w == 0 && g == 0) Lr[r16] = Lh;
#pragma unroll
            for (int vi = 0; vi < VBW; ++vi) {
                const int vb = w + kNW * vi;
                if (vb >= VB) break;
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) ob[128 * vb + 8 * (4 * g + i) + j][r16] = os_r[vi][j][i];
            }
        }
        __syncthreads();
        uint16_t *ob_out = static_cast<uint16_t *>(a.out) + ((int64_t)b * H + h0) * Dv;
        for (int i = tid; i < 16 * (Dv >> 3); i += NT) {
            const int h = i / (Dv >> 3), cq = i % (Dv >> 3);
            if (h0 + h >= H) continue;
            uint32_t r[4] = {0u, 0u, 0u, 0u};
            if (L > 0) {
                const float l = Lr[h];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    r[q] = to_bf16_rne(ob[8 * cq + 2 * q][h] / l) | (to_bf16_rne(ob[8 * cq + 2 * q + 1][h] / l) << 16);
            }
            *reinterpret_cast<uint4 *>(ob_out + (int64_t)h * Dv + 8 * cq) = make_uint4(r[0], r[1], r[2], r[3]);
        }
    }
}

// The fold of the chunk partials, one thread per four output elements
// (request, head group, head, dims 4q .. 4q + 3): it folds chunks 0, 1, ...
// of its head in order, recomputing the head's scalars by the same
// operations; the partials of up to kFoldBatch chunks are loaded before
// they are folded.
constexpr int kFoldBatch = 8;
__global__ __launch_bounds__(256) void mla_fold_kernel(MlaArgs a) {
    const int Dv = a.Dv, H = a.H, HG = (H + 15) >> 4, DQ = Dv >> 2;
    const int64_t per = 16 * (int64_t)DQ;
    const int64_t total = (int64_t)a.B * HG * per;
    const int64_t pstride = 32 + 16 * (int64_t)Dv;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
        const int64_t u = idx / per;
        const int i = (int)(idx - u * per);
        const int h = i / DQ, d = 4 * (i - h * DQ);
        const int b = (int)(u / HG), h0 = (int)(u % HG) * 16;
        if (h0 + h >= H) continue;
        int L = a.lens[b];
        L = L < 0 ? 0 : (L > a.Lmax ? a.Lmax : L);
        const int nc = (L + kMlaChunk - 1) / kMlaChunk;
        const float *pw = a.ws + u * a.nchunk * pstride;
        float M = 0.f, Ls = 0.f, Os[4] = {0.f, 0.f, 0.f, 0.f}, fa, fb;
        for (int cb = 0; cb < nc; cb += kFoldBatch) {
            float mv[kFoldBatch], lv[kFoldBatch];
            float4 ov[kFoldBatch];
#pragma unroll
            for (int k = 0; k < kFoldBatch; ++k) {
                if (cb + k < nc) {
                    const float *pc = pw + (cb + k) * pstride;
                    mv[k] = pc[h];
                    lv[k] = pc[16 + h];
                    ov[k] = *reinterpret_cast<const float4 *>(pc + 32 + (int64_t)h * Dv + d);
                }
            }
#pragma unroll
            for (int k = 0; k < kFoldBatch; ++k) {
                if (cb + k < nc) {
                    const int c = cb + k;
                    fold_head(c, mv[k], lv[k], M, Ls, fa, fb);
                    Os[0] = fold_elem(c, ov[k].x, Os[0], fa, fb);
                    Os[1] = fold_elem(c, ov[k].y, Os[1], fa, fb);
                    Os[2] = fold_elem(c, ov[k].z, Os[2], fa, fb);
                    Os[3] = fold_elem(c, ov[k].w, Os[3], fa, fb);
                }
            }
        }
        uint32_t r[2] = {0u, 0u};
        if (nc > 0) {
            r[0] = to_bf16_rne(Os[0] / Ls) | (to_bf16_rne(Os[1] / Ls) << 16);
            r[1] = to_bf16_rne(Os[2] / Ls) | (to_bf16_rne(Os[3] / Ls) << 16);
        }
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + ((int64_t)b * H + h0 + h) * Dv + d) =
            make_uint2(r[0], r[1]);
    }
}

std::atomic<float *> g_scratch_ptr[kMaxDevices];

}  // namespace

// Library-held scratch for callers that cannot allocate: the chunk partials
// of the chunked schedule, kMlaScratchBytes per GPU, held from the code
// object's load until the process ends.  Host code must never pass this
// name to a kernel (on the host it is only a stand-in for the symbol); it
// uses the device address that hipGetSymbolAddress returns for the current
// device, looked up once per device in mla_scratch.
static __device__ __align__(256) float scratch[kMlaScratchBytes / sizeof(float)];

hipError_t mla_scratch(float **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    float *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        // with `dev` current: each GPU holds its own copy of the array
        e = hipGetSymbolAddress(reinterpret_cast<void **>(&p), HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

int mla_token_capacity(int Lmax) { return Lmax <= 4096 ? 4096 : (Lmax <= kMlaMaxTokens ? kMlaMaxTokens : 0); }

// The compiled (KC, VB) of the MFMA kernel for (Dqk, Dv), or 0 (VALU kernel).
int mla_mfma_variant(int Dqk, int Dv) {
    const int kc = (Dqk + 31) / 32, vb = (Dv + 127) / 128;
    if (kc == 18 && vb == 4) return 1;
    if (kc == 4 && vb == 1) return 2;
    if (kc == 2 && vb == 1) return 3;
    return 0;
}

int64_t mla_workspace_bytes(int B, int H, int Lmax, int Dqk, int Dv) {
    if (!mla_mfma_variant(Dqk, Dv)) return 0;
    const int64_t nch = (Lmax + kMlaChunk - 1) / kMlaChunk;
    return (int64_t)B * ((H + 15) / 16) * nch * (32 + 16 * (int64_t)Dv) * 4;
}

hipError_t launch_mla_decode(const MlaArgs &a, int grid, int fold_grid, hipStream_t st) {
    if (grid < 1 || a.Dqk <= 0 || a.Dqk % 8 || a.Dqk > kMlaMaxDqk || a.Dv <= 0 || a.Dv % 8 ||
        a.Dv > a.Dqk || a.Dv > kMlaMaxDv || a.Lmax < 0)
        return hipErrorInvalidValue;
    const int v = mla_mfma_variant(a.Dqk, a.Dv);
    if (v) {
        if (a.ws && (a.nchunk < 1 || fold_grid < 1)) return hipErrorInvalidValue;
        switch (v) {
            case 1: hipLaunchKernelGGL((mla_mfma_kernel<18, 4>), dim3(grid), dim3((kNW + kNCopy) * 64), 0, st, a); break;
            case 2: hipLaunchKernelGGL((mla_mfma_kernel<4, 1>), dim3(grid), dim3((kNW + kNCopy) * 64), 0, st, a); break;
            default: hipLaunchKernelGGL((mla_mfma_kernel<2, 1>), dim3(grid), dim3((kNW + kNCopy) * 64), 0, st, a); break;
        }
        if (a.ws) {
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(mla_fold_kernel, dim3(fold_grid), dim3(256), 0, st, a);
        }
        return hipGetLastError();
    }
    switch (mla_token_capacity(a.Lmax)) {
        case 4096: hipLaunchKernelGGL(mla_valu_kernel<4096>, dim3(grid), dim3(kNT), 0, st, a); break;
        case kMlaMaxTokens:
            hipLaunchKernelGGL(mla_valu_kernel<kMlaMaxTokens>, dim3(grid), dim3(kNT), 0, st, a);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace bi
