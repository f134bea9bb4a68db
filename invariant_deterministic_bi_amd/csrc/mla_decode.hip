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
// request's tokens form chunks of kMlaChunk.  Within chunk c, wavefront w of
// four takes the chunk's 32-token blocks w, w+4, w+8, ... ascending and
// keeps, per head of a group of 16, a running max m, a weight sum l and an
// fp32 value accumulator O:
//   S^T = K . Q^T        16x16x32 bf16 MFMA, tokens as rows, heads as
//                        columns, Dqk in ascending 32-wide chunks; times scale;
//   m' = max(m, block max);  alpha = exp2((m - m') * log2 e);
//   p_t = exp2((s_t - m') * log2 e)  (hardware exp2; 0 past L_b);
//   l = alpha * l + the lane's p_t in a fixed order;
//   O^T = alpha * O^T + V^T . P_hi^T + V^T . P_lo^T, where P_hi = bf16(p)
//                        and P_lo = bf16(p - P_hi) (the pair carries p to
//                        about 2^-18 relative), V^T transposed in registers.
// The four waves' (m, l, O) are merged in wave order with the factors
// exp2((m_w - M) * log2 e), M the largest m_w, giving the chunk's
// (m_c, l_c, O_c).  The chunks are folded in ascending order (fold_head,
// fold_elem) and o = bf16_rne(O / l).  Either one workgroup per (request,
// head group) walks all chunks and folds them in LDS, or, given a workspace,
// one workgroup per chunk writes (m_c, l_c, O_c) and mla_fold_kernel folds
// them: the same operations, so the same bits.

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

constexpr int kNW = 4;                    // wavefronts per workgroup (MFMA kernel)
constexpr int kQStride = kMlaMaxDqk + 8;  // LDS row of Q, padded: 16 rows conflict-free

constexpr int kOutOfRange = 0x7FFFFFF0;  // a buffer offset past every range: loads read zeros

// 16 bytes at byte offset `off` of the buffer `r`, or zeros past its range.
__device__ __forceinline__ uint4 rload16(gemm_detail::i32x4 r, int off) {
    return __builtin_bit_cast(uint4, bi_raw_buffer_load_b128(r, off, 0, 0));
}

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

template <int KC, int VB>
__global__ __launch_bounds__(kNW * 64, 1) void mla_mfma_kernel(MlaArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t qs[16 * kQStride];
    __shared__ float ob[VB * 128][17];  // this chunk's merged O^T: [dim][head], padded
    __shared__ float os[VB * 128][17];  // the running fold over chunks (one-workgroup path)
    __shared__ float mred[kNW][16], lred[kNW][16], mch[16], lch[16], fah[16], fbh[16], Mr[16], Lr[16];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int Dqk = a.Dqk, Dv = a.Dv, H = a.H;
    const int HG = (H + 15) >> 4;
    const int qrow = (Dqk + 31) & ~31;  // Q columns staged (zero past Dqk)
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
        const int b = (int)(key / ncu), h0 = hg * 16;
        int L = a.lens[b];
        L = L < 0 ? 0 : (L > a.Lmax ? a.Lmax : L);
        const int nc = (L + kMlaChunk - 1) / kMlaChunk;
        const int c0 = a.ws ? (int)(key % ncu) : 0, c1 = a.ws ? c0 + 1 : nc;
        if (c0 >= nc && a.ws) continue;  // a chunk past the request's end (uniform per workgroup)
        const uint16_t *kvb = static_cast<const uint16_t *>(a.kv) + (int64_t)b * a.Lmax * Dqk;
        const uint16_t *qb = static_cast<const uint16_t *>(a.q) + ((int64_t)b * H + h0) * Dqk;

        __syncthreads();  // the previous unit's readers of qs, ob, os and the head arrays are done
        for (int i = tid; i < 16 * (qrow >> 3); i += kNW * 64) {
            const int h = i / (qrow >> 3), d = (i % (qrow >> 3)) * 8;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (h0 + h < H && d < Dqk) v = *reinterpret_cast<const uint4 *>(qb + (int64_t)h * Dqk + d);
            *reinterpret_cast<uint4 *>(qs + h * kQStride + d) = v;
        }
        __syncthreads();

        const int nblk = (L + 31) >> 5;
        // the request's L cached rows; rows at or past L read as zeros
        const gemm_detail::i32x4 rkv = gemm_detail::make_rsrc(kvb, (uint32_t)L * (uint32_t)Dqk * 2u);
        for (int c = c0; c < c1; ++c) {
            f32x4_t o[VB][8];
#pragma unroll
            for (int vb = 0; vb < VB; ++vb)
#pragma unroll
                for (int j = 0; j < 8; ++j) o[vb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            float m_run = -INFINITY, l_part = 0.f;
            const int kb_end = min(nblk, (c + 1) * (kMlaChunk / 32));
            for (int kb = c * (kMlaChunk / 32) + w; kb < kb_end; kb += kNW) {
                const int t0 = kb * 32;
                // scores: lane holds tokens t0 + 16hb + 4g + i of head r16
                f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
                uint4 kk[2][KC];
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    const int t = t0 + 16 * hb + r16;
#pragma unroll
                    for (int cc = 0; cc < KC; ++cc) {
                        const int d = 32 * cc + 8 * g;
                        kk[hb][cc] = rload16(rkv, d < Dqk ? (t * Dqk + d) * 2 : kOutOfRange);
                    }
                }
                // the first value block's loads go out before the score MFMAs
                uint32_t wv0[8][4];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int t = t0 + 16 * (k >> 2) + 4 * g + (k & 3);
                    const uint4 v = rload16(rkv, 8 * r16 < Dv ? (t * Dqk + 8 * r16) * 2 : kOutOfRange);
                    wv0[k][0] = v.x; wv0[k][1] = v.y; wv0[k][2] = v.z; wv0[k][3] = v.w;
                }
                // each Q chunk is read from LDS once and feeds both halves' chains
#pragma unroll
                for (int cc = 0; cc < KC; ++cc) {
                    const uint4 qq = *reinterpret_cast<const uint4 *>(qs + r16 * kQStride + 32 * cc + 8 * g);
                    sacc[0] = mfma16(kk[0][cc], qq, sacc[0]);
                    sacc[1] = mfma16(kk[1][cc], qq, sacc[1]);
                }
                float sv[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int t = t0 + 16 * (k >> 2) + 4 * g + (k & 3);
                    sv[k] = t < L ? sacc[k >> 2][k & 3] * a.scale : -INFINITY;
                }
                float bm = sv[0];
#pragma unroll
                for (int k = 1; k < 8; ++k) bm = fmaxf(bm, sv[k]);
                bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
                bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
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
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t h0b = to_bf16_rne(pv[2 * q]), h1b = to_bf16_rne(pv[2 * q + 1]);
                    const uint32_t l0b = to_bf16_rne(pv[2 * q] - __uint_as_float(h0b << 16));
                    const uint32_t l1b = to_bf16_rne(pv[2 * q + 1] - __uint_as_float(h1b << 16));
                    hi[q] = h0b | (h1b << 16);
                    lo[q] = l0b | (l1b << 16);
                }
                const uint4 phi = make_uint4(hi[0], hi[1], hi[2], hi[3]);
                const uint4 plo = make_uint4(lo[0], lo[1], lo[2], lo[3]);
#pragma unroll
                for (int vb = 0; vb < VB; ++vb)
#pragma unroll
                    for (int j = 0; j < 8; ++j) o[vb][j] *= alpha;
                // values: lane loads its group's 8 tokens x 8 dims (128 vb + 8 r16 ..);
                // block vb + 1's loads go out before block vb's MFMAs
                uint32_t wcur[8][4];
#pragma unroll
                for (int k = 0; k < 8; ++k)
#pragma unroll
                    for (int e = 0; e < 4; ++e) wcur[k][e] = wv0[k][e];
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) {
                    uint32_t wnext[8][4];
                    if (vb + 1 < VB) {
                        const int dn = 128 * (vb + 1) + 8 * r16;
#pragma unroll
                        for (int k = 0; k < 8; ++k) {
                            const int t = t0 + 16 * (k >> 2) + 4 * g + (k & 3);
                            const uint4 v = rload16(rkv, dn < Dv ? (t * Dqk + dn) * 2 : kOutOfRange);
                            wnext[k][0] = v.x; wnext[k][1] = v.y; wnext[k][2] = v.z; wnext[k][3] = v.w;
                        }
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
                        o[vb][j] = mfma16(av, phi, o[vb][j]);
                        o[vb][j] = mfma16(av, plo, o[vb][j]);
                    }
                    if (vb + 1 < VB) {
#pragma unroll
                        for (int k = 0; k < 8; ++k)
#pragma unroll
                            for (int e = 0; e < 4; ++e) wcur[k][e] = wnext[k][e];
                    }
                }
            }

            // merge the chunk's waves in wave order (the chunk holds token c * chunk < L)
            float lw = l_part;
            lw += __shfl_xor(lw, 16, 64);
            lw += __shfl_xor(lw, 32, 64);
            if (g == 0) {
                mred[w][r16] = m_run;
                lred[w][r16] = lw;
            }
            __syncthreads();
            float M = mred[0][r16];
#pragma unroll
            for (int v = 1; v < kNW; ++v) M = fmaxf(M, mred[v][r16]);
            const float f = __builtin_amdgcn_exp2f((m_run - M) * kLog2e);
            if (tid < 16) {
                float lt = __builtin_amdgcn_exp2f((mred[0][tid] - M) * kLog2e) * lred[0][tid];
#pragma unroll
                for (int v = 1; v < kNW; ++v)
                    lt = __builtin_fmaf(__builtin_amdgcn_exp2f((mred[v][tid] - M) * kLog2e), lred[v][tid], lt);
                mch[tid] = M;
                lch[tid] = lt;
            }
            for (int v = 0; v < kNW; ++v) {
                if (w == v) {
#pragma unroll
                    for (int vb = 0; vb < VB; ++vb)
#pragma unroll
                        for (int j = 0; j < 8; ++j)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                float &dst = ob[128 * vb + 8 * (4 * g + i) + j][r16];
                                dst = v == 0 ? f * o[vb][j][i] : __builtin_fmaf(f, o[vb][j][i], dst);
                            }
                }
                __syncthreads();
            }
            if (a.ws) {
                // this chunk's partial: m[16], l[16], O[Dv][16]
                float *pw = a.ws + (((int64_t)b * HG + hg) * ncu + c) * (32 + 16 * (int64_t)Dv);
                if (tid < 16) {
                    pw[tid] = mch[tid];
                    pw[16 + tid] = lch[tid];
                }
                for (int i = tid; i < 16 * Dv; i += kNW * 64) pw[32 + i] = ob[i >> 4][i & 15];
            } else {
                if (tid < 16) {
                    float Mh = Mr[tid], Lh = Lr[tid], fa, fb;
                    fold_head(c, mch[tid], lch[tid], Mh, Lh, fa, fb);
                    Mr[tid] = Mh; Lr[tid] = Lh; fah[tid] = fa; fbh[tid] = fb;
                }
                __syncthreads();
                for (int i = tid; i < 16 * Dv; i += kNW * 64) {
                    const int d = i >> 4, h = i & 15;
                    os[d][h] = fold_elem(c, ob[d][h], os[d][h], fah[h], fbh[h]);
                }
                __syncthreads();
            }
        }
        if (a.ws) continue;
        // out[b][h0 + h][8c .. 8c + 7]
        uint16_t *ob_out = static_cast<uint16_t *>(a.out) + ((int64_t)b * H + h0) * Dv;
        for (int i = tid; i < 16 * (Dv >> 3); i += kNW * 64) {
            const int h = i / (Dv >> 3), cq = i % (Dv >> 3);
            if (h0 + h >= H) continue;
            uint32_t r[4] = {0u, 0u, 0u, 0u};
            if (L > 0) {
                const float l = Lr[h];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    r[q] = to_bf16_rne(os[8 * cq + 2 * q][h] / l) | (to_bf16_rne(os[8 * cq + 2 * q + 1][h] / l) << 16);
            }
            *reinterpret_cast<uint4 *>(ob_out + (int64_t)h * Dv + 8 * cq) = make_uint4(r[0], r[1], r[2], r[3]);
        }
    }
}

// The fold of the chunk partials, one thread per output element (request,
// head group, dim, head): it folds chunks 0, 1, ... of its head in order,
// recomputing the head's scalars by the same operations.
__global__ __launch_bounds__(256) void mla_fold_kernel(MlaArgs a) {
    const int Dv = a.Dv, H = a.H, HG = (H + 15) >> 4;
    const int64_t per = 16 * (int64_t)Dv;
    const int64_t total = (int64_t)a.B * HG * per;
    const int64_t pstride = 32 + per;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
        const int64_t u = idx / per;
        const int i = (int)(idx - u * per);
        const int d = i >> 4, h = i & 15;
        const int b = (int)(u / HG), h0 = (int)(u % HG) * 16;
        if (h0 + h >= H) continue;
        int L = a.lens[b];
        L = L < 0 ? 0 : (L > a.Lmax ? a.Lmax : L);
        const int nc = (L + kMlaChunk - 1) / kMlaChunk;
        const float *pw = a.ws + u * a.nchunk * pstride;
        float M = 0.f, Ls = 0.f, Os = 0.f, fa, fb;
        for (int c = 0; c < nc; ++c) {
            const float *pc = pw + c * pstride;
            fold_head(c, pc[h], pc[16 + h], M, Ls, fa, fb);
            Os = fold_elem(c, pc[32 + i], Os, fa, fb);
        }
        static_cast<uint16_t *>(a.out)[((int64_t)b * H + h0 + h) * Dv + d] = (uint16_t)(nc > 0 ? to_bf16_rne(Os / Ls) : 0u);
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
            case 1: hipLaunchKernelGGL((mla_mfma_kernel<18, 4>), dim3(grid), dim3(kNW * 64), 0, st, a); break;
            case 2: hipLaunchKernelGGL((mla_mfma_kernel<4, 1>), dim3(grid), dim3(kNW * 64), 0, st, a); break;
            default: hipLaunchKernelGGL((mla_mfma_kernel<2, 1>), dim3(grid), dim3(kNW * 64), 0, st, a); break;
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
