// Batch-invariant decode attention over a latent (MLA-absorbed) KV cache.
// The vLLM batch-invariance tracking issue lists the MLA attention backends
// among the operators batch-invariant mode must cover, and the vLLM-Ascend
// guide requires deterministic attention kernels.  For request b (L_b cached
// tokens) and head h the kernel computes, in this order:
//   s_t = (fp32 fma chain from 0 over d ascending of q[d] * kv_t[d]) * scale,
//         one thread per token;
//   m   = max over t of s_t (order-free);
//   p_t = exp2((s_t - m) * log2(e)), the hardware exp2;
//   l   = sum of p_t: thread i sums tokens i, i+256, ... ascending, then a
//         64-lane xor butterfly, then the four wave partials in wave order;
//   o[c] = bf16_rne(u[c] / l) with u[c] = ((u0 + u1) + u2) + u3, where wave
//         w's u_w[c] is the fp32 fma chain over tokens t = w, w+4, w+8, ...
//         ascending of p_t * v_t[c] and v_t is the first Dv components of kv_t.
// One workgroup computes one (b, h) over all of the request's tokens: there
// is no KV split, so every step above depends only on L_b, Dqk and Dv --
// never on the other requests, the batch size, the grid or the launch.

#include "bi_internal.h"

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
__global__ __launch_bounds__(kNT) void mla_decode_kernel(MlaArgs a) {
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

}  // namespace

int mla_token_capacity(int Lmax) { return Lmax <= 4096 ? 4096 : (Lmax <= kMlaMaxTokens ? kMlaMaxTokens : 0); }

hipError_t launch_mla_decode(const MlaArgs &a, int grid, hipStream_t st) {
    if (grid < 1 || a.Dqk <= 0 || a.Dqk % 8 || a.Dqk > kMlaMaxDqk || a.Dv <= 0 || a.Dv % 8 ||
        a.Dv > a.Dqk || a.Dv > kMlaMaxDv || a.Lmax < 0)
        return hipErrorInvalidValue;
    switch (mla_token_capacity(a.Lmax)) {
        case 4096: hipLaunchKernelGGL(mla_decode_kernel<4096>, dim3(grid), dim3(kNT), 0, st, a); break;
        case kMlaMaxTokens:
            hipLaunchKernelGGL(mla_decode_kernel<kMlaMaxTokens>, dim3(grid), dim3(kNT), 0, st, a);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace bi
