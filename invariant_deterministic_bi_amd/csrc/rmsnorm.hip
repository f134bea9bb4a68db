// Batch-invariant RMSNorm for gfx950: one row per workgroup iteration, a
// reduction order fixed by H alone.
//
// For a row of H bf16 values (H % 8 == 0, C = H/8 chunks of 8 elements):
//   1. thread t of T loads chunks c = t, t+T, t+2T, ... (at most CPT of them)
//      and accumulates s_t = fma(x, x, s_t) over those chunks in ascending c,
//      elements of a chunk in ascending order, from +0;
//   2. a 64-lane butterfly: s += shfl_xor(s, d) for d = 32, 16, 8, 4, 2, 1;
//      fp32 addition is commutative, so every lane ends with the same value;
//   3. wave partials are added in wave order: ((w0 + w1) + w2) + w3;
//   4. r = rsqrt(total / H + eps); y = bf16_rne((x * r) * gamma).
// T and CPT depend on H only; rows never share a reduction, and the grid size
// only decides which workgroup handles which row.  The row is held in
// registers between the reduction and the scaling, so Y may alias X.
//
// RMSNorm is the row reduction of the fused all-reduce + RMSNorm on the vLLM
// PR #51292 page (section "Purpose"); its reduction there runs in a
// run-to-run-varying order, which is exactly what this fixed tree rules out.

#include "bi_internal.h"

namespace bi {
namespace {

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int T, int CPT>
__global__ __launch_bounds__(T) void rmsnorm_kernel(RmsArgs p) {
    constexpr int NW = T / 64;
    __shared__ float wsum[NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int chunks = p.H >> 3;
    const uint16_t *gam = static_cast<const uint16_t *>(p.gamma);

    for (int row = blockIdx.x; row < p.M; row += gridDim.x) {
        const uint16_t *x = static_cast<const uint16_t *>(p.X) + (int64_t)row * p.ldx;
        uint16_t *y = static_cast<uint16_t *>(p.Y) + (int64_t)row * p.ldy;
        uint4 v[CPT];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * T;
            v[i] = c < chunks ? *reinterpret_cast<const uint4 *>(x + c * 8) : make_uint4(0, 0, 0, 0);
        }
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float a = bf16_lo(w[j]), b = bf16_hi(w[j]);
                s = __builtin_fmaf(a, a, s);
                s = __builtin_fmaf(b, b, s);
            }
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
        if (lane == 0) wsum[wave] = s;
        __syncthreads();
        float tot = wsum[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) tot += wsum[w];
        __syncthreads();  // wsum is rewritten by the next row
        const float r = rsqrtf(tot / (float)p.H + p.eps);

#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * T;
            if (c < chunks) {
                const uint4 g = *reinterpret_cast<const uint4 *>(gam + c * 8);
                const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
                const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
                uint32_t o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t lo = f32_to_bf16_rne((bf16_lo(w[j]) * r) * bf16_lo(gw[j]));
                    const uint32_t hi = f32_to_bf16_rne((bf16_hi(w[j]) * r) * bf16_hi(gw[j]));
                    o[j] = lo | (hi << 16);
                }
                *reinterpret_cast<uint4 *>(y + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }
}

template <int T, int CPT>
hipError_t launch_one(const RmsArgs &a, int grid, hipStream_t s) {
    hipLaunchKernelGGL((rmsnorm_kernel<T, CPT>), dim3(grid), dim3(T), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm(int threads, int cpt, const RmsArgs &a, int grid, hipStream_t s) {
    if (threads == 64) {
        switch (cpt) {
            case 1: return launch_one<64, 1>(a, grid, s);
            case 2: return launch_one<64, 2>(a, grid, s);
        }
    } else if (threads == 256) {
        switch (cpt) {
            case 1: return launch_one<256, 1>(a, grid, s);
            case 2: return launch_one<256, 2>(a, grid, s);
            case 4: return launch_one<256, 4>(a, grid, s);
            case 8: return launch_one<256, 8>(a, grid, s);
            case 16: return launch_one<256, 16>(a, grid, s);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace bi
