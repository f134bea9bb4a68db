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
// reduce_rmsnorm_kernel is that pair's share on one GPU: the partial outputs
// of a row-parallel layer summed in one fixed (rank) order, then the same
// row normalisation.

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

// Steps 1-4 for one row whose 8-element chunks c = tid + i*T are in v[i]
// (zero beyond the row); writes y.  wsum holds T/64 floats of LDS.
template <int T, int CPT>
__device__ __forceinline__ void rms_row(const uint4 (&v)[CPT], const uint16_t *gam, uint16_t *y, int chunks,
                                        int H, float eps, float *wsum) {
    constexpr int NW = T / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
    const float r = rsqrtf(tot / (float)H + eps);

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

template <int T, int CPT>
__global__ __launch_bounds__(T) void rmsnorm_kernel(RmsArgs p) {
    __shared__ float wsum[T / 64];
    const int tid = threadIdx.x;
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
        rms_row<T, CPT>(v, gam, y, chunks, p.H, p.eps, wsum);
    }
}

// Fixed-order reduction of partial rows, then the same row normalisation:
//   R = bf16_rne( ((t_0 + t_1) + t_2) + ... ) in fp32, where the terms are
//   the residual row (if any) followed by partials 0 .. np-1, each widened
//   exactly from bf16; the first term starts the sum;
//   Y = rms_row(R), the very instruction sequence bi_rmsnorm runs, so Y is
//   bitwise bi_rmsnorm(R).
// All loads of a chunk (at most kMaxPartials + 1) are issued before its adds.
template <int T, int CPT>
__global__ __launch_bounds__(T) void reduce_rmsnorm_kernel(ReduceRmsArgs p) {
    __shared__ float wsum[T / 64];
    const int tid = threadIdx.x;
    const int chunks = p.H >> 3;
    const uint16_t *gam = static_cast<const uint16_t *>(p.gamma);
    const bool has_res = p.res != nullptr;

    for (int row = blockIdx.x; row < p.M; row += gridDim.x) {
        uint16_t *rout = static_cast<uint16_t *>(p.R) + (int64_t)row * p.ldr;
        uint16_t *y = static_cast<uint16_t *>(p.Y) + (int64_t)row * p.ldy;
        uint4 v[CPT];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * T;
            v[i] = make_uint4(0, 0, 0, 0);
            if (c < chunks) {
                uint4 t0 = make_uint4(0, 0, 0, 0), t[kMaxPartials];
                if (has_res)
                    t0 = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.res) +
                                                          (int64_t)row * p.ldres + c * 8);
#pragma unroll
                for (int q = 0; q < kMaxPartials; ++q)
                    t[q] = q < p.np ? *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.P[q]) +
                                                                      (int64_t)row * p.ldp + c * 8)
                                    : make_uint4(0, 0, 0, 0);
                // the first term starts the sum: the residual, else partial 0
                const uint4 f = has_res ? t0 : t[0];
                const uint32_t w0[4] = {f.x, f.y, f.z, f.w};
                float acc[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[2 * j] = bf16_lo(w0[j]);
                    acc[2 * j + 1] = bf16_hi(w0[j]);
                }
#pragma unroll
                for (int q = 0; q < kMaxPartials; ++q)
                    if (q < p.np && (has_res || q > 0)) {
                        const uint32_t w[4] = {t[q].x, t[q].y, t[q].z, t[q].w};
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            acc[2 * j] = acc[2 * j] + bf16_lo(w[j]);
                            acc[2 * j + 1] = acc[2 * j + 1] + bf16_hi(w[j]);
                        }
                    }
                uint32_t o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = f32_to_bf16_rne(acc[2 * j]) | (f32_to_bf16_rne(acc[2 * j + 1]) << 16);
                v[i] = make_uint4(o[0], o[1], o[2], o[3]);
                *reinterpret_cast<uint4 *>(rout + c * 8) = v[i];
            }
        }
        rms_row<T, CPT>(v, gam, y, chunks, p.H, p.eps, wsum);
    }
}

template <int T, int CPT>
hipError_t launch_one(const RmsArgs &a, int grid, hipStream_t s) {
    hipLaunchKernelGGL((rmsnorm_kernel<T, CPT>), dim3(grid), dim3(T), 0, s, a);
    return hipGetLastError();
}

template <int T, int CPT>
hipError_t launch_one(const ReduceRmsArgs &a, int grid, hipStream_t s) {
    hipLaunchKernelGGL((reduce_rmsnorm_kernel<T, CPT>), dim3(grid), dim3(T), 0, s, a);
    return hipGetLastError();
}

template <class Args>
hipError_t launch_shape(int threads, int cpt, const Args &a, int grid, hipStream_t s) {
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

}  // namespace

hipError_t launch_rmsnorm(int threads, int cpt, const RmsArgs &a, int grid, hipStream_t s) {
    return launch_shape(threads, cpt, a, grid, s);
}

hipError_t launch_reduce_rmsnorm(int threads, int cpt, const ReduceRmsArgs &a, int grid, hipStream_t s) {
    if (a.np < 1 || a.np > kMaxPartials) return hipErrorInvalidValue;
    return launch_shape(threads, cpt, a, grid, s);
}

}  // namespace bi
