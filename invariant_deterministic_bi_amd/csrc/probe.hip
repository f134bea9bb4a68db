// Measurement probes: the ceilings the hot path's kernels are judged
// against on the machine at hand, next to the published peaks.
//   * MFMA loop: every wavefront issues the hot path's instruction,
//     v_mfma_f32_16x16x32_bf16, back to back on eight independent
//     accumulators with operands already in registers -- no memory, no
//     LDS.  Each wavefront also records its shader-clock cycles (s_memtime)
//     and constant-rate 100 MHz ticks (s_memrealtime) over the loop, so the
//     clock the matrix cores actually ran at is measured, not assumed.
//   * Read stream: 16-byte loads over a caller buffer, every byte once,
//     folded into a per-thread XOR so no load can be dropped.
//   * LDS read stream: every wavefront reads a 64 KB LDS buffer with 16-byte
//     reads (ds_read_b128), consecutive lanes on consecutive 16-byte slots
//     (no bank conflict), recording its shader-clock cycles over the loop.
// Neither is part of the batch-invariant path; the library exports them so
// that a benchmark can report its kernels against measured ceilings.

#include "bi_internal.h"

namespace bi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeWaves = 8;  // wavefronts per workgroup (two per SIMD)

__global__ __launch_bounds__(kProbeWaves * 64, 1) void mfma_probe_kernel(uint64_t *out, int64_t iters) {
    const int lane = threadIdx.x & 63;
    // operands: small values from the lane number, so no product overflows
    u32x4 a, b;
    a.x = 0x3F803F80u + (uint32_t)(lane & 7);
    a.y = a.x ^ 1u; a.z = a.x ^ 2u; a.w = a.x ^ 3u;
    b.x = 0x3F003F00u + (uint32_t)(lane >> 3);
    b.y = b.x ^ 1u; b.z = b.x ^ 2u; b.w = b.x ^ 3u;
    const bf16x8 av = __builtin_bit_cast(bf16x8, a), bv = __builtin_bit_cast(bf16x8, b);
    f32x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[i], 0, 0, 0);
    }
    // the loop's last MFMA results are read before the second timestamp
    float sink = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) sink += acc[i].x + acc[i].y + acc[i].z + acc[i].w;
    asm volatile("" : "+v"(sink));
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) {
        uint64_t *o = out + ((int64_t)blockIdx.x * kProbeWaves + (threadIdx.x >> 6)) * 3;
        o[0] = t1 - t0;
        o[1] = r1 - r0;
        o[2] = (uint64_t)__float_as_uint(sink);
    }
}

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4 *src, int64_t n16, uint32_t *sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t x = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 v0 = __builtin_nontemporal_load(src + i);
        const u32x4 v1 = __builtin_nontemporal_load(src + i + stride);
        const u32x4 v2 = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 v3 = __builtin_nontemporal_load(src + i + 3 * stride);
        x ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
        x ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = x;
}

constexpr int kLdsProbeSlots = 4096;  // 16-byte slots: 64 KB
constexpr int kLdsProbeReads = 16;    // reads per wavefront per iteration

__global__ __launch_bounds__(kProbeWaves * 64, 1) void lds_probe_kernel(uint64_t *out, int64_t iters) {
    __shared__ u32x4 buf[kLdsProbeSlots];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < kLdsProbeSlots; i += kProbeWaves * 64)
        buf[i] = u32x4{(uint32_t)i, (uint32_t)i * 3u, 7u, 9u};
    __syncthreads();
    u32x4 x = {0u, 0u, 0u, 0u};
    // slot base + 256 r: base < 256, so every index is below 4096; the reads
    // of one instruction are 64 consecutive slots
    int base = (wave * 64 + lane) & 255;
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < kLdsProbeReads; ++r) x += buf[base + r * 256];
        base = (base + 64) & 255;
    }
    // the sum is used (so no read is dropped) before the second timestamp
    asm volatile("" ::"v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w));
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    if (lane == 0) {
        uint64_t *o = out + ((int64_t)blockIdx.x * kProbeWaves + wave) * 2;
        o[0] = t1 - t0;
        o[1] = (uint64_t)(x.x ^ x.y ^ x.z ^ x.w);
    }
}

}  // namespace

hipError_t launch_lds_probe(uint64_t *out, int64_t iters, int grid, hipStream_t s) {
    hipLaunchKernelGGL(lds_probe_kernel, dim3(grid), dim3(kProbeWaves * 64), 0, s, out, iters);
    return hipGetLastError();
}

hipError_t launch_mfma_probe(uint64_t *out, int64_t iters, int grid, hipStream_t s) {
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(grid), dim3(kProbeWaves * 64), 0, s, out, iters);
    return hipGetLastError();
}

hipError_t launch_read_probe(const void *src, int64_t bytes, uint32_t *sink, int grid, hipStream_t s) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(256), 0, s, static_cast<const u32x4 *>(src), bytes / 16,
                       sink);
    return hipGetLastError();
}

}  // namespace bi
