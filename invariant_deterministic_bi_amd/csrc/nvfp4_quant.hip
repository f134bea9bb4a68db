// Row-local NVFP4 quantiser for gfx950: bf16 activations -> FP4 E2M1 codes
// plus one FP8 E4M3 scale per 16 consecutive elements of a row, given a
// per-tensor global scale g.  This is the scaled_fp4_quant(x, global_scale)
// step of the W4A4 path in the vLLM PR #39912 unit test (summary page,
// section "key source snippets"); the pages name it without a definition,
// and the reading implemented here is, per 16-element block:
//   amax = max |x|;  v = min(fp32(fp32(amax * g) / 6), 448);
//   scale code = nearest E4M3 to v (ties to the even code), s = its value;
//   s == 0: every code 0; else r = fp32(g / s) and for each element
//   code = nearest E2M1 magnitude to fp32(|x| * r) (ties to the even code,
//   saturating at 6), sign bit for a negative x with a non-zero code.
// Every floating-point step is one IEEE fp32 operation with round to
// nearest even (division included: no fast-math), so the codes are a
// function of the row and g alone -- the row-local property that makes a
// row quantised alone equal to the same row quantised inside a batch, as
// long as g is fixed by the caller rather than recomputed per batch.
//
// Work split: a thread owns 8 elements (half a block) at a time; lanes 2i
// and 2i+1 hold one block and exchange their partial amax with one shuffle.
// Per half-block slot a wavefront reads 1 KB of contiguous bf16 and writes
// 256 contiguous code bytes and 32 scale bytes.

#include "bi_internal.h"

namespace bi {
namespace {

// Nearest E4M3 (fn) code to v, 0 <= v <= 448, ties to the even code.
__device__ __forceinline__ uint32_t e4m3_nearest(float v) {
    if (v < 0x1p-6f) return (uint32_t)__builtin_rintf(v * 512.0f);  // m * 2^-9, m = 0..8
    uint32_t b = __float_as_uint(v);
    b += 0x7FFFFu + ((b >> 20) & 1u);  // keep 3 mantissa bits, round half to even
    return (b >> 20) - (120u << 3);     // rebias the exponent: 127 -> 7
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
    const uint32_t e = c >> 3, m = c & 7u;
    return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
}

// One half block: 8 bf16 values in v, partner lane holds the other 8 of the
// block.  Returns the 8 codes packed as nibbles and the block's scale code.
__device__ __forceinline__ uint32_t quant_half(const uint4 &v, float g, uint32_t *scale) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t mx = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) mx = max(mx, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 1, 64));
    const float amax = __uint_as_float(mx << 16);
    const float u = amax * g;
    const float vs = fminf(u / 6.0f, 448.0f);
    const uint32_t sc = e4m3_nearest(vs);
    uint32_t codes = 0;
    if (sc != 0) {
        const float r = g / e4m3_decode(sc);
        // Signed products x * r (|x * r| == |x| * r exactly) to E2M1 by the
        // gfx950 converter with a unit scale: nearest, ties to the even code,
        // saturating at 6; byte j receives elements 2j (low nibble) and 2j+1.
        codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, bf16_lo(w[0]) * r, bf16_hi(w[0]) * r, 1.0f, 0);
        codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, bf16_lo(w[1]) * r, bf16_hi(w[1]) * r, 1.0f, 1);
        codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, bf16_lo(w[2]) * r, bf16_hi(w[2]) * r, 1.0f, 2);
        codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, bf16_lo(w[3]) * r, bf16_hi(w[3]) * r, 1.0f, 3);
        // a negative value whose magnitude rounds to 0 gets code 0, not 8 (-0)
        const uint32_t mag = codes & 0x77777777u;
        const uint32_t nz = (mag | (mag >> 1) | (mag >> 2)) & 0x11111111u;
        codes = mag | (codes & (nz << 3));
    }
    *scale = sc;
    return codes;
}

// Row of half block idx: idx / halves_per_row as (idx * magic) >> shift, with
// magic = ceil(2^shift / halves_per_row) and shift = 32 + ceil(log2
// halves_per_row), exact for every idx < 2^32 (the round-up method of
// Granlund and Montgomery); the host computes both.
//
// Each thread takes kU half blocks, kT apart (kT = the grid's thread count),
// and issues their loads before any arithmetic, so a wavefront keeps 4 KB of
// reads in flight.  idx and idx ^ 1 are both below halves or both not
// (halves, kT and the loop step are even), so a lane's shuffle partner is
// always active when it is.
constexpr int kU = 4;

__global__ __launch_bounds__(256) void nvfp4_quant_kernel(QuantArgs p) {
    const int halves_per_row = p.K >> 3;
    const int T = gridDim.x * 256;
    for (int base = blockIdx.x * 256 + threadIdx.x; base < p.halves; base += kU * T) {
        uint4 v[kU];
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            const int idx = base + i * T;
            v[i] = make_uint4(0, 0, 0, 0);
            if (idx < p.halves) {
                const int row = (int)(((uint64_t)idx * p.magic) >> p.shift), h = idx - row * halves_per_row;
                v[i] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.X) +
                                                       (int64_t)row * p.ldx + h * 8);
            }
        }
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            const int idx = base + i * T;
            if (idx < p.halves) {
                uint32_t sc;
                const uint32_t codes = quant_half(v[i], p.g, &sc);
                const int row = (int)(((uint64_t)idx * p.magic) >> p.shift), h = idx - row * halves_per_row;
                uint8_t *q = static_cast<uint8_t *>(p.Q) + (int64_t)row * (p.ldq >> 1) + h * 4;
                *reinterpret_cast<uint32_t *>(q) = codes;
                if ((h & 1) == 0)
                    static_cast<uint8_t *>(p.S)[(int64_t)row * (p.ldq >> 4) + (h >> 1)] = (uint8_t)sc;
            }
        }
    }
}

}  // namespace

hipError_t launch_nvfp4_quant(const QuantArgs &a, int grid, hipStream_t s) {
    if (grid < 1 || (a.halves & 1) || (a.K & 15)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(nvfp4_quant_kernel, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace bi
