// Internal interface between the C-ABI layer (api.cpp) and the kernel
// translation units (gemm.hip, rmsnorm.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi {

// Operand storage modes of the GEMM mainloop.
enum OperandMode : int {
    OPND_BF16_ROWS = 0,  // bf16 [rows, K], K contiguous (GEMM A and B, BMM A)
    OPND_BF16_KN = 1,    // bf16 [K, cols], cols contiguous (BMM B)
    OPND_NVFP4_ROWS = 2, // e2m1 codes [rows, K/2] + e4m3 scales [rows, K/16], via registers
    OPND_NVFP4_RAW = 3   // the same bytes, LDS-DMA into a raw ring, decoded in LDS (K % 64 == 0)
};

// Compiled tile shapes of the GEMM mainloop.  A tile is bm x bn outputs,
// computed by wgm x wgn wavefronts (each owning a (bm/wgm) x (bn/wgn) block).
// K is staged through LDS 64 columns at a time, in a ring of `sa` buffers for
// A and `sb` buffers for B (sb >= sa >= 2): a deep B ring keeps enough of the
// weight in flight per compute unit to stream it at small M.  The shape
// changes which lanes and workgroups compute which outputs, never the
// arithmetic of one output.
struct TileShape {
    int bm, bn, wgm, wgn, sa, sb;
};

constexpr TileShape kTileShapes[] = {
    {256, 256, 4, 2, 2, 2},   // 0
    {256, 128, 2, 2, 2, 4},   // 1
    {256, 128, 4, 2, 2, 4},   // 2
    {128, 128, 2, 2, 3, 4},   // 3
    {256, 64, 4, 1, 2, 8},    // 4
    {128, 64, 2, 2, 3, 8},    // 5
    {64, 64, 2, 2, 4, 8},     // 6
    {256, 32, 4, 1, 2, 16},   // 7
    {128, 32, 4, 1, 3, 16},   // 8
    {256, 128, 4, 2, 3, 4},   // 9
    {128, 128, 2, 2, 4, 4},   // 10
    {128, 128, 4, 2, 4, 4},   // 11
    {256, 256, 4, 2, 2, 3},   // 12
    {256, 256, 2, 4, 2, 3},   // 13: ping-pong schedule (bf16 x bf16, batch 1; else as 12)
    {128, 128, 2, 2, 2, 2},   // 14: 64 KB of LDS, two workgroups per compute unit
    {128, 128, 4, 2, 2, 2},   // 15: the same with eight wavefronts
    {256, 192, 4, 2, 2, 3},   // 16: 256 x 192, classic schedule
    {256, 192, 2, 4, 2, 3},   // 17: 256 x 192, ping-pong schedule (bf16 x bf16, batch 1; else as 16)
    {256, 128, 2, 4, 2, 3},   // 18: 256 x 128, ping-pong schedule (bf16 x bf16, batch 1; else as 9)
};
constexpr int kPingPongVariant = 13;
constexpr int kPingPong192Variant = 17;
constexpr int kPingPong128Variant = 18;
constexpr int kNumTileShapes = sizeof(kTileShapes) / sizeof(kTileShapes[0]);

// LDS bytes of one workgroup: the two rings, or the padded bf16 output tile
// of the epilogue if that is larger.
constexpr int tile_lds_bytes(const TileShape &t) {
    const int pipe = (t.sa * t.bm + t.sb * t.bn) * 64 * 2;
    const int ctile = t.bm * (t.bn * 2 + 16);
    return pipe > ctile ? pipe : ctile;
}
constexpr int kLdsPerCu = 160 * 1024;

// Tile recipe selected from (op, N, K).
struct GemmRecipe {
    int variant;  // index into kTileShapes
};

struct GemmArgs {
    const void *A;        // operand A base
    const void *A_scales; // NVFP4 A scales (mode OPND_NVFP4_ROWS)
    const void *B;
    const void *B_scales;
    void *Y;
    int64_t lda, sA;      // A row stride (elements), head stride (elements)
    int64_t ldb, sB;
    int64_t ldy, sY;
    int M, N, K, batch;
    int tiles_m, tiles_n;
    int num_tiles;
    float alpha;
    int use_alpha;
    // Grouped GEMM (mixture of experts): when set, head e is expert e, whose
    // rows are group_off[e] .. group_off[e+1]-1 of A and Y (device int64
    // [batch+1], clamped to [0, total_rows]); M is then total_rows, the bound
    // of any group, and B's head stride sB is the expert stride.
    const int64_t *group_off;
    int64_t total_rows;
};

// Launchers; they return hipSuccess or the launch error.
hipError_t launch_gemm(int a_mode, int b_mode, const GemmRecipe &r, const GemmArgs &args,
                       int grid, hipStream_t stream);
// Skinny path for 1 <= M <= ma <= 16 (ma = 4, 8 or 16 rows of A staged),
// bf16 A, weight OPND_BF16_ROWS or OPND_NVFP4_RAW, batch 1; one 64-thread
// workgroup per nb-column block (nb = 8 or 16).
hipError_t launch_skinny(int b_mode, int nb, int ma, const GemmArgs &args, int grid, hipStream_t stream);
int skinny_lds_bytes(int b_mode, int M, int nb);
// BMM with a short reduction (K = 64, 128 or 256), B [K, N]: one workgroup
// per (head, 128-column block) keeps the transposed B block in LDS and
// streams 64-row tiles of A; four wavefronts.  Same bits as every tiled
// variant.
bool bmm_short_k_ok(int K);
int bmm_short_k_lds_bytes(int K);
hipError_t launch_bmm_short_k(const GemmArgs &args, int grid, hipStream_t stream);
// 256 x 256 tiles, eight wavefronts in a ping-pong schedule; bf16 x bf16, batch 1.
hipError_t launch_pingpong(const GemmArgs &args, int bn, int grid, hipStream_t stream);
// The same schedule for bf16 A and a raw NVFP4 weight (K % 64 == 0), 256 x
// 256 tiles: one group decodes the raw B stages and hands the fragments to
// the other through LDS.
hipError_t launch_pingpong_nvfp4(const GemmArgs &args, int grid, hipStream_t stream);
// Direct path for 1 <= M <= 16 * rb, bf16 A and bf16 weight [N, K], batch 1:
// one 64-thread workgroup per 16-column item, fragments loaded into
// registers, each weight fragment feeding rb = 1, 2, 4 or 8 16-row blocks of
// A; ap = 1 (rb = 1, M <= 8): one load carries A rows 0-7 of two K chunks.
hipError_t launch_direct(const GemmArgs &args, int rb, int ap, int grid, int depth, hipStream_t stream);
// The same for a raw NVFP4 weight (codes [N, K/2], scales [N, K/16]), K % 128
// == 0, rb = 1, 2 or 4.
hipError_t launch_direct_nvfp4(const GemmArgs &args, int rb, int ap, int grid, int depth, hipStream_t stream);
// Direct path with A staged in LDS once per workgroup (bf16 or raw NVFP4
// weight), for shapes with direct_alds_ok; `waves` streaming wavefronts.
// afp4 (with fp4): A is NVFP4 rows (lda % 32 == 0), decoded into LDS.
bool direct_alds_ok(int M, int K, bool fp4);
// Direct path with A staged in LDS in K chunks (16 < M <= 64): rb = 2 or 4
// row blocks; bf16 A, bf16 or raw NVFP4 weight; `waves` wavefronts.  afp4
// (with fp4): A is NVFP4 rows (lda % 32 == 0), decoded into LDS chunk by
// chunk.
bool direct_achunk_ok(int M, int K, int rb, bool fp4);
hipError_t launch_direct_achunk(const GemmArgs &args, bool fp4, bool afp4, int rb, int waves, int cus, int depth,
                                hipStream_t stream);
hipError_t launch_direct_alds(const GemmArgs &args, bool fp4, bool afp4, int nb, int waves, int cus, int depth,
                              hipStream_t stream);

struct RmsArgs {
    const void *X;
    const void *gamma;
    void *Y;
    int64_t ldx, ldy;
    int M, H;
    float eps;
};

hipError_t launch_rmsnorm(int threads, int chunks_per_thread, const RmsArgs &args, int grid,
                          hipStream_t stream);

constexpr int kMaxPartials = 8;

struct ReduceRmsArgs {
    const void *P[kMaxPartials];  // np partial outputs, bf16 [M, H], row stride ldp
    int np;
    int64_t ldp;
    const void *res;              // residual bf16 [M, H] (row stride ldres) or NULL
    int64_t ldres;
    const void *gamma;
    void *R;                      // reduced rows, bf16 [M, H], row stride ldr
    void *Y;                      // RMSNorm(R), bf16 [M, H], row stride ldy
    int64_t ldr, ldy;
    int M, H;
    float eps;
};

// Same threads / chunks per thread as RMSNorm for H (the row normalisation
// is RMSNorm's own code).
hipError_t launch_reduce_rmsnorm(int threads, int chunks_per_thread, const ReduceRmsArgs &args,
                                 int grid, hipStream_t stream);

struct QuantArgs {
    const void *X;     // bf16 [M, K], row stride ldx elements
    void *Q;           // codes, row stride ldq / 2 bytes
    void *S;           // E4M3 scales, row stride ldq / 16 bytes
    int64_t ldx, ldq;
    int M, K;
    int halves;        // M * K / 8: one thread per 8 elements
    uint64_t magic;    // row of half block i = (i * magic) >> shift
    int shift;
    float g;           // global scale
};

// Row-local NVFP4 quantiser: 256-thread workgroups, a grid-stride loop over
// the 8-element half blocks.
hipError_t launch_nvfp4_quant(const QuantArgs &args, int grid, hipStream_t stream);

// Decode attention over a latent KV cache (one workgroup per request and
// head, no KV split).
constexpr int kMlaMaxTokens = 16384;  // the weights live in LDS
constexpr int kMlaMaxDqk = 1024;
constexpr int kMlaMaxDv = 1024;
constexpr int kMlaChunk = 1024;  // tokens per chunk of the MFMA kernel's fold
struct MlaArgs {
    const void *q;        // bf16 [B, H, Dqk]
    const void *kv;       // bf16 [B, Lmax, Dqk]
    const int32_t *lens;  // device int32 [B], clamped to [0, Lmax]
    void *out;            // bf16 [B, H, Dv]
    int B, H, Lmax, Dqk, Dv;
    float scale;
    float *ws;   // chunk partials (one workgroup per chunk), or null (one per request)
    int nchunk;  // chunks per (request, head group) in ws: ceil(Lmax / kMlaChunk)
};
int mla_token_capacity(int Lmax);     // VALU kernel's LDS capacity; 0 when Lmax is too large
int mla_mfma_variant(int Dqk, int Dv);  // 0: the VALU kernel serves (Dqk, Dv)
// Work units of the MFMA kernel: `keys` (requests, or request chunks) padded
// to a multiple of 8, times the head groups.
__host__ __device__ inline int64_t mla_mfma_units(int64_t keys, int head_groups) {
    return (keys + 7) / 8 * 8 * head_groups;
}
int64_t mla_workspace_bytes(int B, int H, int Lmax, int Dqk, int Dv);  // 0: no workspace used
// The library-held chunk-partial scratch of bi_mla_decode_noalloc: its size,
// and its device address on the current device (looked up once per device).
constexpr int64_t kMlaScratchBytes = (int64_t)32 << 20;
constexpr int kMaxDevices = 64;
hipError_t mla_scratch(float **out);
hipError_t launch_mla_decode(const MlaArgs &args, int grid, int fold_grid, hipStream_t stream);

// Measurement probes (probe.hip): an MFMA-only loop (eight wavefronts per
// workgroup; out: three uint64 per wavefront), a 16-byte read stream (256
// threads per workgroup; sink: one uint32 per thread) and an LDS read loop.
hipError_t launch_mfma_probe(uint64_t *out, int64_t iters, int grid, hipStream_t stream);
hipError_t launch_read_probe(const void *src, int64_t bytes, uint32_t *sink, int grid, hipStream_t stream);
// LDS read probe: eight wavefronts per workgroup, each issuing iters * 16
// conflict-free ds_read_b128; out: two uint64 per wavefront (cycles, sink).
hipError_t launch_lds_probe(uint64_t *out, int64_t iters, int grid, hipStream_t stream);

}  // namespace bi
