// C-ABI layer of libbi: argument validation, the (op, N, K) -> recipe table,
// the kernel regimes, persistent-grid sizing and kernel launch.
// Declarations and the contract are in include/bi.h.
//
// The per-element recipe -- the MFMA instruction, the K order, the
// accumulator and the epilogue -- is the same for every (op, N, K) and M.
// The kernel that runs it does depend on M: at small M a streaming kernel,
// else the tiled kernel with a tile shape from a cost model of M and N
// (classify() below; the ranges are listed by bi_plan_regimes, and
// bi_plan_query reports the large-M shape).  The vLLM PR #39912 summary page (section
// "implementation breakdown") pins one default config instead of M-bucketed
// ones, and the vLLM PR #51292 page's root-cause comment names size-gated
// selection as the failure mode; here every kernel a shape can take runs the
// identical per-element chain, and the bitwise tests walk every regime edge.

#include <atomic>
#include <cstdint>
#include <cstring>

#include <hip/hip_runtime.h>

#include "../../include/bi.h"
#include "bi_internal.h"

namespace {

using bi::GemmArgs;
using bi::GemmRecipe;

constexpr int64_t kI32Max = 2147483647;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Half-open byte range of a [rows, cols] matrix with row stride ld elements of
// esize bytes (esize_num/esize_den to allow half-byte NVFP4 codes).
struct Range {
    uintptr_t lo, hi;
};

Range mat_range(const void *p, int64_t rows, int64_t cols, int64_t ld, int64_t num, int64_t den) {
    Range r;
    r.lo = reinterpret_cast<uintptr_t>(p);
    const int64_t elems = rows > 0 ? (rows - 1) * ld + cols : 0;
    r.hi = r.lo + static_cast<uintptr_t>((elems * num + den - 1) / den);
    return r;
}

bool overlap(const Range &a, const Range &b) { return a.lo < b.hi && b.lo < a.hi && a.lo < a.hi && b.lo < b.hi; }

// Compute-unit count of the current device, cached per device ordinal.
std::atomic<int> g_cu_count[64];

bi_status device_cus(int *out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return BI_ERR_HIP;
    if (dev >= 0 && dev < 64) {
        const int c = g_cu_count[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *out = c;
            return BI_OK;
        }
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return BI_ERR_HIP;
    if (dev >= 0 && dev < 64) g_cu_count[dev].store(n, std::memory_order_relaxed);
    *out = n;
    return BI_OK;
}

// ---------------------------------------------------------------------------
// Tile shapes.  Every output element is computed the same way by every tile
// shape (16x16x32 bf16 MFMA, K ascending in chunks of 32, one lane's fp32
// accumulator); the shape only decides which workgroup computes which
// outputs, so it is chosen for speed alone.
// ---------------------------------------------------------------------------
constexpr int64_t kMaxLd = (int64_t)1 << 22;  // keeps 32-bit in-tile byte offsets

// Tile shape of the batched GEMM: 256 x 128, 8 wavefronts, at every M.
int fixed_variant(int /*op*/, int64_t /*N*/) { return 2; }

// Tile shape of the grouped GEMM from N and the average rows per expert
// (T / E, rounded up; the group sizes themselves are on the device).  Every
// expert adds a partial m-tile, and sizes spread around the average, so an
// m-tile just above the average would double the tiles: the bands sit below
// the multiples of bm.  MI355X, 8 experts of 4096 x 4096 (µs, this choice
// against the best forced tile): 64 rows 47 (47), 128 rows 57 (57), 256 rows
// 91 (91), 512 rows 171 (171), 1024 rows 316 (315).  Every tile shape gives
// the same bits, so each row is still bitwise bi_gemm's.
int grouped_variant(int64_t N, int64_t rows) {
    if (N < 512) return 6;               // 64 x 64
    if (N < 2048 || rows <= 96) return 11;  // 128 x 128, 8 wavefronts
    if (rows <= 192) return 9;           // 256 x 128, 8 wavefronts, 3-deep A ring
    if (rows <= 768) return 16;          // 256 x 192, classic schedule
    return 12;                           // 256 x 256, classic schedule
}

// Cost model of the dense and NVFP4 GEMMs' tiled kernel (batch 1).  A launch
// runs in rounds of one tile per compute unit (every candidate needs more
// than half of a compute unit's LDS, so one workgroup fits), and a round's
// time grows with the tile's operand bytes, not with the number of busy
// compute units: a compute unit streams its tile's A and B at about 45-50
// GB/s whatever the others do, until the tile is large enough to be
// MFMA-bound.  So a call's time is ceil(tiles / CUs) x (round cost) x K, and
// the shape with the least estimate runs (the larger one on a tie).  Round
// costs are MI355X measurements (microseconds per 4096 of K, every shape
// forced at M = 32 ... 8192 on N = 4096 ... 24576); each table lists the
// shapes that won somewhere in that sweep for its operand modes.
struct TileCost {
    int variant;  // index into bi::kTileShapes
    int cost;     // one round, microseconds per 4096 of K
};
constexpr TileCost kCostBf16[] = {{6, 24}, {5, 31}, {11, 45}, {2, 60}, {bi::kPingPong192Variant, 85},
                                  {bi::kPingPongVariant, 100}};
constexpr TileCost kCostNvfp4W[] = {{11, 50}, {2, 82}, {16, 102}, {bi::kPingPongVariant, 113}};
constexpr TileCost kCostW4A4[] = {{10, 64}, {2, 92}, {16, 120}, {12, 128}};
// Above this many rows every shape runs several rounds, and the choice is
// the shape with the least cost per output row, cost x ceil(N / bn) / bm
// (the estimate's limit for large M without the round-up), so that the
// choice stops changing with M.
constexpr int64_t kModelRows = 4096;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

const TileCost *cost_table(int a_mode, int b_mode, int *n) {
    if (a_mode == bi::OPND_NVFP4_ROWS) {
        *n = sizeof kCostW4A4 / sizeof kCostW4A4[0];
        return kCostW4A4;
    }
    if (b_mode == bi::OPND_NVFP4_RAW || b_mode == bi::OPND_NVFP4_ROWS) {
        *n = sizeof kCostNvfp4W / sizeof kCostNvfp4W[0];
        return kCostNvfp4W;
    }
    *n = sizeof kCostBf16 / sizeof kCostBf16[0];
    return kCostBf16;
}

// The tile shape of a dense or NVFP4 GEMM with M rows (M > kModelRows: the
// large-M limit), and its estimate in microseconds per 4096 of K (0 for the
// limit).
int model_variant(int a_mode, int b_mode, int64_t N, int cus, int64_t M, int64_t *est) {
    int n = 0;
    const TileCost *tab = cost_table(a_mode, b_mode, &n);
    int best = -1;
    int64_t be = 0;
    double bl = 0.0;
    for (int i = 0; i < n; ++i) {
        const bi::TileShape &t = bi::kTileShapes[tab[i].variant];
        const int64_t tn = ceil_div(N, t.bn);
        if (M <= kModelRows) {
            const int64_t e = ceil_div(ceil_div(M, t.bm) * tn, cus) * tab[i].cost;
            if (best < 0 || e <= be) {
                best = tab[i].variant;
                be = e;
            }
        } else {
            const double l = static_cast<double>(tab[i].cost) * static_cast<double>(tn) / t.bm;
            if (best < 0 || l <= bl) {
                best = tab[i].variant;
                bl = l;
            }
        }
    }
    *est = M <= kModelRows ? be : 0;
    return best;
}

// The per-(N, K) plan bi_plan_query reports: the shape every call with more
// than kModelRows rows runs (the large-M limit does not depend on the number
// of compute units).
int plan_variant(int op, int64_t N, int64_t K) {
    if (op == BI_OP_GROUPED_GEMM) return grouped_variant(N, kModelRows + 1);
    if (op != BI_OP_GEMM && op != BI_OP_NVFP4_GEMM) return fixed_variant(op, N);
    const int b_mode = op == BI_OP_GEMM ? bi::OPND_BF16_ROWS
                                        : (K % 64 == 0 ? bi::OPND_NVFP4_RAW : bi::OPND_NVFP4_ROWS);
    int64_t est = 0;
    return model_variant(bi::OPND_BF16_ROWS, b_mode, N, 1, kModelRows + 1, &est);
}

// The ping-pong kernels serve their tile shapes for bf16 A with a bf16 weight
// (256, 192 or 128 columns) or a raw NVFP4 weight (256 columns), batch 1;
// other operand modes run the classic schedule of the same shape (same bits).
bool pingpong_ok(int variant, int a_mode, int b_mode, int batch, bool grouped) {
    if (a_mode != bi::OPND_BF16_ROWS || batch != 1 || grouped) return false;
    if (b_mode == bi::OPND_BF16_ROWS)
        return variant == bi::kPingPongVariant || variant == bi::kPingPong192Variant ||
               variant == bi::kPingPong128Variant;
    return b_mode == bi::OPND_NVFP4_RAW && variant == bi::kPingPongVariant;
}

void fill_tile_plan(int op, int variant, bi_plan *out) {
    const bi::TileShape &t = bi::kTileShapes[variant];
    std::memset(out, 0, sizeof *out);
    out->op = op;
    out->bm = t.bm;
    out->bn = t.bn;
    out->bk = 64;
    out->mfma_m = 16;
    out->mfma_n = 16;
    out->mfma_k = 32;
    out->waves = t.wgm * t.wgn;
    out->lds_stages = t.sb;
    out->threads = 64 * t.wgm * t.wgn;
    out->chunks_per_thread = 0;
}

// RMSNorm: T threads per row, CPT 16-byte chunks per thread, from H alone.
bool rms_shape(int64_t H, int *T, int *cpt) {
    if (H <= 0 || H % 8 != 0 || H > 32768) return false;
    const int64_t chunks = H / 8;
    *T = chunks <= 128 ? 64 : 256;
    const int64_t need = (chunks + *T - 1) / *T;
    int c = 1;
    while (c < need) c *= 2;
    *cpt = c;
    return true;
}

int default_grid(int tiles, int cus, const bi_launch_opts *opts, int per_cu) {
    int cap = cus * per_cu;
    if (opts && opts->max_workgroups > 0) cap = opts->max_workgroups;
    return tiles < cap ? tiles : cap;
}

// ---------------------------------------------------------------------------
// Kernel regimes of the GEMM family.  Every kernel below runs the same
// per-element chain -- one 16x16x32 bf16 MFMA per 32-wide K chunk, K
// ascending from +0, one fp32 accumulator per output owned by one lane for
// the whole K range, (alpha x) then bf16 RNE -- so each gives the same bits.
// Which one runs is chosen on the host from the row count M as well as
// (op, N, K):
//   * M <= 16: a streaming kernel spreads 8- or 16-column items of the
//     weight over every compute unit, which no tile can do at so few rows;
//   * 16 < M <= 128: the register-streaming kernel when its estimate beats
//     the tiled kernel's (narrow weights, whose tiles cannot fill the chip);
//   * else the tiled kernel, its tile shape from the cost model above.
// This departs from a single tile per (N, K); it is kept safe by that
// identical chain and by bitwise tests at every regime edge of every
// configured (N, K).  classify() is the whole rule: run_gemm dispatches on it
// and bi_plan_regimes() enumerates it.
// ---------------------------------------------------------------------------
struct Regime {
    int kind;   // bi_kernel_kind
    int rb;     // 16-row MFMA blocks of A per weight fragment (tiled: bm / 16)
    int ap;     // one load carries A rows 0-7 of two K chunks (M <= 8)
    int ma;     // rows of A staged by the LDS-ring kernel (4, 8 or 16)
    int cols;   // output columns per item (tiled: bn)
    int variant;  // tiled: index into kTileShapes
    bool operator==(const Regime &o) const {
        return kind == o.kind && rb == o.rb && ap == o.ap && ma == o.ma && cols == o.cols && variant == o.variant;
    }
};

// Register-streaming kernel (16 < M <= 128): one wavefront per 16-column
// item, up to 16 per compute unit; each item streams its weight columns once
// and re-reads A (rb 16-row blocks) from L2, so a round of one item per
// compute unit costs about 6 + 3.7 rb microseconds per 4096 of K (MI355X,
// bf16 and NVFP4 weights alike).  In hundredths of a microsecond:
int64_t stream_round_cost(int rb) { return 600 + 368 * rb; }

// The chunked-A kernel (A staged in LDS 2048 / rb columns at a time, one
// 16-column item per wavefront, up to eight per compute unit): with w items
// per compute unit (w > 1) a call costs about a + b w microseconds per 4096
// of K (MI355X, N = 6144 ... 24576, M = 17 ... 128).  A bf16 weight is bound
// by the stream (b large); an NVFP4 one by its decode, which two items share
// a SIMD for only above four per compute unit.  Eight row blocks (M > 64)
// re-read 128 rows of A from LDS per weight fragment: they beat the tile
// only for an NVFP4 weight with at least four items per compute unit.  In
// hundredths of a microsecond (kNever: not a candidate):
constexpr int64_t kNever = INT64_MAX / 4;
int64_t achunk_cost(bool fp4, int rb, int64_t items, int cus) {
    const int64_t w100 = items * 100 / cus;  // items per compute unit, x 100
    if (fp4) {
        if (rb == 8) return items >= 4 * static_cast<int64_t>(cus) ? 4000 + 120 * w100 / 100 : kNever;
        return (rb == 2 ? 1350 : 1900) + (rb == 2 ? 125 : 130) * w100 / 100;
    }
    if (rb == 8) return kNever;
    return (rb == 2 ? 1220 : 1660) + (rb == 2 ? 470 : 430) * w100 / 100;
}
// With an NVFP4 A, whose rows each workgroup (of at least four wavefronts)
// decodes into LDS as well (N = 1000 ... 24576, K = 4096 and 12288):
int64_t achunk_cost_w4a4(int rb, int64_t items, int cus) {
    const int64_t w100 = items * 100 / cus;
    if (rb == 8) return 4200 + 150 * w100 / 100;
    return rb == 2 ? 1600 + 110 * w100 / 100 : 2350 + 150 * w100 / 100;
}

Regime classify(int op, int a_mode, int b_mode, int64_t N, int64_t K, int batch, bool grouped, int cus,
                int64_t M) {
    const bool fp4 = b_mode == bi::OPND_NVFP4_RAW;
    const bool stream_modes = a_mode == bi::OPND_BF16_ROWS && (b_mode == bi::OPND_BF16_ROWS || fp4);
    const bool dense = (op == BI_OP_GEMM || op == BI_OP_NVFP4_GEMM) && batch == 1 && !grouped;
    if ((op == BI_OP_GEMM || op == BI_OP_NVFP4_GEMM) && M <= 16 && stream_modes) {
        // A in LDS when its copy into every compute unit (M * K * 2 bytes
        // each) is at most 0.7 times the weight bytes that unit streams; else
        // A is loaded along with the weight fragments.  8-column items when
        // 16-column ones would leave fewer than two per compute unit.
        if (bi::direct_alds_ok(static_cast<int>(M), static_cast<int>(K), fp4) && (fp4 || 10 * M * cus <= 7 * N)) {
            const int nb = (!fp4 && (N + 15) / 16 < 2 * static_cast<int64_t>(cus)) ? 8 : 16;
            return {BI_KERNEL_STREAM_A_LDS, 1, 0, 0, nb, -1};
        }
        if (b_mode == bi::OPND_BF16_ROWS) return {BI_KERNEL_STREAM_REG, 1, M <= 8 ? 1 : 0, 0, 16, -1};
        if (K % 128 == 0 && M <= 8) return {BI_KERNEL_STREAM_REG, 1, 1, 0, 16, -1};
        const int nb = (N + 15) / 16 >= 2 * static_cast<int64_t>(cus) ? 16 : 8;
        return {BI_KERNEL_STREAM_RING, 1, 0, M <= 4 ? 4 : M <= 8 ? 8 : 16, nb, -1};
    }
    // NVFP4 A and weight, M <= 16: the same A-in-LDS streaming kernel, A rows
    // decoded exactly to bf16 into LDS as they are copied
    if (op == BI_OP_NVFP4_GEMM && M <= 16 && a_mode == bi::OPND_NVFP4_ROWS &&
        bi::direct_alds_ok(static_cast<int>(M), static_cast<int>(K), true))
        return {BI_KERNEL_STREAM_A_LDS, 1, 0, 0, 16, -1};
    // BMM with a short reduction: the streaming BMM kernel for every M (its
    // own recipe, chosen from K alone)
    if (op == BI_OP_BMM && bi::bmm_short_k_ok(static_cast<int>(K))) return {BI_KERNEL_BMM_STREAM, 4, 0, 0, 128, -1};
    if (!dense) {
        // grouped: M is the average rows per expert
        const int v = grouped ? grouped_variant(N, M) : fixed_variant(op, N);
        return {BI_KERNEL_TILED, bi::kTileShapes[v].bm / 16, 0, 0, bi::kTileShapes[v].bn, v};
    }
    int64_t est = 0;
    const int v = model_variant(a_mode, b_mode, N, cus, M, &est);
    // bf16 A with 16 < M <= 128 and a bf16 weight, or 16 < M <= 64 and a raw
    // NVFP4 one (K % 128 == 0): the register-streaming kernel with two, four
    // or eight 16-row blocks (one weight fragment feeds each block's chain);
    // with M <= 128 (either weight) and more 16-column items than compute
    // units, also the kernel that keeps A in LDS in K chunks.  The one with
    // the least estimate runs if it is below the tile's.
    const int64_t items = ceil_div(N, 16);
    int64_t best = 100 * est;
    Regime pick{BI_KERNEL_TILED, 0, 0, 0, 0, -1};
    if (a_mode == bi::OPND_BF16_ROWS && M <= 128 && (b_mode == bi::OPND_BF16_ROWS || (fp4 && K % 128 == 0))) {
        const int rb = M > 64 ? 8 : M > 32 ? 4 : 2;
        if (b_mode == bi::OPND_BF16_ROWS || M <= 64) {
            const int64_t e = ceil_div(items, cus) * stream_round_cost(rb);
            if (e < best) {
                best = e;
                pick = {BI_KERNEL_STREAM_REG, rb, 0, 0, 16, -1};
            }
        }
        if (items > cus && bi::direct_achunk_ok(static_cast<int>(M), static_cast<int>(K), rb, fp4)) {
            const int64_t ec = achunk_cost(fp4, rb, items, cus);
            if (ec < best) {
                best = ec;
                pick = {BI_KERNEL_STREAM_A_CHUNKS, rb, 0, 0, 16, -1};
            }
        }
    }
    // NVFP4 A and weight, 16 < M <= 128 (K % 128 == 0): the chunked-A
    // kernel with A's rows decoded into LDS chunk by chunk (at any N: there
    // is no register-streaming kernel for an NVFP4 A)
    if (a_mode == bi::OPND_NVFP4_ROWS && M <= 128 && K % 128 == 0) {
        const int rb = M > 64 ? 8 : M > 32 ? 4 : 2;
        if (bi::direct_achunk_ok(static_cast<int>(M), static_cast<int>(K), rb, true)) {
            const int64_t ec = achunk_cost_w4a4(rb, items, cus);
            if (ec < best) {
                best = ec;
                pick = {BI_KERNEL_STREAM_A_CHUNKS, rb, 0, 0, 16, -1};
            }
        }
    }
    if (pick.kind != BI_KERNEL_TILED) return pick;
    const bi::TileShape &t = bi::kTileShapes[v];
    const bool pp = pingpong_ok(v, a_mode, b_mode, batch, grouped);
    return {pp ? BI_KERNEL_TILED_PINGPONG : BI_KERNEL_TILED, t.bm / 16, 0, 0, t.bn, v};
}

// Operand modes of an op as its entry point sets them.
void op_modes(int op, int a_fmt, int64_t K, int *a_mode, int *b_mode) {
    *a_mode = bi::OPND_BF16_ROWS;
    *b_mode = bi::OPND_BF16_ROWS;
    if (op == BI_OP_BMM) *b_mode = bi::OPND_BF16_KN;
    if (op == BI_OP_NVFP4_GEMM) {
        *a_mode = a_fmt == BI_A_BF16 ? bi::OPND_BF16_ROWS : bi::OPND_NVFP4_ROWS;
        // weight bytes by LDS DMA into a raw ring when the scale rows are
        // dword-aligned (K % 64 == 0); otherwise through registers (same bits)
        *b_mode = (*a_mode == bi::OPND_BF16_ROWS && K % 64 == 0) ? bi::OPND_NVFP4_RAW : bi::OPND_NVFP4_ROWS;
    }
}

bi_status launch_tiled(int a_mode, int b_mode, int op, int variant, const GemmArgs &in, void *stream,
                       const bi_launch_opts *opts, int cus) {
    const bi::TileShape &t = bi::kTileShapes[variant];
    if (op == BI_OP_BMM && (t.bn % 8 != 0)) return BI_ERR_UNSUPPORTED;
    GemmArgs a = in;
    a.tiles_m = static_cast<int>((a.M + t.bm - 1) / t.bm);
    a.tiles_n = static_cast<int>((a.N + t.bn - 1) / t.bn);
    // grouped: the experts' non-empty tiles are enumerated compactly, at most
    // (ceil(T / bm) + E) * tiles_n of them
    const int64_t tiles = a.group_off ? (static_cast<int64_t>(a.tiles_m) + a.batch) * a.tiles_n
                                      : static_cast<int64_t>(a.tiles_m) * a.tiles_n * a.batch;
    if (tiles > kI32Max) return BI_ERR_UNSUPPORTED;
    a.num_tiles = static_cast<int>(tiles);
    int per_cu = bi::kLdsPerCu / bi::tile_lds_bytes(t);
    if (per_cu < 1) per_cu = 1;
    const int grid = default_grid(a.num_tiles, cus, opts, per_cu);
    hipError_t e;
    if (!pingpong_ok(variant, a_mode, b_mode, a.batch, a.group_off != nullptr))
        e = bi::launch_gemm(a_mode, b_mode, GemmRecipe{variant}, a, grid, static_cast<hipStream_t>(stream));
    else if (b_mode == bi::OPND_NVFP4_RAW)
        e = bi::launch_pingpong_nvfp4(a, grid, static_cast<hipStream_t>(stream));
    else
        e = bi::launch_pingpong(a, t.bn, grid, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? BI_OK : BI_ERR_HIP;
}

bi_status run_gemm(int a_mode, int b_mode, int op, const GemmArgs &in, void *stream,
                   const bi_launch_opts *opts) {
    int cus = 0;
    bi_status st = device_cus(&cus);
    if (st != BI_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int depth = opts ? opts->pipeline_depth : 0;
    // a forced tile_variant keeps the tiled kernel, so the kernels can be compared
    if (opts && opts->tile_variant != 0) {
        if (opts->tile_variant < 0 || opts->tile_variant > bi::kNumTileShapes) return BI_ERR_SHAPE;
        return launch_tiled(a_mode, b_mode, op, opts->tile_variant - 1, in, stream, opts, cus);
    }
    // fixed_plan: one tile shape for (op, operand modes, N, K) at every M --
    // the cost model's many-rows choice, which no longer depends on M
    if (opts && opts->fixed_plan && op != BI_OP_BMM) {
        int64_t est = 0;
        const int v = op == BI_OP_GROUPED_GEMM ? grouped_variant(in.N, kModelRows + 1)
                                               : model_variant(a_mode, b_mode, in.N, 1, kModelRows + 1, &est);
        return launch_tiled(a_mode, b_mode, op, v, in, stream, opts, cus);
    }
    // grouped: classify() takes the average rows per expert
    const int64_t m_cls = in.group_off ? (in.M + in.batch - 1) / in.batch : in.M;
    const Regime r = classify(op, a_mode, b_mode, in.N, in.K, in.batch, in.group_off != nullptr, cus, m_cls);
    hipError_t e = hipSuccess;
    switch (r.kind) {
        case BI_KERNEL_STREAM_A_LDS: {
            // one wavefront per item up to three per compute unit; beyond that
            // a bf16 weight streams best from one wavefront per compute unit
            // (fewer concurrent row streams in HBM), an NVFP4 one from one
            // wavefront per item up to eight per compute unit: its decode is
            // VALU work, and a SIMD issues VALU at about half rate for one
            // wavefront, near full rate for two or more
            const bool afp4 = a_mode == bi::OPND_NVFP4_ROWS;
            const bool fp4 = afp4 || b_mode == bi::OPND_NVFP4_RAW;
            const int items = static_cast<int>((in.N + r.cols - 1) / r.cols);
            int waves = items <= 3 * cus ? items : fp4 ? (items < 8 * cus ? items : 8 * cus) : cus;
            if (opts && opts->max_workgroups > 0 && opts->max_workgroups < waves) waves = opts->max_workgroups;
            e = bi::launch_direct_alds(in, fp4, afp4, r.cols, waves, cus, depth, s);
            break;
        }
        case BI_KERNEL_STREAM_A_CHUNKS: {
            // one wavefront per 16-column item, up to eight per compute unit
            const bool afp4 = a_mode == bi::OPND_NVFP4_ROWS;
            const bool fp4 = afp4 || b_mode == bi::OPND_NVFP4_RAW;
            const int items = static_cast<int>((in.N + 15) / 16);
            int waves = items < 8 * cus ? items : 8 * cus;
            if (opts && opts->max_workgroups > 0 && opts->max_workgroups < waves) waves = opts->max_workgroups;
            e = bi::launch_direct_achunk(in, fp4, afp4, r.rb, waves, cus, depth, s);
            break;
        }
        case BI_KERNEL_STREAM_REG: {
            // one wavefront per 16-column item, up to 16 per compute unit
            const int items = static_cast<int>((in.N + 15) / 16);
            const int grid = default_grid(items, cus, opts, 16);
            e = b_mode == bi::OPND_NVFP4_RAW ? bi::launch_direct_nvfp4(in, r.rb, r.ap, grid, depth, s)
                                             : bi::launch_direct(in, r.rb, r.ap, grid, depth, s);
            break;
        }
        case BI_KERNEL_STREAM_RING: {
            const int items = static_cast<int>((in.N + r.cols - 1) / r.cols);
            int per_cu = bi::kLdsPerCu / bi::skinny_lds_bytes(b_mode, static_cast<int>(in.M), r.cols);
            per_cu = per_cu > 8 ? 8 : per_cu < 1 ? 1 : per_cu;
            e = bi::launch_skinny(b_mode, r.cols, r.ma, in, default_grid(items, cus, opts, per_cu), s);
            break;
        }
        case BI_KERNEL_BMM_STREAM: {
            const int64_t units = static_cast<int64_t>(in.batch) * ((in.N + 127) / 128);
            if (units > kI32Max) return BI_ERR_UNSUPPORTED;
            int per_cu = bi::kLdsPerCu / bi::bmm_short_k_lds_bytes(in.K);
            per_cu = per_cu > 2 ? 2 : (per_cu < 1 ? 1 : per_cu);
            e = bi::launch_bmm_short_k(in, default_grid(static_cast<int>(units), cus, opts, per_cu), s);
            break;
        }
        default:
            return launch_tiled(a_mode, b_mode, op, r.variant, in, stream, opts, cus);
    }
    return e == hipSuccess ? BI_OK : BI_ERR_HIP;
}

}  // namespace

extern "C" {

const char *bi_status_str(bi_status s) {
    switch (s) {
        case BI_OK: return "BI_OK";
        case BI_ERR_NULL: return "BI_ERR_NULL: a required pointer is NULL";
        case BI_ERR_SHAPE: return "BI_ERR_SHAPE: invalid sizes or leading dimensions";
        case BI_ERR_ALIGN: return "BI_ERR_ALIGN: pointer or stride not 16-byte aligned";
        case BI_ERR_ALIAS: return "BI_ERR_ALIAS: output overlaps an input";
        case BI_ERR_UNSUPPORTED: return "BI_ERR_UNSUPPORTED: no batch-invariant plan for this shape";
        case BI_ERR_VALUE: return "BI_ERR_VALUE: a scalar argument is outside its domain";
        case BI_ERR_HIP: return "BI_ERR_HIP: the HIP runtime reported an error";
    }
    return "unknown bi_status";
}

const char *bi_version(void) { return "bi 0.2.0 gfx950"; }

bi_status bi_tile_shape(int v, bi_plan *out) {
    if (!out) return BI_ERR_NULL;
    if (v < 0 || v >= bi::kNumTileShapes) return BI_ERR_SHAPE;
    fill_tile_plan(-1, v, out);
    return BI_OK;
}

bi_status bi_plan_query(int op, int64_t N, int64_t K, bi_plan *out) {
    if (!out) return BI_ERR_NULL;
    switch (op) {
        case BI_OP_GEMM:
        case BI_OP_BMM:
        case BI_OP_NVFP4_GEMM:
        case BI_OP_GROUPED_GEMM: {
            if (N <= 0 || K <= 0) return BI_ERR_SHAPE;
            if (op == BI_OP_NVFP4_GEMM ? (K % 32 != 0) : (K % 8 != 0)) return BI_ERR_SHAPE;
            if (op == BI_OP_BMM && N % 8 != 0) return BI_ERR_SHAPE;
            if (N > kI32Max || K > kI32Max) return BI_ERR_UNSUPPORTED;
            if (op == BI_OP_BMM && bi::bmm_short_k_ok(static_cast<int>(K))) {
                // the streaming BMM kernel: 64 x 128 tiles, the whole K staged
                std::memset(out, 0, sizeof *out);
                out->op = op;
                out->bm = 64;
                out->bn = 128;
                out->bk = static_cast<int32_t>(K);
                out->mfma_m = 16;
                out->mfma_n = 16;
                out->mfma_k = 32;
                out->waves = 4;
                out->lds_stages = 1;
                out->threads = 256;
                return BI_OK;
            }
            fill_tile_plan(op, plan_variant(op, N, K), out);
            return BI_OK;
        }
        case BI_OP_RMSNORM:
        case BI_OP_REDUCE_RMSNORM: {
            int T = 0, cpt = 0;
            if (!rms_shape(N, &T, &cpt)) return N > 32768 && N % 8 == 0 ? BI_ERR_UNSUPPORTED : BI_ERR_SHAPE;
            std::memset(out, 0, sizeof *out);
            out->op = op;
            out->threads = T;
            out->waves = T / 64;
            out->chunks_per_thread = cpt;
            return BI_OK;
        }
        case BI_OP_NVFP4_QUANT: {
            if (N <= 0 || N % 16 != 0) return BI_ERR_SHAPE;
            if (N > kI32Max) return BI_ERR_UNSUPPORTED;
            std::memset(out, 0, sizeof *out);
            out->op = op;
            out->threads = 256;
            out->waves = 4;
            out->chunks_per_thread = 1;
            return BI_OK;
        }
    }
    return BI_ERR_UNSUPPORTED;
}

bi_status bi_plan_regimes(int op, int64_t N, int64_t K, int a_fmt, int cus, bi_regime *out, int capacity,
                          int *count) {
    if (!count || (capacity > 0 && !out)) return BI_ERR_NULL;
    *count = 0;
    if (op != BI_OP_GEMM && op != BI_OP_BMM && op != BI_OP_NVFP4_GEMM && op != BI_OP_GROUPED_GEMM)
        return BI_ERR_UNSUPPORTED;
    if (a_fmt != BI_A_BF16 && a_fmt != BI_A_NVFP4) return BI_ERR_SHAPE;
    if (a_fmt == BI_A_NVFP4 && op != BI_OP_NVFP4_GEMM) return BI_ERR_SHAPE;
    bi_plan plan;
    bi_status st = bi_plan_query(op, N, K, &plan);
    if (st != BI_OK) return st;
    if (cus < 0) return BI_ERR_SHAPE;
    if (cus == 0) {
        st = device_cus(&cus);
        if (st != BI_OK) return st;
    }
    int a_mode = 0, b_mode = 0;
    op_modes(op, a_fmt, K, &a_mode, &b_mode);
    // classify() is constant above kModelRows rows: walk M up to there and
    // merge equal neighbours into row ranges
    int n = 0;
    Regime prev{};
    for (int64_t M = 1; M <= kModelRows + 1; ++M) {
        const Regime r = classify(op, a_mode, b_mode, N, K, 1, op == BI_OP_GROUPED_GEMM, cus, M);
        if (M > 1 && r == prev) {
            if (n <= capacity) out[n - 1].m_max = static_cast<int32_t>(M);
            continue;
        }
        if (n < capacity) {
            bi_regime &g = out[n];
            std::memset(&g, 0, sizeof g);
            g.kernel = r.kind;
            g.m_min = g.m_max = static_cast<int32_t>(M);
            g.row_blocks = r.rb;
            g.cols = r.cols;
            g.a_pairs = r.ap;
            g.a_rows_staged = r.ma;
            g.tile_variant = r.variant + 1;
        }
        ++n;
        prev = r;
    }
    if (n <= capacity) out[n - 1].m_max = static_cast<int32_t>(kI32Max);
    *count = n;
    return n <= capacity ? BI_OK : BI_ERR_SHAPE;
}

bi_status bi_gemm_ex(const void *A, int64_t lda, const void *B, int64_t ldb, void *Y, int64_t ldy,
                     int64_t M, int64_t N, int64_t K, void *stream, const bi_launch_opts *opts) {
    if (M < 0 || N <= 0 || K <= 0 || K % 8 != 0) return BI_ERR_SHAPE;
    if (lda < K || ldb < K || ldy < N) return BI_ERR_SHAPE;
    if (M > kI32Max || N > kI32Max || K > kI32Max || lda >= kMaxLd || ldb >= kMaxLd)
        return BI_ERR_UNSUPPORTED;
    if (M == 0) return BI_OK;
    if (!A || !B || !Y) return BI_ERR_NULL;
    if (!aligned16(A) || !aligned16(B) || !aligned16(Y) || lda % 8 || ldb % 8) return BI_ERR_ALIGN;
    const Range ry = mat_range(Y, M, N, ldy, 2, 1);
    if (overlap(ry, mat_range(A, M, K, lda, 2, 1)) || overlap(ry, mat_range(B, N, K, ldb, 2, 1)))
        return BI_ERR_ALIAS;
    GemmArgs a{};
    a.A = A; a.B = B; a.Y = Y;
    a.lda = lda; a.ldb = ldb; a.ldy = ldy;
    a.M = (int)M; a.N = (int)N; a.K = (int)K; a.batch = 1;
    a.alpha = 1.0f;
    return run_gemm(bi::OPND_BF16_ROWS, bi::OPND_BF16_ROWS, BI_OP_GEMM, a, stream, opts);
}

bi_status bi_gemm(const void *A, int64_t lda, const void *B, int64_t ldb, void *Y, int64_t ldy,
                  int64_t M, int64_t N, int64_t K, void *stream) {
    return bi_gemm_ex(A, lda, B, ldb, Y, ldy, M, N, K, stream, nullptr);
}

bi_status bi_bmm_ex(const void *A, int64_t sA, int64_t lda, const void *B, int64_t sB, int64_t ldb,
                    void *Y, int64_t sY, int64_t ldy, int64_t batch, int64_t M, int64_t N, int64_t K,
                    void *stream, const bi_launch_opts *opts) {
    if (M < 0 || N <= 0 || K <= 0 || batch <= 0 || K % 8 != 0 || N % 8 != 0) return BI_ERR_SHAPE;
    if (lda < K || ldb < N || ldy < N) return BI_ERR_SHAPE;
    if (batch > 1 && (sA < (M > 0 ? (M - 1) * lda + K : 0) || sB < (K - 1) * ldb + N ||
                      sY < (M > 0 ? (M - 1) * ldy + N : 0) || sA < 0 || sB < 0 || sY < 0))
        return BI_ERR_SHAPE;
    if (M > kI32Max || N > kI32Max || K > kI32Max || batch > kI32Max || lda >= kMaxLd)
        return BI_ERR_UNSUPPORTED;
    if (M == 0) return BI_OK;
    if (!A || !B || !Y) return BI_ERR_NULL;
    if (!aligned16(A) || !aligned16(B) || !aligned16(Y) || lda % 8 || ldb % 8 || sA % 8 || sB % 8 ||
        sY % 8)
        return BI_ERR_ALIGN;
    // Whole-tensor spans (head strides are >= the per-head extent, checked above).
    const Range ra = mat_range(A, 1, (batch - 1) * sA + (M - 1) * lda + K, 0, 2, 1);
    const Range rb = mat_range(B, 1, (batch - 1) * sB + (K - 1) * ldb + N, 0, 2, 1);
    const Range ry2 = mat_range(Y, 1, (batch - 1) * sY + (M - 1) * ldy + N, 0, 2, 1);
    if (overlap(ry2, ra) || overlap(ry2, rb)) return BI_ERR_ALIAS;
    GemmArgs a{};
    a.A = A; a.B = B; a.Y = Y;
    a.lda = lda; a.ldb = ldb; a.ldy = ldy;
    a.sA = sA; a.sB = sB; a.sY = sY;
    a.M = (int)M; a.N = (int)N; a.K = (int)K; a.batch = (int)batch;
    a.alpha = 1.0f;
    return run_gemm(bi::OPND_BF16_ROWS, bi::OPND_BF16_KN, BI_OP_BMM, a, stream, opts);
}

bi_status bi_bmm(const void *A, int64_t sA, int64_t lda, const void *B, int64_t sB, int64_t ldb,
                 void *Y, int64_t sY, int64_t ldy, int64_t batch, int64_t M, int64_t N, int64_t K,
                 void *stream) {
    return bi_bmm_ex(A, sA, lda, B, sB, ldb, Y, sY, ldy, batch, M, N, K, stream, nullptr);
}

bi_status bi_nvfp4_gemm_ex(const void *A, const void *A_scales, int a_fmt, int64_t lda,
                           const void *W, const void *W_scales, float alpha, void *Y, int64_t ldy,
                           int64_t M, int64_t N, int64_t K, void *stream,
                           const bi_launch_opts *opts) {
    if (a_fmt != BI_A_BF16 && a_fmt != BI_A_NVFP4) return BI_ERR_SHAPE;
    if (M < 0 || N <= 0 || K <= 0 || K % 32 != 0) return BI_ERR_SHAPE;
    if (lda < K || ldy < N) return BI_ERR_SHAPE;
    if (M > kI32Max || N > kI32Max || K > kI32Max || lda >= kMaxLd) return BI_ERR_UNSUPPORTED;
    if (M == 0) return BI_OK;
    if (!A || !W || !W_scales || !Y || (a_fmt == BI_A_NVFP4 && !A_scales)) return BI_ERR_NULL;
    if (!aligned16(A) || !aligned16(W) || !aligned16(W_scales) || !aligned16(Y)) return BI_ERR_ALIGN;
    if (a_fmt == BI_A_NVFP4 && (!aligned16(A_scales) || lda % 32)) return BI_ERR_ALIGN;
    if (a_fmt == BI_A_BF16 && lda % 8) return BI_ERR_ALIGN;
    const Range ry = mat_range(Y, M, N, ldy, 2, 1);
    if (overlap(ry, mat_range(W, N, K, K, 1, 2)) || overlap(ry, mat_range(W_scales, N, K, K, 1, 16)))
        return BI_ERR_ALIAS;
    if (a_fmt == BI_A_BF16) {
        if (overlap(ry, mat_range(A, M, K, lda, 2, 1))) return BI_ERR_ALIAS;
    } else {
        if (overlap(ry, mat_range(A, M, K, lda, 1, 2)) || overlap(ry, mat_range(A_scales, M, K, lda, 1, 16)))
            return BI_ERR_ALIAS;
    }
    GemmArgs a{};
    a.A = A; a.A_scales = A_scales; a.B = W; a.B_scales = W_scales; a.Y = Y;
    a.lda = lda; a.ldb = K; a.ldy = ldy;
    a.M = (int)M; a.N = (int)N; a.K = (int)K; a.batch = 1;
    a.alpha = alpha;
    a.use_alpha = 1;
    const int am = a_fmt == BI_A_BF16 ? bi::OPND_BF16_ROWS : bi::OPND_NVFP4_ROWS;
    // weight bytes by LDS DMA into a raw ring when the scale rows are
    // dword-aligned (K % 64 == 0); otherwise through registers (same bits)
    const int bm = (am == bi::OPND_BF16_ROWS && K % 64 == 0) ? bi::OPND_NVFP4_RAW : bi::OPND_NVFP4_ROWS;
    return run_gemm(am, bm, BI_OP_NVFP4_GEMM, a, stream, opts);
}

bi_status bi_nvfp4_gemm(const void *A, const void *A_scales, int a_fmt, int64_t lda, const void *W,
                        const void *W_scales, float alpha, void *Y, int64_t ldy, int64_t M,
                        int64_t N, int64_t K, void *stream) {
    return bi_nvfp4_gemm_ex(A, A_scales, a_fmt, lda, W, W_scales, alpha, Y, ldy, M, N, K, stream,
                            nullptr);
}

bi_status bi_rmsnorm_ex(const void *X, int64_t ldx, const void *gamma, float eps, void *Y,
                        int64_t ldy, int64_t M, int64_t H, void *stream,
                        const bi_launch_opts *opts) {
    int T = 0, cpt = 0;
    if (M < 0 || H <= 0 || H % 8 != 0) return BI_ERR_SHAPE;
    if (ldx < H || ldy < H) return BI_ERR_SHAPE;
    if (!rms_shape(H, &T, &cpt)) return BI_ERR_UNSUPPORTED;
    if (M > kI32Max) return BI_ERR_UNSUPPORTED;
    if (M == 0) return BI_OK;
    if (!X || !gamma || !Y) return BI_ERR_NULL;
    if (!aligned16(X) || !aligned16(gamma) || !aligned16(Y) || ldx % 8 || ldy % 8) return BI_ERR_ALIGN;
    const Range ry = mat_range(Y, M, H, ldy, 2, 1);
    const Range rx = mat_range(X, M, H, ldx, 2, 1);
    const bool in_place = (X == Y && ldx == ldy);
    if ((!in_place && overlap(ry, rx)) || overlap(ry, mat_range(gamma, 1, H, H, 2, 1)))
        return BI_ERR_ALIAS;
    int cus = 0;
    bi_status st = device_cus(&cus);
    if (st != BI_OK) return st;
    bi::RmsArgs a{};
    a.X = X; a.gamma = gamma; a.Y = Y;
    a.ldx = ldx; a.ldy = ldy;
    a.M = (int)M; a.H = (int)H; a.eps = eps;
    const int grid = default_grid((int)M, cus, opts, 16);
    hipError_t e = bi::launch_rmsnorm(T, cpt, a, grid, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? BI_OK : BI_ERR_HIP;
}

bi_status bi_rmsnorm(const void *X, int64_t ldx, const void *gamma, float eps, void *Y, int64_t ldy,
                     int64_t M, int64_t H, void *stream) {
    return bi_rmsnorm_ex(X, ldx, gamma, eps, Y, ldy, M, H, stream, nullptr);
}

bi_status bi_nvfp4_quant_ex(const void *X, int64_t ldx, float g, void *Q, void *Q_scales, int64_t ldq,
                            int64_t M, int64_t K, void *stream, const bi_launch_opts *opts) {
    if (M < 0 || K <= 0 || K % 16 != 0 || ldx < K || ldq < K) return BI_ERR_SHAPE;
    if (!(g > 0.0f) || !(g <= 3.402823466e38f)) return BI_ERR_VALUE;
    if (M > kI32Max || K > kI32Max || M * (K / 8) >= ((int64_t)1 << 30)) return BI_ERR_UNSUPPORTED;
    if (M == 0) return BI_OK;
    if (!X || !Q || !Q_scales) return BI_ERR_NULL;
    // 16-byte loads of X; 4-byte code stores (row strides ldq/2 bytes); byte scale stores
    if (!aligned16(X) || (reinterpret_cast<uintptr_t>(Q) & 3u) || ldx % 8 || ldq % 16) return BI_ERR_ALIGN;
    const Range rx = mat_range(X, M, K, ldx, 2, 1);
    const Range rq = mat_range(Q, M, K, ldq, 1, 2);
    const Range rs = mat_range(Q_scales, M, K, ldq, 1, 16);
    if (overlap(rq, rx) || overlap(rs, rx) || overlap(rq, rs)) return BI_ERR_ALIAS;
    int cus = 0;
    bi_status st = device_cus(&cus);
    if (st != BI_OK) return st;
    bi::QuantArgs a{};
    a.X = X; a.Q = Q; a.S = Q_scales;
    a.ldx = ldx; a.ldq = ldq;
    a.M = (int)M; a.K = (int)K;
    a.halves = (int)(M * (K / 8));
    {   // exact division by d = K / 8 for every dividend below 2^32
        const uint64_t d = (uint64_t)(K / 8);
        int l = 0;
        while (((uint64_t)1 << l) < d) ++l;
        a.shift = 32 + l;
        a.magic = (((uint64_t)1 << a.shift) + d - 1) / d;
    }
    a.g = g;
    // four half blocks per thread (the kernel's kU), at most 8 workgroups per compute unit
    const int wgs = (int)(((int64_t)a.halves + 4 * 256 - 1) / (4 * 256));
    const int grid = default_grid(wgs, cus, opts, 8);
    hipError_t e = bi::launch_nvfp4_quant(a, grid, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? BI_OK : BI_ERR_HIP;
}

bi_status bi_nvfp4_quant(const void *X, int64_t ldx, float g, void *Q, void *Q_scales, int64_t ldq,
                         int64_t M, int64_t K, void *stream) {
    return bi_nvfp4_quant_ex(X, ldx, g, Q, Q_scales, ldq, M, K, stream, nullptr);
}

bi_status bi_reduce_rmsnorm_ex(const void *const *partials, int n_partials, int64_t ldp,
                               const void *residual, int64_t ldres, const void *gamma, float eps,
                               void *R, int64_t ldr, void *Y, int64_t ldy, int64_t M, int64_t H,
                               void *stream, const bi_launch_opts *opts) {
    int T = 0, cpt = 0;
    if (M < 0 || H <= 0 || H % 8 != 0) return BI_ERR_SHAPE;
    if (n_partials < 1 || n_partials > bi::kMaxPartials) return BI_ERR_SHAPE;
    if (ldp < H || ldr < H || ldy < H || (residual && ldres < H)) return BI_ERR_SHAPE;
    if (!rms_shape(H, &T, &cpt)) return BI_ERR_UNSUPPORTED;
    if (M > kI32Max) return BI_ERR_UNSUPPORTED;
    if (M == 0) return BI_OK;
    if (!partials || !gamma || !R || !Y) return BI_ERR_NULL;
    for (int q = 0; q < n_partials; ++q)
        if (!partials[q]) return BI_ERR_NULL;
    if (!aligned16(gamma) || !aligned16(R) || !aligned16(Y) || ldp % 8 || ldr % 8 || ldy % 8 ||
        (residual && (!aligned16(residual) || ldres % 8)))
        return BI_ERR_ALIGN;
    for (int q = 0; q < n_partials; ++q)
        if (!aligned16(partials[q])) return BI_ERR_ALIGN;
    const Range rr = mat_range(R, M, H, ldr, 2, 1);
    const Range ry = mat_range(Y, M, H, ldy, 2, 1);
    const Range rg = mat_range(gamma, 1, H, H, 2, 1);
    if (overlap(rr, ry) || overlap(rr, rg) || overlap(ry, rg)) return BI_ERR_ALIAS;
    for (int q = 0; q < n_partials; ++q) {
        const Range rp = mat_range(partials[q], M, H, ldp, 2, 1);
        if (overlap(rr, rp) || overlap(ry, rp)) return BI_ERR_ALIAS;
    }
    if (residual) {
        const Range rs = mat_range(residual, M, H, ldres, 2, 1);
        const bool in_place = (residual == R && ldres == ldr);
        if ((!in_place && overlap(rr, rs)) || overlap(ry, rs)) return BI_ERR_ALIAS;
    }
    int cus = 0;
    bi_status st = device_cus(&cus);
    if (st != BI_OK) return st;
    bi::ReduceRmsArgs a{};
    for (int q = 0; q < n_partials; ++q) a.P[q] = partials[q];
    a.np = n_partials;
    a.ldp = ldp;
    a.res = residual;
    a.ldres = residual ? ldres : 0;
    a.gamma = gamma;
    a.R = R; a.Y = Y;
    a.ldr = ldr; a.ldy = ldy;
    a.M = (int)M; a.H = (int)H; a.eps = eps;
    const int grid = default_grid((int)M, cus, opts, 16);
    hipError_t e = bi::launch_reduce_rmsnorm(T, cpt, a, grid, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? BI_OK : BI_ERR_HIP;
}

bi_status bi_reduce_rmsnorm(const void *const *partials, int n_partials, int64_t ldp,
                            const void *residual, int64_t ldres, const void *gamma, float eps,
                            void *R, int64_t ldr, void *Y, int64_t ldy, int64_t M, int64_t H,
                            void *stream) {
    return bi_reduce_rmsnorm_ex(partials, n_partials, ldp, residual, ldres, gamma, eps, R, ldr, Y, ldy,
                                M, H, stream, nullptr);
}

bi_status bi_grouped_gemm_ex(const void *A, int64_t lda, const void *W, int64_t ldw, int64_t sW, void *Y,
                             int64_t ldy, const int64_t *group_offsets, int64_t E, int64_t T, int64_t N,
                             int64_t K, void *stream, const bi_launch_opts *opts) {
    if (T < 0 || E <= 0 || N <= 0 || K <= 0 || K % 8 != 0) return BI_ERR_SHAPE;
    if (lda < K || ldw < K || ldy < N || (E > 1 && sW < (N - 1) * ldw + K) || sW < 0) return BI_ERR_SHAPE;
    if (T > kI32Max || N > kI32Max || K > kI32Max || E > kI32Max || lda >= kMaxLd || ldw >= kMaxLd)
        return BI_ERR_UNSUPPORTED;
    if (T == 0) return BI_OK;
    if (!A || !W || !Y || !group_offsets) return BI_ERR_NULL;
    if (!aligned16(A) || !aligned16(W) || !aligned16(Y) || (reinterpret_cast<uintptr_t>(group_offsets) & 7u) ||
        lda % 8 || ldw % 8 || sW % 8)
        return BI_ERR_ALIGN;
    const Range ry = mat_range(Y, T, N, ldy, 2, 1);
    const Range rw = mat_range(W, 1, (E - 1) * sW + (N - 1) * ldw + K, 0, 2, 1);
    const Range ro = mat_range(group_offsets, 1, E + 1, 0, 8, 1);
    if (overlap(ry, mat_range(A, T, K, lda, 2, 1)) || overlap(ry, rw) || overlap(ry, ro)) return BI_ERR_ALIAS;
    GemmArgs a{};
    a.A = A; a.B = W; a.Y = Y;
    a.lda = lda; a.ldb = ldw; a.ldy = ldy;
    a.sB = sW;
    a.M = (int)T; a.N = (int)N; a.K = (int)K; a.batch = (int)E;
    a.alpha = 1.0f;
    a.group_off = group_offsets;
    a.total_rows = T;
    return run_gemm(bi::OPND_BF16_ROWS, bi::OPND_BF16_ROWS, BI_OP_GROUPED_GEMM, a, stream, opts);
}

bi_status bi_grouped_gemm(const void *A, int64_t lda, const void *W, int64_t ldw, int64_t sW, void *Y,
                          int64_t ldy, const int64_t *group_offsets, int64_t E, int64_t T, int64_t N,
                          int64_t K, void *stream) {
    return bi_grouped_gemm_ex(A, lda, W, ldw, sW, Y, ldy, group_offsets, E, T, N, K, stream, nullptr);
}

bi_status bi_mla_decode_workspace_size(int64_t B, int64_t H, int64_t Lmax, int64_t Dqk, int64_t Dv,
                                       int64_t *bytes) {
    if (!bytes) return BI_ERR_NULL;
    *bytes = 0;
    if (B < 0 || H < 0 || Lmax < 0 || Dqk <= 0 || Dv <= 0 || Dv > Dqk || Dqk % 8 || Dv % 8) return BI_ERR_SHAPE;
    if (Dqk > bi::kMlaMaxDqk || Dv > bi::kMlaMaxDv || Lmax > bi::kMlaMaxTokens) return BI_ERR_UNSUPPORTED;
    if (B > kI32Max || H > kI32Max || B * H > kI32Max) return BI_ERR_UNSUPPORTED;
    *bytes = bi::mla_workspace_bytes((int)B, (int)H, (int)Lmax, (int)Dqk, (int)Dv);
    return BI_OK;
}

}  // extern "C"

namespace {

// Host-side validation shared by the decode-attention entry points; *need is
// the workspace size of the shape.  BI_OK with B == 0 or H == 0 means a no-op.
bi_status mla_check(const void *q, const void *kv, const int32_t *lens, float scale, void *out, int64_t B,
                    int64_t H, int64_t Lmax, int64_t Dqk, int64_t Dv, void *workspace, int64_t workspace_bytes,
                    int64_t *need) {
    bi_status st = bi_mla_decode_workspace_size(B, H, Lmax, Dqk, Dv, need);
    if (st != BI_OK) return st;
    if (!(scale == scale) || scale > 3.402823466e38f || scale < -3.402823466e38f) return BI_ERR_VALUE;
    if (workspace && *need > 0 && workspace_bytes < *need) return BI_ERR_SHAPE;
    if (B == 0 || H == 0) return BI_OK;
    if (!q || !kv || !lens || !out) return BI_ERR_NULL;
    if (!aligned16(q) || !aligned16(kv) || !aligned16(out) || (reinterpret_cast<uintptr_t>(lens) & 3u) ||
        (workspace && !aligned16(workspace)))
        return BI_ERR_ALIGN;
    const Range ro = mat_range(out, B * H, Dv, Dv, 2, 1);
    const Range rq = mat_range(q, B * H, Dqk, Dqk, 2, 1);
    const Range rl = mat_range(lens, 1, B, B, 4, 1);
    const Range rk = Lmax > 0 ? mat_range(kv, B * Lmax, Dqk, Dqk, 2, 1) : Range{0, 0};
    if (overlap(ro, rq) || overlap(ro, rl) || overlap(ro, rk)) return BI_ERR_ALIAS;
    if (workspace && *need > 0) {
        const Range rw = mat_range(workspace, 1, *need, *need, 1, 1);
        if (overlap(rw, ro) || overlap(rw, rq) || overlap(rw, rl) || overlap(rw, rk)) return BI_ERR_ALIAS;
    }
    return BI_OK;
}

}  // namespace

extern "C" {

bi_status bi_mla_decode_ex(const void *q, const void *kv, const int32_t *lens, float scale, void *out,
                           int64_t B, int64_t H, int64_t Lmax, int64_t Dqk, int64_t Dv, void *workspace,
                           int64_t workspace_bytes, void *stream, const bi_launch_opts *opts) {
    int64_t need = 0;
    bi_status st = mla_check(q, kv, lens, scale, out, B, H, Lmax, Dqk, Dv, workspace, workspace_bytes, &need);
    if (st != BI_OK) return st;
    if (B == 0 || H == 0) return BI_OK;
    const bool use_ws = workspace && need > 0;
    int cus = 0;
    st = device_cus(&cus);
    if (st != BI_OK) return st;
    // The chunked schedule pays for its fold only when the (request, head
    // group) units alone leave compute units idle; both give the same bits.
    const int64_t groups = B * ((H + 15) / 16);
    const bool split = use_ws && groups < cus;
    bi::MlaArgs a{};
    a.q = q; a.kv = kv; a.lens = lens; a.out = out;
    a.B = (int)B; a.H = (int)H; a.Lmax = (int)Lmax; a.Dqk = (int)Dqk; a.Dv = (int)Dv;
    a.scale = scale;
    a.ws = split ? static_cast<float *>(workspace) : nullptr;
    a.nchunk = split ? (int)((Lmax + bi::kMlaChunk - 1) / bi::kMlaChunk) : 0;
    // work units: (request, 16-head group[, chunk]) for the MFMA kernel, one
    // workgroup each (a compute unit takes the next as it finishes one, which
    // evens out requests of unequal length); (request, head) for the VALU
    // kernel
    const bool mfma = bi::mla_mfma_variant(a.Dqk, a.Dv) != 0;
    const int64_t units = mfma ? bi::mla_mfma_units(B * (split ? a.nchunk : 1), (int)((H + 15) / 16)) : B * H;
    if (units > kI32Max) return BI_ERR_UNSUPPORTED;
    const int per_cu = mfma ? (int)((units + cus - 1) / cus) : (bi::mla_token_capacity(a.Lmax) == 4096 ? 4 : 1);
    const int grid = default_grid((int)units, cus, opts, per_cu);
    const int64_t fold_blocks = (groups * 4 * Dv + 255) / 256;  // one thread per four output elements
    const int fold_grid = (int)(fold_blocks < (int64_t)cus * 8 ? fold_blocks : (int64_t)cus * 8);
    hipError_t e = bi::launch_mla_decode(a, grid, fold_grid < 1 ? 1 : fold_grid, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? BI_OK : BI_ERR_HIP;
}

bi_status bi_mla_decode_noalloc(const void *q, const void *kv, const int32_t *lens, float scale, void *out,
                                int64_t B, int64_t H, int64_t Lmax, int64_t Dqk, int64_t Dv, void *stream) {
    int64_t need = 0;
    bi_status st = mla_check(q, kv, lens, scale, out, B, H, Lmax, Dqk, Dv, nullptr, 0, &need);
    if (st != BI_OK || B == 0 || H == 0) return st;
    int cus = 0;
    st = device_cus(&cus);
    if (st != BI_OK) return st;
    // The chunked schedule, the only one that needs scratch, runs exactly when
    // bi_mla_decode with a workspace would run it: fewer (request, head group)
    // pairs than compute units.  Its partials then go to the library's array.
    void *ws = nullptr;
    if (need > 0 && B * ((H + 15) / 16) < cus) {
        if (need > bi::kMlaScratchBytes) return BI_ERR_UNSUPPORTED;
        float *p = nullptr;
        if (bi::mla_scratch(&p) != hipSuccess) return BI_ERR_HIP;
        ws = p;
    }
    return bi_mla_decode_ex(q, kv, lens, scale, out, B, H, Lmax, Dqk, Dv, ws, ws ? bi::kMlaScratchBytes : 0, stream,
                            nullptr);
}

bi_status bi_mla_decode(const void *q, const void *kv, const int32_t *lens, float scale, void *out, int64_t B,
                        int64_t H, int64_t Lmax, int64_t Dqk, int64_t Dv, void *workspace, int64_t workspace_bytes,
                        void *stream) {
    return bi_mla_decode_ex(q, kv, lens, scale, out, B, H, Lmax, Dqk, Dv, workspace, workspace_bytes, stream,
                            nullptr);
}

bi_status bi_probe_mfma(void *out, int64_t iters, int grid, void *stream) {
    if (iters < 1 || grid < 1 || iters > ((int64_t)1 << 40)) return BI_ERR_SHAPE;
    if (!out) return BI_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(out) & 7u) return BI_ERR_ALIGN;
    return bi::launch_mfma_probe(static_cast<uint64_t *>(out), iters, grid, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? BI_OK
               : BI_ERR_HIP;
}

bi_status bi_probe_lds(void *out, int64_t iters, int grid, void *stream) {
    if (iters < 1 || grid < 1 || iters > ((int64_t)1 << 40)) return BI_ERR_SHAPE;
    if (!out) return BI_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(out) & 7u) return BI_ERR_ALIGN;
    return bi::launch_lds_probe(static_cast<uint64_t *>(out), iters, grid, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? BI_OK
               : BI_ERR_HIP;
}

bi_status bi_probe_read(const void *src, int64_t bytes, void *sink, int grid, void *stream) {
    if (bytes <= 0 || bytes % 16 || grid < 1) return BI_ERR_SHAPE;
    if (!src || !sink) return BI_ERR_NULL;
    if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return BI_ERR_ALIGN;
    if (overlap(mat_range(sink, 1, (int64_t)grid * 256, 0, 4, 1), mat_range(src, 1, bytes, 0, 1, 1)))
        return BI_ERR_ALIAS;
    return bi::launch_read_probe(src, bytes, static_cast<uint32_t *>(sink), grid, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? BI_OK
               : BI_ERR_HIP;
}

}  // extern "C"
