/*
 * Oracle for the batch-invariant GEMM family and RMSNorm: a plain, slow,
 * fp64 CPU implementation of what each operation computes.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; it consumes the same stored
 * inputs (bf16 bit patterns, NVFP4 code and scale bytes) and nothing else.
 *
 * Every function returns the exact-up-to-fp64-rounding value of the plain
 * definition, never an emulation of a GPU kernel:
 *   - products of two bf16 values are exact in fp64 (8 + 8 significand bits);
 *   - sums are accumulated sequentially in ascending k in fp64;
 *   - nothing is rounded to fp32 or bf16.
 * Alongside y it returns sum_k |a_k * b_k|, the scale the tolerance uses.
 *
 * Sources (the pages' own wording is not reproduced here):
 *   - "NVFP4 CUTLASS batch invariant mode" (vLLM PR #39912 summary page),
 *     section "key source snippets", unit test test_nvfp4_gemm_batch_invariance:
 *     a is [m,k], b is [n,k], k = 2 * packed_k, out = alpha * (a . b^T) with
 *     alpha = 1 / (global_scale_a * global_scale_b).  This fixes the operand
 *     orientation y = A . B^T used for every GEMM here.
 *   - "[Core] Disable fuse_allreduce_rms under VLLM_BATCH_INVARIANT" (vLLM
 *     PR #51292), section Purpose: RMSNorm is the row reduction fused after
 *     the all-reduce.  The pages name it without a formula; the definition
 *     used is the standard one, y = x * gamma / sqrt(mean(x^2) + eps).
 *   - NVFP4 element and scale encodings are named by the pages but not
 *     spelled out; the decoders below follow the OCP 8-bit floating point
 *     (E4M3, "fn" variant: no infinities, one NaN pattern per sign) and the
 *     OCP Microscaling FP4 E2M1 definitions.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

/* bf16 bit pattern -> value: bf16 is the top half of an IEEE binary32. */
static double bf16_value(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* FP4 E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 * Exponent field 0 is subnormal: value = mantissa * 2^(1-1) * 0.5. */
static double e2m1_value(unsigned code) {
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* FP8 E4M3 (fn): bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa.
 * Exponent field 0 is subnormal: m/8 * 2^-6.  S.1111.111 is NaN; there is no
 * infinity, so S.1111.110 = 448 is the largest finite magnitude. */
static double e4m3_value(unsigned code) {
    unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m / 8.0, -6);
    else mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* Exported decoders so the tests can pin them exhaustively. */
double oracle_e2m1_value(uint32_t code) { return e2m1_value(code & 15u); }
double oracle_e4m3_value(uint32_t code) { return e4m3_value(code & 255u); }
double oracle_bf16_value(uint32_t bits) { return bf16_value((uint16_t)bits); }

/* Element k of an NVFP4 row: codes hold two elements per byte, element 2j in
 * the low nibble of byte j and element 2j+1 in the high nibble; one E4M3
 * scale covers 16 consecutive elements.  value = e2m1(code) * e4m3(scale). */
static double nvfp4_elem(const uint8_t *codes, const uint8_t *scales, int64_t k) {
    unsigned byte = codes[k >> 1];
    unsigned code = (k & 1) ? (byte >> 4) : (byte & 15u);
    return e2m1_value(code) * e4m3_value(scales[k >> 4]);
}

/*
 * GEMM: Y[r][j] = sum_{k<K} A[i][k] * B[j][k], i = rows[r] (or r when rows is
 * NULL), for j < N.  A is bf16 [M,K] with row stride lda, B is bf16 [N,K]
 * with row stride ldb.  Y and S are dense [nrows, N]; S gets sum_k |a*b|.
 */
void oracle_gemm(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                 int64_t M, int64_t N, int64_t K, const int64_t *rows, int64_t nrows,
                 double *Y, double *S) {
    if (!rows) nrows = M;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t r = 0; r < nrows; r++) {
        for (int64_t j = 0; j < N; j++) {
            int64_t i = rows ? rows[r] : r;
            const uint16_t *a = A + i * lda, *b = B + j * ldb;
            double y = 0.0, s = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = bf16_value(a[k]) * bf16_value(b[k]);
                y += p;
                s += fabs(p);
            }
            Y[r * N + j] = y;
            S[r * N + j] = s;
        }
    }
}

/*
 * BMM: for each head h, Y[h][i][j] = sum_{k<K} A[h][i][k] * B[h][k][j].
 * A is bf16 [batch,M,K] (head stride sA, row stride lda), B is bf16
 * [batch,K,N] (head stride sB, row stride ldb over k).  Y, S dense
 * [batch,M,N].
 */
void oracle_bmm(const uint16_t *A, int64_t sA, int64_t lda, const uint16_t *B, int64_t sB,
                int64_t ldb, int64_t batch, int64_t M, int64_t N, int64_t K, double *Y,
                double *S) {
#pragma omp parallel for collapse(3) schedule(static)
    for (int64_t h = 0; h < batch; h++) {
        for (int64_t i = 0; i < M; i++) {
            for (int64_t j = 0; j < N; j++) {
                const uint16_t *a = A + h * sA + i * lda;
                const uint16_t *b = B + h * sB + j;
                double y = 0.0, s = 0.0;
                for (int64_t k = 0; k < K; k++) {
                    double p = bf16_value(a[k]) * bf16_value(b[k * ldb]);
                    y += p;
                    s += fabs(p);
                }
                Y[(h * M + i) * N + j] = y;
                S[(h * M + i) * N + j] = s;
            }
        }
    }
}

/*
 * NVFP4 weight GEMM: Y[r][j] = alpha * sum_{k<K} a(i,k) * w(j,k).
 *   w(j,k) = e2m1(W code) * e4m3(W scale), W codes [N, K/2] and W scales
 *   [N, K/16], both dense.
 *   a_fmt 0: a(i,k) = bf16 A[i*lda + k].
 *   a_fmt 1: a(i,k) is the NVFP4 element k of row i: codes at A + i*lda/2
 *            bytes, scales at A_scales + i*lda/16 bytes.
 * alpha is the fp32 argument, widened to fp64 and applied once.
 * S gets |alpha| * sum_k |a * w|.
 */
void oracle_nvfp4_gemm(const void *A, const uint8_t *A_scales, int a_fmt, int64_t lda,
                       const uint8_t *W, const uint8_t *W_scales, float alpha, int64_t M,
                       int64_t N, int64_t K, const int64_t *rows, int64_t nrows, double *Y,
                       double *S) {
    if (!rows) nrows = M;
    double al = (double)alpha;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t r = 0; r < nrows; r++) {
        for (int64_t j = 0; j < N; j++) {
            int64_t i = rows ? rows[r] : r;
            const uint8_t *wc = W + j * (K / 2), *ws = W_scales + j * (K / 16);
            double y = 0.0, s = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double a;
                if (a_fmt == 0)
                    a = bf16_value(((const uint16_t *)A)[i * lda + k]);
                else
                    a = nvfp4_elem((const uint8_t *)A + i * (lda / 2), A_scales + i * (lda / 16), k);
                double p = a * nvfp4_elem(wc, ws, k);
                y += p;
                s += fabs(p);
            }
            Y[r * N + j] = al * y;
            S[r * N + j] = fabs(al) * s;
        }
    }
}

/*
 * RMSNorm: Y[r][h] = x[i][h] * gamma[h] / sqrt((1/H) * sum_h' x[i][h']^2 + eps).
 * X bf16 [M,H] row stride ldx, gamma bf16 [H], eps the fp32 argument widened.
 * Y dense [nrows, H].
 */
void oracle_rmsnorm(const uint16_t *X, int64_t ldx, const uint16_t *gamma, float eps,
                    int64_t M, int64_t H, const int64_t *rows, int64_t nrows, double *Y) {
    if (!rows) nrows = M;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; r++) {
        int64_t i = rows ? rows[r] : r;
        const uint16_t *x = X + i * ldx;
        double ss = 0.0;
        for (int64_t h = 0; h < H; h++) {
            double v = bf16_value(x[h]);
            ss += v * v;
        }
        double denom = sqrt(ss / (double)H + (double)eps);
        for (int64_t h = 0; h < H; h++)
            Y[r * H + h] = bf16_value(x[h]) * bf16_value(gamma[h]) / denom;
    }
}

/*
 * NVFP4 quantiser of activations, row-local: the operation named
 * scaled_fp4_quant(x, global_scale) -> (fp4 codes, block scales) in the vLLM
 * PR #39912 unit test (summary page, section "key source snippets").  The
 * pages name it without defining it; the reading used, step by step for
 * each block of 16 consecutive elements of a row:
 *   1. amax = the largest |x| of the block (bf16 values, exact);
 *   2. v = (amax * g) / 6 with each operation rounded to fp32 (round to
 *      nearest even), then min(v, 448): the block's largest magnitude is to
 *      land on the largest E2M1 magnitude, 6, and 448 is the largest finite
 *      E4M3 value;
 *   3. the scale code is the E4M3 code whose value is nearest to v, ties to
 *      the even code;
 *   4. s = that code's value; when s == 0 every code of the block is 0;
 *      otherwise r = g / s rounded to fp32, and for each element
 *      w = |x| * r rounded to fp32;
 *   5. the element code is the E2M1 magnitude code nearest to w, ties to the
 *      even code, values beyond 6 giving 6; the sign bit is set for a
 *      negative x whose magnitude code is not 0.
 * The fp32 steps decide integers (the codes), so they are taken in the same
 * precision as the GPU kernel takes them; the nearest-code searches are
 * plain scans over every code.  Each row depends only on itself and g.
 * Codes are packed two per byte, element 2j in the low nibble of byte j.
 * Q: codes [M, K/2] with row stride ldq/2 bytes; S: scales [M, K/16] with
 * row stride ldq/16 bytes; X: bf16 [M, K] with row stride ldx.
 */
static unsigned nearest_code(double v, double (*dec)(unsigned), unsigned ncodes) {
    unsigned best = 0;
    double bd = fabs(dec(0) - v);
    for (unsigned c = 1; c < ncodes; c++) {
        double d = fabs(dec(c) - v);
        if (d < bd || (d == bd && (c & 1u) == 0)) {
            best = c;
            bd = d;
        }
    }
    return best;
}

void oracle_nvfp4_quant(const uint16_t *X, int64_t ldx, float g, int64_t M, int64_t K,
                        int64_t ldq, uint8_t *Q, uint8_t *S) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; i++) {
        const uint16_t *x = X + i * ldx;
        uint8_t *q = Q + i * (ldq / 2), *sc = S + i * (ldq / 16);
        for (int64_t b = 0; b < K / 16; b++) {
            float amax = 0.0f;
            for (int j = 0; j < 16; j++) {
                float a = (float)fabs(bf16_value(x[16 * b + j]));
                if (a > amax) amax = a;
            }
            float u = amax * g;
            float v = u / 6.0f;
            if (v > 448.0f) v = 448.0f;
            unsigned scode = nearest_code((double)v, e4m3_value, 127);
            float s = (float)e4m3_value(scode);
            float r = (s != 0.0f) ? g / s : 0.0f;
            unsigned codes[16];
            for (int j = 0; j < 16; j++) {
                double xv = bf16_value(x[16 * b + j]);
                unsigned c = 0;
                if (s != 0.0f) {
                    float w = (float)fabs(xv) * r;
                    if (w > 6.0f) w = 6.0f;
                    c = nearest_code((double)w, e2m1_value, 8);
                    if (c != 0 && signbit(xv)) c |= 8u;
                }
                codes[j] = c;
            }
            for (int j = 0; j < 8; j++) q[8 * b + j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
            sc[b] = (uint8_t)scode;
        }
    }
}

/*
 * Fixed-order reduction of partial outputs followed by RMSNorm: the
 * all-reduce + RMSNorm pair that the vLLM PR #51292 page fuses (section
 * "Purpose"), and whose reduction it requires to run in one fixed order for
 * every batch (the root-cause comment and the test plan: one distinct
 * output over 8 runs).  On one GPU the P partial [M,H] outputs of a
 * row-parallel layer are the inputs.  Plain definition, in fp64:
 *   R[i][h] = residual[i][h] (if given) + sum_p P_p[i][h];
 *   Y[i][h] = R[i][h] * gamma[h] / sqrt((1/H) * sum_h' R[i][h']^2 + eps).
 * P holds the partials back to back, each bf16 [M,H] dense, P_p at P + p*M*H;
 * residual is bf16 [M,H] dense or NULL.  SR gets sum |terms| of each R
 * element, SY gets |gamma| * SR / sqrt(mean(R^2) + eps): the scales of the
 * tolerances.
 */
void oracle_reduce_rmsnorm(const uint16_t *P, int64_t np, const uint16_t *residual,
                           const uint16_t *gamma, float eps, int64_t M, int64_t H, double *R,
                           double *SR, double *Y, double *SY) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; i++) {
        double ss = 0.0;
        for (int64_t h = 0; h < H; h++) {
            double r = 0.0, sr = 0.0;
            if (residual) {
                r = bf16_value(residual[i * H + h]);
                sr = fabs(r);
            }
            for (int64_t p = 0; p < np; p++) {
                double v = bf16_value(P[(p * M + i) * H + h]);
                r += v;
                sr += fabs(v);
            }
            R[i * H + h] = r;
            SR[i * H + h] = sr;
            ss += r * r;
        }
        double denom = sqrt(ss / (double)H + (double)eps);
        for (int64_t h = 0; h < H; h++) {
            double g = bf16_value(gamma[h]);
            Y[i * H + h] = R[i * H + h] * g / denom;
            SY[i * H + h] = fabs(g) * SR[i * H + h] / denom;
        }
    }
}

/*
 * Grouped (mixture-of-experts) GEMM: rows of A are grouped by expert, rows
 * offsets[e] .. offsets[e+1]-1 belonging to expert e, and
 *   Y[t][j] = sum_{k<K} A[t][k] * W_e[j][k]   for t in expert e's rows,
 * W_e the bf16 [N,K] weight of expert e at W + e*sW (row stride ldw).  The
 * vLLM batch-invariance user guide lists mixture-of-experts layers among the
 * operations that must not change with batch composition; the row count of
 * each expert is exactly what changes with it.  Y and S are dense [T, N]
 * (T = offsets[E]); S gets sum_k |a*w|.
 */
void oracle_grouped_gemm(const uint16_t *A, int64_t lda, const uint16_t *W, int64_t ldw, int64_t sW,
                         const int64_t *offsets, int64_t E, int64_t N, int64_t K, double *Y,
                         double *S) {
    for (int64_t e = 0; e < E; e++) {
        const int64_t t0 = offsets[e], t1 = offsets[e + 1];
#pragma omp parallel for collapse(2) schedule(static)
        for (int64_t t = t0; t < t1; t++) {
            for (int64_t j = 0; j < N; j++) {
                const uint16_t *a = A + t * lda, *w = W + e * sW + j * ldw;
                double y = 0.0, s = 0.0;
                for (int64_t k = 0; k < K; k++) {
                    double p = bf16_value(a[k]) * bf16_value(w[k]);
                    y += p;
                    s += fabs(p);
                }
                Y[t * N + j] = y;
                S[t * N + j] = s;
            }
        }
    }
}

/*
 * Decode attention over a latent (MLA-absorbed) KV cache: the attention step
 * the vLLM batch-invariance tracking issue lists (MLA backends) and the
 * vLLM-Ascend guide requires to be deterministic.  Plain definition, fp64,
 * for request b with L_b cached tokens and head h:
 *   s_t = scale * sum_{d < Dqk} q[b][h][d] * kv[b][t][d],   t < L_b;
 *   p_t = exp(s_t - max_t s_t);
 *   o[b][h][c] = sum_t p_t * kv[b][t][c] / sum_t p_t,       c < Dv (Dv <= Dqk:
 *   the value is the first Dv components of the cached latent).
 * q is bf16 [B, H, Dqk] dense; kv is bf16 [B, Lmax, Dqk] dense; lens [B].
 * O and S are dense [B, H, Dv]; S gets sum_t p_t |v_t[c]| / sum_t p_t, the
 * scale of the tolerance.  A request with L_b == 0 gives O = S = 0.
 */
void oracle_mla_decode(const uint16_t *q, const uint16_t *kv, const int64_t *lens, float scale,
                       int64_t B, int64_t H, int64_t Lmax, int64_t Dqk, int64_t Dv, double *O,
                       double *S) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; b++) {
        for (int64_t h = 0; h < H; h++) {
            const int64_t L = lens[b];
            const uint16_t *qq = q + (b * H + h) * Dqk;
            double *o = O + (b * H + h) * Dv, *sv = S + (b * H + h) * Dv;
            for (int64_t c = 0; c < Dv; c++) o[c] = sv[c] = 0.0;
            if (L <= 0) continue;
            double smax = -INFINITY;
            for (int64_t t = 0; t < L; t++) {
                const uint16_t *k = kv + (b * Lmax + t) * Dqk;
                double dot = 0.0;
                for (int64_t d = 0; d < Dqk; d++) dot += bf16_value(qq[d]) * bf16_value(k[d]);
                double st = (double)scale * dot;
                if (st > smax) smax = st;
            }
            double l = 0.0;
            for (int64_t t = 0; t < L; t++) {
                const uint16_t *k = kv + (b * Lmax + t) * Dqk;
                double dot = 0.0;
                for (int64_t d = 0; d < Dqk; d++) dot += bf16_value(qq[d]) * bf16_value(k[d]);
                double pt = exp((double)scale * dot - smax);
                l += pt;
                for (int64_t c = 0; c < Dv; c++) {
                    double v = bf16_value(k[c]);
                    o[c] += pt * v;
                    sv[c] += pt * fabs(v);
                }
            }
            for (int64_t c = 0; c < Dv; c++) {
                o[c] /= l;
                sv[c] /= l;
            }
        }
    }
}

/* Number of OpenMP threads the oracle will use (for reporting). */
int oracle_num_threads(void) { return omp_get_max_threads(); }
