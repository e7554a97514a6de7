/*
 * oracle.c -- the CPU oracle of the batch-invariant matmul library.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library. It shares no code, header, table or
 * helper with the GPU library and never calls it.
 *
 * What it computes, and where the pages define it:
 *
 *  - oracle_gemm_ordered: the order contract quoted on "Reproducible GPU
 *    inference" (section "Three interventions, and what each was worth", the
 *    kernel package's module docstring): each output element is a single
 *    chain over k in increasing order, acc = acc + x*w, where every step
 *    multiplies and rounds to binary32, then adds and rounds again.
 *    "Taming Bitwise Behavior in GPU Kernels with Tensor Core" section 3.2.1
 *    describes the same scalar path (an uncontracted multiply gives two
 *    roundings per element instead of the one of an fma). The accumulator
 *    starts at +0.0f; products and sums are IEEE binary32 round to nearest
 *    even, subnormals kept. The loop nest runs m, then k, then n so the
 *    n-loop vectorises; each output still sees exactly its own chain, in
 *    ascending k, with nothing regrouped.
 *
 *  - oracle_gemm_f64 / oracle_gemm_absdot_f64: the real-number product
 *    sum_k a*w (and sum_k |a*w|), every product exact in binary64, summed
 *    ascending in binary64. This is the reference the MFMA path's error bound
 *    is stated against.
 *
 *  - oracle_gemv_tree: the tree-ordered GEMV. "Taming Bitwise Behavior in GPU
 *    Kernels with Tensor Core", section 3.2.2 (the GEMV paragraph and Figure
 *    2(d)): the lanes deal the k axis among themselves tile by tile, each
 *    taking every countth tile, fold their own tiles as a chain of fused
 *    multiply-adds, and then combine their totals through a butterfly; section
 *    5.1 pins the butterfly to offsets counting up from 1, which makes it a
 *    balanced pairwise tree whose first level adds neighbours. The tile
 *    width (8 k), the number of chains (256) and the operand layout (W given
 *    as its transpose, k contiguous) are this library's reading; they are
 *    fixed for every shape, so the order depends on K alone.
 *
 *  - oracle_freivalds_*: the float Freivalds certificate of "Same Bits on the
 *    CPU and the GPU" (section "The CPU as a checker: a float Freivalds
 *    certificate"): a +-1 vector r, the product of r with W precomputed once
 *    per matrix in binary64, and a residual |r.y - (rW).x| compared with a
 *    bound.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math (no -march, so x86-64 SSE2,
 * which has no fused multiply-add); ORACLE_SRC_SHA256 is the SHA-256 of this
 * file, baked in by the build script so a test can prove which source a
 * library was built from.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifndef ORACLE_SRC_SHA256
#define ORACLE_SRC_SHA256 "unknown"
#endif

const char *oracle_source_sha256(void) { return ORACLE_SRC_SHA256; }

/* bfloat16 is the top half of a binary32: widening is a 16-bit shift. */
static float widen_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* a_dtype: 0 = bfloat16 bit patterns, 1 = binary32. */
static float load_a(const void *A, int a_dtype, int64_t i)
{
    if (a_dtype == 0)
        return widen_bf16(((const uint16_t *)A)[i]);
    return ((const float *)A)[i];
}

static double load_a64(const void *A, int a_dtype, int64_t i)
{
    return (double)load_a(A, a_dtype, i);
}

/*
 * C[m, n] = fold over k = 0 .. K-1 of acc = fl(acc + fl(a[m,k] * w[k,n])),
 * acc = +0.0f at the start. A is [M, K] with row stride lda, W is [K, N]
 * bfloat16 with row stride ldw, C is [M, N] binary32 with row stride ldc.
 */
void oracle_gemm_ordered(const void *A, int a_dtype, int64_t lda,
                         const uint16_t *W, int64_t ldw,
                         float *C, int64_t ldc,
                         int64_t M, int64_t N, int64_t K)
{
    for (int64_t m = 0; m < M; ++m) {
        float *acc = C + m * ldc;
        for (int64_t n = 0; n < N; ++n)
            acc[n] = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            const float a = load_a(A, a_dtype, m * lda + k);
            const uint16_t *wrow = W + k * ldw;
            for (int64_t n = 0; n < N; ++n) {
                const float p = a * widen_bf16(wrow[n]);   /* first rounding  */
                acc[n] = acc[n] + p;                        /* second rounding */
            }
        }
    }
}

/* D[m, n] = sum_k a[m,k] * w[k,n] in binary64, ascending k (products exact). */
void oracle_gemm_f64(const void *A, int a_dtype, int64_t lda,
                     const uint16_t *W, int64_t ldw,
                     double *D, int64_t ldd,
                     int64_t M, int64_t N, int64_t K)
{
    for (int64_t m = 0; m < M; ++m) {
        double *d = D + m * ldd;
        for (int64_t n = 0; n < N; ++n)
            d[n] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = load_a64(A, a_dtype, m * lda + k);
            const uint16_t *wrow = W + k * ldw;
            for (int64_t n = 0; n < N; ++n)
                d[n] += a * (double)widen_bf16(wrow[n]);
        }
    }
}

/* S[m, n] = sum_k |a[m,k] * w[k,n]| in binary64 (the scale of the error bound). */
void oracle_gemm_absdot_f64(const void *A, int a_dtype, int64_t lda,
                            const uint16_t *W, int64_t ldw,
                            double *S, int64_t lds,
                            int64_t M, int64_t N, int64_t K)
{
    for (int64_t m = 0; m < M; ++m) {
        double *s = S + m * lds;
        for (int64_t n = 0; n < N; ++n)
            s[n] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = fabs(load_a64(A, a_dtype, m * lda + k));
            const uint16_t *wrow = W + k * ldw;
            for (int64_t n = 0; n < N; ++n)
                s[n] += a * fabs((double)widen_bf16(wrow[n]));
        }
    }
}

/*
 * Tree-ordered GEMV. x is [M, K] bfloat16 (row stride ldx), WT is the weight
 * transposed, [N, K] bfloat16 (row stride ldwt), y is [M, N] binary32.
 *
 * Tile t holds k = 8t .. 8t+7 (the last tile stops at K). Chain p, for
 * p = 0 .. 255, takes the tiles t = p, p + 256, p + 512, ... in ascending
 * order and folds every k of them in ascending order as
 *     acc = fmaf(x[m,k], WT[n,k], acc),   acc = +0.0f at the start,
 * one rounding per step (fmaf is the correctly rounded C99 fused
 * multiply-add). A chain with no tiles stays +0.0f. Then the 256 chain totals
 * are reduced by halving: level 1 forms part[2i] + part[2i+1], level 2 adds
 * neighbouring level-1 sums, ..., and level 8 gives y[m, n]. Every addition
 * rounds to binary32 (nearest even).
 */
#define TREE_TILE 8
#define TREE_CHAINS 256

void oracle_gemv_tree(const uint16_t *x, int64_t ldx,
                      const uint16_t *WT, int64_t ldwt,
                      float *y, int64_t ldy,
                      int64_t M, int64_t N, int64_t K)
{
    float part[TREE_CHAINS];
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *xr = x + m * ldx;
        for (int64_t n = 0; n < N; ++n) {
            const uint16_t *wr = WT + n * ldwt;
            for (int64_t p = 0; p < TREE_CHAINS; ++p) {
                float acc = 0.0f;
                for (int64_t t = p; t * TREE_TILE < K; t += TREE_CHAINS) {
                    const int64_t k0 = t * TREE_TILE;
                    const int64_t k1 = k0 + TREE_TILE < K ? k0 + TREE_TILE : K;
                    for (int64_t k = k0; k < k1; ++k)
                        acc = fmaf(widen_bf16(xr[k]), widen_bf16(wr[k]), acc);
                }
                part[p] = acc;
            }
            for (int64_t width = TREE_CHAINS; width > 1; width /= 2)
                for (int64_t i = 0; i < width / 2; ++i)
                    part[i] = part[2 * i] + part[2 * i + 1];
            y[m * ldy + n] = part[0];
        }
    }
}

/*
 * Freivalds precompute, once per matrix. With y = x W (y over the output
 * index n), the certificate's "r^T W" is the K-vector s = W r:
 *   s[k] = sum_n w[k,n] * r[n],   q[k] = ||w[k,:]||_2,   a[k] = sum_n |w[k,n]|.
 */
void oracle_freivalds_prepare(const uint16_t *W, int64_t ldw, int64_t K, int64_t N,
                              const int8_t *r, double *s, double *q, double *a)
{
    for (int64_t k = 0; k < K; ++k) {
        double ss = 0.0, qq = 0.0, aa = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double w = (double)widen_bf16(W[k * ldw + n]);
            ss += w * (double)r[n];
            qq += w * w;
            aa += fabs(w);
        }
        s[k] = ss;
        q[k] = sqrt(qq);
        a[k] = aa;
    }
}

/*
 * One check of one sampled output row y (length N) against its input row x
 * (length K, bfloat16):
 *   rho   = | sum_n r[n] y[n] - sum_k x[k] s[k] |
 *   sigma = 2^-24 * sqrt(K) * sum_k |x[k]| q[k]
 *   tau   = c_f * sigma
 *   bound = gamma_{K-1} * sum_k |x[k]| a[k] + host rounding allowance
 * Returns 1 (accept) when rho <= tau, else 0. out[0..3] = rho, sigma, tau, bound.
 */
int oracle_freivalds_check(const double *s, const double *q, const double *a,
                           const int8_t *r, int64_t K, int64_t N,
                           const uint16_t *x, const float *y, double c_f,
                           double *out)
{
    double ry = 0.0, xs = 0.0, sxq = 0.0, sxa = 0.0, mag = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        ry += (double)r[n] * (double)y[n];
        mag += fabs((double)y[n]);
    }
    for (int64_t k = 0; k < K; ++k) {
        const double xk = (double)widen_bf16(x[k]);
        xs += xk * s[k];
        sxq += fabs(xk) * q[k];
        sxa += fabs(xk) * a[k];
        mag += fabs(xk * s[k]);
    }
    const double u = ldexp(1.0, -24);
    const double km1 = (double)(K > 0 ? K - 1 : 0);
    const double gamma = km1 * u / (1.0 - km1 * u);
    const double rho = fabs(ry - xs);
    const double sigma = u * sqrt((double)K) * sxq;
    const double tau = c_f * sigma;
    const double bound = gamma * sxa + 2.0 * (double)(N + K) * ldexp(1.0, -53) * mag;
    out[0] = rho;
    out[1] = sigma;
    out[2] = tau;
    out[3] = bound;
    return rho <= tau ? 1 : 0;
}
