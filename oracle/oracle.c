/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for the fused-chain
 * hot path.  TEST INFRASTRUCTURE ONLY: tests, the smoke check and the CPU
 * baseline leg of the benchmark call it; the product path never does.  It
 * shares no code, header or constant table with the HIP library.
 *
 * Everything is computed in fp64 from the exact values of the stored inputs
 * (fp32, fp16 or bf16 bits).  No blocking, no fusion, no reordering beyond
 * the plain definitions below.  Built with gcc -O2 -ffp-contract=off so the
 * compiler does not fuse the fp64 multiply-adds written here.
 *
 * Sources (the three pages on vertical fusion):
 *  - "C-05. Kernel Fusion 代价边界", section 3 (API / experiment form): the
 *    stage operation y = a_s*y + b_s with ReLU on even stages; naive, fused
 *    and fat forms all compute this same chain.
 *  - "K4 讲解：fusion 的三笔账", section 1 (the four split plans): the chain
 *    mm -> bias -> gelu -> residual on [M,N] outputs.
 *  - "AIGC 基本功｜算子融合与 CUDA Graph-Fusion", section 3.5 (causal mask:
 *    query i sees keys j <= i) and the appendix's attention-tail section (the
 *    max / subtract / exp / sum / divide softmax steps).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

/* ------------------------------------------------------------ storage decode */

/* IEEE binary16 -> double, written out field by field (exact). */
static double half_bits_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal or zero */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 -> double: the bits are the top half of an fp32 word (exact). */
static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_half_to_double(uint16_t h) { return half_bits_to_double(h); }
double oracle_bf16_to_double(uint16_t b) { return bf16_bits_to_double(b); }

/* ------------------------------------------------------------ pointwise chain */

/*
 * K-stage pointwise chain ("C-05", section 3): for s = 0 .. K-1,
 *   y = a_s * y + b_s, then y = max(y, 0) when relu_even and s is even
 * (stages counted from 0, the fused loop's own index).  fp64 throughout.
 */
void oracle_chain_f64(const float *x, double *y, int64_t n,
                      const float *a, const float *b, int K, int relu_even)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double v = (double)x[i];
        for (int s = 0; s < K; ++s) {
            v = (double)a[s] * v + (double)b[s];
            if (relu_even && (s % 2) == 0 && v < 0.0)
                v = 0.0;
        }
        y[i] = v;
    }
}

/*
 * The same chain evaluated in fp32 with exactly one rounding per stage (a
 * correctly rounded fused multiply-add), the precision the chain's data is
 * stored in.  fmaf() from libm is correctly rounded, so this predicts the
 * bits of any fp32 implementation that also rounds once per stage.
 */
void oracle_chain_f32fma(const float *x, float *y, int64_t n,
                         const float *a, const float *b, int K, int relu_even)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float v = x[i];
        for (int s = 0; s < K; ++s) {
            v = fmaf(a[s], v, b[s]);
            if (relu_even && (s % 2) == 0 && v < 0.0f)
                v = 0.0f;
        }
        y[i] = v;
    }
}

/* ------------------------------------------------------------ fat-probe sink */

/*
 * The fat row of "C-05", section 3 (API table): the fused chain plus T live
 * temporaries per thread, added into a sink so that none can be dropped.  The
 * pages give the idea, not a formula; the formula read here is:
 *  - elements go in vectors of four, v = x[4q .. 4q+3], q = 0 .. n/4 - 1; the
 *    n mod 4 trailing elements are not part of any vector and never reach the
 *    sink;
 *  - vector q belongs to lane q mod L of the L lanes of the launch, and a lane
 *    visits its vectors in increasing q;
 *  - for one element with chain values y_s (after stage s and its ReLU):
 *      t_{-1} = 0,  t_j = t_{j-1} / 2 + y_{s(j)},  s(j) = floor(j K / T),
 *      j = 0 .. T-1, and the element's term is t_0 + t_1 + ... + t_{T-1};
 *  - sink[4 lane + c] = sum of the terms of component c over the lane's vectors.
 * T = 0 leaves the sink zero.  L, the lane count, is the launch's.
 */
static void fat_lane_f64(const float *x, int64_t nvec, const float *a, const float *b, int K,
                         int relu_even, int T, int64_t lanes, int64_t lane, double *sink,
                         double *abs_sink)
{
    for (int c = 0; c < 4; ++c) {
        double acc = 0.0, acc_abs = 0.0;
        for (int64_t q = lane; q < nvec; q += lanes) {
            double y = (double)x[4 * q + c];
            double t = 0.0, term = 0.0, term_abs = 0.0;
            int j = 0;
            for (int s = 0; s < K; ++s) {
                y = (double)a[s] * y + (double)b[s];
                if (relu_even && (s % 2) == 0 && y < 0.0)
                    y = 0.0;
                for (; j < T && ((int64_t)j * K) / T == s; ++j) {
                    t = 0.5 * t + y;
                    term += t;
                    term_abs += fabs(t);
                }
            }
            acc += term;
            acc_abs += term_abs;
        }
        sink[4 * lane + c] = acc;
        if (abs_sink)
            abs_sink[4 * lane + c] = acc_abs;
    }
}

/* fp64 sink (and, if abs_sink is not NULL, the same sums of |t_j|, the scale
 * of the rounding error of any fp32 evaluation).  sink: 4 * lanes doubles. */
void oracle_chain_fat_sink_f64(const float *x, int64_t n, const float *a, const float *b, int K,
                               int relu_even, int T, int64_t lanes, double *sink,
                               double *abs_sink)
{
    #pragma omp parallel for schedule(static)
    for (int64_t lane = 0; lane < lanes; ++lane)
        fat_lane_f64(x, n / 4, a, b, K, relu_even, T, lanes, lane, sink, abs_sink);
}

/*
 * The same sink evaluated the way a single-precision thread evaluates it: one
 * correctly rounded fmaf per chain stage, t_j = fmaf(0.5, t_{j-1}, y_{s(j)}),
 * the element's terms added from the last one back,
 * t_0 + (t_1 + (... + (t_{T-2} + t_{T-1}))), and the lane's running fp32 sum
 * taking one term per vector in visiting order.  Every operation is a single
 * IEEE rounding, so this predicts the bits of any evaluation in that order.
 */
void oracle_chain_fat_sink_f32(const float *x, int64_t n, const float *a, const float *b, int K,
                               int relu_even, int T, int64_t lanes, float *sink)
{
    const int64_t nvec = n / 4;
    #pragma omp parallel
    {
        float *t = (float *)malloc((size_t)(T > 0 ? T : 1) * sizeof(float));
        #pragma omp for schedule(static)
        for (int64_t lane = 0; lane < lanes; ++lane) {
            for (int c = 0; c < 4; ++c) {
                float acc = 0.0f;
                for (int64_t q = lane; q < nvec && t; q += lanes) {
                    float y = x[4 * q + c];
                    float prev = 0.0f;
                    int j = 0;
                    for (int s = 0; s < K; ++s) {
                        y = fmaf(a[s], y, b[s]);
                        if (relu_even && (s % 2) == 0 && y < 0.0f)
                            y = 0.0f;
                        for (; j < T && ((int64_t)j * K) / T == s; ++j) {
                            prev = fmaf(0.5f, prev, y);
                            t[j] = prev;
                        }
                    }
                    if (T > 0) {
                        float r = t[T - 1];
                        for (int jj = T - 2; jj >= 0; --jj)
                            r = t[jj] + r;
                        acc = acc + r;
                    }
                }
                sink[4 * lane + c] = t ? acc : NAN;
            }
        }
        free(t);
    }
}

/* ------------------------------------------------------------ GEMM + epilogue */

/* GELU in its erf form: z * Phi(z) = 0.5 * z * (1 + erf(z / sqrt(2))). */
double oracle_gelu(double z)
{
    return 0.5 * z * (1.0 + erf(z / sqrt(2.0)));
}

/* C[i,j] = sum_k A[i,k] * B[k,j]; A [M,K], B [K,N] fp16 row-major. */
static double dot_f16(const uint16_t *A, const uint16_t *B,
                      int64_t N, int64_t K, int64_t i, int64_t j)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
        acc += half_bits_to_double(A[i * K + k]) * half_bits_to_double(B[k * N + j]);
    return acc;
}

void oracle_gemm_f64(const uint16_t *A, const uint16_t *B,
                     int64_t M, int64_t N, int64_t K, double *C)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            C[i * N + j] = dot_f16(A, B, N, K, i, j);
}

/*
 * The four-stage chain of "K4 讲解", section 1, on one output element:
 *   C = A.B ; C' = C + bias[j] ; C'' = GELU(C') ; Y = C'' + R[i,j].
 */
static double epilogue_of(double c, const uint16_t *bias, const uint16_t *R,
                          int64_t N, int64_t i, int64_t j)
{
    double c1 = c + half_bits_to_double(bias[j]);
    double c2 = oracle_gelu(c1);
    return c2 + half_bits_to_double(R[i * N + j]);
}

static double epilogue_at(const uint16_t *A, const uint16_t *B,
                          const uint16_t *bias, const uint16_t *R,
                          int64_t N, int64_t K, int64_t i, int64_t j)
{
    return epilogue_of(dot_f16(A, B, N, K, i, j), bias, R, N, i, j);
}

void oracle_gemm_epilogue_f64(const uint16_t *A, const uint16_t *B,
                              const uint16_t *bias, const uint16_t *R,
                              int64_t M, int64_t N, int64_t K, double *Y)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            Y[i * N + j] = epilogue_at(A, B, bias, R, N, K, i, j);
}

/* The chain's last three stages on a product C = A.B (fp64 [M,N]) that the
 * caller formed with a library matrix product: Y = GELU(C + bias) + R. */
void oracle_epilogue_on_product_f64(const double *C, const uint16_t *bias, const uint16_t *R,
                                    int64_t M, int64_t N, double *Y)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            Y[i * N + j] = epilogue_of(C[i * N + j], bias, R, N, i, j);
}

/* Same chain at cnt sampled (row, col) positions. */
void oracle_gemm_epilogue_at(const uint16_t *A, const uint16_t *B,
                             const uint16_t *bias, const uint16_t *R,
                             int64_t M, int64_t N, int64_t K,
                             const int64_t *rows, const int64_t *cols,
                             int64_t cnt, double *out)
{
    (void)M;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < cnt; ++t)
        out[t] = epilogue_at(A, B, bias, R, N, K, rows[t], cols[t]);
}

/* ------------------------------------------------------------ causal softmax */

/*
 * One row of the causal scaled softmax: query i of a [S,S] score block sees
 * keys j <= i ("AIGC 基本功", section 3.5).  With z_j = scale * s_j:
 *   m = max_{j<=i} z_j ; l = sum_{j<=i} exp(z_j - m) ;
 *   out_j = exp(z_j - m) / l for j <= i, and exactly 0 for j > i.
 */
static void softmax_row(const uint16_t *srow, int64_t S, int64_t i,
                        double scale, double *orow)
{
    double m = -INFINITY;
    for (int64_t j = 0; j <= i; ++j) {
        double z = scale * bf16_bits_to_double(srow[j]);
        if (z > m)
            m = z;
    }
    double l = 0.0;
    for (int64_t j = 0; j <= i; ++j)
        l += exp(scale * bf16_bits_to_double(srow[j]) - m);
    for (int64_t j = 0; j < S; ++j)
        orow[j] = (j <= i) ? exp(scale * bf16_bits_to_double(srow[j]) - m) / l : 0.0;
}

/*
 * scores: bf16 bits [BH, S, S]; row_ids index flattened rows r = bh*S + i;
 * out: nrows x S doubles.
 */
void oracle_causal_softmax_rows(const uint16_t *scores, int64_t S, double scale,
                                const int64_t *row_ids, int64_t nrows, double *out)
{
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = 0; t < nrows; ++t) {
        int64_t r = row_ids[t];
        int64_t i = r % S;
        softmax_row(scores + r * S, S, i, scale, out + t * S);
    }
}

void oracle_causal_softmax_f64(const uint16_t *scores, int64_t BH, int64_t S,
                               double scale, double *out)
{
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < BH * S; ++r)
        softmax_row(scores + r * S, S, r % S, scale, out + r * S);
}

/* ------------------------------------------------------------ causal attention */

/*
 * Causal scaled dot-product attention, the chain the pages' score tensor sits
 * in ("AIGC 基本功", section 3.5: query i sees keys j <= i; the attention-tail
 * section: scale, mask, softmax; and its further-reading list, which names the
 * online-softmax kernel that never materialises the scores as the way to
 * remove that tensor).  Its result is plain attention, written out here:
 *   z_j = scale * sum_d Q[i][d] K[j][d]          for j <= i
 *   m = max_j z_j ; p_j = exp(z_j - m) ; l = sum_j p_j
 *   O[i][d] = sum_j p_j V[j][d] / l
 * Q, K, V: bf16 bits [BH, S, D] row-major; values decoded exactly to fp64.
 */
static void attention_row(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                          int64_t S, int64_t D, int64_t bh, int64_t i, double scale,
                          double *z, double *orow)
{
    const uint16_t *q = Q + (bh * S + i) * D;
    double m = -INFINITY;
    for (int64_t j = 0; j <= i; ++j) {
        const uint16_t *k = K + (bh * S + j) * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d)
            dot += bf16_bits_to_double(q[d]) * bf16_bits_to_double(k[d]);
        z[j] = scale * dot;
        if (z[j] > m)
            m = z[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j <= i; ++j) {
        z[j] = exp(z[j] - m);
        l += z[j];
    }
    for (int64_t d = 0; d < D; ++d)
        orow[d] = 0.0;
    for (int64_t j = 0; j <= i; ++j) {
        const uint16_t *v = V + (bh * S + j) * D;
        for (int64_t d = 0; d < D; ++d)
            orow[d] += z[j] * bf16_bits_to_double(v[d]);
    }
    for (int64_t d = 0; d < D; ++d)
        orow[d] /= l;
}

/* Rows r = bh*S + i of O for the listed row ids; out: nrows x D doubles.
 * Returns 0, or -1 if a row's score buffer cannot be allocated. */
int oracle_causal_attention_rows(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                                 int64_t S, int64_t D, double scale,
                                 const int64_t *row_ids, int64_t nrows, double *out)
{
    int failed = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int64_t t = 0; t < nrows; ++t) {
        int64_t r = row_ids[t];
        double *z = (double *)malloc((size_t)(r % S + 1) * sizeof(double));
        if (!z) {
            failed = 1;
            continue;
        }
        attention_row(Q, K, V, S, D, r / S, r % S, scale, z, out + t * D);
        free(z);
    }
    return failed ? -1 : 0;
}

/* ------------------------------------------------------------ RMSNorm */

/*
 * RMSNorm of each row ("AIGC 基本功", section 3.2 byte ledger and the
 * appendix ledger's RMSNorm entry: square, mean, multiply by the reciprocal
 * root, multiply by the gain):
 *   y[i][j] = x[i][j] / sqrt(mean_j x[i][j]^2 + eps) * g[j]
 * x: fp32 [rows, d]; g: fp32 [d]; y: fp64 [rows, d].
 */
void oracle_rmsnorm_f64(const float *x, const float *g, int64_t rows, int64_t d, double eps,
                        double *y)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        const float *xr = x + i * d;
        double ss = 0.0;
        for (int64_t j = 0; j < d; ++j)
            ss += (double)xr[j] * (double)xr[j];
        const double r = sqrt(ss / (double)d + eps);
        for (int64_t j = 0; j < d; ++j)
            y[i * d + j] = (double)xr[j] / r * (double)g[j];
    }
}
