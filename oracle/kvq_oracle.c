/*
 * kvq_oracle.c -- plain, slow CPU reference of the rotate-then-quantize KV
 * cache path.  TEST INFRASTRUCTURE ONLY: it is built and called by the tests,
 * by the smoke check and by the CPU-baseline leg of the benchmark, never by the
 * library.  It shares no source, header, table or constant with the GPU path.
 *
 * All arithmetic is IEEE double.  Inputs arrive as doubles (fp16 inputs are
 * widened exactly by the caller).  Every routine follows the step order of
 * the method as the pages state it; no blocking, fusion or reordering.
 *
 * Sources (page title / section):
 *  - "PolarQuant: Optimal Gaussian Weight Quantization via Hadamard Rotation"
 *    (gist.science 2603.29078), Technical summary sec. 2 "Methodology":
 *    block L2 normalisation keeping the norm r_i, normalised Walsh-Hadamard
 *    rotation, scaling to unit variance, Lloyd-Max centroids for N(0,1);
 *    dequantisation = centroid lookup, scale, Hadamard (self-inverse), norm.
 *  - "O Que E TurboQuant?" (a2a-mcp.org), "Como Funciona", Stage 1 (random
 *    rotation, per-coordinate Lloyd-Max codes) and Stage 2 (1-bit QJL sign
 *    residual that corrects inner-product bias); "Como Implementar" (codebooks
 *    precomputed per dimension and bit width; query rotated once, scores read
 *    from the indices).
 *  - "NSNQuant: A Double Normalization Approach ..." (gist.science
 *    2505.18231), Technical summary "Metodologia" sec. 1 (Normalize-Shift-
 *    Normalize with byproducts s1, o, s2), sec. 2 (Hadamard), sec. 3 (one
 *    global codebook for N(0,1), k-means on synthetic normal samples).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  rotation y = H (D .* u) with the unnormalised +-1 Sylvester matrix
 *  H_ij = (-1)^popcount(i&j) on the unit vector u, which gives coordinates of
 *  unit variance; bucket index = #{j : t_j < y}; codes packed LSB-first per
 *  vector (coordinate i in bits [b*i, b*i+b)); zero vector -> u = 0.
 */
#define _DEFAULT_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* Standard normal density and probability mass                              */
/* ------------------------------------------------------------------------ */

static double npdf(double x)
{
    if (isinf(x)) return 0.0;
    return exp(-0.5 * x * x) / sqrt(2.0 * M_PI);
}

/* P(a < X < b) for X ~ N(0,1), written so that tail masses do not cancel. */
static double nmass(double a, double b)
{
    const double r2 = sqrt(2.0);
    if (a >= 0.0) return 0.5 * (erfc(a / r2) - erfc(b / r2));
    if (b <= 0.0) return 0.5 * (erfc(-b / r2) - erfc(-a / r2));
    return 1.0 - 0.5 * erfc(-a / r2) - 0.5 * erfc(b / r2);
}

/* ------------------------------------------------------------------------ */
/* Lloyd-Max scalar quantiser for N(0,1)                                      */
/* Lloyd's two optimality conditions iterated to their fixed point:           */
/*   thresholds t_j = (c_j + c_{j+1}) / 2                                     */
/*   centroids  c_j = E[X | t_{j-1} < X < t_j]                                */
/*             = (phi(t_{j-1}) - phi(t_j)) / (Phi(t_j) - Phi(t_{j-1}))        */
/* ------------------------------------------------------------------------ */

ORC_API int kvqo_lloyd_max(int bits, const double *init, int max_iter, double tol,
                           double *c_out, int *iters_out)
{
    if (bits < 1 || bits > 8) return -1;
    const int L = 1 << bits;
    double *c = (double *)malloc(sizeof(double) * L);
    double *t = (double *)malloc(sizeof(double) * (L + 1));
    for (int j = 0; j < L; ++j)
        c[j] = init ? init[j] : (-2.5 + 5.0 * (j + 0.5) / L);
    int it = 0;
    for (; it < max_iter; ++it) {
        t[0] = -INFINITY;
        t[L] = INFINITY;
        for (int j = 1; j < L; ++j) t[j] = 0.5 * (c[j - 1] + c[j]);
        double delta = 0.0;
        for (int j = 0; j < L; ++j) {
            double m = nmass(t[j], t[j + 1]);
            double cn = (npdf(t[j]) - npdf(t[j + 1])) / m;
            double dd = fabs(cn - c[j]);
            if (dd > delta) delta = dd;
            c[j] = cn;
        }
        if (delta < tol) { ++it; break; }
    }
    memcpy(c_out, c, sizeof(double) * L);
    if (iters_out) *iters_out = it;
    free(c);
    free(t);
    return 0;
}

/* Mean squared error of a scalar quantiser (levels c, decision thresholds t
 * between them) on N(0,1), by the exact integral per cell:
 *   int_a^b (x-c)^2 phi = (1+c^2) dPhi - 2c (phi(a)-phi(b)) + a phi(a) - b phi(b)
 */
ORC_API double kvqo_gauss_mse(int bits, const double *c, const double *t)
{
    const int L = 1 << bits;
    double mse = 0.0;
    for (int j = 0; j < L; ++j) {
        double a = (j == 0) ? -INFINITY : t[j - 1];
        double b = (j == L - 1) ? INFINITY : t[j];
        double pa = npdf(a), pb = npdf(b);
        double apa = isinf(a) ? 0.0 : a * pa;
        double bpb = isinf(b) ? 0.0 : b * pb;
        mse += (1.0 + c[j] * c[j]) * nmass(a, b) - 2.0 * c[j] * (pa - pb) + apa - bpb;
    }
    return mse;
}

/* Canonical stored tables: centroids rounded to fp32; thresholds are the
 * fp32 rounding of the midpoint of adjacent fp32 centroids (computed in
 * double, where the sum of two floats is exact). */
ORC_API int kvqo_tables_f32(int bits, float *c32, float *t32)
{
    const int L = 1 << bits;
    double c[256];
    int rc = kvqo_lloyd_max(bits, NULL, 1000000, 1e-13, c, NULL);
    if (rc) return rc;
    for (int j = 0; j < L; ++j) c32[j] = (float)c[j];
    for (int j = 0; j + 1 < L; ++j)
        t32[j] = (float)(((double)c32[j] + (double)c32[j + 1]) * 0.5);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Lloyd-Max for the exact coordinate law at dimension d ("O Que E           */
/* TurboQuant?", Como Funciona, Estagio 1: after the rotation each coordinate */
/* of the unit vector follows Beta((d-1)/2, (d-1)/2) on [-1, 1]; the Lloyd-Max */
/* quantiser is optimised for that law).  With the coordinates scaled by      */
/* sqrt(d) to unit variance, the density on [-sqrt d, sqrt d] is proportional */
/* to g(y) = (1 - y^2/d)^((d-3)/2).  Cell integrals:                          */
/*   m0(a, b) = int_a^b g: F(b) - F(a), F tabulated on a grid of step 1/512   */
/*              by 8-point Gauss-Legendre per step, plus Gauss-Legendre over  */
/*              the partial step;                                             */
/*   m1(a, b) = int_a^b y g = d/(d-1) [G(a) - G(b)], G(y) = (1 - y^2/d)^((d-1)/2). */
/* ------------------------------------------------------------------------ */

static const double kGLx[4] = {0.1834346424956498, 0.5255324099163290, 0.7966664774136267, 0.9602898564975363};
static const double kGLw[4] = {0.3626837833783620, 0.3137066458778873, 0.2223810344533745, 0.1012285362903763};

typedef struct {
    int d;
    double r, h;   /* support radius sqrt(d), grid step */
    int n;         /* grid points */
    double *F;     /* F[i] = int_{-r}^{-r + i h} g */
} beta_law;

static double beta_g(const beta_law *B, double y)
{
    const double u = 1.0 - y * y / B->d;
    return u <= 0.0 ? 0.0 : pow(u, 0.5 * (B->d - 3));
}

static double beta_gl(const beta_law *B, double a, double b)
{
    const double m = 0.5 * (a + b), hw = 0.5 * (b - a);
    double s = 0.0;
    for (int k = 0; k < 4; ++k) s += kGLw[k] * (beta_g(B, m - hw * kGLx[k]) + beta_g(B, m + hw * kGLx[k]));
    return s * hw;
}

static int beta_init(beta_law *B, int d)
{
    B->d = d;
    B->r = sqrt((double)d);
    B->h = 1.0 / 512.0;
    B->n = (int)ceil(2.0 * B->r / B->h) + 1;
    B->F = (double *)malloc(sizeof(double) * B->n);
    if (!B->F) return -1;
    B->F[0] = 0.0;
    for (int i = 1; i < B->n; ++i) {
        const double a = -B->r + (i - 1) * B->h;
        double b = a + B->h;
        if (b > B->r) b = B->r;
        B->F[i] = B->F[i - 1] + beta_gl(B, a, b);
    }
    return 0;
}

static double beta_F(const beta_law *B, double y)
{
    if (y <= -B->r) return 0.0;
    if (y >= B->r) y = B->r;
    int i = (int)floor((y + B->r) / B->h);
    if (i >= B->n - 1) i = B->n - 2;
    const double y0 = -B->r + i * B->h;
    return B->F[i] + beta_gl(B, y0, y);
}

static double beta_G(const beta_law *B, double y)
{
    const double u = 1.0 - y * y / B->d;
    return u <= 0.0 ? 0.0 : pow(u, 0.5 * (B->d - 1));
}

/* Total mass Z = int g over the support, also in closed form:
 * sqrt(d) B(1/2, (d-1)/2) (exposed for the tests). */
ORC_API double kvqo_beta_mass(int d, double a, double b)
{
    beta_law B;
    if (d < 4 || beta_init(&B, d)) return -1.0;
    const double m = beta_F(&B, b) - beta_F(&B, a);
    free(B.F);
    return m;
}

/* Centroids c[2^bits] (fp64) of the Lloyd-Max quantiser for the law above;
 * start from uniform levels on [-2.5, 2.5], iterate until max |dc| < tol. */
ORC_API int kvqo_lloyd_max_beta(int bits, int d, int max_iter, double tol, double *c_out, int *iters_out)
{
    if (bits < 1 || bits > 8 || d < 4) return -1;
    beta_law B;
    if (beta_init(&B, d)) return -1;
    const int L = 1 << bits;
    double c[256], t[257];
    for (int j = 0; j < L; ++j) c[j] = -2.5 + 5.0 * (j + 0.5) / L;
    const double k1 = (double)d / (d - 1);
    int it = 0;
    for (; it < max_iter; ++it) {
        t[0] = -B.r;
        t[L] = B.r;
        for (int j = 1; j < L; ++j) t[j] = 0.5 * (c[j - 1] + c[j]);
        double delta = 0.0;
        for (int j = 0; j < L; ++j) {
            const double m0 = beta_F(&B, t[j + 1]) - beta_F(&B, t[j]);
            const double m1 = k1 * (beta_G(&B, t[j]) - beta_G(&B, t[j + 1]));
            const double cn = m1 / m0;
            if (fabs(cn - c[j]) > delta) delta = fabs(cn - c[j]);
            c[j] = cn;
        }
        if (delta < tol) { ++it; break; }
    }
    memcpy(c_out, c, sizeof(double) * L);
    if (iters_out) *iters_out = it;
    free(B.F);
    return 0;
}

/* Mean squared error of quantiser (c, t) under the law, per coordinate:
 * sum_j int_{t_{j-1}}^{t_j} (y - c_j)^2 g / Z, with int y^2 g by Gauss-Legendre. */
ORC_API double kvqo_beta_mse(int bits, int d, const double *c, const double *t)
{
    beta_law B;
    if (beta_init(&B, d)) return -1.0;
    const int L = 1 << bits;
    const double Z = B.F[B.n - 1];
    double mse = 0.0;
    for (int j = 0; j < L; ++j) {
        const double a = j == 0 ? -B.r : t[j - 1], b = j == L - 1 ? B.r : t[j];
        /* int (y - c)^2 g over [a, b], panel by panel */
        const int np = (int)ceil((b - a) / B.h) + 1;
        const double hp = (b - a) / np;
        double s = 0.0;
        for (int p = 0; p < np; ++p) {
            const double pa = a + p * hp, m = pa + 0.5 * hp, hw = 0.5 * hp;
            for (int k = 0; k < 4; ++k) {
                const double y0 = m - hw * kGLx[k], y1 = m + hw * kGLx[k];
                s += kGLw[k] * hw * ((y0 - c[j]) * (y0 - c[j]) * beta_g(&B, y0) + (y1 - c[j]) * (y1 - c[j]) * beta_g(&B, y1));
            }
        }
        mse += s;
    }
    free(B.F);
    return mse / Z;
}

/* Canonical fp32 tables of the law, rounded as kvqo_tables_f32 rounds. */
ORC_API int kvqo_tables_f32_beta(int bits, int d, float *c32, float *t32)
{
    const int L = 1 << bits;
    double c[256];
    int rc = kvqo_lloyd_max_beta(bits, d, 1000000, 1e-13, c, NULL);
    if (rc) return rc;
    for (int j = 0; j < L; ++j) c32[j] = (float)c[j];
    for (int j = 0; j + 1 < L; ++j)
        t32[j] = (float)(((double)c32[j] + (double)c32[j + 1]) * 0.5);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Walsh-Hadamard                                                             */
/* ------------------------------------------------------------------------ */

static int popcount_u32(uint32_t v)
{
    int n = 0;
    while (v) { n += (int)(v & 1u); v >>= 1; }
    return n;
}

/* Dense Sylvester matrix entry H_ij = (-1)^popcount(i & j). */
ORC_API int kvqo_hadamard_entry(int i, int j)
{
    return (popcount_u32((uint32_t)(i & j)) & 1) ? -1 : 1;
}

/* y = H x with the dense matrix (n^2 work). */
ORC_API void kvqo_hadamard_dense(const double *x, double *y, int n)
{
    for (int i = 0; i < n; ++i) {
        double s = 0.0;
        for (int j = 0; j < n; ++j) s += kvqo_hadamard_entry(i, j) * x[j];
        y[i] = s;
    }
}

/* In-place fast transform: log2(n) butterfly stages, natural order.  Gives
 * the same vector as kvqo_hadamard_dense. */
ORC_API void kvqo_fwht(double *x, int n)
{
    for (int h = 1; h < n; h <<= 1)
        for (int i = 0; i < n; i += 2 * h)
            for (int j = i; j < i + h; ++j) {
                double a = x[j], b = x[j + h];
                x[j] = a + b;
                x[j + h] = a - b;
            }
}

/* ------------------------------------------------------------------------ */
/* Bit packing: LSB-first stream per vector.                                  */
/* ------------------------------------------------------------------------ */

ORC_API void kvqo_pack(const int32_t *idx, int d, int bits, uint8_t *rec)
{
    memset(rec, 0, (size_t)(d * bits + 7) / 8);
    for (int i = 0; i < d; ++i)
        for (int k = 0; k < bits; ++k) {
            int p = i * bits + k;
            if ((idx[i] >> k) & 1) rec[p / 8] |= (uint8_t)(1u << (p % 8));
        }
}

ORC_API void kvqo_unpack(const uint8_t *rec, int d, int bits, int32_t *idx)
{
    for (int i = 0; i < d; ++i) {
        int v = 0;
        for (int k = 0; k < bits; ++k) {
            int p = i * bits + k;
            v |= ((rec[p / 8] >> (p % 8)) & 1) << k;
        }
        idx[i] = v;
    }
}

/* ------------------------------------------------------------------------ */
/* Scalar bucketisation against thresholds t[0..L-2]: idx = #{j : t_j < y}.   */
/* flag = 1 when y lies within `band` of any threshold.                       */
/* ------------------------------------------------------------------------ */

static int bucket(double y, const double *t, int L, double band, int *flag)
{
    int idx = 0;
    int f = 0;
    for (int j = 0; j + 1 < L; ++j) {
        if (t[j] < y) ++idx;
        if (fabs(y - t[j]) < band) f = 1;
    }
    if (flag) *flag = f;
    return idx;
}

/* Quantise an array of scalars with a given fp32 table (for MSE checks). */
ORC_API void kvqo_scalar_quantize(const double *y, int64_t n, int bits, const float *c32,
                                  const float *t32, int32_t *idx, double *yhat)
{
    const int L = 1 << bits;
    double t[255];
    for (int j = 0; j + 1 < L; ++j) t[j] = t32[j];
    for (int64_t i = 0; i < n; ++i) {
        int k = bucket(y[i], t, L, 0.0, NULL);
        if (idx) idx[i] = k;
        if (yhat) yhat[i] = c32[k];
    }
}

/* ------------------------------------------------------------------------ */
/* Quantise KV vectors (MSE codes).                                           */
/* x: [B, H, T, d]; signs: [H, d] (+-1), the random diagonal D of the head.   */
/* Per vector: rho = ||x||; u = x / rho (u = 0 if rho = 0); y = H (D .* u);   */
/* idx_i = #{j : t_j < y_i}; packed record of d*bits/8 bytes.                 */
/* Outputs (any may be NULL except codes/norms): rotated y [.., d], idx       */
/* [.., d], flags [.., d] (1 = within `band` of a threshold).                 */
/* ------------------------------------------------------------------------ */

ORC_API int kvqo_quantize(int d, int bits, int64_t B, int64_t H, int64_t T,
                          const double *x, const int8_t *signs, const float *t32,
                          double band, uint8_t *codes, double *norms, double *y_out,
                          int32_t *idx_out, uint8_t *flags)
{
    if (d <= 0 || (d & (d - 1)) || bits < 1 || bits > 8) return -1;
    const int L = 1 << bits;
    const int rec = d * bits / 8;
    double t[255];
    for (int j = 0; j + 1 < L; ++j) t[j] = t32[j];
    double *u = (double *)malloc(sizeof(double) * d);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * d);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t tt = 0; tt < T; ++tt) {
                int64_t v = (b * H + h) * T + tt;
                const double *xv = x + v * d;
                double ss = 0.0;
                for (int i = 0; i < d; ++i) ss += xv[i] * xv[i];
                double rho = sqrt(ss);
                for (int i = 0; i < d; ++i) {
                    double ui = (rho > 0.0) ? xv[i] / rho : 0.0;
                    u[i] = signs[h * d + i] * ui;
                }
                kvqo_fwht(u, d);
                for (int i = 0; i < d; ++i) {
                    int f = 0;
                    idx[i] = bucket(u[i], t, L, band, &f);
                    if (flags) flags[v * d + i] = (uint8_t)f;
                    if (y_out) y_out[v * d + i] = u[i];
                    if (idx_out) idx_out[v * d + i] = idx[i];
                }
                norms[v] = rho;
                kvqo_pack(idx, d, bits, codes + v * rec);
            }
    free(u);
    free(idx);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dequantisation (PolarQuant, Methodology: centroid lookup, Hadamard is its  */
/* own inverse up to d, restore the norm):                                    */
/*   k_hat = rho * D .* (H c[idx]) / d                                        */
/* ------------------------------------------------------------------------ */

ORC_API void kvqo_dequant(int d, int bits, const uint8_t *rec, double rho,
                          const int8_t *signs, const float *c32, double *out)
{
    int32_t idx[1024];
    kvqo_unpack(rec, d, bits, idx);
    for (int i = 0; i < d; ++i) out[i] = c32[idx[i]];
    kvqo_fwht(out, d);
    for (int i = 0; i < d; ++i) out[i] = rho * signs[i] * out[i] / d;
}

/* QJL residual reconstruction added to a dequantised key:                    */
/*   r_hat = gamma * sqrt(pi/2) / m * S^T sgn,  k_hat += rho * D .* H r_hat / sqrt(d) */
static void qjl_dequant_add(int d, int m, const uint8_t *sg, double gamma, double rho,
                            const int8_t *signs, const double *S, double *k)
{
    double *r = (double *)calloc((size_t)d, sizeof(double));
    const double coef = gamma * sqrt(M_PI / 2.0) / m;
    for (int j = 0; j < m; ++j) {
        double s = ((sg[j / 8] >> (j % 8)) & 1) ? 1.0 : -1.0;
        for (int i = 0; i < d; ++i) r[i] += coef * s * S[(int64_t)j * d + i];
    }
    kvqo_fwht(r, d);
    for (int i = 0; i < d; ++i) k[i] += rho * signs[i] * r[i] / sqrt((double)d);
    free(r);
}

/* ------------------------------------------------------------------------ */
/* Logits <q_h, k_t> for grouped-query heads: q head h reads KV head          */
/* g = h / (Hq / Hkv).  Two independent routes:                               */
/*  route 0: dequantise every key, then a plain dot product;                  */
/*  route 1: rotate the query once, q' = H (D .* q), and score against the    */
/*           centroids directly: rho <q', c[idx]> / d  (+ QJL term           */
/*           rho gamma sqrt(pi/2)/m sum_j sgn_j (S q')_j / sqrt(d)).           */
/* q: [B, Hq, d]; codes [B, Hkv, T, rec]; norms [B, Hkv, T];                   */
/* qjl_signs [B, Hkv, T, m/8] and gamma [B, Hkv, T] or NULL; S [m, d].         */
/* logits: [B, Hq, T].                                                        */
/* ------------------------------------------------------------------------ */

ORC_API int kvqo_logits(int route, int d, int bits, int64_t B, int64_t Hq, int64_t Hkv,
                        int64_t T, const double *q, const uint8_t *codes, const double *norms,
                        const int8_t *signs, const float *c32, const uint8_t *qjl_signs,
                        const double *gamma, const double *S, int m, double *logits)
{
    if (Hkv <= 0 || Hq % Hkv) return -1;
    const int64_t G = Hq / Hkv;
    const int rec = d * bits / 8;
    double *kh = (double *)malloc(sizeof(double) * d);
    double *qr = (double *)malloc(sizeof(double) * d);
    double *pq = (double *)malloc(sizeof(double) * (m > 0 ? m : 1));
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * d);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < Hq; ++h) {
            const int64_t g = h / G;
            const double *qh = q + (b * Hq + h) * d;
            const int8_t *sg = signs + g * d;
            if (route == 1) {
                for (int i = 0; i < d; ++i) qr[i] = sg[i] * qh[i];
                kvqo_fwht(qr, d);
                if (qjl_signs)
                    for (int j = 0; j < m; ++j) {
                        double s = 0.0;
                        for (int i = 0; i < d; ++i) s += S[(int64_t)j * d + i] * qr[i];
                        pq[j] = s / sqrt((double)d);
                    }
            }
            for (int64_t t = 0; t < T; ++t) {
                const int64_t v = (b * Hkv + g) * T + t;
                double acc = 0.0;
                if (route == 0) {
                    kvqo_dequant(d, bits, codes + v * rec, norms[v], sg, c32, kh);
                    if (qjl_signs)
                        qjl_dequant_add(d, m, qjl_signs + v * (m / 8), gamma[v], norms[v], sg, S, kh);
                    for (int i = 0; i < d; ++i) acc += qh[i] * kh[i];
                } else {
                    kvqo_unpack(codes + v * rec, d, bits, idx);
                    for (int i = 0; i < d; ++i) acc += qr[i] * c32[idx[i]];
                    acc *= norms[v] / d;
                    if (qjl_signs) {
                        const uint8_t *sv = qjl_signs + v * (m / 8);
                        double s = 0.0;
                        for (int j = 0; j < m; ++j)
                            s += (((sv[j / 8] >> (j % 8)) & 1) ? 1.0 : -1.0) * pq[j];
                        acc += norms[v] * gamma[v] * sqrt(M_PI / 2.0) / m * s;
                    }
                }
                logits[(b * Hq + h) * T + t] = acc;
            }
        }
    free(kh);
    free(qr);
    free(pq);
    free(idx);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Decode attention over the quantised cache, by definition: dequantise each  */
/* key and value, logits <q, k_hat>, softmax with scale sm_scale (two passes: */
/* maximum, then exponentials), output = sum_t w_t v_hat_t / sum_t w_t.       */
/* q [B,Hq,d]; k/v codes [B,Hkv,T,rec]; norms [B,Hkv,T]; out [B,Hq,d].        */
/* ------------------------------------------------------------------------ */

ORC_API int kvqo_attention(int d, int bits, int64_t B, int64_t Hq, int64_t Hkv, int64_t T,
                           const double *q, const uint8_t *kc, const double *kn,
                           const uint8_t *vc, const double *vn, const int8_t *signs_k,
                           const int8_t *signs_v, const float *c32, double sm_scale,
                           double *out)
{
    if (Hkv <= 0 || Hq % Hkv || T <= 0) return -1;
    const int64_t G = Hq / Hkv;
    const int rec = d * bits / 8;
    double *K = (double *)malloc(sizeof(double) * T * d);
    double *V = (double *)malloc(sizeof(double) * T * d);
    double *s = (double *)malloc(sizeof(double) * T);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t g = 0; g < Hkv; ++g) {
            for (int64_t t = 0; t < T; ++t) {
                const int64_t v = (b * Hkv + g) * T + t;
                kvqo_dequant(d, bits, kc + v * rec, kn[v], signs_k + g * d, c32, K + t * d);
                kvqo_dequant(d, bits, vc + v * rec, vn[v], signs_v + g * d, c32, V + t * d);
            }
            for (int64_t hh = 0; hh < G; ++hh) {
                const int64_t h = g * G + hh;
                const double *qh = q + (b * Hq + h) * d;
                double mx = -INFINITY;
                for (int64_t t = 0; t < T; ++t) {
                    double a = 0.0;
                    for (int i = 0; i < d; ++i) a += qh[i] * K[t * d + i];
                    s[t] = sm_scale * a;
                    if (s[t] > mx) mx = s[t];
                }
                double l = 0.0;
                for (int64_t t = 0; t < T; ++t) {
                    s[t] = exp(s[t] - mx);
                    l += s[t];
                }
                double *o = out + (b * Hq + h) * d;
                for (int i = 0; i < d; ++i) o[i] = 0.0;
                for (int64_t t = 0; t < T; ++t)
                    for (int i = 0; i < d; ++i) o[i] += s[t] * V[t * d + i];
                for (int i = 0; i < d; ++i) o[i] /= l;
            }
        }
    free(K);
    free(V);
    free(s);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dense rotation ("O Que E TurboQuant?", Como Funciona, Estagio 1: a random  */
/* orthogonal transformation independent of the data, from the QR            */
/* decomposition of a Gaussian matrix).  Q [d, d] row-major orthogonal, the   */
/* same for every head and for K and V.  Scaled like the Hadamard path so     */
/* that the coordinates have unit variance:                                   */
/*   y = sqrt(d) Q (x / rho);  k_hat = rho Q^T c[idx] / sqrt(d);              */
/*   <q, k_hat> = rho / d * <sqrt(d) Q q, c[idx]>.                            */
/* ------------------------------------------------------------------------ */

static void matvec(const double *Q, const double *x, double *y, int d, int transpose)
{
    for (int i = 0; i < d; ++i) {
        double s = 0.0;
        for (int j = 0; j < d; ++j) s += (transpose ? Q[(int64_t)j * d + i] : Q[(int64_t)i * d + j]) * x[j];
        y[i] = s;
    }
}

ORC_API int kvqo_quantize_dense(int d, int bits, int64_t B, int64_t H, int64_t T, const double *x,
                                const double *Q, const float *t32, double band, uint8_t *codes, double *norms,
                                double *y_out, int32_t *idx_out, uint8_t *flags)
{
    if (d <= 0 || d > 1024 || bits < 1 || bits > 8) return -1;
    const int L = 1 << bits;
    const int rec = d * bits / 8;
    double t[255];
    for (int j = 0; j + 1 < L; ++j) t[j] = t32[j];
    double *u = (double *)malloc(sizeof(double) * d);
    double *y = (double *)malloc(sizeof(double) * d);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * d);
    for (int64_t v = 0; v < B * H * T; ++v) {
        const double *xv = x + v * d;
        double ss = 0.0;
        for (int i = 0; i < d; ++i) ss += xv[i] * xv[i];
        const double rho = sqrt(ss);
        for (int i = 0; i < d; ++i) u[i] = rho > 0.0 ? xv[i] / rho : 0.0;
        matvec(Q, u, y, d, 0);
        for (int i = 0; i < d; ++i) {
            y[i] *= sqrt((double)d);
            int f = 0;
            idx[i] = bucket(y[i], t, L, band, &f);
            if (flags) flags[v * d + i] = (uint8_t)f;
            if (y_out) y_out[v * d + i] = y[i];
            if (idx_out) idx_out[v * d + i] = idx[i];
        }
        norms[v] = rho;
        kvqo_pack(idx, d, bits, codes + v * rec);
    }
    free(u);
    free(y);
    free(idx);
    return 0;
}

ORC_API void kvqo_dequant_dense(int d, int bits, const uint8_t *rec, double rho, const double *Q,
                                const float *c32, double *out)
{
    int32_t idx[1024];
    double c[1024];
    kvqo_unpack(rec, d, bits, idx);
    for (int i = 0; i < d; ++i) c[i] = c32[idx[i]];
    matvec(Q, c, out, d, 1);
    for (int i = 0; i < d; ++i) out[i] *= rho / sqrt((double)d);
}

/* route 0: dequantise, then <q, k_hat>; route 1: rotated query q' = sqrt(d) Q q. */
/* With QJL signs (qjl_signs, gamma, S [m, d] not NULL; TurboQuant, Como     */
/* Funciona, Estagio 1 + Estagio 2: the dense rotation, then the 1-bit sign   */
/* residual): the residual r = (y - c[idx]) / sqrt(d) lives in the rotated    */
/* space, u - u_hat = Q^T r, and its estimate is                              */
/* r_hat = gamma sqrt(pi/2) / m S^T sgn, so                                   */
/*  route 0: k_hat = rho Q^T (c[idx] / sqrt(d) + r_hat), then <q, k_hat>;     */
/*  route 1: rho <q', c[idx]> / d + rho gamma sqrt(pi/2)/m sum_j sgn_j         */
/*           (S q')_j / sqrt(d) with q' = sqrt(d) Q q.                         */
ORC_API int kvqo_logits_dense(int route, int d, int bits, int64_t B, int64_t Hq, int64_t Hkv, int64_t T,
                              const double *q, const uint8_t *codes, const double *norms, const double *Q,
                              const float *c32, const uint8_t *qjl_signs, const double *gamma, const double *S,
                              int m, double *logits)
{
    if (Hkv <= 0 || Hq % Hkv || d > 1024) return -1;
    const int64_t G = Hq / Hkv;
    const int rec = d * bits / 8;
    double *kh = (double *)malloc(sizeof(double) * d);
    double *qr = (double *)malloc(sizeof(double) * d);
    double *rh = (double *)malloc(sizeof(double) * d);
    double *rq = (double *)malloc(sizeof(double) * d);
    double *pq = (double *)malloc(sizeof(double) * (m > 0 ? m : 1));
    int32_t idx[1024];
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < Hq; ++h) {
            const int64_t g = h / G;
            const double *qh = q + (b * Hq + h) * d;
            matvec(Q, qh, qr, d, 0);
            for (int i = 0; i < d; ++i) qr[i] *= sqrt((double)d);
            if (qjl_signs)
                for (int j = 0; j < m; ++j) {
                    double s = 0.0;
                    for (int i = 0; i < d; ++i) s += S[(int64_t)j * d + i] * qr[i];
                    pq[j] = s / sqrt((double)d);
                }
            for (int64_t t = 0; t < T; ++t) {
                const int64_t v = (b * Hkv + g) * T + t;
                double acc = 0.0;
                if (route == 0) {
                    kvqo_dequant_dense(d, bits, codes + v * rec, norms[v], Q, c32, kh);
                    if (qjl_signs) {
                        const uint8_t *sv = qjl_signs + v * (m / 8);
                        const double coef = gamma[v] * sqrt(M_PI / 2.0) / m;
                        for (int i = 0; i < d; ++i) rh[i] = 0.0;
                        for (int j = 0; j < m; ++j) {
                            const double sg = ((sv[j / 8] >> (j % 8)) & 1) ? 1.0 : -1.0;
                            for (int i = 0; i < d; ++i) rh[i] += coef * sg * S[(int64_t)j * d + i];
                        }
                        matvec(Q, rh, rq, d, 1);
                        for (int i = 0; i < d; ++i) kh[i] += norms[v] * rq[i];
                    }
                    for (int i = 0; i < d; ++i) acc += qh[i] * kh[i];
                } else {
                    kvqo_unpack(codes + v * rec, d, bits, idx);
                    for (int i = 0; i < d; ++i) acc += qr[i] * c32[idx[i]];
                    acc *= norms[v] / d;
                    if (qjl_signs) {
                        const uint8_t *sv = qjl_signs + v * (m / 8);
                        double s = 0.0;
                        for (int j = 0; j < m; ++j) s += (((sv[j / 8] >> (j % 8)) & 1) ? 1.0 : -1.0) * pq[j];
                        acc += norms[v] * gamma[v] * sqrt(M_PI / 2.0) / m * s;
                    }
                }
                logits[(b * Hq + h) * T + t] = acc;
            }
        }
    free(kh);
    free(qr);
    free(rh);
    free(rq);
    free(pq);
    return 0;
}

/* Decode attention with the dense rotation: as kvqo_attention, keys and
 * values dequantised with Q^T. */
ORC_API int kvqo_attention_dense(int d, int bits, int64_t B, int64_t Hq, int64_t Hkv, int64_t T, const double *q,
                                 const uint8_t *kc, const double *kn, const uint8_t *vc, const double *vn,
                                 const double *Q, const float *c32, double sm_scale, double *out)
{
    if (Hkv <= 0 || Hq % Hkv || T <= 0 || d > 1024) return -1;
    const int64_t G = Hq / Hkv;
    const int rec = d * bits / 8;
    double *K = (double *)malloc(sizeof(double) * T * d);
    double *V = (double *)malloc(sizeof(double) * T * d);
    double *s = (double *)malloc(sizeof(double) * T);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t g = 0; g < Hkv; ++g) {
            for (int64_t t = 0; t < T; ++t) {
                const int64_t v = (b * Hkv + g) * T + t;
                kvqo_dequant_dense(d, bits, kc + v * rec, kn[v], Q, c32, K + t * d);
                kvqo_dequant_dense(d, bits, vc + v * rec, vn[v], Q, c32, V + t * d);
            }
            for (int64_t hh = 0; hh < G; ++hh) {
                const double *qh = q + (b * Hq + g * G + hh) * d;
                double mx = -INFINITY;
                for (int64_t t = 0; t < T; ++t) {
                    double a = 0.0;
                    for (int i = 0; i < d; ++i) a += qh[i] * K[t * d + i];
                    s[t] = sm_scale * a;
                    if (s[t] > mx) mx = s[t];
                }
                double l = 0.0;
                for (int64_t t = 0; t < T; ++t) {
                    s[t] = exp(s[t] - mx);
                    l += s[t];
                }
                double *o = out + (b * Hq + g * G + hh) * d;
                for (int i = 0; i < d; ++i) o[i] = 0.0;
                for (int64_t t = 0; t < T; ++t)
                    for (int i = 0; i < d; ++i) o[i] += s[t] * V[t * d + i];
                for (int i = 0; i < d; ++i) o[i] /= l;
            }
        }
    free(K);
    free(V);
    free(s);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Decode attention over a cache split into a quantised part and a full-     */
/* precision residual (NSNQuant, "Detalhes de Implementacao": following KIVI, */
/* the residual is quantised and appended when it fills).  Token order: the  */
/* T quantised tokens, then the R residual ones (kt, vt [B, Hkv, R, d]);     */
/* keys and values are the dequantised prefix followed by the residual rows, */
/* then the same two-pass softmax as kvqo_attention over all T + R tokens.   */
/* ------------------------------------------------------------------------ */

ORC_API int kvqo_attention_stream(int d, int bits, int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t R,
                                  const double *q, const uint8_t *kc, const double *kn, const uint8_t *vc,
                                  const double *vn, const double *kt, const double *vt,
                                  const int8_t *signs_k, const int8_t *signs_v, const float *c32,
                                  double sm_scale, double *out)
{
    if (Hkv <= 0 || Hq % Hkv || T < 0 || R < 0 || T + R <= 0) return -1;
    const int64_t G = Hq / Hkv, N = T + R;
    const int rec = d * bits / 8;
    double *K = (double *)malloc(sizeof(double) * N * d);
    double *V = (double *)malloc(sizeof(double) * N * d);
    double *s = (double *)malloc(sizeof(double) * N);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t g = 0; g < Hkv; ++g) {
            for (int64_t t = 0; t < T; ++t) {
                const int64_t v = (b * Hkv + g) * T + t;
                kvqo_dequant(d, bits, kc + v * rec, kn[v], signs_k + g * d, c32, K + t * d);
                kvqo_dequant(d, bits, vc + v * rec, vn[v], signs_v + g * d, c32, V + t * d);
            }
            for (int64_t t = 0; t < R; ++t)
                for (int i = 0; i < d; ++i) {
                    K[(T + t) * d + i] = kt[((b * Hkv + g) * R + t) * d + i];
                    V[(T + t) * d + i] = vt[((b * Hkv + g) * R + t) * d + i];
                }
            for (int64_t hh = 0; hh < G; ++hh) {
                const double *qh = q + (b * Hq + g * G + hh) * d;
                double mx = -INFINITY;
                for (int64_t t = 0; t < N; ++t) {
                    double a = 0.0;
                    for (int i = 0; i < d; ++i) a += qh[i] * K[t * d + i];
                    s[t] = sm_scale * a;
                    if (s[t] > mx) mx = s[t];
                }
                double l = 0.0;
                for (int64_t t = 0; t < N; ++t) {
                    s[t] = exp(s[t] - mx);
                    l += s[t];
                }
                double *o = out + (b * Hq + g * G + hh) * d;
                for (int i = 0; i < d; ++i) o[i] = 0.0;
                for (int64_t t = 0; t < N; ++t)
                    for (int i = 0; i < d; ++i) o[i] += s[t] * V[t * d + i];
                for (int i = 0; i < d; ++i) o[i] /= l;
            }
        }
    free(K);
    free(V);
    free(s);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* QJL 1-bit residual (TurboQuant, Stage 2).  Reading: the residual lives in  */
/* the orthonormal rotated space, r = (y - c[idx]) / sqrt(d); gamma = ||r||;  */
/* z = S r with S [m, d] of N(0,1) entries; sign bit sgn_j = [z_j >= 0].      */
/* y [n, d] rotated coordinates, idx [n, d] the MSE codes actually stored.    */
/* Outputs: packed sign bits [n, m/8] (LSB-first), gamma [n], flags [n, m]    */
/* (1 when |z_j| < band * gamma).                                             */
/* ------------------------------------------------------------------------ */

ORC_API int kvqo_qjl(int d, int m, int64_t n, const double *y, const int32_t *idx,
                     const float *c32, const double *S, double band, uint8_t *sgn,
                     double *gamma, uint8_t *flags)
{
    if (m % 8) return -1;
    double *r = (double *)malloc(sizeof(double) * d);
    for (int64_t v = 0; v < n; ++v) {
        double g2 = 0.0;
        for (int i = 0; i < d; ++i) {
            r[i] = (y[v * d + i] - c32[idx[v * d + i]]) / sqrt((double)d);
            g2 += r[i] * r[i];
        }
        double gm = sqrt(g2);
        gamma[v] = gm;
        uint8_t *out = sgn + v * (m / 8);
        memset(out, 0, (size_t)(m / 8));
        for (int j = 0; j < m; ++j) {
            double z = 0.0;
            for (int i = 0; i < d; ++i) z += S[(int64_t)j * d + i] * r[i];
            if (z >= 0.0) out[j / 8] |= (uint8_t)(1u << (j % 8));
            if (flags) flags[v * m + j] = (uint8_t)(fabs(z) < band * gm);
        }
    }
    free(r);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* NSN + Hadamard + vector quantisation (NSNQuant, Metodologia 1-3).          */
/* x [H, T, d].  Per head, over the T tokens of the call:                     */
/*   a_t = sqrt(d) x_t / ||x_t||,   s1_t = ||x_t|| / sqrt(d)   (normalise)    */
/*   o   = mean_t a_t                                          (shift)        */
/*   b_t = a_t - o,  s2_t = ||b_t|| / sqrt(d),  xt_t = b_t / s2_t (normalise) */
/*   z_t = H xt_t / sqrt(d)                                   (Hadamard)      */
/* then each sub-vector of `sub` coordinates is replaced by the index of the  */
/* nearest of K codebook entries (squared Euclidean distance, lowest index on */
/* exact ties).  flags: 1 when z is within `band` of the bisecting hyperplane */
/* of the winner and some other entry.  Degenerate tokens: ||x_t|| = 0 gives  */
/* a_t = 0; s2_t = 0 gives xt_t = 0.                                          */
/* o_given: NULL, or a mean [H, d] to use instead of the mean of these T      */
/* tokens (to encode a sample of a longer sequence).                         */
/* adaptive: 1 for the adaptive scale (NSNQuant, Metodologia sec. 3, "Ajuste  */
/* de Escala": the quantised vector is scaled so that its component along    */
/* the original is preserved): zq = the selected entries, alpha =            */
/* ||z||^2 / <z, zq> (1 when <z, zq> <= 0), and the returned s2 is           */
/* alpha * s2, so that s1 (s2 H zq / sqrt(d) + o) reconstructs with the       */
/* scaled zq and every other use of the byproducts is unchanged.            */
/* ------------------------------------------------------------------------ */

ORC_API int kvqo_nsn_vq(int d, int sub, int K, int64_t H, int64_t T, const double *x,
                        const double *codebook, double band, uint8_t *codes, double *s1,
                        double *s2, double *o, double *z_out, uint8_t *flags,
                        const double *o_given, int adaptive)
{
    if (d % sub || T <= 0) return -1;
    const int nsub = d / sub;
    const double sd = sqrt((double)d);
    double *a = (double *)malloc(sizeof(double) * T * d);
    double *z = (double *)malloc(sizeof(double) * d);
    double *dist = (double *)malloc(sizeof(double) * K);
    for (int64_t h = 0; h < H; ++h) {
        const double *xh = x + h * T * d;
        double *oh = o + h * d;
        for (int i = 0; i < d; ++i) oh[i] = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            double ss = 0.0;
            for (int i = 0; i < d; ++i) ss += xh[t * d + i] * xh[t * d + i];
            double nx = sqrt(ss);
            s1[h * T + t] = nx / sd;
            for (int i = 0; i < d; ++i) a[t * d + i] = nx > 0.0 ? sd * xh[t * d + i] / nx : 0.0;
        }
        for (int64_t t = 0; t < T; ++t)
            for (int i = 0; i < d; ++i) oh[i] += a[t * d + i];
        for (int i = 0; i < d; ++i) oh[i] = o_given ? o_given[h * d + i] : oh[i] / (double)T;
        for (int64_t t = 0; t < T; ++t) {
            double ss = 0.0;
            for (int i = 0; i < d; ++i) {
                double bi = a[t * d + i] - oh[i];
                z[i] = bi;
                ss += bi * bi;
            }
            double nb = sqrt(ss);
            s2[h * T + t] = nb / sd;
            for (int i = 0; i < d; ++i) z[i] = nb > 0.0 ? z[i] / (nb / sd) : 0.0;
            kvqo_fwht(z, d);
            for (int i = 0; i < d; ++i) z[i] /= sd;
            if (z_out)
                for (int i = 0; i < d; ++i) z_out[(h * T + t) * d + i] = z[i];
            for (int s = 0; s < nsub; ++s) {
                int best = 0;
                for (int j = 0; j < K; ++j) {
                    double dd = 0.0;
                    for (int k = 0; k < sub; ++k) {
                        double e = z[s * sub + k] - codebook[j * sub + k];
                        dd += e * e;
                    }
                    dist[j] = dd;
                    if (dd < dist[best]) best = j;
                }
                codes[(h * T + t) * nsub + s] = (uint8_t)best;
                if (flags) {
                    double mind = INFINITY;
                    for (int j = 0; j < K; ++j) {
                        if (j == best) continue;
                        double cc = 0.0;
                        for (int k = 0; k < sub; ++k) {
                            double e = codebook[j * sub + k] - codebook[best * sub + k];
                            cc += e * e;
                        }
                        double md = cc > 0.0 ? (dist[j] - dist[best]) / (2.0 * sqrt(cc)) : 0.0;
                        if (md < mind) mind = md;
                    }
                    flags[(h * T + t) * nsub + s] = (uint8_t)(mind < band);
                }
            }
            if (adaptive) {
                double zz = 0.0, zq = 0.0;
                for (int s = 0; s < nsub; ++s) {
                    const int c = codes[(h * T + t) * nsub + s];
                    for (int k = 0; k < sub; ++k) {
                        zz += z[s * sub + k] * z[s * sub + k];
                        zq += z[s * sub + k] * codebook[c * sub + k];
                    }
                }
                if (zq > 0.0) s2[h * T + t] *= zz / zq;
            }
        }
    }
    free(a);
    free(z);
    free(dist);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 4-bit double quantisation (NSNQuant, Metodologia sec. 3, "Double          */
/* Quantization": the NSN parameters o and s1, and the codebook entries, are  */
/* stored with 4 bits).  The page gives no scheme; the reading here is the    */
/* plain uniform min-max quantiser of a block of n values:                    */
/*   lo = min v,  step = (max v - lo) / 15,                                   */
/*   code = floor((v - lo) / step + 1/2) in [0, 15]  (all 0 when step = 0),   */
/*   stored value lo + code * step.                                           */
/* flags: 1 when (v - lo) / step lies within `band` of a half-integer, where  */
/* another precision may round the other way.                                */
/* ------------------------------------------------------------------------ */
ORC_API int kvqo_dq4(int64_t n, const double *v, double band, uint8_t *code, double *lo_out,
                     double *step_out, uint8_t *flags)
{
    if (n <= 0) return -1;
    double lo = v[0], hi = v[0];
    for (int64_t i = 1; i < n; ++i) {
        if (v[i] < lo) lo = v[i];
        if (v[i] > hi) hi = v[i];
    }
    const double step = (hi - lo) / 15.0;
    for (int64_t i = 0; i < n; ++i) {
        int c = 0, f = 0;
        if (step > 0.0) {
            const double u = (v[i] - lo) / step;
            c = (int)floor(u + 0.5);
            if (c < 0) c = 0;
            if (c > 15) c = 15;
            f = fabs(u - floor(u) - 0.5) < band;
        }
        code[i] = (uint8_t)c;
        if (flags) flags[i] = (uint8_t)f;
    }
    *lo_out = lo;
    *step_out = step;
    return 0;
}

/* Reconstruction from the NSN byproducts and a rotated vector zq [d]:        */
/*   x_hat = s1 * (s2 * H zq / sqrt(d) + o)                                   */
ORC_API void kvqo_nsn_reconstruct(int d, const double *zq, double s1, double s2,
                                  const double *o, double *x_hat)
{
    for (int i = 0; i < d; ++i) x_hat[i] = zq[i];
    kvqo_fwht(x_hat, d);
    for (int i = 0; i < d; ++i) x_hat[i] = s1 * (s2 * x_hat[i] / sqrt((double)d) + o[i]);
}

/* ------------------------------------------------------------------------ */
/* Attention over NSN-VQ codes (NSNQuant, "Detalhes de Implementacao": the    */
/* score uses the byproducts s1, s2, o inside the attention kernels).  The    */
/* reconstruction inverts Metodologia 1-2: x_hat = s1 (s2 H zq / sqrt(d) + o), */
/* zq the 16 codebook entries the codes name, in sub-vector order.            */
/* codes [B, Hkv, T, d/sub]; s1, s2 [B, Hkv, T]; o [B, Hkv, d]; q [B, Hq, d]; */
/* KV head of query head h = h / (Hq / Hkv).                                   */
/* ------------------------------------------------------------------------ */

static void nsn_entries(int d, int sub, const uint8_t *code, const double *cb, double *zq)
{
    for (int s = 0; s < d / sub; ++s)
        for (int k = 0; k < sub; ++k) zq[s * sub + k] = cb[(int)code[s] * sub + k];
}

/* route 1: <q, x_hat> with x_hat reconstructed.  route 2: the query is
 * rotated once, q' = H q / sqrt(d), and
 *   logit = s1 (s2 sum_s <q'_s, C[code_s]> + <q, o>),
 * which is route 1 with H symmetric moved onto q. */
ORC_API int kvqo_nsn_logits(int route, int d, int sub, int64_t B, int64_t Hq, int64_t Hkv, int64_t T,
                            const double *q, const uint8_t *codes, const double *s1, const double *s2,
                            const double *o, const double *cb, double *logits)
{
    if (Hkv <= 0 || Hq % Hkv || d % sub) return -1;
    const int64_t G = Hq / Hkv;
    const int ns = d / sub;
    double *zq = (double *)malloc(sizeof(double) * d);
    double *xh = (double *)malloc(sizeof(double) * d);
    double *qr = (double *)malloc(sizeof(double) * d);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < Hq; ++h) {
            const int64_t g = h / G;
            const double *qh = q + (b * Hq + h) * d;
            const double *og = o + (b * Hkv + g) * d;
            double qo = 0.0;
            for (int i = 0; i < d; ++i) qo += qh[i] * og[i];
            for (int i = 0; i < d; ++i) qr[i] = qh[i];
            kvqo_fwht(qr, d);
            for (int i = 0; i < d; ++i) qr[i] /= sqrt((double)d);
            for (int64_t t = 0; t < T; ++t) {
                const int64_t v = (b * Hkv + g) * T + t;
                double acc = 0.0;
                if (route == 1) {
                    nsn_entries(d, sub, codes + v * ns, cb, zq);
                    kvqo_nsn_reconstruct(d, zq, s1[v], s2[v], og, xh);
                    for (int i = 0; i < d; ++i) acc += qh[i] * xh[i];
                } else {
                    for (int sidx = 0; sidx < ns; ++sidx) {
                        const double *c = cb + (int)codes[v * ns + sidx] * sub;
                        for (int k = 0; k < sub; ++k) acc += qr[sidx * sub + k] * c[k];
                    }
                    acc = s1[v] * (s2[v] * acc + qo);
                }
                logits[(b * Hq + h) * T + t] = acc;
            }
        }
    free(zq);
    free(xh);
    free(qr);
    return 0;
}

/* Decode attention by definition: reconstruct every key and value, logits
 * <q, k_hat> times sm_scale, softmax in two passes (maximum, exponentials),
 * out = sum_t w_t v_hat_t / sum_t w_t. */
ORC_API int kvqo_nsn_attention(int d, int sub, int64_t B, int64_t Hq, int64_t Hkv, int64_t T,
                               const double *q, const uint8_t *kc, const double *ks1, const double *ks2,
                               const double *ko, const uint8_t *vc, const double *vs1, const double *vs2,
                               const double *vo, const double *cb, double sm_scale, double *out)
{
    if (Hkv <= 0 || Hq % Hkv || T <= 0 || d % sub) return -1;
    const int64_t G = Hq / Hkv;
    const int ns = d / sub;
    double *K = (double *)malloc(sizeof(double) * T * d);
    double *V = (double *)malloc(sizeof(double) * T * d);
    double *zq = (double *)malloc(sizeof(double) * d);
    double *w = (double *)malloc(sizeof(double) * T);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t g = 0; g < Hkv; ++g) {
            const int64_t bg = b * Hkv + g;
            for (int64_t t = 0; t < T; ++t) {
                const int64_t v = bg * T + t;
                nsn_entries(d, sub, kc + v * ns, cb, zq);
                kvqo_nsn_reconstruct(d, zq, ks1[v], ks2[v], ko + bg * d, K + t * d);
                nsn_entries(d, sub, vc + v * ns, cb, zq);
                kvqo_nsn_reconstruct(d, zq, vs1[v], vs2[v], vo + bg * d, V + t * d);
            }
            for (int64_t hh = 0; hh < G; ++hh) {
                const double *qh = q + (b * Hq + g * G + hh) * d;
                double mx = -INFINITY;
                for (int64_t t = 0; t < T; ++t) {
                    double a = 0.0;
                    for (int i = 0; i < d; ++i) a += qh[i] * K[t * d + i];
                    w[t] = sm_scale * a;
                    if (w[t] > mx) mx = w[t];
                }
                double l = 0.0;
                for (int64_t t = 0; t < T; ++t) {
                    w[t] = exp(w[t] - mx);
                    l += w[t];
                }
                double *oh = out + (b * Hq + g * G + hh) * d;
                for (int i = 0; i < d; ++i) oh[i] = 0.0;
                for (int64_t t = 0; t < T; ++t)
                    for (int i = 0; i < d; ++i) oh[i] += w[t] * V[t * d + i];
                for (int i = 0; i < d; ++i) oh[i] /= l;
            }
        }
    free(K);
    free(V);
    free(zq);
    free(w);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* k-means (Lloyd's algorithm) for the NSN vector codebook, on synthetic      */
/* N(0, I) samples (NSNQuant, Metodologia 3).  samples [n, dim]; init [K]     */
/* distinct sample indices; stops when no assignment changes or after         */
/* max_iter passes; an empty cluster is re-seeded with the sample farthest    */
/* from its current centroid.  distortion[it] = mean squared distance per     */
/* dimension after the assignment step of pass it.  Returns passes done.      */
/* ------------------------------------------------------------------------ */

ORC_API int kvqo_kmeans(int64_t n, int dim, int K, const double *samples, const int64_t *init,
                        int max_iter, double *codebook, double *distortion)
{
    int32_t *asg = (int32_t *)malloc(sizeof(int32_t) * n);
    double *dmin = (double *)malloc(sizeof(double) * n);
    double *sum = (double *)malloc(sizeof(double) * K * dim);
    int64_t *cnt = (int64_t *)malloc(sizeof(int64_t) * K);
    for (int j = 0; j < K; ++j)
        for (int k = 0; k < dim; ++k) codebook[j * dim + k] = samples[init[j] * dim + k];
    for (int64_t i = 0; i < n; ++i) asg[i] = -1;
    int it = 0;
    for (; it < max_iter; ++it) {
        int64_t changed = 0;
        double tot = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            int best = 0;
            double bd = INFINITY;
            for (int j = 0; j < K; ++j) {
                double dd = 0.0;
                for (int k = 0; k < dim; ++k) {
                    double e = samples[i * dim + k] - codebook[j * dim + k];
                    dd += e * e;
                }
                if (dd < bd) { bd = dd; best = j; }
            }
            if (best != asg[i]) ++changed;
            asg[i] = best;
            dmin[i] = bd;
            tot += bd;
        }
        if (distortion) distortion[it] = tot / ((double)n * dim);
        if (changed == 0) { ++it; break; }
        memset(sum, 0, sizeof(double) * K * dim);
        memset(cnt, 0, sizeof(int64_t) * K);
        for (int64_t i = 0; i < n; ++i) {
            ++cnt[asg[i]];
            for (int k = 0; k < dim; ++k) sum[asg[i] * dim + k] += samples[i * dim + k];
        }
        for (int j = 0; j < K; ++j) {
            if (cnt[j] > 0) {
                for (int k = 0; k < dim; ++k) codebook[j * dim + k] = sum[j * dim + k] / cnt[j];
            } else {
                int64_t far = 0;
                for (int64_t i = 1; i < n; ++i)
                    if (dmin[i] > dmin[far]) far = i;
                for (int k = 0; k < dim; ++k) codebook[j * dim + k] = samples[far * dim + k];
                dmin[far] = 0.0;
            }
        }
    }
    free(asg);
    free(dmin);
    free(sum);
    free(cnt);
    return it;
}

/* ------------------------------------------------------------------------ */
/* Decode attention over an NSN-VQ streaming cache (NSNQuant, Detalhes de     */
/* Implementacao, Residuos: following KIVI the cache is a quantised part and  */
/* a full-precision residual that is quantised and appended when it fills;   */
/* read with Metodologia sec. 1, each flushed group of Gs tokens is encoded   */
/* as one call, with its own channel mean).  Packed token t of (b, g) is      */
/* reconstructed with the mean of its group t / Gs:                           */
/*   x_hat_t = s1_t (s2_t H zq_t / sqrt(d) + o_{t / Gs}),                      */
/* followed by the R window tokens as they are; one softmax over all T + R.  */
/* kc, vc [B, Hkv, T, d/sub]; ks1.. [B, Hkv, T]; ko, vo [B, Hkv, T / Gs, d]    */
/* (T a multiple of Gs; T = 0 allowed); kt, vt [B, Hkv, R, d].               */
/* ------------------------------------------------------------------------ */

ORC_API int kvqo_nsn_attention_stream(int d, int sub, int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t Gs,
                                      int64_t R, const double *q, const uint8_t *kc, const double *ks1,
                                      const double *ks2, const double *ko, const uint8_t *vc, const double *vs1,
                                      const double *vs2, const double *vo, const double *kt, const double *vt,
                                      const double *cb, double sm_scale, double *out)
{
    if (Hkv <= 0 || Hq % Hkv || T < 0 || R < 0 || T + R <= 0 || d % sub || Gs <= 0 || T % Gs) return -1;
    const int64_t G = Hq / Hkv, N = T + R, ng = T / Gs;
    const int ns = d / sub;
    double *K = (double *)malloc(sizeof(double) * N * d);
    double *V = (double *)malloc(sizeof(double) * N * d);
    double *zq = (double *)malloc(sizeof(double) * d);
    double *w = (double *)malloc(sizeof(double) * N);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t g = 0; g < Hkv; ++g) {
            const int64_t bg = b * Hkv + g;
            for (int64_t t = 0; t < T; ++t) {
                const int64_t v = bg * T + t;
                const double *okg = ko + (bg * ng + t / Gs) * d, *ovg = vo + (bg * ng + t / Gs) * d;
                nsn_entries(d, sub, kc + v * ns, cb, zq);
                kvqo_nsn_reconstruct(d, zq, ks1[v], ks2[v], okg, K + t * d);
                nsn_entries(d, sub, vc + v * ns, cb, zq);
                kvqo_nsn_reconstruct(d, zq, vs1[v], vs2[v], ovg, V + t * d);
            }
            for (int64_t t = 0; t < R; ++t)
                for (int i = 0; i < d; ++i) {
                    K[(T + t) * d + i] = kt[(bg * R + t) * d + i];
                    V[(T + t) * d + i] = vt[(bg * R + t) * d + i];
                }
            for (int64_t hh = 0; hh < G; ++hh) {
                const double *qh = q + (b * Hq + g * G + hh) * d;
                double mx = -INFINITY;
                for (int64_t t = 0; t < N; ++t) {
                    double a = 0.0;
                    for (int i = 0; i < d; ++i) a += qh[i] * K[t * d + i];
                    w[t] = sm_scale * a;
                    if (w[t] > mx) mx = w[t];
                }
                double l = 0.0;
                for (int64_t t = 0; t < N; ++t) {
                    w[t] = exp(w[t] - mx);
                    l += w[t];
                }
                double *oh = out + (b * Hq + g * G + hh) * d;
                for (int i = 0; i < d; ++i) oh[i] = 0.0;
                for (int64_t t = 0; t < N; ++t)
                    for (int i = 0; i < d; ++i) oh[i] += w[t] * V[t * d + i];
                for (int i = 0; i < d; ++i) oh[i] /= l;
            }
        }
    free(K);
    free(V);
    free(zq);
    free(w);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Cosine refinement of a codebook (NSNQuant, Metodologia sec. 3: the k-means */
/* codebook on standard-normal samples is refined to minimise the cosine     */
/* distance between the vectors and their quantised versions).  Reading:     */
/* each pass assigns every sample to its nearest entry (squared Euclidean    */
/* distance, lowest index on ties: the quantiser in use), then moves each     */
/* entry to the direction u = sum over its cell of x / ||x|| (the direction  */
/* that maximises the cell's summed cosine similarity), with the length that */
/* is least-squares optimal along u, mean over the cell of <x, u>.  Entries  */
/* with an empty cell, or a zero direction sum, are kept.  mean_cos[i] is the */
/* mean cosine similarity of the samples with their entries at the           */
/* assignment of pass i (zero samples count as 1).  Returns the passes run.  */
/* ------------------------------------------------------------------------ */

ORC_API int kvqo_cosine_refine(int64_t n, int dim, int K, const double *samples, double *codebook, int passes,
                               double *mean_cos)
{
    int32_t *asg = (int32_t *)malloc(sizeof(int32_t) * n);
    double *usum = (double *)malloc(sizeof(double) * K * dim);
    double *proj = (double *)malloc(sizeof(double) * K);
    int64_t *cnt = (int64_t *)malloc(sizeof(int64_t) * K);
    int it = 0;
    for (; it < passes; ++it) {
        double cs = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            const double *x = samples + i * dim;
            int best = 0;
            double bd = INFINITY;
            for (int j = 0; j < K; ++j) {
                double dd = 0.0;
                for (int k = 0; k < dim; ++k) {
                    const double e = x[k] - codebook[j * dim + k];
                    dd += e * e;
                }
                if (dd < bd) { bd = dd; best = j; }
            }
            asg[i] = best;
            double xx = 0.0, cc = 0.0, xc = 0.0;
            for (int k = 0; k < dim; ++k) {
                xx += x[k] * x[k];
                cc += codebook[best * dim + k] * codebook[best * dim + k];
                xc += x[k] * codebook[best * dim + k];
            }
            cs += (xx > 0.0 && cc > 0.0) ? xc / sqrt(xx * cc) : 1.0;
        }
        if (mean_cos) mean_cos[it] = cs / (double)n;
        memset(usum, 0, sizeof(double) * K * dim);
        memset(cnt, 0, sizeof(int64_t) * K);
        for (int64_t i = 0; i < n; ++i) {
            const double *x = samples + i * dim;
            double xx = 0.0;
            for (int k = 0; k < dim; ++k) xx += x[k] * x[k];
            if (xx <= 0.0) continue;
            const double inv = 1.0 / sqrt(xx);
            ++cnt[asg[i]];
            for (int k = 0; k < dim; ++k) usum[asg[i] * dim + k] += x[k] * inv;
        }
        for (int j = 0; j < K; ++j) {
            double uu = 0.0;
            for (int k = 0; k < dim; ++k) uu += usum[j * dim + k] * usum[j * dim + k];
            if (cnt[j] == 0 || uu <= 0.0) { proj[j] = -1.0; continue; }
            const double inv = 1.0 / sqrt(uu);
            for (int k = 0; k < dim; ++k) usum[j * dim + k] *= inv; /* unit direction */
            proj[j] = 0.0;
        }
        for (int64_t i = 0; i < n; ++i) {
            const int j = asg[i];
            if (proj[j] < 0.0) continue;
            double xu = 0.0;
            for (int k = 0; k < dim; ++k) xu += samples[i * dim + k] * usum[j * dim + k];
            proj[j] += xu;
        }
        for (int j = 0; j < K; ++j) {
            if (proj[j] < 0.0) continue;
            const double len = proj[j] / (double)cnt[j];
            for (int k = 0; k < dim; ++k) codebook[j * dim + k] = len * usum[j * dim + k];
        }
    }
    free(asg);
    free(usum);
    free(proj);
    free(cnt);
    return it;
}

/* ------------------------------------------------------------------------ */
/* NSN front end alone (NSNQuant, Metodologia 1-2): the steps of kvqo_nsn_vq */
/* up to the rotated vector z, without the codebook search.  x [H, T, d];    */
/* s1, s2 [H, T]; o [H, d] (the mean of the T tokens, or o_given); z [H,T,d]. */
/* ------------------------------------------------------------------------ */
ORC_API int kvqo_nsn_front(int d, int64_t H, int64_t T, const double *x, const double *o_given, double *s1,
                           double *s2, double *o, double *z)
{
    if (T <= 0) return -1;
    const double sd = sqrt((double)d);
    double *a = (double *)malloc(sizeof(double) * T * d);
    for (int64_t h = 0; h < H; ++h) {
        const double *xh = x + h * T * d;
        double *oh = o + h * d;
        for (int i = 0; i < d; ++i) oh[i] = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            double ss = 0.0;
            for (int i = 0; i < d; ++i) ss += xh[t * d + i] * xh[t * d + i];
            const double nx = sqrt(ss);
            s1[h * T + t] = nx / sd;
            for (int i = 0; i < d; ++i) a[t * d + i] = nx > 0.0 ? sd * xh[t * d + i] / nx : 0.0;
        }
        for (int64_t t = 0; t < T; ++t)
            for (int i = 0; i < d; ++i) oh[i] += a[t * d + i];
        for (int i = 0; i < d; ++i) oh[i] = o_given ? o_given[h * d + i] : oh[i] / (double)T;
        for (int64_t t = 0; t < T; ++t) {
            double *zt = z + (h * T + t) * d;
            double ss = 0.0;
            for (int i = 0; i < d; ++i) {
                zt[i] = a[t * d + i] - oh[i];
                ss += zt[i] * zt[i];
            }
            const double nb = sqrt(ss);
            s2[h * T + t] = nb / sd;
            for (int i = 0; i < d; ++i) zt[i] = nb > 0.0 ? zt[i] / (nb / sd) : 0.0;
            kvqo_fwht(zt, d);
            for (int i = 0; i < d; ++i) zt[i] /= sd;
        }
    }
    free(a);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Gain-shape residual quantisation ("GSRQ: Quantitzacio Residual de Forma-  */
/* Guanys per a Cau KV de Menys d'1 Bit", q2bstudio): gain-shape k-means     */
/* (GSKM) keeps the norm (gain) of the reproduction apart from its direction */
/* (shape), so that the averaging of k-means does not shrink it; GSKM stages */
/* inside a residual quantisation pipeline give GSRQ.  The page gives no     */
/* dimensions, stage count or training recipe; the reading here:             */
/*  - GSKM on n samples of dimension m: K unit shapes, initialised from K     */
/*    given samples (normalised); a pass assigns every sample to the shape of */
/*    largest projection <x, s_j> (lowest j on ties), then moves each shape   */
/*    to the normalised sum of its samples (the unit vector with the largest  */
/*    summed projection over the cell); a shape with no sample or a zero sum  */
/*    is kept.  objective[it] = mean best projection at pass it's assignment. */
/*  - gain levels: Lloyd's algorithm in one dimension on the best            */
/*    projections (levels = cell means, thresholds = midpoints), started at   */
/*    the (i + 1/2) / L quantiles.                                            */
/*  - encoding of a sub-vector, stage k = 1, 2 on the running residual r      */
/*    (r = z first): j = argmax_j <r, S_k[j]> (lowest j on ties),             */
/*    p = <r, S_k[j]>, c = #{l : t_k[l] < p} (t_k the midpoints of the sorted */
/*    levels G_k), r <- r - G_k[c] S_k[j]; the reproduction is z - r.        */
/* ------------------------------------------------------------------------ */

ORC_API int kvqo_gskm(int64_t n, int m, int K, const double *x, const int64_t *init, int passes, double *shapes,
                      double *objective)
{
    int32_t *asg = (int32_t *)malloc(sizeof(int32_t) * n);
    double *sum = (double *)malloc(sizeof(double) * K * m);
    for (int j = 0; j < K; ++j) {
        double ss = 0.0;
        for (int k = 0; k < m; ++k) ss += x[init[j] * m + k] * x[init[j] * m + k];
        const double inv = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
        for (int k = 0; k < m; ++k) shapes[j * m + k] = x[init[j] * m + k] * inv;
    }
    int it = 0;
    for (; it < passes; ++it) {
        double tot = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            int best = 0;
            double bp = -INFINITY;
            for (int j = 0; j < K; ++j) {
                double p = 0.0;
                for (int k = 0; k < m; ++k) p += x[i * m + k] * shapes[j * m + k];
                if (p > bp) { bp = p; best = j; }
            }
            asg[i] = best;
            tot += bp;
        }
        if (objective) objective[it] = tot / (double)n;
        memset(sum, 0, sizeof(double) * K * m);
        for (int64_t i = 0; i < n; ++i)
            for (int k = 0; k < m; ++k) sum[asg[i] * m + k] += x[i * m + k];
        for (int j = 0; j < K; ++j) {
            double ss = 0.0;
            for (int k = 0; k < m; ++k) ss += sum[j * m + k] * sum[j * m + k];
            if (ss <= 0.0) continue;
            const double inv = 1.0 / sqrt(ss);
            for (int k = 0; k < m; ++k) shapes[j * m + k] = sum[j * m + k] * inv;
        }
    }
    free(asg);
    free(sum);
    return it;
}

static int cmp_double(const void *a, const void *b)
{
    const double x = *(const double *)a, y = *(const double *)b;
    return x < y ? -1 : x > y ? 1 : 0;
}

/* Returns 0 (passes run as given). */
ORC_API int kvqo_lloyd_1d(int64_t n, const double *v, int L, int passes, double *levels)
{
    if (n <= 0 || L <= 0) return -1;
    double *sv = (double *)malloc(sizeof(double) * n);
    double *sum = (double *)malloc(sizeof(double) * L);
    int64_t *cnt = (int64_t *)malloc(sizeof(int64_t) * L);
    memcpy(sv, v, sizeof(double) * n);
    qsort(sv, (size_t)n, sizeof(double), cmp_double);
    for (int l = 0; l < L; ++l) {
        int64_t i = (int64_t)(((double)l + 0.5) / L * (double)n);
        if (i >= n) i = n - 1;
        levels[l] = sv[i];
    }
    int it = 0;
    for (; it < passes; ++it) {
        memset(sum, 0, sizeof(double) * L);
        memset(cnt, 0, sizeof(int64_t) * L);
        for (int64_t i = 0; i < n; ++i) {
            int c = 0;
            while (c < L - 1 && 0.5 * (levels[c] + levels[c + 1]) < sv[i]) ++c;
            sum[c] += sv[i];
            ++cnt[c];
        }
        for (int l = 0; l < L; ++l)
            if (cnt[l] > 0) levels[l] = sum[l] / (double)cnt[l];
    }
    free(sv);
    free(sum);
    free(cnt);
    return 0;
}

/* One stage on residual r [m]: the shape index, the gain index and flags   */
/* (bit 0: best projection within band of the runner-up; bit 1: projection */
/* within band of a gain threshold); r is updated.                          */
static void gsrq_stage(int m, int K, int L, double *r, const double *S, const double *G, double band, int *j_out,
                       int *c_out, int *flags)
{
    int best = 0;
    double bp = -INFINITY, second = -INFINITY;
    for (int j = 0; j < K; ++j) {
        double p = 0.0;
        for (int k = 0; k < m; ++k) p += r[k] * S[j * m + k];
        if (p > bp) { second = bp; bp = p; best = j; }
        else if (p > second) second = p;
    }
    int c = 0, f = 0;
    for (int l = 0; l + 1 < L; ++l) {
        const double t = 0.5 * (G[l] + G[l + 1]);
        if (t < bp) ++c;
        if (fabs(bp - t) < band) f |= 2;
    }
    if (bp - second < band) f |= 1;
    for (int k = 0; k < m; ++k) r[k] -= G[c] * S[best * m + k];
    *j_out = best;
    *c_out = c;
    *flags = f;
}

/* n sub-vectors z [n][m] -> codes [n][3] = (j1, j2, c1 | c2 << 4), the       */
/* reproductions zhat [n][m] and flags [n] (stage-1 bits 0-1, stage-2 2-3).  */
/* K <= 256 shapes and L <= 16 sorted levels per stage.                      */
ORC_API int kvqo_gsrq_encode(int64_t n, int m, int K, int L, const double *z, const double *S1, const double *G1,
                             const double *S2, const double *G2, double band, uint8_t *codes, double *zhat,
                             uint8_t *flags)
{
    if (K > 256 || L > 16 || m > 256) return -1;
    double r[256];
    for (int64_t i = 0; i < n; ++i) {
        for (int k = 0; k < m; ++k) r[k] = z[i * m + k];
        int j1, c1, f1, j2, c2, f2;
        gsrq_stage(m, K, L, r, S1, G1, band, &j1, &c1, &f1);
        gsrq_stage(m, K, L, r, S2, G2, band, &j2, &c2, &f2);
        codes[i * 3] = (uint8_t)j1;
        codes[i * 3 + 1] = (uint8_t)j2;
        codes[i * 3 + 2] = (uint8_t)(c1 | (c2 << 4));
        if (zhat)
            for (int k = 0; k < m; ++k) zhat[i * m + k] = z[i * m + k] - r[k];
        if (flags) flags[i] = (uint8_t)(f1 | (f2 << 2));
    }
    return 0;
}

/* Reproduction of a whole vector from its record: P = d / m sub-vectors,    */
/* record bytes [j1 of each sub-vector][j2 of each][c1 | c2 << 4 of each].    */
static void gsrq_entries(int d, int m, const uint8_t *rec, const double *S1, const double *G1, const double *S2,
                         const double *G2, double *zq)
{
    const int P = d / m;
    for (int s = 0; s < P; ++s) {
        const int j1 = rec[s], j2 = rec[P + s], c1 = rec[2 * P + s] & 15, c2 = rec[2 * P + s] >> 4;
        for (int k = 0; k < m; ++k) zq[s * m + k] = G1[c1] * S1[j1 * m + k] + G2[c2] * S2[j2 * m + k];
    }
}

/* Logits and decode attention over GSRQ records with the NSN byproducts      */
/* (x_hat = s1 (s2 H zq / sqrt(d) + o), as for NSN-VQ).  route 1: reconstruct */
/* then dot; route 2: q' = H q / sqrt(d) and                                  */
/*   logit = s1 (s2 sum_s (G1[c1] <q'_s, S1[j1]> + G2[c2] <q'_s, S2[j2]>) + <q, o>). */
ORC_API int kvqo_gsrq_logits(int route, int d, int m, int64_t B, int64_t Hq, int64_t Hkv, int64_t T,
                             const double *q, const uint8_t *codes, const double *s1, const double *s2,
                             const double *o, const double *S1, const double *G1, const double *S2,
                             const double *G2, double *logits)
{
    if (Hkv <= 0 || Hq % Hkv || d % m) return -1;
    const int64_t G = Hq / Hkv;
    const int P = d / m, rb = 3 * P;
    double *zq = (double *)malloc(sizeof(double) * d);
    double *xh = (double *)malloc(sizeof(double) * d);
    double *qr = (double *)malloc(sizeof(double) * d);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < Hq; ++h) {
            const int64_t g = h / G;
            const double *qh = q + (b * Hq + h) * d;
            const double *og = o + (b * Hkv + g) * d;
            double qo = 0.0;
            for (int i = 0; i < d; ++i) qo += qh[i] * og[i];
            for (int i = 0; i < d; ++i) qr[i] = qh[i];
            kvqo_fwht(qr, d);
            for (int i = 0; i < d; ++i) qr[i] /= sqrt((double)d);
            for (int64_t t = 0; t < T; ++t) {
                const int64_t v = (b * Hkv + g) * T + t;
                const uint8_t *rec = codes + v * rb;
                double acc = 0.0;
                if (route == 1) {
                    gsrq_entries(d, m, rec, S1, G1, S2, G2, zq);
                    kvqo_nsn_reconstruct(d, zq, s1[v], s2[v], og, xh);
                    for (int i = 0; i < d; ++i) acc += qh[i] * xh[i];
                } else {
                    for (int s = 0; s < P; ++s) {
                        const int j1 = rec[s], j2 = rec[P + s], c1 = rec[2 * P + s] & 15, c2 = rec[2 * P + s] >> 4;
                        double a1 = 0.0, a2 = 0.0;
                        for (int k = 0; k < m; ++k) {
                            a1 += qr[s * m + k] * S1[j1 * m + k];
                            a2 += qr[s * m + k] * S2[j2 * m + k];
                        }
                        acc += G1[c1] * a1 + G2[c2] * a2;
                    }
                    acc = s1[v] * (s2[v] * acc + qo);
                }
                logits[(b * Hq + h) * T + t] = acc;
            }
        }
    free(zq);
    free(xh);
    free(qr);
    return 0;
}

ORC_API int kvqo_gsrq_attention(int d, int m, int64_t B, int64_t Hq, int64_t Hkv, int64_t T, const double *q,
                                const uint8_t *kc, const double *ks1, const double *ks2, const double *ko,
                                const uint8_t *vc, const double *vs1, const double *vs2, const double *vo,
                                const double *S1, const double *G1, const double *S2, const double *G2,
                                double sm_scale, double *out)
{
    if (Hkv <= 0 || Hq % Hkv || T <= 0 || d % m) return -1;
    const int64_t G = Hq / Hkv;
    const int rb = 3 * (d / m);
    double *K = (double *)malloc(sizeof(double) * T * d);
    double *V = (double *)malloc(sizeof(double) * T * d);
    double *zq = (double *)malloc(sizeof(double) * d);
    double *w = (double *)malloc(sizeof(double) * T);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t g = 0; g < Hkv; ++g) {
            const int64_t bg = b * Hkv + g;
            for (int64_t t = 0; t < T; ++t) {
                const int64_t v = bg * T + t;
                gsrq_entries(d, m, kc + v * rb, S1, G1, S2, G2, zq);
                kvqo_nsn_reconstruct(d, zq, ks1[v], ks2[v], ko + bg * d, K + t * d);
                gsrq_entries(d, m, vc + v * rb, S1, G1, S2, G2, zq);
                kvqo_nsn_reconstruct(d, zq, vs1[v], vs2[v], vo + bg * d, V + t * d);
            }
            for (int64_t hh = 0; hh < G; ++hh) {
                const double *qh = q + (b * Hq + g * G + hh) * d;
                double mx = -INFINITY;
                for (int64_t t = 0; t < T; ++t) {
                    double a = 0.0;
                    for (int i = 0; i < d; ++i) a += qh[i] * K[t * d + i];
                    w[t] = sm_scale * a;
                    if (w[t] > mx) mx = w[t];
                }
                double l = 0.0;
                for (int64_t t = 0; t < T; ++t) {
                    w[t] = exp(w[t] - mx);
                    l += w[t];
                }
                double *oh = out + (b * Hq + g * G + hh) * d;
                for (int i = 0; i < d; ++i) oh[i] = 0.0;
                for (int64_t t = 0; t < T; ++t)
                    for (int i = 0; i < d; ++i) oh[i] += w[t] * V[t * d + i];
                for (int i = 0; i < d; ++i) oh[i] /= l;
            }
        }
    free(K);
    free(V);
    free(zq);
    free(w);
    return 0;
}
