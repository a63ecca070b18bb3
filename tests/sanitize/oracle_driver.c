/* Runs every routine of the CPU oracle once on small seeded inputs, for a
 * build with the address and undefined-behaviour sanitizers (test
 * infrastructure; the results are checked elsewhere, here only that every
 * access stays in bounds and no arithmetic is undefined).  Prints "oracle ok". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kvqo_lloyd_max(int bits, const double *init, int max_iter, double tol, double *c_out, int *iters_out);
double kvqo_gauss_mse(int bits, const double *c, const double *t);
int kvqo_tables_f32(int bits, float *c32, float *t32);
double kvqo_beta_mass(int d, double a, double b);
int kvqo_lloyd_max_beta(int bits, int d, int max_iter, double tol, double *c_out, int *iters_out);
double kvqo_beta_mse(int bits, int d, const double *c, const double *t);
int kvqo_tables_f32_beta(int bits, int d, float *c32, float *t32);
int kvqo_hadamard_entry(int i, int j);
void kvqo_hadamard_dense(const double *x, double *y, int n);
void kvqo_fwht(double *x, int n);
void kvqo_pack(const int32_t *idx, int d, int bits, uint8_t *rec);
void kvqo_unpack(const uint8_t *rec, int d, int bits, int32_t *idx);
void kvqo_scalar_quantize(const double *y, int64_t n, int bits, const float *c32, const float *t32, int32_t *idx,
                          double *yhat);
int kvqo_quantize(int d, int bits, int64_t B, int64_t H, int64_t T, const double *x, const int8_t *signs,
                  const float *t32, double band, uint8_t *codes, double *norms, double *y_out, int32_t *idx_out,
                  uint8_t *flags);
void kvqo_dequant(int d, int bits, const uint8_t *rec, double rho, const int8_t *signs, const float *c32,
                  double *out);
int kvqo_logits(int route, int d, int bits, int64_t B, int64_t Hq, int64_t Hkv, int64_t T, const double *q,
                const uint8_t *codes, const double *norms, const int8_t *signs, const float *c32,
                const uint8_t *qjl_signs, const double *gamma, const double *S, int m, double *logits);
int kvqo_attention(int d, int bits, int64_t B, int64_t Hq, int64_t Hkv, int64_t T, const double *q,
                   const uint8_t *kc, const double *kn, const uint8_t *vc, const double *vn, const int8_t *signs_k,
                   const int8_t *signs_v, const float *c32, double sm_scale, double *out);
int kvqo_quantize_dense(int d, int bits, int64_t B, int64_t H, int64_t T, const double *x, const double *Q,
                        const float *t32, double band, uint8_t *codes, double *norms, double *y_out,
                        int32_t *idx_out, uint8_t *flags);
void kvqo_dequant_dense(int d, int bits, const uint8_t *rec, double rho, const double *Q, const float *c32,
                        double *out);
int kvqo_logits_dense(int route, int d, int bits, int64_t B, int64_t Hq, int64_t Hkv, int64_t T, const double *q,
                      const uint8_t *codes, const double *norms, const double *Q, const float *c32,
                      const uint8_t *qjl_signs, const double *gamma, const double *S, int m, double *logits);
int kvqo_attention_dense(int d, int bits, int64_t B, int64_t Hq, int64_t Hkv, int64_t T, const double *q,
                         const uint8_t *kc, const double *kn, const uint8_t *vc, const double *vn, const double *Q,
                         const float *c32, double sm_scale, double *out);
int kvqo_attention_stream(int d, int bits, int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t R, const double *q,
                          const uint8_t *kc, const double *kn, const uint8_t *vc, const double *vn, const double *kt,
                          const double *vt, const int8_t *signs_k, const int8_t *signs_v, const float *c32,
                          double sm_scale, double *out);
int kvqo_qjl(int d, int m, int64_t n, const double *y, const int32_t *idx, const float *c32, const double *S,
             double band, uint8_t *sgn, double *gamma, uint8_t *flags);
int kvqo_nsn_vq(int d, int sub, int K, int64_t H, int64_t T, const double *x, const double *codebook, double band,
                uint8_t *codes, double *s1, double *s2, double *o, double *z_out, uint8_t *flags,
                const double *o_given, int adaptive);
void kvqo_nsn_reconstruct(int d, const double *zq, double s1, double s2, const double *o, double *x_hat);
int kvqo_nsn_logits(int route, int d, int sub, int64_t B, int64_t Hq, int64_t Hkv, int64_t T, const double *q,
                    const uint8_t *codes, const double *s1, const double *s2, const double *o, const double *cb,
                    double *logits);
int kvqo_nsn_attention(int d, int sub, int64_t B, int64_t Hq, int64_t Hkv, int64_t T, const double *q,
                       const uint8_t *kc, const double *ks1, const double *ks2, const double *ko, const uint8_t *vc,
                       const double *vs1, const double *vs2, const double *vo, const double *cb, double sm_scale,
                       double *out);
int kvqo_nsn_attention_stream(int d, int sub, int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t Gs, int64_t R,
                              const double *q, const uint8_t *kc, const double *ks1, const double *ks2,
                              const double *ko, const uint8_t *vc, const double *vs1, const double *vs2,
                              const double *vo, const double *kt, const double *vt, const double *cb,
                              double sm_scale, double *out);
int kvqo_kmeans(int64_t n, int dim, int K, const double *samples, const int64_t *init, int max_iter,
                double *codebook, double *distortion);
int kvqo_cosine_refine(int64_t n, int dim, int K, const double *samples, double *codebook, int passes,
                       double *mean_cos);

static uint64_t rs = 88172645463325252ull;
static double urand(void)
{
    rs ^= rs << 13;
    rs ^= rs >> 7;
    rs ^= rs << 17;
    return (double)(rs >> 11) / 9007199254740992.0;
}
static double nrand(void)
{
    double u = urand() + 1e-300, v = urand();
    return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}
static void *zalloc(size_t n) { void *p = calloc(n ? n : 1, 1); if (!p) abort(); return p; }
#define CHECK(e) do { if (!(e)) { fprintf(stderr, "check failed: %s (line %d)\n", #e, __LINE__); return 1; } } while (0)

int main(void)
{
    const int d = 128, B = 2, H = 2, Hq = 4, T = 37, R = 5, m = 128;
    const int64_t nv = (int64_t)B * H * T;
    double *x = zalloc(sizeof(double) * nv * d), *v = zalloc(sizeof(double) * nv * d);
    for (int64_t i = 0; i < nv * d; ++i) { x[i] = nrand(); v[i] = nrand(); }
    memset(x + 5 * d, 0, sizeof(double) * d); /* a zero vector */
    int8_t *sg = zalloc((size_t)H * d);
    for (int i = 0; i < H * d; ++i) sg[i] = urand() < 0.5 ? -1 : 1;
    double *q = zalloc(sizeof(double) * B * Hq * d);
    for (int i = 0; i < B * Hq * d; ++i) q[i] = nrand();
    double *S = zalloc(sizeof(double) * m * d), *Q = zalloc(sizeof(double) * d * d);
    for (int i = 0; i < m * d; ++i) S[i] = nrand();
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) Q[i * d + j] = kvqo_hadamard_entry(i, j) / sqrt((double)d);
    for (int bits = 1; bits <= 4; ++bits) {
        const int L = 1 << bits, rec = d * bits / 8;
        double c[16], t[16];
        int it = 0;
        CHECK(kvqo_lloyd_max(bits, NULL, 100000, 1e-12, c, &it) == 0);
        for (int j = 0; j + 1 < L; ++j) t[j] = 0.5 * (c[j] + c[j + 1]);
        CHECK(kvqo_gauss_mse(bits, c, t) > 0.0);
        float c32[16], t32[16], cb32[16], tb32[16];
        CHECK(kvqo_tables_f32(bits, c32, t32) == 0);
        CHECK(kvqo_tables_f32_beta(bits, d, cb32, tb32) == 0);
        double cb[16], tb[16];
        CHECK(kvqo_lloyd_max_beta(bits, d, 100000, 1e-12, cb, &it) == 0);
        for (int j = 0; j + 1 < L; ++j) tb[j] = 0.5 * (cb[j] + cb[j + 1]);
        CHECK(kvqo_beta_mse(bits, d, cb, tb) > 0.0);
        uint8_t *kc = zalloc((size_t)nv * rec), *vc = zalloc((size_t)nv * rec), *fl = zalloc((size_t)nv * d);
        double *kn = zalloc(sizeof(double) * nv), *vn = zalloc(sizeof(double) * nv), *y = zalloc(sizeof(double) * nv * d);
        int32_t *idx = zalloc(sizeof(int32_t) * nv * d);
        CHECK(kvqo_quantize(d, bits, B, H, T, x, sg, t32, 1e-5, kc, kn, y, idx, fl) == 0);
        CHECK(kvqo_quantize(d, bits, B, H, T, v, sg, t32, 1e-5, vc, vn, NULL, NULL, NULL) == 0);
        double out[128], *lg = zalloc(sizeof(double) * B * Hq * T), *att = zalloc(sizeof(double) * B * Hq * d);
        kvqo_dequant(d, bits, kc, kn[0], sg, c32, out);
        uint8_t *qs = zalloc((size_t)nv * m / 8), *qf = zalloc((size_t)nv * m);
        double *gm = zalloc(sizeof(double) * nv);
        CHECK(kvqo_qjl(d, m, nv, y, idx, c32, S, 1e-5, qs, gm, qf) == 0);
        for (int route = 1; route <= 2; ++route) {
            CHECK(kvqo_logits(route, d, bits, B, Hq, H, T, q, kc, kn, sg, c32, NULL, NULL, NULL, 0, lg) == 0);
            CHECK(kvqo_logits(route, d, bits, B, Hq, H, T, q, kc, kn, sg, c32, qs, gm, S, m, lg) == 0);
            CHECK(kvqo_logits_dense(route, d, bits, B, Hq, H, T, q, kc, kn, Q, c32, NULL, NULL, NULL, 0, lg) == 0);
            CHECK(kvqo_logits_dense(route, d, bits, B, Hq, H, T, q, kc, kn, Q, c32, qs, gm, S, m, lg) == 0);
        }
        CHECK(kvqo_attention(d, bits, B, Hq, H, T, q, kc, kn, vc, vn, sg, sg, c32, 0.1, att) == 0);
        CHECK(kvqo_attention_dense(d, bits, B, Hq, H, T, q, kc, kn, vc, vn, Q, c32, 0.1, att) == 0);
        double *kt = zalloc(sizeof(double) * B * H * R * d);
        for (int i = 0; i < B * H * R * d; ++i) kt[i] = nrand();
        CHECK(kvqo_attention_stream(d, bits, B, Hq, H, T, R, q, kc, kn, vc, vn, kt, kt, sg, sg, c32, 0.1, att) == 0);
        CHECK(kvqo_attention_stream(d, bits, B, Hq, H, 0, R, q, kc, kn, vc, vn, kt, kt, sg, sg, c32, 0.1, att) == 0);
        CHECK(kvqo_quantize_dense(d, bits, B, H, T, x, Q, t32, 1e-5, kc, kn, y, idx, fl) == 0);
        kvqo_dequant_dense(d, bits, kc, kn[1], Q, c32, out);
        double yy[64];
        int32_t ii[64];
        for (int i = 0; i < 64; ++i) yy[i] = 3.0 * nrand();
        kvqo_scalar_quantize(yy, 64, bits, c32, t32, ii, yy);
        free(kc); free(vc); free(fl); free(kn); free(vn); free(y); free(idx); free(lg); free(att);
        free(qs); free(qf); free(gm); free(kt);
    }
    for (int bits = 1; bits <= 8; ++bits) {
        int32_t idx[128], back[128];
        uint8_t rec[128];
        for (int i = 0; i < d; ++i) idx[i] = (int32_t)(urand() * (1 << bits));
        kvqo_pack(idx, d, bits, rec);
        kvqo_unpack(rec, d, bits, back);
        CHECK(memcmp(idx, back, sizeof(idx)) == 0);
    }
    double hx[128], hy[128];
    for (int i = 0; i < d; ++i) hx[i] = nrand();
    kvqo_hadamard_dense(hx, hy, d);
    kvqo_fwht(hx, d);
    CHECK(kvqo_beta_mass(d, -1.0, 1.0) > 0.0);
    /* NSN + VQ with a small random codebook */
    const int K = 256, sub = 8;
    double *cbk = zalloc(sizeof(double) * K * sub);
    for (int i = 0; i < K * sub; ++i) cbk[i] = nrand();
    uint8_t *codes = zalloc((size_t)nv * (d / sub)), *fl = zalloc((size_t)nv * (d / sub));
    double *s1 = zalloc(sizeof(double) * nv), *s2 = zalloc(sizeof(double) * nv), *o = zalloc(sizeof(double) * B * H * d);
    double *z = zalloc(sizeof(double) * nv * d);
    CHECK(kvqo_nsn_vq(d, sub, K, B * H, T, x, cbk, 1e-5, codes, s1, s2, o, z, fl, NULL, 0) == 0);
    CHECK(kvqo_nsn_vq(d, sub, K, B * H, T, x, cbk, 1e-5, codes, s1, s2, o, z, fl, NULL, 1) == 0);
    CHECK(kvqo_nsn_vq(d, sub, K, B * H, T, x, cbk, 1e-5, codes, s1, s2, o, NULL, NULL, o, 1) == 0);
    double xh[128];
    kvqo_nsn_reconstruct(d, z, s1[0], s2[0], o, xh);
    double *lg = zalloc(sizeof(double) * B * Hq * T), *att = zalloc(sizeof(double) * B * Hq * d);
    for (int route = 1; route <= 2; ++route)
        CHECK(kvqo_nsn_logits(route, d, sub, B, Hq, H, T, q, codes, s1, s2, o, cbk, lg) == 0);
    CHECK(kvqo_nsn_attention(d, sub, B, Hq, H, T, q, codes, s1, s2, o, codes, s1, s2, o, cbk, 0.1, att) == 0);
    {   /* one group of T tokens (the means o are per (b, g)), and a window of R */
        double *kt2 = zalloc(sizeof(double) * B * H * 5 * d);
        for (int i = 0; i < B * H * 5 * d; ++i) kt2[i] = nrand();
        CHECK(kvqo_nsn_attention_stream(d, sub, B, Hq, H, T, T, 5, q, codes, s1, s2, o, codes, s1, s2, o, kt2, kt2,
                                        cbk, 0.1, att) == 0);
        CHECK(kvqo_nsn_attention_stream(d, sub, B, Hq, H, 0, 1, 5, q, codes, s1, s2, o, codes, s1, s2, o, kt2, kt2,
                                        cbk, 0.1, att) == 0);
        free(kt2);
    }
    /* k-means on a few samples */
    const int64_t ns = 2000;
    double *smp = zalloc(sizeof(double) * ns * sub), *kcb = zalloc(sizeof(double) * 16 * sub), dist[10];
    int64_t init[16];
    for (int64_t i = 0; i < ns * sub; ++i) smp[i] = nrand();
    for (int i = 0; i < 16; ++i) init[i] = i * 7;
    CHECK(kvqo_kmeans(ns, sub, 16, smp, init, 10, kcb, dist) > 0);
    CHECK(kvqo_cosine_refine(ns, sub, 16, smp, kcb, 5, dist) == 5);
    free(cbk); free(codes); free(fl); free(s1); free(s2); free(o); free(z); free(lg); free(att); free(smp); free(kcb);
    free(x); free(v); free(sg); free(q); free(S); free(Q);
    printf("oracle ok\n");
    return 0;
}
