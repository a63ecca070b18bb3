// libkvq host side: context lifetime, the Lloyd-Max table builders (N(0,1) and
// the exact law at d = 128),
// argument validation and kernel launches behind the C ABI of kvq.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>

#include "kvq_internal.h"

namespace {

// ---------------------------------------------------------------------------
// Lloyd-Max quantiser for N(0,1) ("PolarQuant", Methodology: Lloyd-Max
// centroids, optimal in MSE for the Gaussian; "TurboQuant", Como Implementar:
// tables precomputed per bit width).  The Gaussian is symmetric, so only the
// 2^(b-1) positive levels m_k are iterated; cell k of the positive half is
// [tau_k, tau_{k+1}) with tau_0 = 0, tau_k = (m_{k-1} + m_k)/2 and
// tau_{half} = +inf, and each level is moved to its cell's conditional mean
//   m_k = (phi(tau_k) - phi(tau_{k+1})) / (Q(tau_k) - Q(tau_{k+1})),
// Q the upper tail.  The negative half is the mirror image, so the table is
// exactly antisymmetric.
// ---------------------------------------------------------------------------
double phi(double x) { return std::isinf(x) ? 0.0 : std::exp(-0.5 * x * x) * 0.3989422804014327; }
double upper_tail(double x) { return std::isinf(x) ? 0.0 : 0.5 * std::erfc(x * 0.7071067811865476); }

void build_codebook(int bits, kvq::Codebook *cb)
{
    const int L = 1 << bits, half = L / 2;
    double m[8];
    for (int k = 0; k < half; ++k) m[k] = 3.0 * (k + 0.5) / half;  // spread over [0, 3]
    for (int it = 0; it < 200000; ++it) {
        double tau[9];
        tau[0] = 0.0;
        for (int k = 1; k < half; ++k) tau[k] = 0.5 * (m[k - 1] + m[k]);
        tau[half] = INFINITY;
        double change = 0.0;
        for (int k = 0; k < half; ++k) {
            double nm = (phi(tau[k]) - phi(tau[k + 1])) / (upper_tail(tau[k]) - upper_tail(tau[k + 1]));
            change = std::fmax(change, std::fabs(nm - m[k]));
            m[k] = nm;
        }
        if (change <= 1e-16) break;
    }
    std::memset(cb, 0, sizeof(*cb));
    cb->bits = bits;
    for (int k = 0; k < half; ++k) {
        cb->c[half + k] = (float)m[k];
        cb->c[half - 1 - k] = -(float)m[k];
    }
    // Stored thresholds: fp32 midpoints of adjacent fp32 centroids.
    for (int j = 0; j + 1 < L; ++j) cb->t[j] = (float)(((double)cb->c[j] + (double)cb->c[j + 1]) * 0.5);
}

// ---------------------------------------------------------------------------
// Lloyd-Max quantiser for the exact coordinate law at dimension d
// ("TurboQuant", Como Funciona, Estagio 1: after the rotation a coordinate of
// the unit vector follows Beta((d-1)/2, (d-1)/2) on [-1, 1]; the quantiser is
// optimised for that law).  Scaled by sqrt(d) (unit variance) the density is
// proportional to g(y) = (1 - y^2/d)^((d-3)/2) on [-sqrt d, sqrt d].  As for
// the Gaussian only the positive levels are iterated; the cell integrals of g
// and y g come from cumulative Simpson sums from 0 on a grid of step 1/2048,
// plus one Simpson step over the partial interval.
// ---------------------------------------------------------------------------
struct BetaHalf {
    int d;
    double r, h;
    int n;
    double *m0, *m1;  // int_0^{i h} g, int_0^{i h} y g
    double g(double y) const
    {
        const double u = 1.0 - y * y / d;
        return u <= 0.0 ? 0.0 : std::pow(u, 0.5 * (d - 3));
    }
    void simpson(double a, double b, double &s0, double &s1) const
    {
        const double m = 0.5 * (a + b), ga = g(a), gm = g(m), gb = g(b), w = (b - a) / 6.0;
        s0 = w * (ga + 4.0 * gm + gb);
        s1 = w * (a * ga + 4.0 * m * gm + b * gb);
    }
    bool init(int dim)
    {
        d = dim;
        r = std::sqrt((double)d);
        h = 1.0 / 2048.0;
        n = (int)std::ceil(r / h) + 1;
        m0 = (double *)std::malloc(sizeof(double) * n);
        m1 = (double *)std::malloc(sizeof(double) * n);
        if (!m0 || !m1) return false;
        m0[0] = m1[0] = 0.0;
        for (int i = 1; i < n; ++i) {
            double s0, s1;
            simpson((i - 1) * h, std::fmin(i * h, r), s0, s1);
            m0[i] = m0[i - 1] + s0;
            m1[i] = m1[i - 1] + s1;
        }
        return true;
    }
    void at(double y, double &a0, double &a1) const  // int_0^y of g and y g
    {
        y = std::fmin(y, r);
        int i = (int)(y / h);
        if (i > n - 1) i = n - 1;
        double s0 = 0.0, s1 = 0.0;
        if (y > i * h) simpson(i * h, y, s0, s1);
        a0 = m0[i] + s0;
        a1 = m1[i] + s1;
    }
    ~BetaHalf()
    {
        std::free(m0);
        std::free(m1);
    }
};

bool build_codebook_beta(int bits, int d, kvq::Codebook *cb)
{
    BetaHalf B{};
    if (!B.init(d)) return false;
    const int L = 1 << bits, half = L / 2;
    double m[8];
    for (int k = 0; k < half; ++k) m[k] = 3.0 * (k + 0.5) / half;
    for (int it = 0; it < 200000; ++it) {
        double tau[9];
        tau[0] = 0.0;
        for (int k = 1; k < half; ++k) tau[k] = 0.5 * (m[k - 1] + m[k]);
        tau[half] = B.r;
        double change = 0.0, lo0, lo1, hi0, hi1;
        B.at(tau[0], lo0, lo1);
        for (int k = 0; k < half; ++k) {
            B.at(tau[k + 1], hi0, hi1);
            const double nm = (hi1 - lo1) / (hi0 - lo0);
            change = std::fmax(change, std::fabs(nm - m[k]));
            m[k] = nm;
            lo0 = hi0;
            lo1 = hi1;
        }
        if (change <= 1e-15) break;
    }
    std::memset(cb, 0, sizeof(*cb));
    cb->bits = bits;
    for (int k = 0; k < half; ++k) {
        cb->c[half + k] = (float)m[k];
        cb->c[half - 1 - k] = -(float)m[k];
    }
    for (int j = 0; j + 1 < L; ++j) cb->t[j] = (float)(((double)cb->c[j] + (double)cb->c[j + 1]) * 0.5);
    return true;
}

struct DeviceGuard {
    int prev = -1;
    bool ok = false;
    explicit DeviceGuard(int dev)
    {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        ok = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard()
    {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

void free_ctx(kvq_ctx *c)
{
    if (!c) return;
    (void)hipFree(c->d_sgnmask);
    (void)hipFree(c->d_signs);
    (void)hipFree(c->d_S);
    (void)hipFree(c->d_S16);
    (void)hipFree(c->d_vq);
    (void)hipFree(c->d_Q);
    (void)hipFree(c->d_Qt);
    (void)hipFree(c->d_Q16);
    (void)hipFree(c->d_vq16);
    (void)hipFree(c->d_vqbias);
    (void)hipFree(c->d_gsrq);
    (void)hipFree(c->d_gsrq16);
    std::free(c->h_signs);
    delete c;
}

// SplitMix64 (Steele, Lea and Flood 2014): output n (counting from 0) of the
// generator seeded with `seed`.
uint64_t splitmix64(uint64_t seed, uint64_t n)
{
    uint64_t z = seed + (n + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

template <class T>
kvq_status upload(T **dst, const T *src, size_t n)
{
    if (hipMalloc((void **)dst, n * sizeof(T)) != hipSuccess) {
        *dst = nullptr;
        return KVQ_E_NOMEM;
    }
    if (hipMemcpy(*dst, src, n * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) return KVQ_E_DEVICE;
    return KVQ_OK;
}

kvq_status launch_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_E_DEVICE; }

bool mse_mode(int m) { return m == KVQ_MODE_MSE || m == KVQ_MODE_MSE_QJL; }

// The codebook's n values in 4 bits ([NSN] Metodologia sec. 3, double
// quantisation): one block, lo = min, step = (max - lo) / 15, each value
// replaced by lo + code step with code the nearest level; decided in double.
// GSRQ tables: 2 x (256 x 32 shape values, 16 strictly increasing levels),
// all finite.
constexpr size_t kGsrqShape = (size_t)kvq::kVqK * 32;
bool gsrq_tables_ok(const float *t)
{
    if (!t) return false;
    for (int st = 0; st < 2; ++st) {
        const float *S = t + st * (kGsrqShape + 16), *G = S + kGsrqShape;
        for (size_t i = 0; i < kGsrqShape; ++i)
            if (!std::isfinite(S[i])) return false;
        for (int l = 0; l < 16; ++l)
            if (!std::isfinite(G[l]) || (l > 0 && !(G[l] > G[l - 1]))) return false;
    }
    return true;
}

void dq4_codebook(float *v, size_t n)
{
    double lo = v[0], hi = v[0];
    for (size_t i = 1; i < n; ++i) {
        lo = std::min(lo, (double)v[i]);
        hi = std::max(hi, (double)v[i]);
    }
    const double step = (hi - lo) / 15.0;
    if (!(step > 0.0)) return;
    for (size_t i = 0; i < n; ++i) {
        int c = (int)std::floor(((double)v[i] - lo) / step + 0.5);
        c = std::min(15, std::max(0, c));
        v[i] = (float)(lo + c * step);
    }
}

// Query heads per KV head that the kernels are built for.
bool logits_group_built(int64_t G) { return G == 1 || G == 2 || G == 4 || G == 8; }
bool decode_group_built(int64_t G) { return G == 1 || G == 2 || G == 4; }

}  // namespace

// KVQ_SPLITS: a positive integer in the environment replaces the automatic
// split count of the decode entry points (read once per process; an explicit
// n_split still wins, and the usual clamps apply).
static int env_splits()
{
    static const int v = [] {
        const char *e = std::getenv("KVQ_SPLITS");
        if (!e || !*e) return 0;
        char *end = nullptr;
        const long n = std::strtol(e, &end, 10);
        return (*end == '\0' && n > 0 && n <= (1L << 20)) ? (int)n : 0;
    }();
    return v;
}
static int auto_splits(int automatic) { return env_splits() ? env_splits() : automatic; }

extern "C" {

int32_t kvq_debug_build(void) { return KVQ_DEBUG_ON; }

uint32_t kvq_debug_take(void)
{
    // every file's record is read (and so cleared); the first non-zero one is returned
    const uint32_t r[] = {kvq::debug_take_quantize(), kvq::debug_take_score(), kvq::debug_take_nsn(),
                          kvq::debug_take_nsn_score(), kvq::debug_take_dense(), kvq::debug_take_stream()};
    for (uint32_t v : r)
        if (v) return v;
    return 0u;
}

const char *kvq_strerror(kvq_status s)
{
    // a C caller may pass any int: read it as an int, not as the enum type
    int v;
    std::memcpy(&v, &s, sizeof v);
    switch (v) {
    case KVQ_OK: return "ok";
    case KVQ_E_INVAL: return "invalid argument";
    case KVQ_E_UNSUPPORTED: return "unsupported configuration";
    case KVQ_E_DEVICE: return "device or HIP runtime error";
    case KVQ_E_NOMEM: return "out of memory";
    case KVQ_E_WORKSPACE: return "workspace too small";
    }
    return "unknown status";
}

kvq_status kvq_create(const kvq_config *cfg, kvq_ctx **out)
{
    if (!out) return KVQ_E_INVAL;
    *out = nullptr;
    if (!cfg) return KVQ_E_INVAL;
    if (cfg->d != kvq::kD || cfg->n_kv_heads < 1 || cfg->n_kv_heads > 4096) return KVQ_E_INVAL;
    const int mode = cfg->mode;
    if (!mse_mode(mode) && mode != KVQ_MODE_NSN_VQ && mode != KVQ_MODE_GSRQ) return KVQ_E_INVAL;
    const int H = cfg->n_kv_heads;
    if (mse_mode(mode)) {
        if (cfg->bits < 1 || cfg->bits > 4) return KVQ_E_INVAL;
        for (int i = 0; i < H * kvq::kD; ++i) {
            if (cfg->signs_k && cfg->signs_k[i] != 1 && cfg->signs_k[i] != -1) return KVQ_E_INVAL;
            if (cfg->signs_v && cfg->signs_v[i] != 1 && cfg->signs_v[i] != -1) return KVQ_E_INVAL;
        }
    }
    if (mode == KVQ_MODE_MSE_QJL && !cfg->qjl_S) return KVQ_E_INVAL;
    if (mode == KVQ_MODE_NSN_VQ && !cfg->vq_codebook) return KVQ_E_INVAL;
    if (mode == KVQ_MODE_GSRQ && !gsrq_tables_ok(cfg->gsrq_tables)) return KVQ_E_INVAL;
    if (cfg->codebook != KVQ_CODEBOOK_GAUSS && cfg->codebook != KVQ_CODEBOOK_BETA) return KVQ_E_INVAL;
    if (cfg->codebook == KVQ_CODEBOOK_BETA && !mse_mode(mode)) return KVQ_E_INVAL;
    if (cfg->rotation != KVQ_ROTATION_HADAMARD && cfg->rotation != KVQ_ROTATION_DENSE) return KVQ_E_INVAL;
    if (cfg->nsn_options & ~(KVQ_NSN_ADAPTIVE_SCALE | KVQ_NSN_DQ_CODEBOOK)) return KVQ_E_INVAL;
    if (cfg->nsn_options && mode != KVQ_MODE_NSN_VQ) return KVQ_E_INVAL;
    if (cfg->rotation == KVQ_ROTATION_DENSE) {
        if (!mse_mode(mode)) return KVQ_E_UNSUPPORTED;
        if (!cfg->rot_Q) return KVQ_E_INVAL;
        for (int i = 0; i < kvq::kD * kvq::kD; ++i)
            if (!std::isfinite(cfg->rot_Q[i]) || std::fabs(cfg->rot_Q[i]) > 1.0f) return KVQ_E_INVAL;
        // orthogonal to within 1e-3: max |Q Q^T - I| over all entries, in double
        const float *Q = cfg->rot_Q;
        for (int i = 0; i < kvq::kD; ++i)
            for (int j = i; j < kvq::kD; ++j) {
                double dot = 0.0;
                for (int k = 0; k < kvq::kD; ++k) dot += (double)Q[i * kvq::kD + k] * (double)Q[j * kvq::kD + k];
                if (std::fabs(dot - (i == j ? 1.0 : 0.0)) > 1e-3) return KVQ_E_INVAL;
            }
    }

    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || cfg->device < 0 || cfg->device >= ndev)
        return KVQ_E_DEVICE;
    DeviceGuard g(cfg->device);
    if (!g.ok) return KVQ_E_DEVICE;
    // scratch of kvq_attn_decode_noalloc on this device (once per device)
    if (kvq::noalloc_setup(cfg->device) != hipSuccess) return KVQ_E_DEVICE;

    kvq_ctx *c = new (std::nothrow) kvq_ctx();
    if (!c) return KVQ_E_NOMEM;
    c->d = cfg->d;
    c->bits = mse_mode(mode) ? cfg->bits : 1;
    c->mode = mode;
    c->rotation = cfg->rotation;
    c->nsn_options = cfg->nsn_options;
    c->H = H;
    c->device = cfg->device;
    if (hipDeviceGetAttribute(&c->n_cu, hipDeviceAttributeMultiprocessorCount, cfg->device) != hipSuccess ||
        c->n_cu < 1)
        c->n_cu = 256;
    if (cfg->codebook == KVQ_CODEBOOK_BETA) {
        if (!build_codebook_beta(c->bits, kvq::kD, &c->cb)) {
            free_ctx(c);
            return KVQ_E_NOMEM;
        }
    } else {
        build_codebook(c->bits, &c->cb);
    }

    kvq_status st = KVQ_OK;
    if (mse_mode(mode)) {
        const size_t n = (size_t)H * kvq::kD;
        uint32_t *mask = (uint32_t *)std::calloc(2 * n / 2, sizeof(uint32_t));
        float *sg = (float *)std::malloc(2 * n * sizeof(float));
        c->h_signs = (int8_t *)std::malloc(2 * n);
        if (!mask || !sg || !c->h_signs) st = KVQ_E_NOMEM;
        for (int kind = 0; st == KVQ_OK && kind < 2; ++kind) {
            const int8_t *src = kind ? cfg->signs_v : cfg->signs_k;
            int8_t *dst = c->h_signs + kind * n;
            for (size_t i = 0; i < n; ++i)
                dst[i] = src ? src[i] : ((splitmix64(cfg->seed, ((uint64_t)kind << 32) + i) >> 63) ? -1 : 1);
            for (size_t i = 0; i < n; ++i) {
                sg[kind * n + i] = (float)dst[i];
                if (dst[i] < 0) mask[(kind * n + i) / 2] |= (i & 1) ? 0x80000000u : 0x8000u;
            }
        }
        if (st == KVQ_OK) st = upload(&c->d_sgnmask, mask, n);
        if (st == KVQ_OK) st = upload(&c->d_signs, sg, 2 * n);
        std::free(mask);
        std::free(sg);
    }
    if (st == KVQ_OK && mode == KVQ_MODE_MSE_QJL) {
        const size_t n = (size_t)kvq::kD * kvq::kD;
        _Float16 *s16 = (_Float16 *)std::malloc(2 * n * sizeof(_Float16));
        if (!s16) st = KVQ_E_NOMEM;
        bool exact = true;
        for (size_t i = 0; st == KVQ_OK && i < n; ++i) {
            const float v = cfg->qjl_S[i];
            if (!std::isfinite(v) || std::fabs(v) > 60000.f) st = KVQ_E_INVAL;
            const _Float16 hi = (_Float16)v;
            const _Float16 lo = (_Float16)(v - (float)hi);
            s16[i] = hi;
            s16[n + i] = lo;
            if ((float)lo != 0.0f) exact = false;
        }
        c->S_exact_f16 = exact;
        // fp32 S transposed for the query projection of the score kernels
        float *st_t = st == KVQ_OK ? (float *)std::malloc(n * sizeof(float)) : nullptr;
        if (st == KVQ_OK && !st_t) st = KVQ_E_NOMEM;
        for (int i = 0; st == KVQ_OK && i < kvq::kD; ++i)
            for (int j = 0; j < kvq::kD; ++j) st_t[i * kvq::kD + j] = cfg->qjl_S[j * kvq::kD + i];
        if (st == KVQ_OK) st = upload(&c->d_S, st_t, n);
        std::free(st_t);
        if (st == KVQ_OK) st = upload(&c->d_S16, s16, 2 * n);
        std::free(s16);
    }
    if (st == KVQ_OK && mode == KVQ_MODE_NSN_VQ) {
        const size_t n = (size_t)kvq::kVqK * kvq::kVqSub;
        float bias[kvq::kVqK];
        _Float16 *c16 = (_Float16 *)std::malloc(2 * n * sizeof(_Float16));
        float *cbv = (float *)std::malloc(n * sizeof(float));
        if (!c16 || !cbv) st = KVQ_E_NOMEM;
        for (size_t i = 0; st == KVQ_OK && i < n; ++i) {
            cbv[i] = cfg->vq_codebook[i];
            if (!std::isfinite(cbv[i])) st = KVQ_E_INVAL;
        }
        if (st == KVQ_OK && (cfg->nsn_options & KVQ_NSN_DQ_CODEBOOK)) dq4_codebook(cbv, n);
        bool exact = true;
        for (int j = 0; st == KVQ_OK && j < kvq::kVqK; ++j) {
            double sq = 0.0;
            for (int k = 0; k < kvq::kVqSub; ++k) {
                const float v = cbv[j * kvq::kVqSub + k];
                if (!std::isfinite(v) || std::fabs(v) > 60000.f) st = KVQ_E_INVAL;
                sq += (double)v * v;
                const _Float16 hi = (_Float16)v;
                const _Float16 lo = (_Float16)(v - (float)hi);
                c16[j * kvq::kVqSub + k] = hi;
                c16[n + j * kvq::kVqSub + k] = lo;
                if ((float)lo != 0.0f) exact = false;
            }
            bias[j] = (float)(-0.5 * sq);
        }
        c->vq_exact_f16 = exact;
        if (st == KVQ_OK) st = upload(&c->d_vq, cbv, n);
        if (st == KVQ_OK) st = upload(&c->d_vq16, c16, 2 * n);
        if (st == KVQ_OK) st = upload(&c->d_vqbias, bias, (size_t)kvq::kVqK);
        std::free(c16);
        std::free(cbv);
    }
    if (st == KVQ_OK && mode == KVQ_MODE_GSRQ) {
        // device layout: shapes [2][256][32], levels [2][16], thresholds [2][15]
        // (midpoints of adjacent levels, in double, rounded once)
        const size_t n = 2 * kGsrqShape + 2 * 16 + 2 * 15;
        float *t = (float *)std::malloc(n * sizeof(float));
        if (!t) st = KVQ_E_NOMEM;
        for (int k = 0; st == KVQ_OK && k < 2; ++k) {
            const float *S = cfg->gsrq_tables + k * (kGsrqShape + 16), *G = S + kGsrqShape;
            std::memcpy(t + k * kGsrqShape, S, kGsrqShape * sizeof(float));
            std::memcpy(t + 2 * kGsrqShape + 16 * k, G, 16 * sizeof(float));
            for (int l = 0; l < 15; ++l)
                t[2 * kGsrqShape + 32 + 15 * k + l] = (float)(0.5 * ((double)G[l] + (double)G[l + 1]));
        }
        if (st == KVQ_OK) st = upload(&c->d_gsrq, t, n);
        // the shapes as exact fp16 pairs (high part, rounding of the rest) for
        // the matrix-core search: [part][stage][cw = 2 c + h][shape j][4], the
        // four dims 8 c + 4 h .. + 3 of shape j (so that consecutive shapes'
        // words of one (c, h) are adjacent)
        _Float16 *t16 = st == KVQ_OK ? (_Float16 *)std::malloc(4 * kGsrqShape * sizeof(_Float16)) : nullptr;
        if (st == KVQ_OK && !t16) st = KVQ_E_NOMEM;
        for (size_t k = 0; st == KVQ_OK && k < 2; ++k)
            for (size_t j = 0; j < (size_t)kvq::kVqK; ++j)
                for (size_t d = 0; d < 32; ++d) {
                    const float v = t[k * kGsrqShape + j * 32 + d];
                    const _Float16 hi = (_Float16)v;
                    const size_t cw = d / 4, at = ((k * 8 + cw) * kvq::kVqK + j) * 4 + d % 4;
                    t16[at] = hi;
                    t16[2 * kGsrqShape + at] = (_Float16)(v - (float)hi);
                }
        if (st == KVQ_OK) st = upload(&c->d_gsrq16, t16, 4 * kGsrqShape);
        std::free(t16);
        std::free(t);
    }
    if (st == KVQ_OK && cfg->rotation == KVQ_ROTATION_DENSE) {
        const size_t n = (size_t)kvq::kD * kvq::kD;
        float *qt = (float *)std::malloc(n * sizeof(float));
        _Float16 *q16 = (_Float16 *)std::malloc(2 * n * sizeof(_Float16));
        if (!qt || !q16) st = KVQ_E_NOMEM;
        for (int i = 0; st == KVQ_OK && i < kvq::kD; ++i)
            for (int j = 0; j < kvq::kD; ++j) {
                const float v = cfg->rot_Q[i * kvq::kD + j];
                qt[j * kvq::kD + i] = v;
                const _Float16 hi = (_Float16)v;
                q16[i * kvq::kD + j] = hi;
                q16[n + i * kvq::kD + j] = (_Float16)(v - (float)hi);
            }
        if (st == KVQ_OK) st = upload(&c->d_Q, cfg->rot_Q, n);
        if (st == KVQ_OK) st = upload(&c->d_Qt, qt, n);
        if (st == KVQ_OK) st = upload(&c->d_Q16, q16, 2 * n);
        std::free(qt);
        std::free(q16);
    }
    if (st != KVQ_OK) {
        free_ctx(c);
        return st;
    }
    *out = c;
    return KVQ_OK;
}

kvq_status kvq_destroy(kvq_ctx *ctx)
{
    if (!ctx) return KVQ_OK;
    DeviceGuard g(ctx->device);
    free_ctx(ctx);
    return KVQ_OK;
}

kvq_status kvq_get_tables(const kvq_ctx *ctx, float *centroids, float *thresholds, int8_t *signs_k,
                          int8_t *signs_v)
{
    if (!ctx) return KVQ_E_INVAL;
    if ((signs_k || signs_v) && !ctx->h_signs) return KVQ_E_INVAL;
    const int L = 1 << ctx->bits;
    const size_t n = (size_t)ctx->H * kvq::kD;
    if (centroids) std::memcpy(centroids, ctx->cb.c, L * sizeof(float));
    if (thresholds) std::memcpy(thresholds, ctx->cb.t, (L - 1) * sizeof(float));
    if (signs_k) std::memcpy(signs_k, ctx->h_signs, n);
    if (signs_v) std::memcpy(signs_v, ctx->h_signs + n, n);
    return KVQ_OK;
}

kvq_status kvq_codebook(int32_t bits, float *centroids, float *thresholds)
{
    if (bits < 1 || bits > 4 || !centroids || !thresholds) return KVQ_E_INVAL;
    kvq::Codebook cb;
    build_codebook(bits, &cb);
    std::memcpy(centroids, cb.c, (1 << bits) * sizeof(float));
    std::memcpy(thresholds, cb.t, ((1 << bits) - 1) * sizeof(float));
    return KVQ_OK;
}

int64_t kvq_code_bytes_per_vec(const kvq_ctx *ctx)
{
    if (!ctx) return 0;
    if (ctx->mode == KVQ_MODE_GSRQ) return kvq::kGsrqRec;
    return ctx->mode == KVQ_MODE_NSN_VQ ? kvq::kD / kvq::kVqSub : 16 * ctx->bits;
}

kvq_status kvq_quantize(kvq_ctx *ctx, int32_t kind, const void *x_f16, int64_t B, int64_t H_kv,
                        int64_t T, uint8_t *codes, float *norms, uint8_t *qjl_signs,
                        float *qjl_gamma, void *stream)
{
    if (!ctx || !mse_mode(ctx->mode)) return KVQ_E_INVAL;
    if (kind != KVQ_KIND_K && kind != KVQ_KIND_V) return KVQ_E_INVAL;
    if (B < 0 || T < 0 || H_kv != ctx->H) return KVQ_E_INVAL;
    const bool want_qjl = ctx->mode == KVQ_MODE_MSE_QJL && kind == KVQ_KIND_K;
    if (want_qjl != (qjl_signs != nullptr) || want_qjl != (qjl_gamma != nullptr)) return KVQ_E_INVAL;
    if (B == 0 || T == 0) return KVQ_OK;
    if (!x_f16 || !codes || !norms) return KVQ_E_INVAL;
    if (!aligned(x_f16, 16) || !aligned(codes, 16) || !aligned(norms, 4)) return KVQ_E_INVAL;
    if (want_qjl && (!aligned(qjl_signs, 16) || !aligned(qjl_gamma, 4))) return KVQ_E_INVAL;
    if (B * H_kv > (int64_t(1) << 40) || T > (int64_t(1) << 31)) return KVQ_E_INVAL;
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVQ_E_DEVICE;
    if (ctx->rotation == KVQ_ROTATION_DENSE && want_qjl)
        return launch_status(kvq::launch_quantize_dense_qjl(ctx, x_f16, B * H_kv * T, codes, norms, qjl_signs,
                                                            qjl_gamma, (hipStream_t)stream));
    if (ctx->rotation == KVQ_ROTATION_DENSE)
        return launch_status(kvq::launch_quantize_dense(ctx, x_f16, nullptr, B * H_kv * T, codes, norms, nullptr,
                                                        nullptr, (hipStream_t)stream));
    return launch_status(kvq::launch_quantize(ctx, kind, x_f16, B, T, codes, norms, qjl_signs,
                                              qjl_gamma, (hipStream_t)stream));
}

kvq_status kvq_quantize_kv(kvq_ctx *ctx, const void *k_f16, const void *v_f16, int64_t B, int64_t H_kv,
                           int64_t T, uint8_t *k_codes, float *k_norms, uint8_t *v_codes, float *v_norms,
                           void *stream)
{
    if (!ctx || ctx->mode != KVQ_MODE_MSE) return KVQ_E_INVAL;
    if (B < 0 || T < 0 || H_kv != ctx->H) return KVQ_E_INVAL;
    if (B == 0 || T == 0) return KVQ_OK;
    if (!k_f16 || !v_f16 || !k_codes || !k_norms || !v_codes || !v_norms) return KVQ_E_INVAL;
    if (!aligned(k_f16, 16) || !aligned(v_f16, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
        !aligned(k_norms, 4) || !aligned(v_norms, 4))
        return KVQ_E_INVAL;
    if (B * H_kv > (int64_t(1) << 40) || T > (int64_t(1) << 31)) return KVQ_E_INVAL;
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVQ_E_DEVICE;
    if (ctx->rotation == KVQ_ROTATION_DENSE)
        return launch_status(kvq::launch_quantize_dense(ctx, k_f16, v_f16, B * H_kv * T, k_codes, k_norms,
                                                        v_codes, v_norms, (hipStream_t)stream));
    return launch_status(kvq::launch_quantize_kv(ctx, k_f16, v_f16, B, T, k_codes, k_norms, v_codes, v_norms,
                                                 (hipStream_t)stream));
}

kvq_status kvq_logits(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                      const uint8_t *codes, const float *norms, const uint8_t *qjl_signs,
                      const float *qjl_gamma, float *logits, void *stream)
{
    if (!ctx || !mse_mode(ctx->mode)) return KVQ_E_INVAL;
    if (B < 0 || T < 0 || H_q < 1 || H_q % ctx->H) return KVQ_E_INVAL;
    if (!logits_group_built(H_q / ctx->H)) return KVQ_E_UNSUPPORTED;
    const bool want_qjl = ctx->mode == KVQ_MODE_MSE_QJL;
    if (want_qjl != (qjl_signs != nullptr) || want_qjl != (qjl_gamma != nullptr)) return KVQ_E_INVAL;
    if (B == 0 || T == 0) return KVQ_OK;
    if (!q_f16 || !codes || !norms || !logits) return KVQ_E_INVAL;
    if (!aligned(q_f16, 16) || !aligned(codes, 16) || !aligned(norms, 4) || !aligned(logits, 4))
        return KVQ_E_INVAL;
    if (want_qjl && (!aligned(qjl_signs, 16) || !aligned(qjl_gamma, 4))) return KVQ_E_INVAL;
    if (T > (int64_t(1) << 31)) return KVQ_E_INVAL;
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVQ_E_DEVICE;
    return launch_status(kvq::launch_logits(ctx, q_f16, B, H_q, T, codes, norms, qjl_signs, qjl_gamma,
                                            logits, (hipStream_t)stream));
}

size_t kvq_attn_decode_ws_bytes(const kvq_ctx *ctx, int64_t B, int64_t H_q, int64_t T)
{
    if (!ctx || B < 1 || T < 1 || H_q < 1) return 0;
    return kvq::decode_ws_bytes(B, H_q, ctx->H, T);
}

kvq_status kvq_attn_decode_splits(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q,
                                  int64_t T, const uint8_t *k_codes, const float *k_norms,
                                  const uint8_t *v_codes, const float *v_norms, float sm_scale,
                                  float *out, void *ws, size_t ws_bytes, int32_t n_split,
                                  void *stream)
{
    if (!ctx || ctx->mode != KVQ_MODE_MSE) return KVQ_E_INVAL;
    if (B < 0 || T < 1 || H_q < 1 || H_q % ctx->H) return KVQ_E_INVAL;
    if (!decode_group_built(H_q / ctx->H)) return KVQ_E_UNSUPPORTED;
    if (n_split < 0 || !std::isfinite(sm_scale) || sm_scale < 0.f) return KVQ_E_INVAL;
    if (B == 0) return KVQ_OK;
    if (!q_f16 || !k_codes || !k_norms || !v_codes || !v_norms || !out || !ws) return KVQ_E_INVAL;
    if (!aligned(q_f16, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(k_norms, 4) ||
        !aligned(v_norms, 4) || !aligned(out, 16) || !aligned(ws, 256))
        return KVQ_E_INVAL;
    if (T > (int64_t(1) << 31)) return KVQ_E_INVAL;
    if (ws_bytes < kvq::decode_ws_bytes(B, H_q, ctx->H, T)) return KVQ_E_WORKSPACE;
    const int64_t max_split = kvq::decode_max_splits(T);
    int ns = n_split == 0 ? auto_splits(kvq::decode_auto_splits(B, ctx->H, T)) : n_split;
    if (ns > max_split) ns = (int)max_split;
    if (ns < 1) ns = 1;
    if (sm_scale == 0.f) sm_scale = 1.0f / std::sqrt((float)kvq::kD);
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVQ_E_DEVICE;
    return launch_status(kvq::launch_decode(ctx, q_f16, B, H_q, T, k_codes, k_norms, v_codes, v_norms,
                                            sm_scale, out, ws, ns, (hipStream_t)stream));
}

kvq_status kvq_attn_decode(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                           const uint8_t *k_codes, const float *k_norms, const uint8_t *v_codes,
                           const float *v_norms, float sm_scale, float *out, void *ws,
                           size_t ws_bytes, void *stream)
{
    return kvq_attn_decode_splits(ctx, q_f16, B, H_q, T, k_codes, k_norms, v_codes, v_norms, sm_scale,
                                  out, ws, ws_bytes, 0, stream);
}

kvq_status kvq_attn_decode_noalloc(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                                   const uint8_t *k_codes, const float *k_norms, const uint8_t *v_codes,
                                   const float *v_norms, float sm_scale, float *out, void *stream)
{
    if (!ctx || ctx->mode != KVQ_MODE_MSE) return KVQ_E_INVAL;
    if (B < 0 || T < 1 || H_q < 1 || H_q % ctx->H) return KVQ_E_INVAL;
    if (!decode_group_built(H_q / ctx->H)) return KVQ_E_UNSUPPORTED;
    if (!std::isfinite(sm_scale) || sm_scale < 0.f) return KVQ_E_INVAL;
    if (B == 0) return KVQ_OK;
    if (!q_f16 || !k_codes || !k_norms || !v_codes || !v_norms || !out) return KVQ_E_INVAL;
    if (!aligned(q_f16, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(k_norms, 4) ||
        !aligned(v_norms, 4) || !aligned(out, 16))
        return KVQ_E_INVAL;
    if (T > (int64_t(1) << 31) || B * H_q > (int64_t(1) << 31)) return KVQ_E_INVAL;
    const bool dense = ctx->rotation == KVQ_ROTATION_DENSE;
    // the split count kvq_attn_decode would take, lowered until the scratch holds it
    int64_t ns = std::min<int64_t>(auto_splits(kvq::decode_auto_splits(B, ctx->H, T)), kvq::decode_max_splits(T));
    if (ns < 1) ns = 1;
    while (ns > 1 && kvq::noalloc_decode_bytes(B, H_q, ctx->H, (int)ns, dense) > kvq::kNoAllocScratchBytes) --ns;
    if (kvq::noalloc_decode_bytes(B, H_q, ctx->H, (int)ns, dense) > kvq::kNoAllocScratchBytes) return KVQ_E_WORKSPACE;
    if (sm_scale == 0.f) sm_scale = 1.0f / std::sqrt((float)kvq::kD);
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVQ_E_DEVICE;
    return launch_status(kvq::launch_decode_noalloc(ctx, q_f16, B, H_q, T, k_codes, k_norms, v_codes, v_norms,
                                                    sm_scale, out, (int)ns, (hipStream_t)stream));
}

size_t kvq_nsn_vq_ws_bytes(const kvq_ctx *ctx, int64_t H, int64_t T)
{
    if (!ctx || H < 1 || T < 1) return 0;
    return kvq::nsn_ws_bytes(H, T);
}

kvq_status kvq_nsn_vq_quantize(kvq_ctx *ctx, const void *x_f16, int64_t H, int64_t T, uint8_t *codes,
                               float *s1, float *s2, float *o, void *ws, size_t ws_bytes,
                               void *stream)
{
    if (!ctx || ctx->mode != KVQ_MODE_NSN_VQ) return KVQ_E_INVAL;
    if (H < 1 || T < 1 || T > (int64_t(1) << 31) || H > (int64_t(1) << 20)) return KVQ_E_INVAL;
    if (H * ((T + 2047) / 2048) > INT32_MAX) return KVQ_E_INVAL;  // one stats block per 2048 tokens
    if (!x_f16 || !codes || !s1 || !s2 || !o || !ws) return KVQ_E_INVAL;
    if (!aligned(x_f16, 16) || !aligned(codes, 16) || !aligned(s1, 4) || !aligned(s2, 4) ||
        !aligned(o, 4) || !aligned(ws, 256))
        return KVQ_E_INVAL;
    if (ws_bytes < kvq::nsn_ws_bytes(H, T)) return KVQ_E_WORKSPACE;
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVQ_E_DEVICE;
    return launch_status(kvq::launch_nsn_vq(ctx, x_f16, H, T, codes, s1, s2, o, ws, (hipStream_t)stream));
}


size_t kvq_attn_decode_stream_ws_bytes(const kvq_ctx *ctx, int64_t B, int64_t H_q, int64_t T_cap)
{
    if (!ctx || B < 1 || T_cap < 0 || H_q < 1) return 0;
    const int64_t bhs = B * ctx->H;
    const int64_t slots = (T_cap > 0 ? kvq::decode_max_splits(T_cap) : 0) + 1;  // splits + the window's slot
    return kvq::decode_count_bytes(bhs) + (size_t)(B * H_q) * (size_t)slots * (kvq::kD + 2) * 4;
}

kvq_status kvq_attn_decode_stream(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                                  int64_t T_cap, const uint8_t *k_codes, const float *k_norms,
                                  const uint8_t *v_codes, const float *v_norms, int64_t R, int64_t R_cap,
                                  const void *k_tail_f16, const void *v_tail_f16, float sm_scale, float *out,
                                  void *ws, size_t ws_bytes, void *stream)
{
    if (!ctx || ctx->mode != KVQ_MODE_MSE) return KVQ_E_INVAL;
    if (ctx->rotation != KVQ_ROTATION_HADAMARD) return KVQ_E_UNSUPPORTED;
    if (B < 0 || H_q < 1 || H_q % ctx->H) return KVQ_E_INVAL;
    const int64_t G = H_q / ctx->H;
    if (G != 1 && G != 2 && G != 4) return KVQ_E_INVAL;
    if (T < 0 || T > T_cap || R < 0 || R > R_cap || T + R < 1) return KVQ_E_INVAL;
    if (!std::isfinite(sm_scale) || sm_scale < 0.f) return KVQ_E_INVAL;
    if (B == 0) return KVQ_OK;
    if (!q_f16 || !out || !ws) return KVQ_E_INVAL;
    if (T > 0 && (!k_codes || !k_norms || !v_codes || !v_norms)) return KVQ_E_INVAL;
    if (R > 0 && (!k_tail_f16 || !v_tail_f16)) return KVQ_E_INVAL;
    if (!aligned(q_f16, 16) || !aligned(out, 16) || !aligned(ws, 256)) return KVQ_E_INVAL;
    if (T > 0 && (!aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(k_norms, 4) || !aligned(v_norms, 4)))
        return KVQ_E_INVAL;
    if (R > 0 && (!aligned(k_tail_f16, 16) || !aligned(v_tail_f16, 16))) return KVQ_E_INVAL;
    if (T_cap > (int64_t(1) << 31) || R_cap > (int64_t(1) << 31) || B * ctx->H > (int64_t(1) << 31))
        return KVQ_E_INVAL;
    if (ws_bytes < kvq_attn_decode_stream_ws_bytes(ctx, B, H_q, T_cap)) return KVQ_E_WORKSPACE;
    int ns = 1;
    if (T > 0) {
        ns = auto_splits(kvq::decode_auto_splits(B, ctx->H, T));
        const int64_t cap = std::min<int64_t>(kvq::decode_max_splits(T), kvq::kMaxSplits - 1);
        if (ns > cap) ns = (int)cap;
        if (ns < 1) ns = 1;
    }
    if (sm_scale == 0.f) sm_scale = 1.0f / std::sqrt((float)kvq::kD);
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVQ_E_DEVICE;
    const kvq::DecodeTail tail{k_tail_f16, v_tail_f16, R, R_cap};
    return launch_status(kvq::launch_decode_stream(ctx, q_f16, B, H_q, T, T_cap, k_codes, k_norms, v_codes, v_norms,
                                                   R > 0 ? &tail : nullptr, sm_scale, out, ws, ns,
                                                   (hipStream_t)stream));
}

kvq_status kvq_flush(kvq_ctx *ctx, const void *k_tail_f16, const void *v_tail_f16, int64_t B, int64_t H_kv, int64_t R,
                     int64_t R_cap, uint8_t *k_codes, float *k_norms, uint8_t *v_codes, float *v_norms, int64_t T0,
                     int64_t T_cap, void *stream)
{
    if (!ctx || ctx->mode != KVQ_MODE_MSE) return KVQ_E_INVAL;
    if (ctx->rotation != KVQ_ROTATION_HADAMARD) return KVQ_E_UNSUPPORTED;
    if (B < 0 || H_kv != ctx->H || R < 0 || R > R_cap || T0 < 0 || T0 + R > T_cap) return KVQ_E_INVAL;
    if (B == 0 || R == 0) return KVQ_OK;
    if (!k_tail_f16 || !v_tail_f16 || !k_codes || !k_norms || !v_codes || !v_norms) return KVQ_E_INVAL;
    if (!aligned(k_tail_f16, 16) || !aligned(v_tail_f16, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
        !aligned(k_norms, 4) || !aligned(v_norms, 4))
        return KVQ_E_INVAL;
    if (T_cap > (int64_t(1) << 31) || R_cap > (int64_t(1) << 31) || 2 * B * H_kv * R > (int64_t(1) << 32))
        return KVQ_E_INVAL;
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVQ_E_DEVICE;
    return launch_status(kvq::launch_flush(ctx, k_tail_f16, v_tail_f16, B, R, R_cap, k_codes, k_norms, v_codes,
                                           v_norms, T0, T_cap, (hipStream_t)stream));
}

namespace {
bool nsn_group_ok(const kvq_ctx *ctx, int64_t H_q)
{
    if (H_q < 1 || H_q % ctx->H) return false;
    const int64_t G = H_q / ctx->H;
    return G == 1 || G == 2 || G == 4 || G == 8;
}
}  // namespace

kvq_status kvq_nsn_logits(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                          const uint8_t *codes, const float *s1, const float *s2, const float *o, float *logits,
                          void *stream)
{
    if (!ctx || ctx->mode != KVQ_MODE_NSN_VQ) return KVQ_E_INVAL;
    if (B < 0 || T < 0 || !nsn_group_ok(ctx, H_q)) return KVQ_E_INVAL;
    if (B == 0 || T == 0) return KVQ_OK;
    if (!q_f16 || !codes || !s1 || !s2 || !o || !logits) return KVQ_E_INVAL;
    if (!aligned(q_f16, 16) || !aligned(codes, 16) || !aligned(s1, 4) || !aligned(s2, 4) || !aligned(o, 16) ||
        !aligned(logits, 4))
        return KVQ_E_INVAL;
    if (T > (int64_t(1) << 31) || B * ctx->H > 65535) return KVQ_E_INVAL;
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVQ_E_DEVICE;
    return launch_status(
        kvq::launch_nsn_logits(ctx, q_f16, B, H_q, T, codes, s1, s2, o, logits, (hipStream_t)stream));
}

size_t kvq_nsn_attn_decode_ws_bytes(const kvq_ctx *ctx, int64_t B, int64_t H_q, int64_t T)
{
    if (!ctx || B < 1 || T < 1 || H_q < 1) return 0;
    return kvq::nsn_decode_ws_bytes(B, H_q, T);
}

kvq_status kvq_nsn_attn_decode_splits(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                                      const uint8_t *k_codes, const float *k_s1, const float *k_s2,
                                      const float *k_o, const uint8_t *v_codes, const float *v_s1,
                                      const float *v_s2, const float *v_o, float sm_scale, float *out, void *ws,
                                      size_t ws_bytes, int32_t n_split, void *stream)
{
    if (!ctx || ctx->mode != KVQ_MODE_NSN_VQ) return KVQ_E_INVAL;
    if (B < 0 || T < 1 || !nsn_group_ok(ctx, H_q)) return KVQ_E_INVAL;
    if (n_split < 0 || !std::isfinite(sm_scale) || sm_scale < 0.f) return KVQ_E_INVAL;
    if (B == 0) return KVQ_OK;
    if (!q_f16 || !k_codes || !k_s1 || !k_s2 || !k_o || !v_codes || !v_s1 || !v_s2 || !v_o || !out || !ws)
        return KVQ_E_INVAL;
    if (!aligned(q_f16, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(k_s1, 4) ||
        !aligned(k_s2, 4) || !aligned(v_s1, 4) || !aligned(v_s2, 4) || !aligned(k_o, 16) || !aligned(v_o, 16) ||
        !aligned(out, 16) || !aligned(ws, 256))
        return KVQ_E_INVAL;
    if (T > (int64_t(1) << 31) || B * ctx->H > 65535) return KVQ_E_INVAL;
    if (ws_bytes < kvq::nsn_decode_ws_bytes(B, H_q, T)) return KVQ_E_WORKSPACE;
    const int64_t max_split = kvq::decode_max_splits(T);
    int ns = n_split == 0 ? auto_splits(kvq::nsn_decode_auto_splits(ctx, B, T)) : n_split;
    if (ns > max_split) ns = (int)max_split;
    if (ns < 1) ns = 1;
    if (sm_scale == 0.f) sm_scale = 1.0f / std::sqrt((float)kvq::kD);
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVQ_E_DEVICE;
    const kvq::NsnKV kv{k_codes, k_s1, k_s2, k_o, v_codes, v_s1, v_s2, v_o};
    return launch_status(
        kvq::launch_nsn_decode(ctx, q_f16, B, H_q, T, kv, sm_scale, out, ws, ns, (hipStream_t)stream));
}

size_t kvq_gsrq_ws_bytes(const kvq_ctx *ctx, int64_t H, int64_t T)
{
    if (!ctx || H < 1 || T < 1) return 0;
    return kvq::nsn_ws_bytes(H, T);
}

kvq_status kvq_gsrq_quantize(kvq_ctx *ctx, const void *x_f16, int64_t H, int64_t T, uint8_t *codes, float *s1,
                             float *s2, float *o, void *ws, size_t ws_bytes, void *stream)
{
    if (!ctx || ctx->mode != KVQ_MODE_GSRQ) return KVQ_E_INVAL;
    if (H < 1 || T < 1 || T > (int64_t(1) << 31) || H > (int64_t(1) << 20)) return KVQ_E_INVAL;
    if (H * ((T + 2047) / 2048) > INT32_MAX || H * ((T + 63) / 64) > INT32_MAX) return KVQ_E_INVAL;
    if (!x_f16 || !codes || !s1 || !s2 || !o || !ws) return KVQ_E_INVAL;
    if (!aligned(x_f16, 16) || !aligned(codes, 4) || !aligned(s1, 4) || !aligned(s2, 4) || !aligned(o, 16) ||
        !aligned(ws, 256))
        return KVQ_E_INVAL;
    if (ws_bytes < kvq::nsn_ws_bytes(H, T)) return KVQ_E_WORKSPACE;
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVQ_E_DEVICE;
    return launch_status(kvq::launch_gsrq(ctx, x_f16, H, T, codes, s1, s2, o, ws, (hipStream_t)stream));
}

kvq_status kvq_gsrq_logits(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T, const uint8_t *codes,
                           const float *s1, const float *s2, const float *o, float *logits, void *stream)
{
    if (!ctx || ctx->mode != KVQ_MODE_GSRQ) return KVQ_E_INVAL;
    if (B < 0 || T < 0 || !nsn_group_ok(ctx, H_q)) return KVQ_E_INVAL;
    if (B == 0 || T == 0) return KVQ_OK;
    if (!q_f16 || !codes || !s1 || !s2 || !o || !logits) return KVQ_E_INVAL;
    if (!aligned(q_f16, 16) || !aligned(codes, 4) || !aligned(s1, 4) || !aligned(s2, 4) || !aligned(o, 16) ||
        !aligned(logits, 4))
        return KVQ_E_INVAL;
    if (T > (int64_t(1) << 31) || B * ctx->H > 65535) return KVQ_E_INVAL;
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVQ_E_DEVICE;
    return launch_status(
        kvq::launch_gsrq_logits(ctx, q_f16, B, H_q, T, codes, s1, s2, o, logits, (hipStream_t)stream));
}

kvq_status kvq_gsrq_attn_decode(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                                const uint8_t *k_codes, const float *k_s1, const float *k_s2, const float *k_o,
                                const uint8_t *v_codes, const float *v_s1, const float *v_s2, const float *v_o,
                                float sm_scale, float *out, void *ws, size_t ws_bytes, int32_t n_split, void *stream)
{
    if (!ctx || ctx->mode != KVQ_MODE_GSRQ) return KVQ_E_INVAL;
    if (B < 0 || T < 1 || H_q < 1 || H_q % ctx->H) return KVQ_E_INVAL;
    const int64_t G = H_q / ctx->H;
    if (G != 1 && G != 2 && G != 4) return KVQ_E_INVAL;
    if (n_split < 0 || !std::isfinite(sm_scale) || sm_scale < 0.f) return KVQ_E_INVAL;
    if (B == 0) return KVQ_OK;
    if (!q_f16 || !k_codes || !k_s1 || !k_s2 || !k_o || !v_codes || !v_s1 || !v_s2 || !v_o || !out || !ws)
        return KVQ_E_INVAL;
    if (!aligned(q_f16, 16) || !aligned(k_codes, 4) || !aligned(v_codes, 4) || !aligned(k_s1, 4) ||
        !aligned(k_s2, 4) || !aligned(v_s1, 4) || !aligned(v_s2, 4) || !aligned(k_o, 16) || !aligned(v_o, 16) ||
        !aligned(out, 16) || !aligned(ws, 256))
        return KVQ_E_INVAL;
    if (T > (int64_t(1) << 31) || B * ctx->H > 65535) return KVQ_E_INVAL;
    if (ws_bytes < kvq::nsn_decode_ws_bytes(B, H_q, T)) return KVQ_E_WORKSPACE;
    const int64_t max_split = kvq::decode_max_splits(T);
    int ns = n_split == 0 ? auto_splits(kvq::nsn_decode_auto_splits(ctx, B, T)) : n_split;
    if (ns > max_split) ns = (int)max_split;
    if (ns < 1) ns = 1;
    if (sm_scale == 0.f) sm_scale = 1.0f / std::sqrt((float)kvq::kD);
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVQ_E_DEVICE;
    const kvq::NsnKV kv{k_codes, k_s1, k_s2, k_o, v_codes, v_s1, v_s2, v_o};
    return launch_status(
        kvq::launch_gsrq_decode(ctx, q_f16, B, H_q, T, kv, sm_scale, out, ws, ns, (hipStream_t)stream));
}

size_t kvq_nsn_vq_dq_ws_bytes(const kvq_ctx *ctx, int64_t H, int64_t T)
{
    if (!ctx || H < 1 || T < 1) return 0;
    return kvq::nsn_dq_ws_bytes(H, T);
}

kvq_status kvq_nsn_vq_quantize_dq(kvq_ctx *ctx, const void *x_f16, int64_t H, int64_t T, uint8_t *codes,
                                  uint8_t *s1q, float *s1p, float *s2, uint8_t *oq, float *op, void *ws,
                                  size_t ws_bytes, void *stream)
{
    if (!ctx || ctx->mode != KVQ_MODE_NSN_VQ) return KVQ_E_INVAL;
    if (H < 1 || T < 1 || T > (int64_t(1) << 31) || H > (int64_t(1) << 20)) return KVQ_E_INVAL;
    if (H * ((T + 2047) / 2048) > INT32_MAX) return KVQ_E_INVAL;
    if (!x_f16 || !codes || !s1q || !s1p || !s2 || !oq || !op || !ws) return KVQ_E_INVAL;
    if (!aligned(x_f16, 16) || !aligned(codes, 16) || !aligned(s1p, 8) || !aligned(s2, 4) || !aligned(op, 8) ||
        !aligned(ws, 256))
        return KVQ_E_INVAL;
    if (ws_bytes < kvq::nsn_dq_ws_bytes(H, T)) return KVQ_E_WORKSPACE;
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVQ_E_DEVICE;
    const kvq::NsnDq dq{s1q, s1p, oq, op};
    return launch_status(kvq::launch_nsn_vq_dq(ctx, x_f16, H, T, codes, s2, dq, ws, (hipStream_t)stream));
}

namespace {
bool dq_in_ok(const uint8_t *s1q, const float *s1p, const float *s2, const uint8_t *oq, const float *op)
{
    return s1q && s1p && s2 && oq && op && aligned(s1p, 8) && aligned(s2, 4) && aligned(op, 8);
}
}  // namespace

kvq_status kvq_nsn_logits_dq(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                             const uint8_t *codes, const uint8_t *s1q, const float *s1p, const float *s2,
                             const uint8_t *oq, const float *op, float *logits, void *stream)
{
    if (!ctx || ctx->mode != KVQ_MODE_NSN_VQ) return KVQ_E_INVAL;
    if (B < 0 || T < 0 || !nsn_group_ok(ctx, H_q)) return KVQ_E_INVAL;
    if (B == 0 || T == 0) return KVQ_OK;
    if (!q_f16 || !codes || !logits || !dq_in_ok(s1q, s1p, s2, oq, op)) return KVQ_E_INVAL;
    if (!aligned(q_f16, 16) || !aligned(codes, 16) || !aligned(logits, 4)) return KVQ_E_INVAL;
    if (T > (int64_t(1) << 31) || B * ctx->H > 65535) return KVQ_E_INVAL;
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVQ_E_DEVICE;
    const kvq::NsnDqIn dq{s1q, s1p, oq, op};
    return launch_status(kvq::launch_nsn_logits_dq(ctx, q_f16, B, H_q, T, codes, dq, s2, logits, (hipStream_t)stream));
}

kvq_status kvq_nsn_attn_decode_dq(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                                  const uint8_t *k_codes, const uint8_t *k_s1q, const float *k_s1p,
                                  const float *k_s2, const uint8_t *k_oq, const float *k_op,
                                  const uint8_t *v_codes, const uint8_t *v_s1q, const float *v_s1p,
                                  const float *v_s2, const uint8_t *v_oq, const float *v_op, float sm_scale,
                                  float *out, void *ws, size_t ws_bytes, int32_t n_split, void *stream)
{
    if (!ctx || ctx->mode != KVQ_MODE_NSN_VQ) return KVQ_E_INVAL;
    if (B < 0 || T < 1 || !nsn_group_ok(ctx, H_q)) return KVQ_E_INVAL;
    if (n_split < 0 || !std::isfinite(sm_scale) || sm_scale < 0.f) return KVQ_E_INVAL;
    if (B == 0) return KVQ_OK;
    if (!q_f16 || !k_codes || !v_codes || !out || !ws || !dq_in_ok(k_s1q, k_s1p, k_s2, k_oq, k_op) ||
        !dq_in_ok(v_s1q, v_s1p, v_s2, v_oq, v_op))
        return KVQ_E_INVAL;
    if (!aligned(q_f16, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(out, 16) ||
        !aligned(ws, 256))
        return KVQ_E_INVAL;
    if (T > (int64_t(1) << 31) || B * ctx->H > 65535) return KVQ_E_INVAL;
    if (ws_bytes < kvq::nsn_decode_ws_bytes(B, H_q, T)) return KVQ_E_WORKSPACE;
    const int64_t max_split = kvq::decode_max_splits(T);
    int ns = n_split == 0 ? auto_splits(kvq::nsn_decode_auto_splits(ctx, B, T)) : n_split;
    if (ns > max_split) ns = (int)max_split;
    if (ns < 1) ns = 1;
    if (sm_scale == 0.f) sm_scale = 1.0f / std::sqrt((float)kvq::kD);
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVQ_E_DEVICE;
    kvq::NsnKV kv{k_codes, nullptr, k_s2, nullptr, v_codes, nullptr, v_s2, nullptr, true,
                  kvq::NsnDqIn{k_s1q, k_s1p, k_oq, k_op}, kvq::NsnDqIn{v_s1q, v_s1p, v_oq, v_op}};
    return launch_status(
        kvq::launch_nsn_decode(ctx, q_f16, B, H_q, T, kv, sm_scale, out, ws, ns, (hipStream_t)stream));
}

size_t kvq_nsn_flush_ws_bytes(const kvq_ctx *ctx, int64_t B, int64_t Gs)
{
    if (!ctx || B < 1 || Gs < 1) return 0;
    return kvq::nsn_ws_bytes(B * ctx->H, Gs);
}

kvq_status kvq_nsn_flush(kvq_ctx *ctx, const void *k_tail_f16, const void *v_tail_f16, int64_t B, int64_t H_kv,
                         int64_t Gs, int64_t R_cap, uint8_t *k_codes, float *k_s1, float *k_s2, float *k_o,
                         uint8_t *v_codes, float *v_s1, float *v_s2, float *v_o, int64_t T0, int64_t T_cap, void *ws,
                         size_t ws_bytes, void *stream)
{
    if (!ctx || ctx->mode != KVQ_MODE_NSN_VQ) return KVQ_E_INVAL;
    if (B < 0 || H_kv != ctx->H || Gs < 64 || Gs % 64 || Gs > R_cap || T0 < 0 || T0 % Gs || T_cap % Gs ||
        T0 + Gs > T_cap)
        return KVQ_E_INVAL;
    if (B == 0) return KVQ_OK;
    if (!k_tail_f16 || !v_tail_f16 || !k_codes || !k_s1 || !k_s2 || !k_o || !v_codes || !v_s1 || !v_s2 || !v_o || !ws)
        return KVQ_E_INVAL;
    if (!aligned(k_tail_f16, 16) || !aligned(v_tail_f16, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
        !aligned(k_s1, 4) || !aligned(k_s2, 4) || !aligned(v_s1, 4) || !aligned(v_s2, 4) || !aligned(k_o, 16) ||
        !aligned(v_o, 16) || !aligned(ws, 256))
        return KVQ_E_INVAL;
    if (T_cap > (int64_t(1) << 31) || R_cap > (int64_t(1) << 31) || B * H_kv > (int64_t(1) << 20)) return KVQ_E_INVAL;
    if (ws_bytes < kvq::nsn_ws_bytes(B * H_kv, Gs)) return KVQ_E_WORKSPACE;
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVQ_E_DEVICE;
    const int64_t H = B * H_kv, grp = T0 / Gs, ldo = (T_cap / Gs) * kvq::kD;
    hipError_t e = kvq::launch_nsn_vq_strided(ctx, k_tail_f16, H, Gs, R_cap, k_codes + T0 * 16, k_s1 + T0, k_s2 + T0,
                                              T_cap, k_o + grp * kvq::kD, ldo, ws, (hipStream_t)stream);
    if (e == hipSuccess)
        e = kvq::launch_nsn_vq_strided(ctx, v_tail_f16, H, Gs, R_cap, v_codes + T0 * 16, v_s1 + T0, v_s2 + T0, T_cap,
                                       v_o + grp * kvq::kD, ldo, ws, (hipStream_t)stream);
    return launch_status(e);
}

size_t kvq_nsn_attn_decode_stream_ws_bytes(const kvq_ctx *ctx, int64_t B, int64_t H_q, int64_t T_cap)
{
    if (!ctx || B < 1 || H_q < 1 || T_cap < 0) return 0;
    return kvq::nsn_stream_ws_bytes(B, H_q, T_cap);
}

kvq_status kvq_nsn_attn_decode_stream(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                                      int64_t T_cap, int64_t Gs, const uint8_t *k_codes, const float *k_s1,
                                      const float *k_s2, const float *k_o, const uint8_t *v_codes, const float *v_s1,
                                      const float *v_s2, const float *v_o, int64_t R, int64_t R_cap,
                                      const void *k_tail_f16, const void *v_tail_f16, float sm_scale, float *out,
                                      void *ws, size_t ws_bytes, int32_t n_split, void *stream)
{
    if (!ctx || ctx->mode != KVQ_MODE_NSN_VQ) return KVQ_E_INVAL;
    if (B < 0 || H_q < 1 || H_q % ctx->H) return KVQ_E_INVAL;
    const int64_t G = H_q / ctx->H;
    if (G != 1 && G != 2 && G != 4) return KVQ_E_INVAL;
    if (Gs < 64 || Gs % 64 || T < 0 || T > T_cap || T % Gs || T_cap % Gs) return KVQ_E_INVAL;
    if (R < 0 || R > R_cap || T + R < 1 || n_split < 0) return KVQ_E_INVAL;
    if (!std::isfinite(sm_scale) || sm_scale < 0.f) return KVQ_E_INVAL;
    if (T_cap > (int64_t(1) << 31) || R_cap > (int64_t(1) << 31) || B * ctx->H > 65535) return KVQ_E_INVAL;
    if (T > (int64_t)(kvq::kMaxSplits - 1) * kvq::kNsnMaxGroupsBlk * Gs) return KVQ_E_INVAL;
    if (B == 0) return KVQ_OK;
    if (!q_f16 || !out || !ws) return KVQ_E_INVAL;
    if (T > 0 && (!k_codes || !k_s1 || !k_s2 || !k_o || !v_codes || !v_s1 || !v_s2 || !v_o)) return KVQ_E_INVAL;
    if (R > 0 && (!k_tail_f16 || !v_tail_f16)) return KVQ_E_INVAL;
    if (!aligned(q_f16, 16) || !aligned(out, 16) || !aligned(ws, 256)) return KVQ_E_INVAL;
    if (T > 0 && (!aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(k_s1, 4) || !aligned(k_s2, 4) ||
                  !aligned(v_s1, 4) || !aligned(v_s2, 4) || !aligned(k_o, 16) || !aligned(v_o, 16)))
        return KVQ_E_INVAL;
    if (R > 0 && (!aligned(k_tail_f16, 16) || !aligned(v_tail_f16, 16))) return KVQ_E_INVAL;
    if (ws_bytes < kvq::nsn_stream_ws_bytes(B, H_q, T_cap)) return KVQ_E_WORKSPACE;
    int ns = 1;
    if (T > 0) {
        ns = n_split == 0 ? auto_splits(kvq::nsn_decode_auto_splits(ctx, B, T)) : n_split;
        const int64_t cap = std::min<int64_t>(T / 64, kvq::kMaxSplits - 1);
        if (ns > cap) ns = (int)cap;
        if (ns < 1) ns = 1;
    }
    if (sm_scale == 0.f) sm_scale = 1.0f / std::sqrt((float)kvq::kD);
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVQ_E_DEVICE;
    const kvq::NsnKV kv{k_codes, k_s1, k_s2, k_o, v_codes, v_s1, v_s2, v_o};
    const kvq::NsnStream st{T_cap, Gs, k_tail_f16, v_tail_f16, R, R_cap};
    return launch_status(kvq::launch_nsn_decode_stream(ctx, q_f16, B, H_q, T, kv, st, sm_scale, out, ws, ns,
                                                       (hipStream_t)stream));
}

kvq_status kvq_nsn_attn_decode(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                               const uint8_t *k_codes, const float *k_s1, const float *k_s2, const float *k_o,
                               const uint8_t *v_codes, const float *v_s1, const float *v_s2, const float *v_o,
                               float sm_scale, float *out, void *ws, size_t ws_bytes, void *stream)
{
    return kvq_nsn_attn_decode_splits(ctx, q_f16, B, H_q, T, k_codes, k_s1, k_s2, k_o, v_codes, v_s1, v_s2, v_o,
                                      sm_scale, out, ws, ws_bytes, 0, stream);
}

}  // extern "C"
