// Attention scores read straight from the packed codes ("TurboQuant", Como
// Funciona, Estagio 2, and Como Implementar: the query is rotated once and
// dot products are taken against the indices; QJL sign residual for unbiased
// inner products) and one decode step of attention over the quantised cache
// ("PolarQuant", Technical summary sec. 2 for the dequantisation).
//
// Both kernels start with the same prologue per (batch, KV head): the G query
// heads of the group are rotated once in LDS, q' = H (D_K .* q), and turned
// into lookup tables over fields of the packed key record.  A field holds the
// codes of F consecutive coordinates (F = 2 for b <= 3, F = 1 for b = 4), and
// entry e of field f of head h is sum_k q'_h[F f + k] c[code_k(e)] / d.  A
// key's logit is then rho times the sum of one table entry per field, which
// replaces 128 multiply-adds per head with 128/F LDS reads that serve all G
// heads at once (the G entries of one (field, value) pair are contiguous).
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half_t;
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

template <int BITS>
struct Fields {
    static constexpr int F = BITS == 4 ? 1 : 2;          // coordinates per field
    static constexpr int NF = kD / F;                    // fields per record
    static constexpr int E = 1 << (F * BITS);            // entries per field
    static constexpr int W = 4 * BITS;                   // dwords per record
};

// Value of field f (F*BITS bits starting at bit F*BITS*f) of a record held in
// dwords W.
template <int BITS>
__device__ __forceinline__ uint32_t field(const uint32_t *Wd, int f)
{
    constexpr int nb = Fields<BITS>::F * BITS;
    const int p = nb * f, wd = p >> 5, sh = p & 31;
    uint32_t v;
    if (sh + nb <= 32)
        v = Wd[wd] >> sh;
    else
        v = __builtin_amdgcn_alignbit(Wd[wd + 1], Wd[wd], (uint32_t)sh);
    return v & ((1u << nb) - 1u);
}

// Prologue shared by the score kernels: qr[G][128] <- H (D .* q_h) for the G
// query heads of KV head g of batch b, then the field tables.  All threads of
// the block participate; ends with a barrier.
template <int BITS, int G>
__device__ void rotate_queries(const half_t *__restrict__ q, const float *__restrict__ signs,
                               int64_t b, int g, int Hq, float *qr)
{
    const int tid = threadIdx.x, nthr = blockDim.x;
    for (int idx = tid; idx < G * kD; idx += nthr) {
        const int h = idx >> 7, i = idx & (kD - 1);
        qr[idx] = (float)q[((int64_t)b * Hq + (int64_t)g * G + h) * kD + i] * signs[g * kD + i];
    }
    for (int s = 1; s < kD; s <<= 1) {
        __syncthreads();
        for (int pidx = tid; pidx < G * kD / 2; pidx += nthr) {
            const int h = pidx >> 6, j = pidx & 63;
            const int i0 = (j / s) * 2 * s + (j % s);
            float *r = qr + h * kD;
            const float a = r[i0], c = r[i0 + s];
            r[i0] = a + c;
            r[i0 + s] = a - c;
        }
    }
    __syncthreads();
}

template <int BITS, int G>
__device__ void build_tables(const float *qr, const Codebook &cb, float *lut)
{
    using FD = Fields<BITS>;
    constexpr uint32_t mask = (1u << BITS) - 1u;
    const float inv_d = 1.0f / kD;
    for (int idx = threadIdx.x; idx < FD::NF * FD::E * G; idx += blockDim.x) {
        const int h = idx % G;
        const int e = (idx / G) % FD::E;
        const int f = idx / (G * FD::E);
        float v = 0.0f;
#pragma unroll
        for (int k = 0; k < FD::F; ++k) v += qr[h * kD + FD::F * f + k] * cb.c[(e >> (BITS * k)) & mask];
        lut[idx] = v * inv_d;
    }
}

// Sum of the table entries of one record for the G heads.
template <int BITS, int G>
__device__ __forceinline__ void score_record(const uint32_t *Wd, const float *lut, float *acc)
{
    using FD = Fields<BITS>;
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.0f;
#pragma unroll
    for (int f = 0; f < FD::NF; ++f) {
        const float *e = lut + (f * FD::E + (int)field<BITS>(Wd, f)) * G;
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] += e[h];
    }
}

template <int BITS>
__device__ __forceinline__ void load_record(const uint8_t *codes, int64_t v, uint32_t *Wd)
{
    const u4_t *src = reinterpret_cast<const u4_t *>(codes) + v * BITS;
#pragma unroll
    for (int k = 0; k < BITS; ++k) {
        const u4_t x = src[k];
        Wd[4 * k] = x.x;
        Wd[4 * k + 1] = x.y;
        Wd[4 * k + 2] = x.z;
        Wd[4 * k + 3] = x.w;
    }
    Wd[4 * BITS] = 0u;  // guard word for fields that end on the last dword
}

// ---------------------------------------------------------------------------
// kvq_logits: logits[b, g*G + h, t] for the tokens of one block.
// QJL: + rho gamma sqrt(pi/2)/m sum_j (2 sgn_j - 1) p_h[j], p_h = S q'_h / sqrt(d),
// read through a second table over the 32 nibbles of the 128 sign bits.
// ---------------------------------------------------------------------------
template <int BITS, int G, bool QJL>
__global__ __launch_bounds__(kThreads) void k_logits(
    const half_t *__restrict__ q, const uint8_t *__restrict__ codes, const float *__restrict__ norms,
    const uint32_t *__restrict__ qjl_signs, const float *__restrict__ qjl_gamma,
    const float *__restrict__ signs, const float *__restrict__ S, Codebook cb,
    float *__restrict__ logits, int64_t T, int H, int Hq, int64_t tokens_per_block,
    int64_t blocks_per_bh)
{
    using FD = Fields<BITS>;
    extern __shared__ float smem[];
    float *qr = smem;                       // [G][128]
    float *lut = qr + G * kD;               // [NF][E][G]
    float *slut = lut + FD::NF * FD::E * G; // [32][16][G] (QJL)
    float *pq = slut + (QJL ? 32 * 16 * G : 0);  // [G][128] (QJL)

    const int64_t bh = blockIdx.x / blocks_per_bh;
    const int64_t part = blockIdx.x - bh * blocks_per_bh;
    const int64_t b = bh / H;
    const int g = (int)(bh - b * H);

    rotate_queries<BITS, G>(q, signs, b, g, Hq, qr);
    build_tables<BITS, G>(qr, cb, lut);
    if constexpr (QJL) {
        const float inv_sqrt_d = 0.08838834764831845f;
        for (int idx = threadIdx.x; idx < G * kD; idx += kThreads) {
            const int h = idx >> 7, j = idx & (kD - 1);
            float s = 0.0f;
            for (int i = 0; i < kD; ++i) s += S[j * kD + i] * qr[h * kD + i];
            pq[idx] = s * inv_sqrt_d;
        }
        __syncthreads();
        const float coef = 1.2533141373155003f / kD;  // sqrt(pi/2) / m
        for (int idx = threadIdx.x; idx < 32 * 16 * G; idx += kThreads) {
            const int h = idx % G, e = (idx / G) & 15, f = idx / (16 * G);
            float v = 0.0f;
#pragma unroll
            for (int k = 0; k < 4; ++k) v += ((e >> k) & 1) ? pq[h * kD + 4 * f + k] : -pq[h * kD + 4 * f + k];
            slut[idx] = v * coef;
        }
    }
    __syncthreads();

    const int64_t t_begin = part * tokens_per_block;
    const int64_t t_end = min(T, t_begin + tokens_per_block);
    for (int64_t t = t_begin + threadIdx.x; t < t_end; t += kThreads) {
        const int64_t v = bh * T + t;
        uint32_t Wd[FD::W + 1];
        load_record<BITS>(codes, v, Wd);
        float acc[G];
        score_record<BITS, G>(Wd, lut, acc);
        const float rho = norms[v];
        if constexpr (QJL) {
            const u4_t sg = reinterpret_cast<const u4_t *>(qjl_signs)[v];
            const uint32_t sw[4] = {sg.x, sg.y, sg.z, sg.w};
            float qa[G];
#pragma unroll
            for (int h = 0; h < G; ++h) qa[h] = 0.0f;
#pragma unroll
            for (int f = 0; f < 32; ++f) {
                const float *e = slut + (f * 16 + (int)((sw[f >> 3] >> (4 * (f & 7))) & 15u)) * G;
#pragma unroll
                for (int h = 0; h < G; ++h) qa[h] += e[h];
            }
            const float gm = qjl_gamma[v];
#pragma unroll
            for (int h = 0; h < G; ++h) acc[h] = fmaf(gm, qa[h], acc[h]);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) logits[((b * Hq) + (int64_t)g * G + h) * T + t] = rho * acc[h];
    }
}

// ---------------------------------------------------------------------------
// kvq_attn_decode: split-K flash decoding.  Block (b, g, split) scores its
// token range tile by tile (one key per thread), keeps a running max m and
// sum l per head (base-2 exponentials of the logits scaled by
// sm_scale*log2(e)), and accumulates the V codes in the rotated domain:
// acc_h[i] += p_h,t rho_t c[idx_t,i].  Each block writes (m, l, acc) for its
// G heads; the last block of a (b, g) to finish (arrival counter) merges the
// splits and applies the inverse rotation once: out_h = D_V .* H acc / (d l).
// ---------------------------------------------------------------------------
constexpr int kDecThreads = 512;
constexpr int kDecTile = kDecThreads;  // tokens per tile, one per thread for K
constexpr int kVPhases = kDecThreads / 64;  // V: 64 coordinate pairs x phases

template <int BITS, int G>
struct DecSmem {
    using FD = Fields<BITS>;
    static constexpr int qr = 0;
    static constexpr int lut = qr + G * kD;
    static constexpr int pw = lut + FD::NF * FD::E * G;          // [tile][G] weights p*rho_V
    static constexpr int vrec = pw + kDecTile * G;               // [tile][W+1] V records (dwords)
    static constexpr int red = vrec + kDecTile * (FD::W + 1);   // [16][G] reductions
    static constexpr int c2 = red + 16 * G;                      // [2^(2b)][2] centroid pairs
    static constexpr int total = c2 + 2 * (1 << (2 * BITS));
    // the phase reduction and the split merge at the end reuse pw and vrec
    static_assert(red - pw >= kVPhases * G * kD, "phase buffer does not fit");
    static_assert(red - pw >= 2 * kMaxSplits * G, "merge buffer does not fit kMaxSplits splits");
};

template <int BITS, int G>
__global__ __launch_bounds__(kDecThreads) void k_decode(
    const half_t *__restrict__ q, const uint8_t *__restrict__ kc, const float *__restrict__ kn,
    const uint8_t *__restrict__ vc, const float *__restrict__ vn, const float *__restrict__ signs_k,
    const float *__restrict__ signs_v, Codebook cb, float scale_log2, float *__restrict__ out,
    float *__restrict__ part, unsigned *__restrict__ counters, int64_t T, int H, int Hq,
    int n_split, int64_t chunk)
{
    using FD = Fields<BITS>;
    using SM = DecSmem<BITS, G>;
    extern __shared__ float smem[];
    float *qr = smem + SM::qr;
    float *lut = smem + SM::lut;
    float *pw = smem + SM::pw;
    uint32_t *vrec = reinterpret_cast<uint32_t *>(smem + SM::vrec);
    float *red = smem + SM::red;
    float *c2 = smem + SM::c2;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t bh = blockIdx.x / n_split;
    const int split = (int)(blockIdx.x - bh * n_split);
    const int64_t b = bh / H;
    const int g = (int)(bh - b * H);

    rotate_queries<BITS, G>(q, signs_k, b, g, Hq, qr);
    build_tables<BITS, G>(qr, cb, lut);
    constexpr uint32_t cm = (1u << BITS) - 1u;
    for (int e = tid; e < (1 << (2 * BITS)); e += kDecThreads) {
        c2[2 * e] = cb.c[e & cm];
        c2[2 * e + 1] = cb.c[(e >> BITS) & cm];
    }
    __syncthreads();

    // V work split: thread -> coordinate pair cp (coordinates 2cp, 2cp+1) and
    // token phase ph (tokens ph, ph + kVPhases, ... of the tile).
    const int cp = tid & 63, ph = tid >> 6;
    float m_run[G], l_run[G], acc0[G], acc1[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.0f;
        acc0[h] = 0.0f;
        acc1[h] = 0.0f;
    }

    const int64_t t_begin = (int64_t)split * chunk;
    const int64_t t_end = min(T, t_begin + chunk);
    for (int64_t t0 = t_begin; t0 < t_end; t0 += kDecTile) {
        const int nt = (int)min((int64_t)kDecTile, t_end - t0);
        // K: one key per thread.
        float s[G];
        const bool valid = tid < nt;
        if (valid) {
            const int64_t v = bh * T + t0 + tid;
            uint32_t Wd[FD::W + 1];
            load_record<BITS>(kc, v, Wd);
            score_record<BITS, G>(Wd, lut, s);
            const float rs = kn[v] * scale_log2;
#pragma unroll
            for (int h = 0; h < G; ++h) s[h] *= rs;
            // stage the V record of this token
            const u4_t *src = reinterpret_cast<const u4_t *>(vc) + v * BITS;
#pragma unroll
            for (int k = 0; k < BITS; ++k) {
                const u4_t x = src[k];
                uint32_t *d = vrec + tid * (FD::W + 1) + 4 * k;
                d[0] = x.x;
                d[1] = x.y;
                d[2] = x.z;
                d[3] = x.w;
            }
            vrec[tid * (FD::W + 1) + FD::W] = 0u;
        } else {
#pragma unroll
            for (int h = 0; h < G; ++h) s[h] = -INFINITY;
        }
        // tile maximum per head
        float mt[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float x = s[h];
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
            mt[h] = x;
        }
        if (lane == 0)
#pragma unroll
            for (int h = 0; h < G; ++h) red[wv * G + h] = mt[h];
        __syncthreads();
        float alpha[G], mnew[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float x = red[h];
            for (int w = 1; w < kDecThreads / 64; ++w) x = fmaxf(x, red[w * G + h]);
            mnew[h] = fmaxf(m_run[h], x);
            alpha[h] = exp2f(m_run[h] - mnew[h]);  // m_run = -inf on the first tile -> 0
            m_run[h] = mnew[h];
        }
        // weights and tile sums
        const float rv = valid ? vn[bh * T + t0 + tid] : 0.0f;
        float ps[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float p = valid ? exp2f(s[h] - mnew[h]) : 0.0f;
            pw[tid * G + h] = p * rv;
            float x = p;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
            ps[h] = x;
        }
        __syncthreads();  // red (max) consumed, pw and vrec written
        if (lane == 0)
#pragma unroll
            for (int h = 0; h < G; ++h) red[wv * G + h] = ps[h];
        // V accumulation in the rotated domain
#pragma unroll
        for (int h = 0; h < G; ++h) {
            acc0[h] *= alpha[h];
            acc1[h] *= alpha[h];
        }
        for (int tt = ph; tt < nt; tt += kVPhases) {
            const uint32_t *r = vrec + tt * (FD::W + 1);
            const int p = 2 * BITS * cp, wd = p >> 5, sh = p & 31;
            const uint32_t fv = __builtin_amdgcn_alignbit(r[wd + 1], r[wd], (uint32_t)sh) &
                                ((1u << (2 * BITS)) - 1u);
            const float ca = c2[2 * fv], cb2 = c2[2 * fv + 1];
            const float *w = pw + tt * G;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                acc0[h] = fmaf(w[h], ca, acc0[h]);
                acc1[h] = fmaf(w[h], cb2, acc1[h]);
            }
        }
        __syncthreads();  // red (sums) written; vrec/pw free for the next tile
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float x = 0.0f;
            for (int w = 0; w < kDecThreads / 64; ++w) x += red[w * G + h];
            l_run[h] = l_run[h] * alpha[h] + x;
        }
        __syncthreads();  // red consumed before the next tile reuses it
    }

    // Reduce the token phases: partial acc of coordinate pair cp, phase ph.
    float *accs = pw;  // reuse: [phases][G][128]
    for (int h = 0; h < G; ++h) {
        accs[(ph * G + h) * kD + 2 * cp] = acc0[h];
        accs[(ph * G + h) * kD + 2 * cp + 1] = acc1[h];
    }
    __syncthreads();
    float *my = part + ((bh * n_split + split) * G) * (kD + 2);
    for (int idx = tid; idx < G * kD; idx += kDecThreads) {
        const int h = idx >> 7, i = idx & (kD - 1);
        float x = 0.0f;
        for (int p2 = 0; p2 < kVPhases; ++p2) x += accs[(p2 * G + h) * kD + i];
        my[h * (kD + 2) + 2 + i] = x;
    }
    if (tid < G) {
        my[tid * (kD + 2)] = m_run[tid];
        my[tid * (kD + 2) + 1] = l_run[tid];
    }

    // Arrival: the last split of (b, g) merges.  Every thread publishes its own
    // partial stores at device scope before the block signals arrival.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    __shared__ unsigned last;
    if (tid == 0) {
        const unsigned prev = atomicAdd(counters + bh, 1u);
        last = (prev == (unsigned)(n_split - 1)) ? 1u : 0u;
    }
    __syncthreads();
    if (!last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

    // Merge weights per (split, head): f = 2^(m_s - M) / (d L), L = sum_s l_s 2^(m_s - M).
    float *ms = pw;                   // reuse: [n_split][G] split maxima, then weights
    float *ls = pw + n_split * G;     // [n_split][G] split sums
    float *o = qr;                    // reuse: [G][128]
    const float *all = part + (bh * n_split) * G * (kD + 2);
    for (int idx = tid; idx < n_split * G; idx += kDecThreads) {
        ms[idx] = all[idx * (kD + 2)];
        ls[idx] = all[idx * (kD + 2) + 1];
    }
    __syncthreads();
    if (tid < G) {
        float M = -INFINITY;
        for (int sp = 0; sp < n_split; ++sp) M = fmaxf(M, ms[sp * G + tid]);
        float L = 0.0f;
        for (int sp = 0; sp < n_split; ++sp) L += ls[sp * G + tid] * exp2f(ms[sp * G + tid] - M);
        const float inv = 1.0f / (L * kD);
        for (int sp = 0; sp < n_split; ++sp) ms[sp * G + tid] = exp2f(ms[sp * G + tid] - M) * inv;
    }
    __syncthreads();
    for (int idx = tid; idx < G * kD; idx += kDecThreads) {
        const int h = idx >> 7, i = idx & (kD - 1);
        const float *col = all + h * (kD + 2) + 2 + i;
        float A = 0.0f;
        int sp = 0;
        for (; sp + 8 <= n_split; sp += 8) {  // 8 independent loads in flight
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = col[(int64_t)(sp + u) * G * (kD + 2)];
#pragma unroll
            for (int u = 0; u < 8; ++u) A = fmaf(ms[(sp + u) * G + h], v[u], A);
        }
        for (; sp < n_split; ++sp) A = fmaf(ms[sp * G + h], col[(int64_t)sp * G * (kD + 2)], A);
        o[idx] = A;
    }
    // inverse rotation: out = D_V .* H o
    for (int s2 = 1; s2 < kD; s2 <<= 1) {
        __syncthreads();
        for (int pidx = tid; pidx < G * kD / 2; pidx += kDecThreads) {
            const int h = pidx >> 6, j = pidx & 63;
            const int i0 = (j / s2) * 2 * s2 + (j % s2);
            float *r = o + h * kD;
            const float a = r[i0], c = r[i0 + s2];
            r[i0] = a + c;
            r[i0 + s2] = a - c;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < G * kD; idx += kDecThreads) {
        const int h = idx >> 7, i = idx & (kD - 1);
        out[((b * Hq) + (int64_t)g * G + h) * kD + i] = o[idx] * signs_v[g * kD + i];
    }
    if (tid == 0) counters[bh] = 0u;  // leave the counter ready for the next call
}

template <int BITS, int G, bool QJL>
hipError_t run_logits(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                      const uint8_t *codes, const float *norms, const uint8_t *qjl_signs,
                      const float *qjl_gamma, float *logits, hipStream_t s)
{
    using FD = Fields<BITS>;
    const int64_t bhs = B * ctx->H;
    // enough blocks to fill the chip, but at least 1024 tokens per block to
    // amortise the table build
    int64_t per = (T + 1023) / 1024;
    const int64_t want = (2048 + bhs - 1) / bhs;
    if (per > want) per = want;
    if (per < 1) per = 1;
    const int64_t tpb = (T + per - 1) / per;
    const int64_t blocks_per_bh = (T + tpb - 1) / tpb;
    const size_t shm = sizeof(float) * (G * kD + FD::NF * FD::E * G + (QJL ? 32 * 16 * G + G * kD : 0));
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute((const void *)k_logits<BITS, G, QJL>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        attr_set = true;
    }
    hipLaunchKernelGGL((k_logits<BITS, G, QJL>), dim3((unsigned)(bhs * blocks_per_bh)), dim3(kThreads), shm,
                       s, (const half_t *)q, codes, norms, (const uint32_t *)qjl_signs, qjl_gamma,
                       ctx->d_signs, ctx->d_S, ctx->cb, logits, T, ctx->H, (int)Hq, tpb, blocks_per_bh);
    return hipGetLastError();
}

template <int BITS, int G>
hipError_t run_decode(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                      const uint8_t *kc, const float *kn, const uint8_t *vc, const float *vn,
                      float sm_scale, float *out, void *ws, int n_split, hipStream_t s)
{
    using SM = DecSmem<BITS, G>;
    const int64_t bhs = B * ctx->H;
    const int64_t chunk = (T + n_split - 1) / n_split;
    n_split = (int)((T + chunk - 1) / chunk);  // no empty split
    unsigned *counters = (unsigned *)ws;
    float *part = (float *)((char *)ws + ((bhs * sizeof(unsigned) + 255) / 256) * 256);
    const size_t shm = sizeof(float) * SM::total;
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute((const void *)k_decode<BITS, G>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)shm);
        attr_set = true;
    }
    hipLaunchKernelGGL((k_decode<BITS, G>), dim3((unsigned)(bhs * n_split)), dim3(kDecThreads), shm, s,
                       (const half_t *)q, kc, kn, vc, vn, ctx->d_signs, ctx->d_signs + ctx->H * kD, ctx->cb,
                       sm_scale * 1.4426950408889634f, out, part, counters, T, ctx->H, (int)Hq, n_split,
                       chunk);
    return hipGetLastError();
}

template <int BITS>
hipError_t dispatch_logits(const kvq_ctx *ctx, int G, bool qjl, const void *q, int64_t B, int64_t Hq,
                           int64_t T, const uint8_t *codes, const float *norms, const uint8_t *qs,
                           const float *qg, float *lg, hipStream_t s)
{
#define KVQ_LG(GG)                                                                                  \
    case GG:                                                                                        \
        return qjl ? run_logits<BITS, GG, true>(ctx, q, B, Hq, T, codes, norms, qs, qg, lg, s)      \
                   : run_logits<BITS, GG, false>(ctx, q, B, Hq, T, codes, norms, qs, qg, lg, s);
    switch (G) {
        KVQ_LG(1)
        KVQ_LG(2)
        KVQ_LG(4)
        KVQ_LG(8)
    }
#undef KVQ_LG
    return hipErrorNotSupported;
}

template <int BITS>
hipError_t dispatch_decode(const kvq_ctx *ctx, int G, const void *q, int64_t B, int64_t Hq, int64_t T,
                           const uint8_t *kc, const float *kn, const uint8_t *vc, const float *vn,
                           float sm, float *out, void *ws, int ns, hipStream_t s)
{
    switch (G) {
    case 1: return run_decode<BITS, 1>(ctx, q, B, Hq, T, kc, kn, vc, vn, sm, out, ws, ns, s);
    case 2: return run_decode<BITS, 2>(ctx, q, B, Hq, T, kc, kn, vc, vn, sm, out, ws, ns, s);
    case 4: return run_decode<BITS, 4>(ctx, q, B, Hq, T, kc, kn, vc, vn, sm, out, ws, ns, s);
    }
    return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_logits(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                         const uint8_t *codes, const float *norms, const uint8_t *qjl_signs,
                         const float *qjl_gamma, float *logits, hipStream_t s)
{
    const int G = (int)(Hq / ctx->H);
    const bool qjl = qjl_signs != nullptr;
    switch (ctx->bits) {
    case 1: return dispatch_logits<1>(ctx, G, qjl, q, B, Hq, T, codes, norms, qjl_signs, qjl_gamma, logits, s);
    case 2: return dispatch_logits<2>(ctx, G, qjl, q, B, Hq, T, codes, norms, qjl_signs, qjl_gamma, logits, s);
    case 3: return dispatch_logits<3>(ctx, G, qjl, q, B, Hq, T, codes, norms, qjl_signs, qjl_gamma, logits, s);
    case 4: return dispatch_logits<4>(ctx, G, qjl, q, B, Hq, T, codes, norms, qjl_signs, qjl_gamma, logits, s);
    }
    return hipErrorInvalidValue;
}

size_t decode_ws_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t T)
{
    const int64_t bhs = B * Hkv;
    const int64_t max_split = decode_max_splits(T);
    return ((bhs * sizeof(unsigned) + 255) / 256) * 256 +
           (size_t)(B * Hq) * (size_t)max_split * (kD + 2) * sizeof(float);
}

int decode_auto_splits(int64_t B, int64_t Hkv, int64_t T)
{
    // about two blocks per compute unit, and at least 1024 tokens per block
    const int64_t bhs = B * Hkv;
    int64_t ns = (512 + bhs - 1) / bhs;
    const int64_t cap = (T + 1023) / 1024;
    if (ns > cap) ns = cap;
    return (int)(ns < 1 ? 1 : ns);
}

hipError_t launch_decode(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                         const uint8_t *kc, const float *kn, const uint8_t *vc, const float *vn,
                         float sm_scale, float *out, void *ws, int n_split, hipStream_t s)
{
    const int G = (int)(Hq / ctx->H);
    switch (ctx->bits) {
    case 1: return dispatch_decode<1>(ctx, G, q, B, Hq, T, kc, kn, vc, vn, sm_scale, out, ws, n_split, s);
    case 2: return dispatch_decode<2>(ctx, G, q, B, Hq, T, kc, kn, vc, vn, sm_scale, out, ws, n_split, s);
    case 3: return dispatch_decode<3>(ctx, G, q, B, Hq, T, kc, kn, vc, vn, sm_scale, out, ws, n_split, s);
    case 4: return dispatch_decode<4>(ctx, G, q, B, Hq, T, kc, kn, vc, vn, sm_scale, out, ws, n_split, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace kvq
