// Attention over NSN-VQ codes: logits (k_nsn_logits) and one decode step
// (k_nsn_part, then k_nsn_merge).  "NSNQuant", Detalhes de Implementacao: the
// attention kernels take the byproducts s1, s2, o directly; the
// reconstruction x_hat = s1 (s2 H zq / sqrt(d) + o) inverts Metodologia 1-2,
// zq being the 16 codebook entries a token's codes name.
//
// H is symmetric, so with the query rotated once, q' = H q / sqrt(d),
//   <q, x_hat_t> = s1_t (s2_t sum_s <q'_s, C[code_t,s]> + <q, o>).
// Every block builds the table T[s][j] = <q'_s, C_j> (16 sub-vectors x 256
// entries) in LDS for the G query heads of its KV head, the G values of one
// (s, j) pair contiguous, so that a key costs 16 reads that serve all G heads.
//
// Values: sum_t w_t x_hat_t = H (sum_t w_t s1_t s2_t zq_t) / sqrt(d)
// + (sum_t w_t s1_t) o, so decode accumulates in the code domain (128 sums
// and one scalar per head) and applies the Hadamard once, in the merge.
#include "kvq_internal.h"
#include "kvq_wave.h"

namespace kvq {
namespace {

typedef _Float16 half_t;
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef float f2_t __attribute__((ext_vector_type(2)));

constexpr int kNS = kD / kVqSub;     // 16 sub-vectors
constexpr int kThreadsN = 512;       // threads of a logits block
// waves of a decode block: 8, or 4 for G = 8, whose 128 KiB table leaves LDS
// for only four waves' staging
template <int G>
constexpr int dec_waves() { return G == 8 ? 4 : 8; }
constexpr int kLogitChunk = 2048;    // tokens per logits block
constexpr float kInvSqrtD = 0.08838834764831845f;
constexpr float kLog2e = 1.4426950408889634f;

template <int G>
struct alignas(16) NsnSmem {
    static constexpr int TAB = kNS * kVqK * G;           // floats of the table
    float tab[TAB];
    float cb[kVqK * kVqSub];                             // fp32 codebook
    float qs[G * kD];                                    // q' = H q / sqrt(d)
    float qo[G];                                         // <q, o>
};

// Prologue of both kernels: codebook into LDS, q' and <q, o> for the G query
// heads of KV head g of batch b (one wave per head), then the table.  Ends
// with a barrier.  Table entry (s, j, h) = sum_k q'_h[8 s + k] C_j[k], one
// fp32 chain over k.
template <int G, int NT>
__device__ void nsn_tables(const half_t *__restrict__ q, const float *__restrict__ o, const float *__restrict__ cb,
                           int64_t bg, int64_t qbase, NsnSmem<G> &sm)
{
    static_assert(NT % kVqK == 0, "one thread per entry and sub-vector group");
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    for (int i = tid; i < kVqK * kVqSub / 4; i += NT)
        reinterpret_cast<f4_t *>(sm.cb)[i] = reinterpret_cast<const f4_t *>(cb)[i];
    for (int h = wv; h < G; h += NT / 64) {
        const h2_t pr = reinterpret_cast<const h2_t *>(q + (qbase + h) * kD)[lane];
        const f2_t ov = reinterpret_cast<const f2_t *>(o + bg * kD)[lane];
        float x0 = (float)pr.x, x1 = (float)pr.y;
        const float qo = wave_sum(fmaf(x1, ov.y, x0 * ov.x));
        wave_fwht(x0, x1, lane);
        reinterpret_cast<f2_t *>(sm.qs + h * kD)[lane] = f2_t{x0 * kInvSqrtD, x1 * kInvSqrtD};
        if (lane == 0) sm.qo[h] = qo;
    }
    __syncthreads();
    const int j = tid & (kVqK - 1);
    const f4_t c0 = reinterpret_cast<const f4_t *>(sm.cb + j * kVqSub)[0];
    const f4_t c1 = reinterpret_cast<const f4_t *>(sm.cb + j * kVqSub)[1];
    for (int s = tid / kVqK; s < kNS; s += NT / kVqK) {
        float v[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const f4_t a0 = reinterpret_cast<const f4_t *>(sm.qs + h * kD + s * kVqSub)[0];
            const f4_t a1 = reinterpret_cast<const f4_t *>(sm.qs + h * kD + s * kVqSub)[1];
            float acc = a0.x * c0.x;
            acc = fmaf(a0.y, c0.y, acc);
            acc = fmaf(a0.z, c0.z, acc);
            acc = fmaf(a0.w, c0.w, acc);
            acc = fmaf(a1.x, c1.x, acc);
            acc = fmaf(a1.y, c1.y, acc);
            acc = fmaf(a1.z, c1.z, acc);
            v[h] = fmaf(a1.w, c1.w, acc);
        }
        float *e = sm.tab + (s * kVqK + j) * G;
#pragma unroll
        for (int h = 0; h < G; ++h) e[h] = v[h];
    }
    __syncthreads();
}

// sum_s T[s][code_s] for the G heads, in sub-vector order.  The G values of
// an entry are read as one vector (16-byte aligned for G >= 4).
template <int G>
__device__ __forceinline__ void nsn_key_sum(const u4_t code, const float *tab, float (&acc)[G])
{
    typedef float fg_t __attribute__((ext_vector_type(G)));
    fg_t sum = 0.0f;
#pragma unroll
    for (int s = 0; s < kNS; ++s) {
        const uint32_t w = s < 4 ? code.x : s < 8 ? code.y : s < 12 ? code.z : code.w;
        const uint32_t j = (w >> (8 * (s & 3))) & 0xFFu;
        sum += *reinterpret_cast<const fg_t *>(tab + (s * kVqK + j) * G);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = sum[h];
}

// logits[b, g G + h, t] = s1_t (s2_t sum_s T_h[s][code_t,s] + <q_h, o>).
// Block (chunk of kLogitChunk tokens, b * Hkv + g); one thread per token.
template <int G>
__global__ __launch_bounds__(kThreadsN) void k_nsn_logits(const half_t *__restrict__ q, const u4_t *__restrict__ codes,
                                                          const float *__restrict__ s1, const float *__restrict__ s2,
                                                          const float *__restrict__ o, const float *__restrict__ cb,
                                                          float *__restrict__ logits, int64_t Hkv, int64_t T)
{
    constexpr int NT = kLogitChunk / kThreadsN;  // tokens per thread
    __shared__ NsnSmem<G> sm;
    const int64_t bg = blockIdx.y, b = bg / Hkv, g = bg % Hkv;
    const int64_t Hq = Hkv * G, qbase = b * Hq + g * G;
    const int64_t c0 = (int64_t)blockIdx.x * kLogitChunk, c1 = min(T, c0 + kLogitChunk);
    // the keys' loads go out before the prologue (a token past the end
    // re-reads the chunk's first one and is not stored)
    u4_t code[NT];
    float a[NT], c[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int64_t t = c0 + threadIdx.x + i * kThreadsN;
        const int64_t v = bg * T + (t < c1 ? t : c0);
        code[i] = codes[v];
        a[i] = s1[v];
        c[i] = s2[v];
    }
    nsn_tables<G, kThreadsN>(q, o, cb, bg, qbase, sm);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int64_t t = c0 + threadIdx.x + i * kThreadsN;
        float acc[G];
        nsn_key_sum<G>(code[i], sm.tab, acc);
        if (t < c1) {
#pragma unroll
            for (int h = 0; h < G; ++h) logits[(qbase + h) * T + t] = a[i] * fmaf(c[i], acc[h], sm.qo[h]);
        }
    }
}

// Decode, part 1.  Block (split, b * Hkv + g) covers tokens [c0, c1) in
// 64-token tiles, one per wave at a time (lane = token).  Per tile and head:
// online softmax in base 2 (running maximum m, per-lane sums l of p and wo of
// p s1_V), then the value sums in the code domain with lanes as dimensions:
// lane (s, k) = (l / 4, 2 (l % 4)) owns dimensions 8 s + k, 8 s + k + 1 of
// all G heads and walks the tile's tokens, reading each token's entry index
// and its weights p s1_V s2_V from LDS.  The waves then merge in LDS and the
// block writes {acc[128], M, L, WO} per head to the workspace.
template <int G>
struct DecodeSmem {
    NsnSmem<G> t;
    u4_t vcode[dec_waves<G>()][64];
    float wts[dec_waves<G>()][64][G];
};
// One lane's token of a decode tile: K and V codes and byproducts.
struct TileIn {
    u4_t kcode, vcode;
    float a, c, e1, e2;  // s1_K, s2_K, s1_V, s2_V
};
__device__ __forceinline__ TileIn load_tile(const u4_t *kc, const float *ks1, const float *ks2, const u4_t *vc,
                                            const float *vs1, const float *vs2, int64_t base, int64_t t)
{
    const int64_t v = base + t;
    return TileIn{kc[v], vc[v], ks1[v], ks2[v], vs1[v], vs2[v]};
}
constexpr int kPartStride = kNsnPartStride;  // floats per (split, head) partial: acc[128], M, L, WO, pad

template <int G>
__global__ __launch_bounds__(64 * dec_waves<G>()) void k_nsn_part(const half_t *__restrict__ q, const u4_t *__restrict__ kc,
                                                        const float *__restrict__ ks1, const float *__restrict__ ks2,
                                                        const float *__restrict__ ko, const u4_t *__restrict__ vc,
                                                        const float *__restrict__ vs1, const float *__restrict__ vs2,
                                                        const float *__restrict__ cb, float *__restrict__ part,
                                                        int64_t Hkv, int64_t T, int64_t chunk, float scale2)
{
    constexpr int NW = dec_waves<G>();
    __shared__ DecodeSmem<G> sm;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bg = blockIdx.y, b = bg / Hkv, g = bg % Hkv;
    const int64_t qbase = b * Hkv * G + g * G;
    const int64_t c0 = (int64_t)blockIdx.x * chunk, c1 = min(T, c0 + chunk);
    // The first tile's loads go out before the prologue, every later tile's
    // before the current one is processed.
    int64_t t0 = c0 + 64 * wv;
    TileIn cur = load_tile(kc, ks1, ks2, vc, vs1, vs2, bg * T, t0 + lane < c1 ? t0 + lane : t0);
    nsn_tables<G, 64 * NW>(q, ko, cb, bg, qbase, sm.t);

    float m[G], l[G], wo[G], acc[G][2];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -__builtin_inff();
        l[h] = wo[h] = acc[h][0] = acc[h][1] = 0.0f;
    }
    const int vs = lane >> 2, vk = 2 * (lane & 3);
    const uint8_t *vcb = reinterpret_cast<const uint8_t *>(sm.vcode[wv]) + vs;
    const float *cbk = sm.t.cb + vk;

    for (; t0 < c1; t0 += 64 * NW) {
        const bool valid = t0 + lane < c1;
        const int64_t tn = t0 + 64 * NW;
        TileIn nxt = cur;
        if (tn < c1) nxt = load_tile(kc, ks1, ks2, vc, vs1, vs2, bg * T, tn + lane < c1 ? tn + lane : tn);
        float ks[G];
        nsn_key_sum<G>(cur.kcode, sm.t.tab, ks);
        float w[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float lg = valid ? cur.a * fmaf(cur.c, ks[h], sm.t.qo[h]) * scale2 : -__builtin_inff();
            const float mn = fmaxf(m[h], wave_max(lg));
            const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);
            const float p = __builtin_amdgcn_exp2f(lg - mn);
            m[h] = mn;
            l[h] = fmaf(l[h], alpha, p);
            wo[h] = fmaf(wo[h], alpha, p * cur.e1);
            acc[h][0] *= alpha;
            acc[h][1] *= alpha;
            w[h] = p * cur.e1 * cur.e2;
        }
        sm.vcode[wv][lane] = cur.vcode;
#pragma unroll
        for (int h = 0; h < G; ++h) sm.wts[wv][lane][h] = w[h];
        wave_lds_sync();
        // all 64 tokens: past the end the weights are 0 and the staged index
        // is that of the tile's first token
#pragma unroll
        for (int i = 0; i < 64; ++i) {
            const uint32_t j = vcb[16 * i];
            const f2_t ce = *reinterpret_cast<const f2_t *>(cbk + j * kVqSub);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float wh = sm.wts[wv][i][h];
                acc[h][0] = fmaf(wh, ce.x, acc[h][0]);
                acc[h][1] = fmaf(wh, ce.y, acc[h][1]);
            }
        }
        wave_lds_sync();
        cur = nxt;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        l[h] = wave_sum(l[h]);
        wo[h] = wave_sum(wo[h]);
    }
    // Merge of the waves (the table is no longer read: its space holds the
    // per-wave partials, laid out [wave][head][kPartStride]).
    __syncthreads();
    float *mw = sm.t.tab;
    static_assert(NW * G * kPartStride <= NsnSmem<G>::TAB, "wave partials fit in the table space");
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float *p = mw + (wv * G + h) * kPartStride;
        *reinterpret_cast<f2_t *>(p + 8 * vs + vk) = f2_t{acc[h][0], acc[h][1]};
        if (lane == 0) {
            p[kD] = m[h];
            p[kD + 1] = l[h];
            p[kD + 2] = wo[h];
        }
    }
    __syncthreads();
    const int64_t split = blockIdx.x, n_split = gridDim.x;
    for (int i = threadIdx.x; i < G * kD; i += 64 * NW) {
        const int h = i / kD, dim = i % kD;
        float M = -__builtin_inff();
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) M = fmaxf(M, mw[(w2 * G + h) * kPartStride + kD]);
        float A = 0.0f, L = 0.0f, WO = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
            const float *p = mw + (w2 * G + h) * kPartStride;
            const float f = __builtin_amdgcn_exp2f(p[kD] - M);  // waves without tokens: 2^-inf = 0
            A = fmaf(f, p[dim], A);
            L = fmaf(f, p[kD + 1], L);
            WO = fmaf(f, p[kD + 2], WO);
        }
        float *dst = part + ((bg * n_split + split) * G + h) * kPartStride;
        dst[dim] = A;
        if (dim == 0) {
            dst[kD] = M;
            dst[kD + 1] = L;
            dst[kD + 2] = WO;
        }
    }
}

// Decode, part 2.  Block b * Hkv + g, one wave per head h (lane: dimensions
// 2 lane, 2 lane + 1): merge of the splits, f_s = 2^(M_s - M), then
// out = (H acc / sqrt(d) + WO o_V) / L.
template <int G>
__global__ __launch_bounds__(64 * G) void k_nsn_merge(const float *__restrict__ part, const float *__restrict__ vo,
                                                      float *__restrict__ out, int64_t Hkv, int n_split)
{
    const int lane = threadIdx.x & 63, h = threadIdx.x >> 6;
    const int64_t bg = blockIdx.x, b = bg / Hkv, g = bg % Hkv;
    const float *p0 = part + (bg * n_split * G + h) * kPartStride;
    const int64_t sst = (int64_t)G * kPartStride;  // split stride
    // split headers (M, L, WO) one split per lane, all loads in flight
    __shared__ float fw[G][kMaxSplits];
    constexpr int kPer = kMaxSplits / 64;
    float mv[kPer], lv[kPer], ov_[kPer];
    float M = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int sp = lane + 64 * k;
        const bool in = sp < n_split;
        mv[k] = in ? p0[sp * sst + kD] : -__builtin_inff();
        lv[k] = in ? p0[sp * sst + kD + 1] : 0.0f;
        ov_[k] = in ? p0[sp * sst + kD + 2] : 0.0f;
        M = fmaxf(M, mv[k]);
    }
    M = wave_max(M);
    float L = 0.0f, WO = 0.0f;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int sp = lane + 64 * k;
        const float f = __builtin_amdgcn_exp2f(mv[k] - M);  // 0 past the last split
        L = fmaf(f, lv[k], L);
        WO = fmaf(f, ov_[k], WO);
        if (sp < n_split) fw[h][sp] = f;
    }
    L = wave_sum(L);
    WO = wave_sum(WO);
    wave_lds_sync();
    // accumulators: 16 splits' loads in flight at a time
    float x0 = 0.0f, x1 = 0.0f;
    for (int s0 = 0; s0 < n_split; s0 += 16) {
        f2_t a[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
            a[u] = s0 + u < n_split ? reinterpret_cast<const f2_t *>(p0 + (s0 + u) * sst)[lane] : f2_t{0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const float f = s0 + u < n_split ? fw[h][s0 + u] : 0.0f;
            x0 = fmaf(f, a[u].x, x0);
            x1 = fmaf(f, a[u].y, x1);
        }
    }
    wave_fwht(x0, x1, lane);
    const f2_t ov = reinterpret_cast<const f2_t *>(vo + bg * kD)[lane];
    const float inv = 1.0f / L;
    reinterpret_cast<f2_t *>(out + ((b * Hkv + g) * G + h) * kD)[lane] =
        f2_t{fmaf(x0, kInvSqrtD, WO * ov.x) * inv, fmaf(x1, kInvSqrtD, WO * ov.y) * inv};
}

template <int G>
hipError_t logits_g(const kvq_ctx *ctx, const void *q, int64_t B, int64_t T, const uint8_t *codes, const float *s1,
                    const float *s2, const float *o, float *logits, hipStream_t s)
{
    const int64_t n_chunks = (T + kLogitChunk - 1) / kLogitChunk;
    hipLaunchKernelGGL(k_nsn_logits<G>, dim3((unsigned)n_chunks, (unsigned)(B * ctx->H)), dim3(kThreadsN), 0, s,
                       (const half_t *)q, (const u4_t *)codes, s1, s2, o, ctx->d_vq, logits, (int64_t)ctx->H, T);
    return hipGetLastError();
}

template <int G>
hipError_t decode_g(const kvq_ctx *ctx, const void *q, int64_t B, int64_t T, const NsnKV &kv, float sm_scale,
                    float *out, void *ws, int n_split, hipStream_t s)
{
    const int64_t chunk = nsn_decode_chunk(T, n_split);
    const int ns = (int)((T + chunk - 1) / chunk);
    float *part = (float *)ws;
    hipLaunchKernelGGL(k_nsn_part<G>, dim3((unsigned)ns, (unsigned)(B * ctx->H)), dim3(64 * dec_waves<G>()), 0, s,
                       (const half_t *)q, (const u4_t *)kv.kc, kv.ks1, kv.ks2, kv.ko, (const u4_t *)kv.vc, kv.vs1,
                       kv.vs2, ctx->d_vq, part, (int64_t)ctx->H, T, chunk, sm_scale * kLog2e);
    hipLaunchKernelGGL(k_nsn_merge<G>, dim3((unsigned)(B * ctx->H)), dim3(64 * G), 0, s, part, kv.vo, out,
                       (int64_t)ctx->H, ns);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_nsn_logits(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                             const uint8_t *codes, const float *s1, const float *s2, const float *o, float *logits,
                             hipStream_t s)
{
    switch (Hq / ctx->H) {
        case 1: return logits_g<1>(ctx, q, B, T, codes, s1, s2, o, logits, s);
        case 2: return logits_g<2>(ctx, q, B, T, codes, s1, s2, o, logits, s);
        case 4: return logits_g<4>(ctx, q, B, T, codes, s1, s2, o, logits, s);
        case 8: return logits_g<8>(ctx, q, B, T, codes, s1, s2, o, logits, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_nsn_decode(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T, const NsnKV &kv,
                             float sm_scale, float *out, void *ws, int n_split, hipStream_t s)
{
    switch (Hq / ctx->H) {
        case 1: return decode_g<1>(ctx, q, B, T, kv, sm_scale, out, ws, n_split, s);
        case 2: return decode_g<2>(ctx, q, B, T, kv, sm_scale, out, ws, n_split, s);
        case 4: return decode_g<4>(ctx, q, B, T, kv, sm_scale, out, ws, n_split, s);
        case 8: return decode_g<8>(ctx, q, B, T, kv, sm_scale, out, ws, n_split, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
