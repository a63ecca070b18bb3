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
KVQ_DEBUG_UNIT(nsn_score, 4)
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

// Double quantisation of the byproducts (the *_dq calls): s1 of token t of
// row bg is its 4-bit code in the block of kNsnDqBlock tokens, lo + code
// step with that block's (lo, step); the means are 4-bit codes with one
// (lo, step) per row.
__device__ __forceinline__ float dq_s1(const NsnDqIn &dq, int64_t bg, int64_t T, int64_t t)
{
    const int64_t ldq = (T + 1) / 2, nblk = (T + kNsnDqBlock - 1) / kNsnDqBlock;
    const uint32_t byte = dq.s1q[bg * ldq + (t >> 1)];
    const uint32_t c = (byte >> (4 * (uint32_t)(t & 1))) & 15u;
    const f2_t p = reinterpret_cast<const f2_t *>(dq.s1p)[bg * nblk + t / kNsnDqBlock];
    return fmaf((float)c, p.y, p.x);
}
// Means of channels 2 lane, 2 lane + 1: from the fp32 row `orow`, or (DQ)
// from the 4-bit codes of row bg.
template <bool DQ>
__device__ __forceinline__ f2_t load_mean(const float *orow, const NsnDqIn &dq, int64_t bg, int lane)
{
    if constexpr (DQ) {
        const uint32_t byte = dq.oq[bg * (kD / 2) + lane];
        const f2_t p = reinterpret_cast<const f2_t *>(dq.op)[bg];
        return f2_t{fmaf((float)(byte & 15u), p.y, p.x), fmaf((float)(byte >> 4), p.y, p.x)};
    } else {
        return reinterpret_cast<const f2_t *>(orow)[lane];
    }
}

// Prologue of both kernels: codebook into LDS, q' and <q, o> for the G query
// heads of KV head g of batch b (one wave per head), then the table.  Ends
// with a barrier.  Table entry (s, j, h) = sum_k q'_h[8 s + k] C_j[k], one
// fp32 chain over k.
template <int G, int NT, bool DQ = false>
__device__ void nsn_tables(const half_t *__restrict__ q, const float *__restrict__ obg, const float *__restrict__ cb,
                           int64_t qbase, NsnSmem<G> &sm, const NsnDqIn &dq = NsnDqIn{}, int64_t bg = 0)
{
    static_assert(NT % kVqK == 0, "one thread per entry and sub-vector group");
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    for (int i = tid; i < kVqK * kVqSub / 4; i += NT)
        reinterpret_cast<f4_t *>(sm.cb)[i] = reinterpret_cast<const f4_t *>(cb)[i];
    for (int h = wv; h < G; h += NT / 64) {
        const h2_t pr = reinterpret_cast<const h2_t *>(q + (qbase + h) * kD)[lane];
        const f2_t ov = load_mean<DQ>(obg, dq, bg, lane);
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
template <int G, bool DQ>
__global__ __launch_bounds__(kThreadsN) void k_nsn_logits(const half_t *__restrict__ q, const u4_t *__restrict__ codes,
                                                          const float *__restrict__ s1, const float *__restrict__ s2,
                                                          const float *__restrict__ o, const float *__restrict__ cb,
                                                          float *__restrict__ logits, int64_t Hkv, int64_t T,
                                                          NsnDqIn dq)
{
    constexpr int NT = kLogitChunk / kThreadsN;  // tokens per thread
    __shared__ NsnSmem<G> sm;
    const int64_t bg = blockIdx.y, b = bg / Hkv, g = bg % Hkv;
    const int64_t Hq = Hkv * G, qbase = b * Hq + g * G;
    const int64_t c0 = (int64_t)blockIdx.x * kLogitChunk, c1 = min(T, c0 + kLogitChunk);
    KVQ_CHECK(c0 < c1 && g < Hkv);
    KVQ_POISON_LDS(&sm, sizeof(sm) / 4, threadIdx.x, kThreadsN);
    if (KVQ_DEBUG_ON) __syncthreads();
    // the keys' loads go out before the prologue (a token past the end
    // re-reads the chunk's first one and is not stored)
    u4_t code[NT];
    float a[NT], c[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int64_t t = c0 + threadIdx.x + i * kThreadsN;
        const int64_t tc = t < c1 ? t : c0, v = bg * T + tc;
        code[i] = codes[v];
        a[i] = DQ ? dq_s1(dq, bg, T, tc) : s1[v];
        c[i] = s2[v];
    }
    nsn_tables<G, kThreadsN, DQ>(q, DQ ? nullptr : o + bg * kD, cb, qbase, sm, dq, bg);
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
// Streaming cache (GROUPED): the packed tokens were flushed in groups of
// gsize tokens, each with its own means; a block's range covers at most
// kMaxGroupsBlk groups, whose K means enter the logits as <q, o^K_g> and whose
// V means enter the value sums in the code domain as H o^V_g / sqrt(d) times
// the tile's sum of p s1_V (a 64-token tile lies in one group).
constexpr int kMaxGroupsBlk = kNsnMaxGroupsBlk;
template <int G, bool GROUPED>
struct DecodeSmem {
    NsnSmem<G> t;
    u4_t vcode[dec_waves<G>()][64];
    float wts[dec_waves<G>()][64][G];
    float og[GROUPED ? kMaxGroupsBlk : 1][kD];  // H o^V_g / sqrt(d)
    float qog[GROUPED ? kMaxGroupsBlk : 1][G];  // <q_h, o^K_g>
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
// The same with s1 of K and V from their 4-bit forms (rows of T tokens).
__device__ __forceinline__ TileIn load_tile_dq(const u4_t *kc, const NsnDqIn &kdq, const float *ks2, const u4_t *vc,
                                               const NsnDqIn &vdq, const float *vs2, int64_t bg, int64_t T, int64_t t)
{
    const int64_t v = bg * T + t;
    return TileIn{kc[v], vc[v], dq_s1(kdq, bg, T, t), ks2[v], dq_s1(vdq, bg, T, t), vs2[v]};
}
constexpr int kPartStride = kNsnPartStride;  // floats per (split, head) partial: acc[128], M, L, WO, pad

// ldt: tokens between (b, g) rows of the packed arrays; n_part: partial
// slots per (b, g) (one more than the splits when a window partial follows);
// GROUPED: ko, vo are per-group means [B Hkv][ngc][128] of groups of gsize
// tokens (gsize and the range start multiples of 64 and of gsize), else the
// per-(b, g) means [B Hkv][128].
// DQ: s1 and the K means from their 4-bit forms (kdq, vdq; rows of T tokens).
template <int G, bool GROUPED, bool DQ>
__global__ __launch_bounds__(64 * dec_waves<G>()) void k_nsn_part(const half_t *__restrict__ q, const u4_t *__restrict__ kc,
                                                        const float *__restrict__ ks1, const float *__restrict__ ks2,
                                                        const float *__restrict__ ko, const u4_t *__restrict__ vc,
                                                        const float *__restrict__ vs1, const float *__restrict__ vs2,
                                                        const float *__restrict__ cb, float *__restrict__ part,
                                                        int64_t Hkv, int64_t T, int64_t chunk, float scale2,
                                                        int64_t ldt, int n_part, const float *__restrict__ vo,
                                                        int64_t gsize, int64_t ngc, NsnDqIn kdq, NsnDqIn vdq)
{
    static_assert(!(GROUPED && DQ), "the streaming cache keeps fp32 byproducts");
    constexpr int NW = dec_waves<G>();
    __shared__ DecodeSmem<G, GROUPED> sm;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bg = blockIdx.y, b = bg / Hkv, g = bg % Hkv;
    const int64_t qbase = b * Hkv * G + g * G;
    const int64_t c0 = (int64_t)blockIdx.x * chunk, c1 = min(T, c0 + chunk);
    KVQ_CHECK(c0 < c1 && (DQ || T <= ldt) && (int64_t)blockIdx.x < n_part &&
              (!GROUPED || (c0 % gsize == 0 && (c1 + gsize - 1) / gsize <= ngc)));
    KVQ_POISON_LDS(&sm, sizeof(sm) / 4, threadIdx.x, 64 * NW);
    if (KVQ_DEBUG_ON) __syncthreads();
    // The first tile's loads go out before the prologue, every later tile's
    // before the current one is processed.  Lanes past the end of the range
    // (and every lane of a wave the range gives no tile) load the range's
    // first token, whose weight is then 0.
    int64_t t0 = c0 + 64 * wv;
    auto fetch = [&](int64_t t) {
        if constexpr (DQ) return load_tile_dq(kc, kdq, ks2, vc, vdq, vs2, bg, T, t);
        else return load_tile(kc, ks1, ks2, vc, vs1, vs2, bg * ldt, t);
    };
    TileIn cur = fetch(t0 + lane < c1 ? t0 + lane : c0);
    const int64_t gfirst = GROUPED ? c0 / gsize : 0;
    nsn_tables<G, 64 * NW, DQ>(q, DQ ? nullptr : GROUPED ? ko + (bg * ngc + gfirst) * kD : ko + bg * kD, cb, qbase,
                               sm.t, kdq, bg);
    if constexpr (GROUPED) {
        // the block's groups: rotated V means and <q_h, o^K_g> = <q'_h, H o^K_g / sqrt(d)>
        const int ngb = (int)((c1 - c0 + gsize - 1) / gsize);
        for (int gi = wv; gi < ngb; gi += NW) {
            const int64_t row = (bg * ngc + gfirst + gi) * kD;
            const f2_t ovv = reinterpret_cast<const f2_t *>(vo + row)[lane];
            const f2_t okk = reinterpret_cast<const f2_t *>(ko + row)[lane];
            float v0 = ovv.x, v1 = ovv.y, k0 = okk.x, k1 = okk.y;
            wave_fwht(v0, v1, lane);
            wave_fwht(k0, k1, lane);
            reinterpret_cast<f2_t *>(sm.og[gi])[lane] = f2_t{v0 * kInvSqrtD, v1 * kInvSqrtD};
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const f2_t qq = reinterpret_cast<const f2_t *>(sm.t.qs + h * kD)[lane];
                const float d = wave_sum(fmaf(qq.x, k0 * kInvSqrtD, qq.y * (k1 * kInvSqrtD)));
                if (lane == 0) sm.qog[gi][h] = d;
            }
        }
        __syncthreads();
    }

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
        if (tn < c1) nxt = fetch(tn + lane < c1 ? tn + lane : c0);
        float ks[G];
        nsn_key_sum<G>(cur.kcode, sm.t.tab, ks);
        float w[G];
        const int gi = GROUPED ? (int)((t0 - c0) / gsize) : 0;  // the tile's group (wave-uniform)
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float qoh = GROUPED ? sm.qog[gi][h] : sm.t.qo[h];
            const float lg = valid ? cur.a * fmaf(cur.c, ks[h], qoh) * scale2 : -__builtin_inff();
            const float mn = fmaxf(m[h], wave_max(lg));
            const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);
            const float p = __builtin_amdgcn_exp2f(lg - mn);
            m[h] = mn;
            l[h] = fmaf(l[h], alpha, p);
            acc[h][0] *= alpha;
            acc[h][1] *= alpha;
            if constexpr (GROUPED) {
                // the tile's sum of p s1_V times its group's rotated V mean
                const float wt = wave_sum(p * cur.e1);
                acc[h][0] = fmaf(wt, sm.og[gi][8 * vs + vk], acc[h][0]);
                acc[h][1] = fmaf(wt, sm.og[gi][8 * vs + vk + 1], acc[h][1]);
            } else {
                wo[h] = fmaf(wo[h], alpha, p * cur.e1);
            }
            w[h] = p * cur.e1 * cur.e2;
        }
        sm.vcode[wv][lane] = cur.vcode;
#pragma unroll
        for (int h = 0; h < G; ++h) sm.wts[wv][lane][h] = w[h];
        wave_lds_sync();
        // all 64 tokens: past the end the weights are 0 and the staged index
        // is that of the range's first token
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
    const int64_t split = blockIdx.x;
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
        float *dst = part + ((bg * n_part + split) * G + h) * kPartStride;
        dst[dim] = A;
        if (dim == 0) {
            dst[kD] = M;
            dst[kD + 1] = L;
            dst[kD + 2] = WO;
        }
    }
}

// Decode, part 2.  Block b * Hkv + g, one wave per head h (lane: dimensions
// 2 lane, 2 lane + 1): merge of the n_split partial slots, f_s = 2^(M_s - M),
// then out = (H acc / sqrt(d) + WO o_V) / L (vo NULL: the V means are already
// in acc, WO = 0).
template <int G, bool DQ>
__global__ __launch_bounds__(64 * G) void k_nsn_merge(const float *__restrict__ part, const float *__restrict__ vo,
                                                      float *__restrict__ out, int64_t Hkv, int n_split, NsnDqIn vdq)
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
    const f2_t ov = DQ ? load_mean<true>(nullptr, vdq, bg, lane)
                       : vo ? load_mean<false>(vo + bg * kD, vdq, bg, lane) : f2_t{0.0f, 0.0f};
    const float inv = 1.0f / L;
    reinterpret_cast<f2_t *>(out + ((b * Hkv + g) * G + h) * kD)[lane] =
        f2_t{fmaf(x0, kInvSqrtD, WO * ov.x) * inv, fmaf(x1, kInvSqrtD, WO * ov.y) * inv};
}

// Window of a streaming cache: the partial of its R fp16 tokens for the G
// query heads of (b, g) in the convention of k_nsn_part (base-2 scores,
// acc = H (sum_t 2^(s_t - M) v_t) / sqrt(d) so that the merge's transform
// returns the plain sum, WO = 0), written to slot `slot` of n_part; with no
// packed tokens (direct) the output itself.  One wave per query head.
template <int G>
__global__ __launch_bounds__(64 * G) void k_nsn_tail(const half_t *__restrict__ q, const half_t *__restrict__ kt,
                                                     const half_t *__restrict__ vt, float scale2,
                                                     float *__restrict__ part, float *__restrict__ out, int64_t R,
                                                     int64_t R_cap, int n_part, int slot, bool direct)
{
    __shared__ __align__(16) float qf[G][kD];
    const int lane = threadIdx.x & 63, h = threadIdx.x >> 6;
    const int64_t bg = blockIdx.x;
    const int64_t qrow = bg * G + h;  // (b Hkv + g) G + h = b Hq + g G + h
    const WindowPartial w = window_partial(qf[h], kt + bg * R_cap * kD, vt + bg * R_cap * kD, R, scale2, lane, [&] {
        const h2_t pr = reinterpret_cast<const h2_t *>(q + qrow * kD)[lane];
        reinterpret_cast<f2_t *>(qf[h])[lane] = f2_t{(float)pr.x, (float)pr.y};
    });
    if (direct) {
        const float inv = 1.0f / w.l;
        reinterpret_cast<f2_t *>(out + qrow * kD)[lane] = f2_t{w.a0 * inv, w.a1 * inv};
        return;
    }
    float x0 = w.a0, x1 = w.a1;
    wave_fwht(x0, x1, lane);
    float *dst = part + ((bg * n_part + slot) * G + h) * kPartStride;
    reinterpret_cast<f2_t *>(dst)[lane] = f2_t{x0 * kInvSqrtD, x1 * kInvSqrtD};
    if (lane == 0) {
        dst[kD] = w.m;
        dst[kD + 1] = w.l;
        dst[kD + 2] = 0.0f;
    }
}

template <int G, bool DQ>
hipError_t logits_g(const kvq_ctx *ctx, const void *q, int64_t B, int64_t T, const uint8_t *codes, const float *s1,
                    const float *s2, const float *o, float *logits, const NsnDqIn &dq, hipStream_t s)
{
    const int64_t n_chunks = (T + kLogitChunk - 1) / kLogitChunk;
    hipLaunchKernelGGL((k_nsn_logits<G, DQ>), dim3((unsigned)n_chunks, (unsigned)(B * ctx->H)), dim3(kThreadsN), 0, s,
                       (const half_t *)q, (const u4_t *)codes, s1, s2, o, ctx->d_vq, logits, (int64_t)ctx->H, T, dq);
    return hipGetLastError();
}

template <int G>
hipError_t decode_g(const kvq_ctx *ctx, const void *q, int64_t B, int64_t T, const NsnKV &kv, float sm_scale,
                    float *out, void *ws, int n_split, hipStream_t s)
{
    const int64_t chunk = nsn_decode_chunk(T, n_split);
    const int ns = (int)((T + chunk - 1) / chunk);
    float *part = (float *)ws;
#define KVQ_NSN_PART(DQ)                                                                                        \
    hipLaunchKernelGGL((k_nsn_part<G, false, DQ>), dim3((unsigned)ns, (unsigned)(B * ctx->H)),                   \
                       dim3(64 * dec_waves<G>()), 0, s, (const half_t *)q, (const u4_t *)kv.kc, kv.ks1, kv.ks2, kv.ko, \
                       (const u4_t *)kv.vc, kv.vs1, kv.vs2, ctx->d_vq, part, (int64_t)ctx->H, T, chunk,           \
                       sm_scale * kLog2e, T, ns, (const float *)nullptr, (int64_t)0, (int64_t)0, kv.kdq, kv.vdq);   \
    hipLaunchKernelGGL((k_nsn_merge<G, DQ>), dim3((unsigned)(B * ctx->H)), dim3(64 * G), 0, s, part, kv.vo, out,  \
                       (int64_t)ctx->H, ns, kv.vdq)
    if (kv.dq) {
        KVQ_NSN_PART(true);
    } else {
        KVQ_NSN_PART(false);
    }
#undef KVQ_NSN_PART
    return hipGetLastError();
}

// Streaming cache: the window's partial (slot ns, or the output when T = 0),
// the packed tokens' splits with per-group means, then the merge.
template <int G>
hipError_t decode_stream_g(const kvq_ctx *ctx, const void *q, int64_t B, int64_t T, const NsnKV &kv,
                           const NsnStream &st, float sm_scale, float *out, void *ws, int n_split, hipStream_t s)
{
    static_assert(G <= 4, "the grouped decode block fits LDS for up to 4 query heads per KV head");
    const float scale2 = sm_scale * kLog2e;
    float *part = (float *)ws;
    const int64_t bgs = B * ctx->H;
    int ns = 0, n_part = 1;
    int64_t chunk = 0;
    if (T > 0) {
        chunk = nsn_stream_chunk(T, n_split, st.Gs);
        if (chunk == 0) return hipErrorInvalidValue;  // more splits than partial slots
        ns = (int)((T + chunk - 1) / chunk);
        n_part = ns + (st.R > 0 ? 1 : 0);
    }
    if (st.R > 0)
        hipLaunchKernelGGL(k_nsn_tail<G>, dim3((unsigned)bgs), dim3(64 * G), 0, s, (const half_t *)q,
                           (const half_t *)st.kt, (const half_t *)st.vt, scale2, part, out, st.R, st.R_cap, n_part,
                           ns, T == 0);
    if (T == 0) return hipGetLastError();
    hipLaunchKernelGGL((k_nsn_part<G, true, false>), dim3((unsigned)ns, (unsigned)bgs), dim3(64 * dec_waves<G>()), 0,
                       s, (const half_t *)q, (const u4_t *)kv.kc, kv.ks1, kv.ks2, kv.ko, (const u4_t *)kv.vc, kv.vs1,
                       kv.vs2, ctx->d_vq, part, (int64_t)ctx->H, T, chunk, scale2, st.T_cap, n_part, kv.vo, st.Gs,
                       st.T_cap / st.Gs, NsnDqIn{}, NsnDqIn{});
    hipLaunchKernelGGL((k_nsn_merge<G, false>), dim3((unsigned)bgs), dim3(64 * G), 0, s, part, (const float *)nullptr,
                       out, (int64_t)ctx->H, n_part, NsnDqIn{});
    return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Scoring over GSRQ records ("GSRQ", gain-shape residual quantisation, on the
// NSN byproducts): zq of sub-vector s = G1[c1] S1[j1] + G2[c2] S2[j2], so with
// q' = H q / sqrt(d)
//   <q, x_hat> = s1 (s2 sum_s (G1[c1_s] T1[s][j1_s] + G2[c2_s] T2[s][j2_s]) + <q, o>),
// T_k[s][j] = <q'_s, S_k[j]> (4 sub-vectors of 32 x 256 shapes per stage).
constexpr int kGM = 32, kGP = kD / kGM;  // sub-vector length, sub-vectors per vector
template <int G>
struct GsrqTab {
    float tab[2][kGP][kVqK][G];  // stage, sub-vector, shape, head
    float qs[G * kD];
    float qo[G];
    float lv[2][16];
};

// Prologue: levels, q' and <q, o> of the G heads (one wave per head), then
// the two tables from the shapes in global memory; ends with a barrier.
template <int G, int NT>
__device__ void gsrq_tables(const half_t *__restrict__ q, const float *__restrict__ obg,
                            const float *__restrict__ gs, int64_t qbase, GsrqTab<G> &sm)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (tid < 32) sm.lv[tid >> 4][tid & 15] = gs[2 * kVqK * kGM + tid];
    for (int h = wv; h < G; h += NT / 64) {
        const h2_t pr = reinterpret_cast<const h2_t *>(q + (qbase + h) * kD)[lane];
        const f2_t ov = reinterpret_cast<const f2_t *>(obg)[lane];
        float x0 = (float)pr.x, x1 = (float)pr.y;
        const float qo = wave_sum(fmaf(x1, ov.y, x0 * ov.x));
        wave_fwht(x0, x1, lane);
        reinterpret_cast<f2_t *>(sm.qs + h * kD)[lane] = f2_t{x0 * kInvSqrtD, x1 * kInvSqrtD};
        if (lane == 0) sm.qo[h] = qo;
    }
    __syncthreads();
    for (int e = tid; e < 2 * kVqK; e += NT) {
        const int st = e / kVqK, j = e % kVqK;
        const f4_t *sh = reinterpret_cast<const f4_t *>(gs + (st * kVqK + j) * kGM);
        f4_t row[kGM / 4];
#pragma unroll
        for (int i = 0; i < kGM / 4; ++i) row[i] = sh[i];
#pragma unroll
        for (int sv = 0; sv < kGP; ++sv) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const f4_t *qv = reinterpret_cast<const f4_t *>(sm.qs + h * kD + sv * kGM);
                float acc = 0.0f;
#pragma unroll
                for (int i = 0; i < kGM / 4; ++i) {
                    const f4_t a = qv[i];
                    acc = fmaf(a.x, row[i].x, acc);
                    acc = fmaf(a.y, row[i].y, acc);
                    acc = fmaf(a.z, row[i].z, acc);
                    acc = fmaf(a.w, row[i].w, acc);
                }
                sm.tab[st][sv][j][h] = acc;
            }
        }
    }
    __syncthreads();
}

// sum_s (G1[c1] T1[s][j1] + G2[c2] T2[s][j2]) for the G heads of one record.
template <int G>
__device__ __forceinline__ void gsrq_key_sum(uint32_t w0, uint32_t w1, uint32_t w2, const GsrqTab<G> &sm,
                                             float (&acc)[G])
{
    typedef float fg_t __attribute__((ext_vector_type(G)));
    fg_t sum = 0.0f;
#pragma unroll
    for (int sv = 0; sv < kGP; ++sv) {
        const uint32_t j1 = (w0 >> (8 * sv)) & 0xFFu, j2 = (w1 >> (8 * sv)) & 0xFFu, g = (w2 >> (8 * sv)) & 0xFFu;
        const float a1 = sm.lv[0][g & 15u], a2 = sm.lv[1][g >> 4];
        sum += a1 * *reinterpret_cast<const fg_t *>(&sm.tab[0][sv][j1][0]);
        sum += a2 * *reinterpret_cast<const fg_t *>(&sm.tab[1][sv][j2][0]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = sum[h];
}

// logits[b, g G + h, t]: block (chunk of kLogitChunk tokens, b * Hkv + g),
// one thread per token.
template <int G>
__global__ __launch_bounds__(kThreadsN) void k_gsrq_logits(const half_t *__restrict__ q, const uint32_t *__restrict__ codes,
                                                           const float *__restrict__ s1, const float *__restrict__ s2,
                                                           const float *__restrict__ o, const float *__restrict__ gs,
                                                           float *__restrict__ logits, int64_t Hkv, int64_t T)
{
    constexpr int NT = kLogitChunk / kThreadsN;
    __shared__ GsrqTab<G> sm;
    const int64_t bg = blockIdx.y, b = bg / Hkv, g = bg % Hkv;
    const int64_t qbase = b * Hkv * G + g * G;
    const int64_t c0 = (int64_t)blockIdx.x * kLogitChunk, c1 = min(T, c0 + kLogitChunk);
    uint32_t r0[NT], r1[NT], r2[NT];
    float a[NT], c[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int64_t t = c0 + threadIdx.x + i * kThreadsN;
        const int64_t v = bg * T + (t < c1 ? t : c0);
        r0[i] = codes[3 * v];
        r1[i] = codes[3 * v + 1];
        r2[i] = codes[3 * v + 2];
        a[i] = s1[v];
        c[i] = s2[v];
    }
    gsrq_tables<G, kThreadsN>(q, o + bg * kD, gs, qbase, sm);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int64_t t = c0 + threadIdx.x + i * kThreadsN;
        float acc[G];
        gsrq_key_sum<G>(r0[i], r1[i], r2[i], sm, acc);
        if (t < c1) {
#pragma unroll
            for (int h = 0; h < G; ++h) logits[(qbase + h) * T + t] = a[i] * fmaf(c[i], acc[h], sm.qo[h]);
        }
    }
}

// Decode, part 1, over GSRQ records: as k_nsn_part (64-token tiles, online
// softmax, value sums in the code domain with lanes as dimensions), with the
// value of a token in dimension pair (2 l, 2 l + 1) of sub-vector l / 16
// being G1[c1] S1[j1][.] + G2[c2] S2[j2][.] (shapes staged in LDS).
template <int G>
struct GsrqDecSmem {
    static constexpr int NW = 8;
    GsrqTab<G> t;
    float shapes[2][kVqK][kGM];
    u4_t vrec[NW][64];
    float wts[NW][64][G];
};

template <int G>
__global__ __launch_bounds__(512) void k_gsrq_part(const half_t *__restrict__ q, const uint32_t *__restrict__ kc,
                                                   const float *__restrict__ ks1, const float *__restrict__ ks2,
                                                   const float *__restrict__ ko, const uint32_t *__restrict__ vc,
                                                   const float *__restrict__ vs1, const float *__restrict__ vs2,
                                                   const float *__restrict__ gs, float *__restrict__ part,
                                                   int64_t Hkv, int64_t T, int64_t chunk, float scale2)
{
    using SM = GsrqDecSmem<G>;
    constexpr int NW = SM::NW;
    __shared__ SM sm;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bg = blockIdx.y, b = bg / Hkv, g = bg % Hkv;
    const int64_t qbase = b * Hkv * G + g * G;
    const int64_t c0 = (int64_t)blockIdx.x * chunk, c1 = min(T, c0 + chunk);
    for (int i = threadIdx.x; i < 2 * kVqK * kGM / 4; i += 64 * NW)
        reinterpret_cast<f4_t *>(&sm.shapes[0][0][0])[i] = reinterpret_cast<const f4_t *>(gs)[i];
    gsrq_tables<G, 64 * NW>(q, ko + bg * kD, gs, qbase, sm.t);

    float m[G], l[G], wo[G], acc[G][2];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -__builtin_inff();
        l[h] = wo[h] = acc[h][0] = acc[h][1] = 0.0f;
    }
    const int vsub = lane >> 4, vk = 2 * (lane & 15);  // the lane's sub-vector and dimension pair in it
    // tokens past the end of the range (and whole waves without a tile) load
    // the range's first token, with weight 0
    for (int64_t t0 = c0 + 64 * wv; t0 < c1; t0 += 64 * NW) {
        const bool valid = t0 + lane < c1;
        const int64_t v = bg * T + (valid ? t0 + lane : c0);
        const uint32_t k0 = kc[3 * v], k1 = kc[3 * v + 1], k2 = kc[3 * v + 2];
        const u4_t vr = u4_t{vc[3 * v], vc[3 * v + 1], vc[3 * v + 2], 0u};
        const float a = ks1[v], c = ks2[v], e1 = vs1[v], e2 = vs2[v];
        float ks[G];
        gsrq_key_sum<G>(k0, k1, k2, sm.t, ks);
        float w[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float lg = valid ? a * fmaf(c, ks[h], sm.t.qo[h]) * scale2 : -__builtin_inff();
            const float mn = fmaxf(m[h], wave_max(lg));
            const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);
            const float p = __builtin_amdgcn_exp2f(lg - mn);
            m[h] = mn;
            l[h] = fmaf(l[h], alpha, p);
            wo[h] = fmaf(wo[h], alpha, p * e1);
            acc[h][0] *= alpha;
            acc[h][1] *= alpha;
            w[h] = p * e1 * e2;
        }
        sm.vrec[wv][lane] = vr;
#pragma unroll
        for (int h = 0; h < G; ++h) sm.wts[wv][lane][h] = w[h];
        wave_lds_sync();
#pragma unroll 8
        for (int i = 0; i < 64; ++i) {
            const u4_t r = sm.vrec[wv][i];
            const uint32_t j1 = (r.x >> (8 * vsub)) & 0xFFu, j2 = (r.y >> (8 * vsub)) & 0xFFu;
            const uint32_t gg = (r.z >> (8 * vsub)) & 0xFFu;
            const float a1 = sm.t.lv[0][gg & 15u], a2 = sm.t.lv[1][gg >> 4];
            const f2_t s1v = *reinterpret_cast<const f2_t *>(&sm.shapes[0][j1][vk]);
            const f2_t s2v = *reinterpret_cast<const f2_t *>(&sm.shapes[1][j2][vk]);
            const float e0 = fmaf(a2, s2v.x, a1 * s1v.x), ee1 = fmaf(a2, s2v.y, a1 * s1v.y);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float wh = sm.wts[wv][i][h];
                acc[h][0] = fmaf(wh, e0, acc[h][0]);
                acc[h][1] = fmaf(wh, ee1, acc[h][1]);
            }
        }
        wave_lds_sync();
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        l[h] = wave_sum(l[h]);
        wo[h] = wave_sum(wo[h]);
    }
    // merge of the waves through the (no longer read) shape space
    __syncthreads();
    float *mw = &sm.shapes[0][0][0];
    static_assert(NW * G * kPartStride <= 2 * kVqK * kGM, "wave partials fit in the shape space");
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float *p = mw + (wv * G + h) * kPartStride;
        *reinterpret_cast<f2_t *>(p + 2 * lane) = f2_t{acc[h][0], acc[h][1]};
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
            const float f = __builtin_amdgcn_exp2f(p[kD] - M);
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

template <int G>
hipError_t gsrq_logits_g(const kvq_ctx *ctx, const void *q, int64_t B, int64_t T, const uint8_t *codes,
                         const float *s1, const float *s2, const float *o, float *logits, hipStream_t s)
{
    const int64_t n_chunks = (T + kLogitChunk - 1) / kLogitChunk;
    hipLaunchKernelGGL(k_gsrq_logits<G>, dim3((unsigned)n_chunks, (unsigned)(B * ctx->H)), dim3(kThreadsN), 0, s,
                       (const half_t *)q, (const uint32_t *)codes, s1, s2, o, ctx->d_gsrq, logits, (int64_t)ctx->H, T);
    return hipGetLastError();
}

template <int G>
hipError_t gsrq_decode_g(const kvq_ctx *ctx, const void *q, int64_t B, int64_t T, const NsnKV &kv, float sm_scale,
                         float *out, void *ws, int n_split, hipStream_t s)
{
    const int64_t chunk = nsn_decode_chunk(T, n_split);
    const int ns = (int)((T + chunk - 1) / chunk);
    float *part = (float *)ws;
    hipLaunchKernelGGL(k_gsrq_part<G>, dim3((unsigned)ns, (unsigned)(B * ctx->H)), dim3(512), 0, s, (const half_t *)q,
                       (const uint32_t *)kv.kc, kv.ks1, kv.ks2, kv.ko, (const uint32_t *)kv.vc, kv.vs1, kv.vs2,
                       ctx->d_gsrq, part, (int64_t)ctx->H, T, chunk, sm_scale * kLog2e);
    hipLaunchKernelGGL((k_nsn_merge<G, false>), dim3((unsigned)(B * ctx->H)), dim3(64 * G), 0, s, part, kv.vo, out,
                       (int64_t)ctx->H, ns, NsnDqIn{});
    return hipGetLastError();
}

}  // namespace

hipError_t launch_nsn_logits(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                             const uint8_t *codes, const float *s1, const float *s2, const float *o, float *logits,
                             hipStream_t s)
{
    const NsnDqIn none{};
    switch (Hq / ctx->H) {
        case 1: return logits_g<1, false>(ctx, q, B, T, codes, s1, s2, o, logits, none, s);
        case 2: return logits_g<2, false>(ctx, q, B, T, codes, s1, s2, o, logits, none, s);
        case 4: return logits_g<4, false>(ctx, q, B, T, codes, s1, s2, o, logits, none, s);
        case 8: return logits_g<8, false>(ctx, q, B, T, codes, s1, s2, o, logits, none, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_nsn_logits_dq(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                                const uint8_t *codes, const NsnDqIn &dq, const float *s2, float *logits, hipStream_t s)
{
    switch (Hq / ctx->H) {
        case 1: return logits_g<1, true>(ctx, q, B, T, codes, nullptr, s2, nullptr, logits, dq, s);
        case 2: return logits_g<2, true>(ctx, q, B, T, codes, nullptr, s2, nullptr, logits, dq, s);
        case 4: return logits_g<4, true>(ctx, q, B, T, codes, nullptr, s2, nullptr, logits, dq, s);
        case 8: return logits_g<8, true>(ctx, q, B, T, codes, nullptr, s2, nullptr, logits, dq, s);
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

hipError_t launch_nsn_decode_stream(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                                    const NsnKV &kv, const NsnStream &st, float sm_scale, float *out, void *ws,
                                    int n_split, hipStream_t s)
{
    switch (Hq / ctx->H) {
        case 1: return decode_stream_g<1>(ctx, q, B, T, kv, st, sm_scale, out, ws, n_split, s);
        case 2: return decode_stream_g<2>(ctx, q, B, T, kv, st, sm_scale, out, ws, n_split, s);
        case 4: return decode_stream_g<4>(ctx, q, B, T, kv, st, sm_scale, out, ws, n_split, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gsrq_logits(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                              const uint8_t *codes, const float *s1, const float *s2, const float *o, float *logits,
                              hipStream_t s)
{
    switch (Hq / ctx->H) {
        case 1: return gsrq_logits_g<1>(ctx, q, B, T, codes, s1, s2, o, logits, s);
        case 2: return gsrq_logits_g<2>(ctx, q, B, T, codes, s1, s2, o, logits, s);
        case 4: return gsrq_logits_g<4>(ctx, q, B, T, codes, s1, s2, o, logits, s);
        case 8: return gsrq_logits_g<8>(ctx, q, B, T, codes, s1, s2, o, logits, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gsrq_decode(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T, const NsnKV &kv,
                              float sm_scale, float *out, void *ws, int n_split, hipStream_t s)
{
    switch (Hq / ctx->H) {
        case 1: return gsrq_decode_g<1>(ctx, q, B, T, kv, sm_scale, out, ws, n_split, s);
        case 2: return gsrq_decode_g<2>(ctx, q, B, T, kv, sm_scale, out, ws, n_split, s);
        case 4: return gsrq_decode_g<4>(ctx, q, B, T, kv, sm_scale, out, ws, n_split, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
