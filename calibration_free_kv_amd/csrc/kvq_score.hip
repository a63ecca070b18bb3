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
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

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

// One Walsh-Hadamard transform of 128 values held two per lane (lane l holds
// coordinates 2l and 2l+1): the first stage inside the lane, the other six
// across lanes with shuffles.
__device__ __forceinline__ void wave_fwht(float &x0, float &x1, int lane)
{
    const float a = x0 + x1;
    x1 = x0 - x1;
    x0 = a;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const float p0 = __shfl_xor(x0, m), p1 = __shfl_xor(x1, m);
        const bool up = (lane & m) != 0;
        x0 = up ? p0 - x0 : x0 + p0;
        x1 = up ? p1 - x1 : x1 + p1;
    }
}

// Prologue shared by the score kernels: qr[G][128] <- H (D .* q_h) for the G
// query heads of KV head g of batch b, one wave per head.  Ends with a barrier.
template <int G>
__device__ void rotate_queries(const half_t *__restrict__ q, const float *__restrict__ signs,
                               int64_t b, int g, int Hq, float *qr)
{
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
    for (int h = wv; h < G; h += nw) {
        const uint32_t pr =
            reinterpret_cast<const uint32_t *>(q + ((int64_t)b * Hq + (int64_t)g * G + h) * kD)[lane];
        const f2_t sg = reinterpret_cast<const f2_t *>(signs + g * kD)[lane];
        float x0 = (float)__builtin_bit_cast(h2_t, pr).x * sg.x;
        float x1 = (float)__builtin_bit_cast(h2_t, pr).y * sg.y;
        wave_fwht(x0, x1, lane);
        reinterpret_cast<f2_t *>(qr + h * kD)[lane] = f2_t{x0, x1};
    }
    __syncthreads();
}

// ctab: the 2^b centroids already in LDS.  One thread per (field, value)
// pair computes the G heads' entries together (the field's query values and
// the pair's centroids are read once) and writes them contiguously.
template <int BITS, int G>
__device__ void build_tables(const float *qr, const float *ctab, float *lut)
{
    using FD = Fields<BITS>;
    constexpr uint32_t mask = (1u << BITS) - 1u;
    const float inv_d = 1.0f / kD;
    for (int fe = threadIdx.x; fe < FD::NF * FD::E; fe += blockDim.x) {
        const int e = fe % FD::E, f = fe / FD::E;
        float c[FD::F];
#pragma unroll
        for (int k = 0; k < FD::F; ++k) c[k] = ctab[(e >> (BITS * k)) & mask] * inv_d;
        float v[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            v[h] = 0.0f;
#pragma unroll
            for (int k = 0; k < FD::F; ++k) v[h] = fmaf(qr[h * kD + FD::F * f + k], c[k], v[h]);
        }
        if constexpr (G % 4 == 0) {
#pragma unroll
            for (int h4 = 0; h4 < G / 4; ++h4)
                reinterpret_cast<f4_t *>(lut)[fe * (G / 4) + h4] =
                    f4_t{v[4 * h4], v[4 * h4 + 1], v[4 * h4 + 2], v[4 * h4 + 3]};
        } else {
#pragma unroll
            for (int h = 0; h < G; ++h) lut[fe * G + h] = v[h];
        }
    }
}

__device__ __forceinline__ void stage_centroids(const Codebook &cb, float *ctab)
{
    if (threadIdx.x < 16) ctab[threadIdx.x] = cb.c[threadIdx.x];
}

// Sum of the table entries of one record for the G heads (the G entries of a
// (field, value) pair are read with one 16- or 8-byte LDS load), in groups of
// 8 fields: the scheduler may not move address computations or reads across
// groups, so at most 8 entries are in flight (all 64 at once would not fit
// in the registers of a wave).
template <int BITS, int G>
__device__ __forceinline__ void score_record_grouped(const uint32_t *Wd, const float *lut, float *acc)
{
    using FD = Fields<BITS>;
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.0f;
#pragma unroll
    for (int f = 0; f < FD::NF; ++f) {
        if (f % 8 == 0) __builtin_amdgcn_sched_barrier(0);
        const int e = f * FD::E + (int)field<BITS>(Wd, f);
        if constexpr (G % 4 == 0) {
#pragma unroll
            for (int h4 = 0; h4 < G / 4; ++h4) {
                const f4_t x = reinterpret_cast<const f4_t *>(lut)[e * (G / 4) + h4];
                acc[4 * h4] += x.x;
                acc[4 * h4 + 1] += x.y;
                acc[4 * h4 + 2] += x.z;
                acc[4 * h4 + 3] += x.w;
            }
        } else if constexpr (G == 2) {
            const f2_t x = reinterpret_cast<const f2_t *>(lut)[e];
            acc[0] += x.x;
            acc[1] += x.y;
        } else {
            acc[0] += lut[e];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
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
// One block of 16 waves per (batch, KV head, token range), about one block per
// CU: the prologue (tables, and for QJL the projection of the G queries) is
// built by 1024 threads and amortised over a long range.
constexpr int kLgThreads = 1024;

template <int BITS, int G, bool QJL>
__global__ __launch_bounds__(kLgThreads) void k_logits(
    const half_t *__restrict__ q, const uint8_t *__restrict__ codes, const float *__restrict__ norms,
    const uint32_t *__restrict__ qjl_signs, const float *__restrict__ qjl_gamma,
    const float *__restrict__ signs, const float *__restrict__ St, Codebook cb,
    float *__restrict__ logits, int64_t T, int H, int Hq, int64_t tokens_per_block,
    int64_t blocks_per_bh)
{
    using FD = Fields<BITS>;
    extern __shared__ __align__(16) float smem[];
    float *qr = smem;                       // [G][128]
    float *lut = qr + G * kD;               // [NF][E][G]
    float *slut = lut + FD::NF * FD::E * G; // [32][16][G] (QJL)
    float *pq = slut + (QJL ? 32 * 16 * G : 0);  // [G][128] (QJL)
    float *ctab = pq + (QJL ? G * kD : 0);       // [16] centroids

    const int64_t bh = blockIdx.x / blocks_per_bh;
    const int64_t part = blockIdx.x - bh * blocks_per_bh;
    const int64_t b = bh / H;
    const int g = (int)(bh - b * H);

    stage_centroids(cb, ctab);
    rotate_queries<G>(q, signs, b, g, Hq, qr);
    build_tables<BITS, G>(qr, ctab, lut);
    if constexpr (QJL) {
        // p_h[j] = sum_i S[j][i] q'_h[i] / sqrt(d): thread (h, j) walks row i of
        // S^T, so that the 128 threads of a head read 512 contiguous bytes per
        // step; the steps are unrolled to keep many loads in flight
        const float inv_sqrt_d = 0.08838834764831845f;
        for (int idx = threadIdx.x; idx < G * kD; idx += kLgThreads) {
            const int h = idx >> 7, j = idx & (kD - 1);
            float s = 0.0f;
#pragma unroll 16
            for (int i = 0; i < kD; ++i) s = fmaf(St[i * kD + j], qr[h * kD + i], s);
            pq[idx] = s * inv_sqrt_d;
        }
        __syncthreads();
        const float coef = 1.2533141373155003f / kD;  // sqrt(pi/2) / m
        for (int idx = threadIdx.x; idx < 32 * 16 * G; idx += kLgThreads) {
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
    // Register prefetch: a thread loads its next token's records before it
    // scores the current one.  The loads are unconditional (indexes past the
    // range re-read its last token), so the compiler's wait before the scoring
    // counts exactly the prefetch loads issued after them.
    uint32_t Wn[FD::W + 1];
    float rn = 0.0f, gn = 0.0f;
    u4_t sn = {};
    auto fetch = [&](int64_t t) {
        const int64_t v = bh * T + min(t, t_end - 1);
        load_record<BITS>(codes, v, Wn);
        rn = norms[v];
        if constexpr (QJL) {
            sn = reinterpret_cast<const u4_t *>(qjl_signs)[v];
            gn = qjl_gamma[v];
        }
    };
    int64_t t = t_begin + threadIdx.x;
    fetch(t);
    for (; t < t_end; t += kLgThreads) {
        uint32_t Wd[FD::W + 1];
#pragma unroll
        for (int k = 0; k <= FD::W; ++k) Wd[k] = Wn[k];
        const float rho = rn, gm = gn;
        const u4_t sg = sn;
        fetch(t + kLgThreads);
        float acc[G];
        score_record_grouped<BITS, G>(Wd, lut, acc);
        if constexpr (QJL) {
            const uint32_t sw[4] = {sg.x, sg.y, sg.z, sg.w};
            float qa[G];
#pragma unroll
            for (int h = 0; h < G; ++h) qa[h] = 0.0f;
#pragma unroll
            for (int f = 0; f < 32; ++f) {
                if (f % 8 == 0) __builtin_amdgcn_sched_barrier(0);  // at most 8 entries in flight
                const float *e = slut + (f * 16 + (int)((sw[f >> 3] >> (4 * (f & 7))) & 15u)) * G;
#pragma unroll
                for (int h = 0; h < G; ++h) qa[h] += e[h];
            }
#pragma unroll
            for (int h = 0; h < G; ++h) acc[h] = fmaf(gm, qa[h], acc[h]);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) logits[((b * Hq) + (int64_t)g * G + h) * T + t] = rho * acc[h];
    }
}

// ---------------------------------------------------------------------------
// kvq_attn_decode: split-K flash decoding.  Block (b, g, split) owns a token
// range of one (batch, KV head).  After the shared prologue (rotated queries,
// K field tables) every wave works alone on 64-token tiles of the range:
//  K  lane = token: logit from the field tables, scaled by rho_K and by
//     sm_scale*log2(e); wave max / sum give a running (m, l) per head
//     (base-2 exponentials);
//  V  lane = 8 consecutive coordinates (an octet) and one of four token
//     phases: the weights p_h,t rho_V,t and the staged V records are read
//     from the wave's LDS and accumulated in the rotated domain,
//     acc_h[i] += p rho_V c[idx_t,i].
// The block's waves merge once at the end; the block writes (m, l, acc) for
// its G heads and the last block of a (b, g) to finish (arrival counter)
// merges the splits and applies the inverse rotation once:
// out_h = D_V .* H acc / (d l).
// ---------------------------------------------------------------------------
constexpr int kDecWaves = 16;
constexpr int kDecThreads = kDecWaves * 64;

template <int BITS, int G>
struct DecSmem {
    using FD = Fields<BITS>;
    // staged V record stride in dwords: at least one word past the record
    // (the funnel shift of the last octet reads it), 16 when that suffices
    static constexpr int RW = FD::W + 1 <= 16 ? 16 : FD::W + 1;
    // the field tables come first: with a constant base, every field's part
    // of an entry address fits the 16-bit offset of an LDS instruction
    static constexpr int lut = 0;                                 // [NF][E][G]
    static constexpr int c2 = lut + FD::NF * FD::E * G;           // [2^(2b)][2] centroid pairs
    static constexpr int vbuf = c2 + 2 * (1 << (2 * BITS));       // [waves][64][RW] V records
    static constexpr int wbuf = vbuf + kDecWaves * 64 * RW;       // [waves][64][G] weights
    static constexpr int qr = wbuf + kDecWaves * 64 * G;          // [G][128] rotated queries
    static constexpr int wm = qr + G * kD;                        // [waves][G] wave maxima
    static constexpr int wl = wm + kDecWaves * G;                 // [waves][G] wave sums
    static constexpr int ctab = wl + kDecWaves * G;               // [16] centroids
    static constexpr int flag = ctab + 16;                        // [1] last-arrival flag
    static constexpr int total = flag + 4;
    // end-of-block reuse of vbuf..wbuf: per-wave accumulators, split merge
    static_assert(qr - vbuf >= kDecWaves * G * kD, "wave merge buffer does not fit");
    static_assert(qr - vbuf >= 2 * kMaxSplits * G, "split merge buffer does not fit");
    static_assert(FD::NF * FD::E * G * 4 <= 65536, "field offsets must fit an LDS immediate");
};

// Cross-row exchanges on the VALU (gfx950 lane swaps): with the same value in
// both operands, the swap of odd and even rows yields lane l ^ 16 in one
// result and lane l in the other, and likewise for halves (l ^ 32).
__device__ __forceinline__ float2 swap16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                    false, false);
    return float2{__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1])};
}
__device__ __forceinline__ float2 swap32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                    false, false);
    return float2{__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1])};
}

// Wave-wide max / sum, result in every lane: four DPP steps inside each row
// of 16 lanes, then the exchanges across rows and halves.
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float wave_max(float x)
{
    x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
    x = fmaxf(x, dpp<0x140>(x));  // row_mirror
    float2 p = swap16(x);
    x = fmaxf(p.x, p.y);
    p = swap32(x);
    return fmaxf(p.x, p.y);
}
__device__ __forceinline__ float wave_sum(float x)
{
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    x += dpp<0x140>(x);
    float2 p = swap16(x);
    x = p.x + p.y;
    p = swap32(x);
    return p.x + p.y;
}
// A value that is the same in every lane, moved to a scalar register.
__device__ __forceinline__ float uniform(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}
// LDS written by some lanes of a wave is read by other lanes of the same wave.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One V step of a lane: the octet of token tt's staged record (bits of 8
// coordinates, as four fields of two), its four centroid pairs, the G weights
// of the token, 8 G multiply-adds.
template <int BITS, int G>
__device__ __forceinline__ void v_step(const uint32_t *rec, const float *wrow, const float *c2, int owd, int osh,
                                       float (&acc)[G][8])
{
    constexpr uint32_t fmask = (1u << (2 * BITS)) - 1u;
    const uint32_t bits = __builtin_amdgcn_alignbit(rec[owd + 1], rec[owd], (uint32_t)osh);
    f2_t cp[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) cp[k] = reinterpret_cast<const f2_t *>(c2)[(bits >> (2 * BITS * k)) & fmask];
    float wv[G];
    if constexpr (G % 4 == 0) {
#pragma unroll
        for (int h4 = 0; h4 < G / 4; ++h4) {
            const f4_t x = reinterpret_cast<const f4_t *>(wrow)[h4];
            wv[4 * h4] = x.x;
            wv[4 * h4 + 1] = x.y;
            wv[4 * h4 + 2] = x.z;
            wv[4 * h4 + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int h = 0; h < G; ++h) wv[h] = wrow[h];
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            acc[h][2 * k] = fmaf(wv[h], cp[k].x, acc[h][2 * k]);
            acc[h][2 * k + 1] = fmaf(wv[h], cp[k].y, acc[h][2 * k + 1]);
        }
}

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
    constexpr int RW = SM::RW;
    extern __shared__ __align__(16) float smem[];
    float *qr = smem + SM::qr;
    float *lut = smem + SM::lut;
    float *c2 = smem + SM::c2;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t *vbuf = reinterpret_cast<uint32_t *>(smem + SM::vbuf) + wv * 64 * RW;
    float *wbuf = smem + SM::wbuf + wv * 64 * G;
    const int64_t bh = blockIdx.x / n_split;
    const int split = (int)(blockIdx.x - bh * n_split);
    const int64_t b = bh / H;
    const int g = (int)(bh - b * H);

    // V lane roles: coordinate octet co (coordinates 8co .. 8co+7) and token
    // phase ph (tokens ph, ph+4, ...): the 8b bits of an octet come from one
    // funnel shift of two record dwords, its four centroid pairs from four
    // 8-byte LDS reads.
    const int co = lane & 15, ph = lane >> 4;
    constexpr int OB = 8 * BITS;  // bits of an octet
    const int obit = OB * co, owd = obit >> 5, osh = obit & 31;

    float m_run[G], l_run[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[h][k] = 0.0f;
    }

    const int64_t t_begin = (int64_t)split * chunk;
    const int64_t t_end = min(T, t_begin + chunk);
    // The query loads go out first: memory operations complete in issue order,
    // so loads issued after the records would make the prologue wait for them.
    uint32_t qv = 0u;
    f2_t qs = f2_t{0.0f, 0.0f};
    if (wv < G) {
        qv = reinterpret_cast<const uint32_t *>(q + ((int64_t)b * Hq + (int64_t)g * G + wv) * kD)[lane];
        qs = reinterpret_cast<const f2_t *>(signs_k + g * kD)[lane];
    }
    // The records of the wave's next tile are held in registers: loaded before
    // the prologue for the first tile, and right after the current tile's
    // records have been consumed for the others.
    uint32_t Kw[FD::W + 1], Vw[FD::W];
    float rk = 0.0f, rv = 0.0f;
    // Every lane loads (tokens past the end re-read the last one of the
    // range), so the loads carry no lane-dependent branch and the compiler's
    // wait for the query values counts exactly the loads issued after them.
    // Addresses: a wave-uniform 64-bit base for the tile plus a 32-bit lane
    // offset (scalar-base loads; one VGPR of address per load).
    auto fetch = [&](int64_t t0) {
        t0 = min(t0, t_end - 1);  // a wave without a tile loads the range's last token
        const int64_t v0 = bh * T + t0;
        const uint32_t l = (uint32_t)min((int64_t)lane, t_end - 1 - t0);  // >= 0
        const uint32_t off = l * (16u * BITS);  // bytes
        const char *ks = reinterpret_cast<const char *>(kc) + v0 * (16 * BITS) + off;
        const char *vs = reinterpret_cast<const char *>(vc) + v0 * (16 * BITS) + off;
#pragma unroll
        for (int k = 0; k < BITS; ++k) {
            const u4_t x = reinterpret_cast<const u4_t *>(ks)[k], y = reinterpret_cast<const u4_t *>(vs)[k];
            Kw[4 * k] = x.x;
            Kw[4 * k + 1] = x.y;
            Kw[4 * k + 2] = x.z;
            Kw[4 * k + 3] = x.w;
            Vw[4 * k] = y.x;
            Vw[4 * k + 1] = y.y;
            Vw[4 * k + 2] = y.z;
            Vw[4 * k + 3] = y.w;
        }
        Kw[4 * BITS] = 0u;  // guard word for fields that end on the last dword
        rk = *reinterpret_cast<const float *>(reinterpret_cast<const char *>(kn + v0) + 4 * l);
        rv = *reinterpret_cast<const float *>(reinterpret_cast<const char *>(vn + v0) + 4 * l);
    };
    constexpr int64_t kStride = (int64_t)kDecWaves * 64;
    // the centroids too: indexed at run time, they are read from memory
    float cen = 0.0f;
    if (tid < 16) cen = cb.c[tid];
    __builtin_amdgcn_sched_barrier(0);  // keep the prologue's loads ahead of the records
    fetch(t_begin + (int64_t)wv * 64);
    float *ctab = smem + SM::ctab;
    if (tid < 16) ctab[tid] = cen;
    if (wv < G) {  // one wave per head: qr[h] = H (D_K .* q_h)
        float x0 = (float)__builtin_bit_cast(h2_t, qv).x * qs.x;
        float x1 = (float)__builtin_bit_cast(h2_t, qv).y * qs.y;
        wave_fwht(x0, x1, lane);
        reinterpret_cast<f2_t *>(qr + wv * kD)[lane] = f2_t{x0, x1};
    }
    __syncthreads();
    constexpr uint32_t cm = (1u << BITS) - 1u;
    for (int e = tid; e < (1 << (2 * BITS)); e += kDecThreads) {
        c2[2 * e] = ctab[e & cm];
        c2[2 * e + 1] = ctab[(e >> BITS) & cm];
    }
    build_tables<BITS, G>(qr, ctab, lut);
    __syncthreads();

    const uint32_t *vrow = vbuf + ph * RW;  // this lane's token phase in the staged records
    const float *wrow = wbuf + ph * G;
    for (int64_t t0 = t_begin + (int64_t)wv * 64; t0 < t_end; t0 += kStride) {
        const int nt = (int)min((int64_t)64, t_end - t0);
        const bool valid = lane < nt;
        float s[G];
        const float rvc = rv;
        // lanes past the end hold a copy of the last record: staged (never
        // read) and scored (then discarded)
        if constexpr (RW % 4 == 0) {  // 16-byte aligned rows
#pragma unroll
            for (int k = 0; k < FD::W / 4; ++k)
                reinterpret_cast<u4_t *>(vbuf + lane * RW)[k] = u4_t{Vw[4 * k], Vw[4 * k + 1], Vw[4 * k + 2], Vw[4 * k + 3]};
        } else {
#pragma unroll
            for (int k = 0; k < FD::W; ++k) vbuf[lane * RW + k] = Vw[k];
        }
        score_record_grouped<BITS, G>(Kw, lut, s);
        const float rs = rk * scale_log2;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            s[h] = valid ? s[h] * rs : -INFINITY;
            // the sums are formed here, not sunk past the loads below (which
            // would keep all 64 table entries live in registers meanwhile)
            asm volatile("" : : "v"(s[h]));
        }
        if (t0 + kStride < t_end) fetch(t0 + kStride);  // this tile's records are consumed
        // m, l and the rescale factor are the same in every lane: kept in
        // scalar registers
        float alpha[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mn = uniform(fmaxf(m_run[h], wave_max(s[h])));
            alpha[h] = uniform(__builtin_amdgcn_exp2f(m_run[h] - mn));  // 0 on the first tile (m_run = -inf)
            m_run[h] = mn;
            const float p = valid ? __builtin_amdgcn_exp2f(s[h] - mn) : 0.0f;
            l_run[h] = uniform(l_run[h] * alpha[h] + wave_sum(p));
            s[h] = p * rvc;
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[h][k] *= alpha[h];
        }
        if constexpr (G % 4 == 0) {
#pragma unroll
            for (int h4 = 0; h4 < G / 4; ++h4)
                reinterpret_cast<f4_t *>(wbuf + lane * G)[h4] = f4_t{s[4 * h4], s[4 * h4 + 1], s[4 * h4 + 2], s[4 * h4 + 3]};
        } else {
#pragma unroll
            for (int h = 0; h < G; ++h) wbuf[lane * G + h] = s[h];
        }
        wave_lds_sync();
        if (nt == 64) {  // full tile: 16 steps with constant LDS offsets
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                // at most two steps' loads in flight: hoisting all sixteen
                // would need far more registers than a wave has
                __builtin_amdgcn_sched_barrier(0);
                v_step<BITS, G>(vrow + 4 * j * RW, wrow + 4 * j * G, c2, owd, osh, acc);
            }
        } else {
            for (int tt = ph; tt < nt; tt += 4) v_step<BITS, G>(vbuf + tt * RW, wbuf + tt * G, c2, owd, osh, acc);
        }
        wave_lds_sync();  // vbuf / wbuf are rewritten by the next tile
    }

    // Sum the four token phases (lanes l, l^16, l^32, l^48 hold partial sums
    // of the same coordinates) with lane swaps: one swap and one add per
    // register and level.  Afterwards register r of red[] holds in row k
    // (lanes 16k .. 16k+15, coordinate octet co) the total of accumulator
    // 4r + k, accumulator a = 8h + j being coordinate 8co + j of head h.
    constexpr int NA = 8 * G;
    float red[NA / 4];
    {
        float s1[NA / 2];
#pragma unroll
        for (int i = 0; i < NA / 2; ++i) {  // level 1: pairs (2i, 2i+1) across halves
            const float a = acc[(2 * i) / 8][(2 * i) % 8], c = acc[(2 * i + 1) / 8][(2 * i + 1) % 8];
            const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a),
                                                            __builtin_bit_cast(unsigned, c), false, false);
            // lanes 0-31: a's halves summed; lanes 32-63: c's
            s1[i] = __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
        }
#pragma unroll
        for (int i = 0; i < NA / 4; ++i) {  // level 2: pairs (2i, 2i+1) across rows
            const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, s1[2 * i]),
                                                            __builtin_bit_cast(unsigned, s1[2 * i + 1]), false, false);
            red[i] = __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
        }
    }

    // Block merge of the waves: M = max_w m_w, acc = sum_w 2^(m_w - M) acc_w, same for l.
    float *wacc = smem + SM::vbuf;  // reuse: [waves][G][128]
    float *wm = smem + SM::wm;
    float *wl = smem + SM::wl;
    __syncthreads();  // all waves done with vbuf / wbuf
    {
        // level-1 result i holds accumulator 2i (lanes 0-31) and 2i+1 (lanes
        // 32-63); level 2 combined level-1 results 2i (rows 0, 2 -> rows 0, 2)
        // and 2i+1 (rows 1, 3): row k of red[i] is accumulator
        // {4i, 4i+2, 4i+1, 4i+3}[k]
        const int k = ph;
        const int sel = (k == 0) ? 0 : (k == 1) ? 2 : (k == 2) ? 1 : 3;
#pragma unroll
        for (int i = 0; i < NA / 4; ++i) {
            const int a = 4 * i + sel, h = a >> 3, j = a & 7;
            wacc[(wv * G + h) * kD + 8 * co + j] = red[i];
        }
    }
    if (lane == 0)
#pragma unroll
        for (int h = 0; h < G; ++h) {
            wm[wv * G + h] = m_run[h];
            wl[wv * G + h] = l_run[h];
        }
    __syncthreads();
    float *my = part + ((bh * n_split + split) * G) * (kD + 2);
    for (int idx = tid; idx < G * kD; idx += kDecThreads) {
        const int h = idx >> 7, i = idx & (kD - 1);
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, wm[w * G + h]);
        float A = 0.0f, L = 0.0f;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) {
            const float f = __builtin_amdgcn_exp2f(wm[w * G + h] - M);  // empty wave: 2^-inf = 0
            A = fmaf(f, wacc[(w * G + h) * kD + i], A);
            L = fmaf(f, wl[w * G + h], L);
        }
        my[h * (kD + 2) + 2 + i] = A;
        if (i == 0) {
            my[h * (kD + 2)] = M;
            my[h * (kD + 2) + 1] = L;
        }
    }

    // Arrival: the last split of (b, g) merges.  Each wave waits for its own
    // partial stores, the barrier joins the waves, and one device-scope release by thread 0 then
    // publishes them (the L2 write-back it implies is a whole-cache operation,
    // so one per block suffices) before the counter is incremented.  The last
    // block performs one device-scope acquire (L2 invalidate) before reading
    // the other blocks' partials.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores have reached L2
    __syncthreads();
    unsigned &last = *reinterpret_cast<unsigned *>(smem + SM::flag);
    if (wv == 0) {  // wave-uniform: cache write-back / invalidate act per wave
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        unsigned prev = 0;
        if (lane == 0) prev = atomicAdd(counters + bh, 1u);
        const unsigned is_last = __builtin_amdgcn_readfirstlane(prev) == (unsigned)(n_split - 1);
        if (is_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (lane == 0) last = is_last;
    }
    __syncthreads();
    if (!last) return;

    // Merge of the splits, one wave per head (the other waves are done):
    // f_s = 2^(m_s - M) / (d L) with M = max_s m_s, L = sum_s l_s 2^(m_s - M);
    // lane l accumulates coordinates 2l, 2l+1 over the splits, then the
    // inverse rotation out = D_V .* H (sum_s f_s acc_s) in the same wave.
    float *fw = smem + SM::vbuf;  // reuse: [G][n_split] merge weights
    const float *all = part + (bh * n_split) * G * (kD + 2);
    const int64_t sst = (int64_t)G * (kD + 2);  // split stride
    constexpr int kPerLane = kMaxSplits / 64;
    for (int h = wv; h < G; h += kDecWaves) {
        const float *ah = all + h * (kD + 2);
        float mv[kPerLane], lv[kPerLane];
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            const int sp = lane + 64 * k;
            mv[k] = sp < n_split ? ah[sp * sst] : -INFINITY;
            lv[k] = sp < n_split ? ah[sp * sst + 1] : 0.0f;
            M = fmaxf(M, mv[k]);
        }
        M = wave_max(M);
        float L = 0.0f;
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) L = fmaf(lv[k], __builtin_amdgcn_exp2f(mv[k] - M), L);
        L = wave_sum(L);
        const float inv = 1.0f / (L * kD);
        float *fh = fw + h * n_split;
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            const int sp = lane + 64 * k;
            if (sp < n_split) fh[sp] = __builtin_amdgcn_exp2f(mv[k] - M) * inv;
        }
        wave_lds_sync();
        const float *col = ah + 2 + 2 * lane;
        float a0 = 0.0f, a1 = 0.0f;
        int sp = 0;
        for (; sp + 16 <= n_split; sp += 16) {  // 16 independent loads in flight
            f2_t v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = *reinterpret_cast<const f2_t *>(col + (sp + u) * sst);
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                a0 = fmaf(fh[sp + u], v[u].x, a0);
                a1 = fmaf(fh[sp + u], v[u].y, a1);
            }
        }
        for (; sp < n_split; ++sp) {
            const f2_t v = *reinterpret_cast<const f2_t *>(col + sp * sst);
            a0 = fmaf(fh[sp], v.x, a0);
            a1 = fmaf(fh[sp], v.y, a1);
        }
        wave_fwht(a0, a1, lane);
        const f2_t sv = reinterpret_cast<const f2_t *>(signs_v + g * kD)[lane];
        reinterpret_cast<f2_t *>(out + ((b * Hq) + (int64_t)g * G + h) * kD)[lane] = f2_t{a0 * sv.x, a1 * sv.y};
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
    // about one block per CU, and at least 1024 tokens per block to amortise
    // the prologue
    int64_t per = (T + 1023) / 1024;
    const int64_t want = ((int64_t)ctx->n_cu + bhs - 1) / bhs;
    if (per > want) per = want;
    if (per < 1) per = 1;
    const int64_t tpb = (T + per - 1) / per;
    const int64_t blocks_per_bh = (T + tpb - 1) / tpb;
    const size_t shm = sizeof(float) * (G * kD + FD::NF * FD::E * G + (QJL ? 32 * 16 * G + G * kD : 0) + 16);
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute((const void *)k_logits<BITS, G, QJL>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        attr_set = true;
    }
    hipLaunchKernelGGL((k_logits<BITS, G, QJL>), dim3((unsigned)(bhs * blocks_per_bh)), dim3(kLgThreads), shm,
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
    // about one block (16 waves) per compute unit, and at least 1024 tokens per block
    const int64_t bhs = B * Hkv;
    int64_t ns = (256 + bhs - 1) / bhs;
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
