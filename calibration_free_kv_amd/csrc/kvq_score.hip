// Attention scores read straight from the packed codes ("TurboQuant", Como
// Funciona, Estagio 2, and Como Implementar: the query is rotated once and
// dot products are taken against the indices; QJL sign residual for unbiased
// inner products) and one decode step of attention over the quantised cache
// ("PolarQuant", Technical summary sec. 2 for the dequantisation).
//
// Both kernels rotate the G query heads of a (batch, KV head) group once,
// q' = H (D_K .* q).  The logits kernel turns them into lookup tables over
// fields of the packed key record.  A field holds the codes of F consecutive
// coordinates (F = 2 for b <= 3, F = 1 for b = 4), and entry e of field f of
// head h is sum_k q'_h[F f + k] c[code_k(e)] / d.  A key's logit is then rho
// times the sum of one table entry per field, which replaces 128
// multiply-adds per head with 128/F LDS reads that serve all G heads at once
// (the G entries of one (field, value) pair are contiguous).  The decode
// kernel instead runs its two contractions (logits over coordinates, values
// over tokens) on the matrix cores; see its own description below.
#include <atomic>
#include <mutex>

#include "kvq_internal.h"
#include "kvq_wave.h"

// Device memory of the decode entry point that allocates nothing
// (kvq_attn_decode_noalloc): arrival counters, split partials and, with the
// dense rotation, the rotated queries, laid out as in a caller's decode
// workspace.  Each device holds its own copy until the process ends.  Host
// code never passes this name to a kernel: it is a host-side stand-in, and
// the device address comes from hipGetSymbolAddress (kvq::noalloc_setup).
static __device__ __align__(256) unsigned char scratch[kvq::kNoAllocScratchBytes];

namespace kvq {
KVQ_DEBUG_UNIT(score, 2)
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


// Prologue shared by the score kernels: qr[G][128] <- H (D .* q_h) for the G
// query heads of KV head g of batch b, one wave per head; with a dense
// rotation Q (not null) instead qr <- sqrt(d) Q q_h by the whole block of NT
// threads, with (NT / 128) G 128 floats of LDS at `red`.  Ends with a
// barrier.
template <int G, int NT>
__device__ void rotate_queries(const half_t *__restrict__ q, const float *__restrict__ signs,
                               int64_t b, int g, int Hq, float *qr, const float *__restrict__ Qm, float *red)
{
    const int tid = threadIdx.x;
    const half_t *qb = q + ((int64_t)b * Hq + (int64_t)g * G) * kD;
    if (Qm) {  // uniform
        GemvSlice<NT> qs;
        gemv_load<NT>(Qm, tid, qs);  // in flight while q is staged
        for (int i = tid; i < G * kD; i += NT) qr[i] = (float)qb[i];
        __syncthreads();
        const float y = block_gemv<G, NT>(qs, qr, red, tid);  // every read of qr precedes its barrier
        if (tid < G * kD) qr[tid] = y * 11.313708498984761f;
        __syncthreads();
        return;
    }
    const int lane = tid & 63, wv = tid >> 6;
    for (int h = wv; h < G; h += NT / 64) {
        const uint32_t pr = reinterpret_cast<const uint32_t *>(qb + h * kD)[lane];
        float x0 = (float)__builtin_bit_cast(h2_t, pr).x;
        float x1 = (float)__builtin_bit_cast(h2_t, pr).y;
        const f2_t sg = reinterpret_cast<const f2_t *>(signs + g * kD)[lane];
        x0 *= sg.x;
        x1 *= sg.y;
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
    int64_t blocks_per_bh, const float *__restrict__ Qm)
{
    using FD = Fields<BITS>;
    extern __shared__ __align__(16) float smem[];
    float *qr = smem;                       // [G][128]
    float *lut = qr + G * kD;               // [NF][E][G]
    // the tables' area also holds the dense rotation's partial sums
    constexpr int LA = FD::NF * FD::E > kLgThreads ? FD::NF * FD::E : kLgThreads;
    float *slut = lut + LA * G;             // [32][16][G] (QJL)
    float *pq = slut + (QJL ? 32 * 16 * G : 0);  // [G][128] (QJL)
    float *ctab = pq + (QJL ? G * kD : 0);       // [16] centroids

    const int64_t bh = blockIdx.x / blocks_per_bh;
    const int64_t part = blockIdx.x - bh * blocks_per_bh;
    const int64_t b = bh / H;
    const int g = (int)(bh - b * H);
    const int64_t nbh = gridDim.x / blocks_per_bh;  // B H (b, g) groups
    KVQ_CHECK(gridDim.x % blocks_per_bh == 0 && nbh % H == 0 && Hq == G * H && T >= 1 &&
              tokens_per_block * blocks_per_bh >= T);
    KVQ_POISON_LDS(smem, (ctab - smem) + 16, threadIdx.x, kLgThreads);
    if (KVQ_DEBUG_ON) __syncthreads();

    stage_centroids(cb, ctab);
    rotate_queries<G, kLgThreads>(q, signs, b, g, Hq, qr, Qm, lut);
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
    KVQ_CHECK(t_begin < t_end && bh < nbh);
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
        KVQ_CHECK(t >= t_begin && t < t_end);
    }
}

// ---------------------------------------------------------------------------
// kvq_attn_decode: split-K flash decoding on the matrix cores.  Block
// (b, g, split) owns a token range of one (batch, KV head); each of its
// waves works alone on 64-token tiles of the range, and both contractions of
// a tile are 16x16x32 fp16 matrix products with fp32 accumulation:
//  K  logits^T = Q' K^T, contracted over the 128 coordinates.  Q' holds the
//     rotated, power-of-two-scaled query of each head split into an fp16
//     high part and an fp16 low part (two rows per head), and K^T the fp16
//     high and low parts of the key centroids, read from a table indexed by
//     the codes of two adjacent coordinates; the two products give the logit
//     to about 2^-22 relative.
//  V  acc = P' V, contracted over tokens.  P' holds the fp16 high and low
//     parts (two rows per head) of the weights 2^(s + log2 rho_V - mv) with
//     mv the running maximum of that exponent; V the centroid high and low
//     parts of one code each (the two parts sit at adjacent positions of the
//     contraction, against two copies of the weight).  Dividing out rho_V in
//     the exponent keeps every weight in [0, 1], so no fp16 operand can
//     overflow whatever the norms are.
// The running softmax state per head is (m, l) over 2^s and mv over the
// numerator; a wave converts its accumulator to the 2^(s - m) scale once at
// the end.  The waves of a block merge in LDS; the block writes (m, l, acc)
// for its G heads and the last block of a (b, g) to finish (arrival counter)
// merges the splits and applies the inverse rotation once:
// out_h = D_V .* H acc / (d l).
//
// Lane roles in a tile (lane = 16 kg + n):
//  logits  B operand: token 16 rg + n (rg = 0..3), coordinates 32 kg .. 32 kg
//          + 31, which are BITS consecutive dwords of the record, loaded
//          straight from memory; result rows 4 kg, 4 kg + 1 are head kg.
//  weights head kg, tokens 16 rg + n.
//  values  B operand: coordinates 8 n .. 8 n + 7 (one per product nb) of
//          tokens 16 kq + 4 kg .. + 3, from the wave's V records staged in
//          LDS transposed (dword w of token t at [w][t]); accumulator nb of
//          the lane holds rows 4 kg, 4 kg + 1 (head kg) of coordinate 8 n + nb.
// ---------------------------------------------------------------------------
constexpr int kDecWaves = 16;
constexpr int kDecThreads = kDecWaves * 64;

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

// Dynamic LDS of the decode kernel (the centroid tables are static arrays,
// whose addresses fold into the offsets of the LDS instructions).
template <int BITS, int G>
struct DecSmem {
    static constexpr int W = 4 * BITS;             // dwords per record
    static constexpr int NP = 1 << (2 * BITS);     // codes of a coordinate pair
    static constexpr int QS = 136;                 // halves per query row (padded as below)
    static constexpr int ctab = 0;                 // [16] fp32 centroids
    static constexpr int qh = ctab + 16;           // [2G + 1][QS] fp16 query rows: high, low parts; zeros
    static constexpr int qf = qh + (2 * G + 1) * QS / 2;  // [G] logit factor of each head
    static constexpr int wm = qf + 4;              // [waves][G] wave maxima
    static constexpr int wl = wm + kDecWaves * G;  // [waves][G] wave sums
    static constexpr int flag = wl + kDecWaves * G;  // [1] last-arrival flag, [1] published query heads
    // per-wave staging, from `stage` on: V records transposed [W + 1][VS]
    // (the last row is only ever read as the unused upper bits of a funnel
    // shift), then the weight operand [16 rows][PS] fp16.  The padded row
    // strides (4 banks, resp. 2 banks, past a multiple of the bank count) put
    // the rows that the lanes of one read group fetch in distinct banks.
    static constexpr int VS = 68;                  // dwords per transposed V row
    static constexpr int PS = 68;                  // halves per weight row
    static constexpr int PT = VS * (W + 1);
    static constexpr int STG = PT + 16 * PS / 2;
    static constexpr int stage = (flag + 4 + 63) / 64 * 64;
    static constexpr int total = stage + kDecWaves * STG;
    // end-of-block reuse of the staging area: per-wave accumulators, split merge
    static_assert(kDecWaves * STG >= kDecWaves * G * kD, "wave merge buffer does not fit");
    static_assert(kDecWaves * STG >= kDecWaves * (kMaxSplits + kD), "split merge buffers do not fit");
    static_assert(kDecWaves * STG >= kDecWaves * kMaxSplits + (1 + kDecThreads / kD) * G * kD,
                  "dense output rotation buffers do not fit");
};

// o[r] = x of lane 16 r + (l & 15), for r = 0..3: row r broadcast to every row.
__device__ __forceinline__ void row_broadcast(float x, float (&o)[4])
{
    const float2 h = swap32(x);   // rows (0, 1, 0, 1) and (2, 3, 2, 3)
    const float2 a = swap16(h.x), c = swap16(h.y);
    o[0] = a.x;
    o[1] = a.y;
    o[2] = c.x;
    o[3] = c.y;
}

// NB bits at bit offset O (compile time) of a window of consecutive dwords.
template <int O, int NB, int N>
__device__ __forceinline__ uint32_t window_bits(const uint32_t (&w)[N])
{
    constexpr int wd = O >> 5, sh = O & 31;
    static_assert(wd < N, "field outside the window");
    if constexpr (sh + NB <= 32) {
        return (w[wd] >> sh) & ((1u << NB) - 1u);
    } else {
        static_assert(wd + 1 < N, "field outside the window");
        return __builtin_amdgcn_alignbit(w[wd + 1], w[wd], (uint32_t)sh) & ((1u << NB) - 1u);
    }
}

// fp16 high part of x (round to nearest) and the fp16 rounding of the rest.
__device__ __forceinline__ void split_f16(float x, _Float16 &hi, _Float16 &lo)
{
    hi = (_Float16)x;
    lo = (_Float16)(x - (float)hi);
}
__device__ __forceinline__ uint32_t pack_h2(_Float16 a, _Float16 b)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// B operands of the logits for coordinates 32 kg + 8 CB .. + 7 of one token:
// the four coordinate pairs of the lane's window, high and low parts (entry e
// of the lane's copy of the pair tables at khi[KREP e], klo[KREP e]).
template <int BITS, int CB, int KREP>
__device__ __forceinline__ void key_operands(const uint32_t (&win)[BITS], const uint32_t *khi, const uint32_t *klo,
                                             u4_t &bh, u4_t &bl)
{
    constexpr uint32_t NB = 2 * BITS;
    const uint32_t e0 = window_bits<8 * BITS * CB + 0 * NB, NB>(win);
    const uint32_t e1 = window_bits<8 * BITS * CB + 1 * NB, NB>(win);
    const uint32_t e2 = window_bits<8 * BITS * CB + 2 * NB, NB>(win);
    const uint32_t e3 = window_bits<8 * BITS * CB + 3 * NB, NB>(win);
    bh = u4_t{khi[KREP * e0], khi[KREP * e1], khi[KREP * e2], khi[KREP * e3]};
    bl = u4_t{klo[KREP * e0], klo[KREP * e1], klo[KREP * e2], klo[KREP * e3]};
}

// Logit partial sums of one 16-token row group (tokens 16 rg + n) over the
// 128 coordinates: eight products, the operands of each block looked up
// while the previous block's products run.
template <int BITS, int KREP>
__device__ __forceinline__ f4_t logit_group(const uint32_t (&win)[BITS], const uint32_t *khi, const uint32_t *klo,
                                            const h8_t (&aq)[4])
{
    f4_t d = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
    u4_t h0, l0, h1, l1;
    key_operands<BITS, 0, KREP>(win, khi, klo, h0, l0);
    key_operands<BITS, 1, KREP>(win, khi, klo, h1, l1);
    __builtin_amdgcn_sched_barrier(0);
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[0], __builtin_bit_cast(h8_t, h0), d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[0], __builtin_bit_cast(h8_t, l0), d, 0, 0, 0);
    key_operands<BITS, 2, KREP>(win, khi, klo, h0, l0);
    __builtin_amdgcn_sched_barrier(0);
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[1], __builtin_bit_cast(h8_t, h1), d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[1], __builtin_bit_cast(h8_t, l1), d, 0, 0, 0);
    key_operands<BITS, 3, KREP>(win, khi, klo, h1, l1);
    __builtin_amdgcn_sched_barrier(0);
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[2], __builtin_bit_cast(h8_t, h0), d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[2], __builtin_bit_cast(h8_t, l0), d, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[3], __builtin_bit_cast(h8_t, h1), d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[3], __builtin_bit_cast(h8_t, l1), d, 0, 0, 0);
    return d;
}

// B operand of the values for coordinate 8 n + NB of the lane's four tokens.
template <int BITS, int NB>
__device__ __forceinline__ u4_t value_operand(const uint32_t (&oc)[4], const uint32_t *vtab)
{
    constexpr uint32_t cm = (1u << BITS) - 1u;
    return u4_t{vtab[(oc[0] >> (BITS * NB)) & cm], vtab[(oc[1] >> (BITS * NB)) & cm],
                vtab[(oc[2] >> (BITS * NB)) & cm], vtab[(oc[3] >> (BITS * NB)) & cm]};
}

template <int BITS, int G>
__global__ __launch_bounds__(kDecThreads) void k_decode(
    const half_t *__restrict__ q, const uint8_t *__restrict__ kc, const float *__restrict__ kn,
    const uint8_t *__restrict__ vc, const float *__restrict__ vn, const float *__restrict__ signs_k,
    const float *__restrict__ signs_v, Codebook cb, float scale_log2, float *__restrict__ out,
    float *__restrict__ part, unsigned *__restrict__ counters, int64_t T, int64_t ldt, int H, int Hq,
    int n_split, int n_part, int64_t chunk, const float *__restrict__ qrot, const float *__restrict__ Qtm)
{
    // qrot, Qtm (dense rotation, or null): the rotated queries sqrt(d) Q q,
    // [B Hq][128] fp32 computed beforehand, and Q^T; the output is rotated
    // back as sqrt(d) Q^T acc instead of with the randomized Hadamard transform.
    // T valid tokens of each (b, g) in arrays of ldt tokens per (b, g); the
    // partials of (b, g) occupy n_part slots (n_split blocks, plus one slot
    // written beforehand by the residual-window kernel when n_part > n_split)
    static_assert(G == 1 || G == 2 || G == 4, "two rows per head in one 16-row operand");
    using SM = DecSmem<BITS, G>;
    constexpr int W = SM::W;
    constexpr uint32_t cm = (1u << BITS) - 1u;
    extern __shared__ __align__(16) float smem[];
    // centroid tables, fp16 high part in the low half of a dword and low part
    // in the high half where one code is looked up; for a coordinate pair,
    // the high (khi) and low (klo) parts of both centroids.  For b <= 3 the
    // pair tables hold one copy per LDS bank (entry e of copy c at dword
    // 32 e + c) and lane l reads copy l mod 32 only, so the lanes' random
    // lookups never meet in a bank (with one copy, 2^(2b) entries over 32
    // banks cost about 2.5 conflict cycles per lookup at b = 3).  klo lies
    // KLO dwords past khi: more than 1020 bytes and not a multiple of 256
    // bytes, out of reach of the paired LDS reads (ds_read2 and its stride-64
    // form), which would return a high and a low part in adjacent registers,
    // to be moved apart again for the two products.  The 16-dword shift keeps
    // the lanes of a copy in distinct banks.
    constexpr int KREP = BITS <= 3 ? 32 : 1;
    constexpr int KLO = BITS <= 3 ? (SM::NP * KREP > 256 ? SM::NP * KREP : 256) + 16 : 260;
    static_assert(SM::NP * KREP <= KLO && KLO * 4 > 1020 && (KLO * 4) % 256 != 0, "pair table placement");
    __shared__ uint32_t ktab[KLO + SM::NP * KREP], vtab[1 << BITS];

    const int tid = threadIdx.x, lane = tid & 63;
    const uint32_t *khi = ktab + (KREP > 1 ? (lane & 31) : 0), *klo = khi + KLO;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = lane >> 4, n = lane & 15;
    uint32_t *stg = reinterpret_cast<uint32_t *>(smem + SM::stage) + wv * SM::STG;
    _Float16 *pT = reinterpret_cast<_Float16 *>(stg + SM::PT);
    const int64_t bh = blockIdx.x / n_split;
    const int split = (int)(blockIdx.x - bh * n_split);
    const int64_t b = bh / H;
    const int g = (int)(bh - b * H);

    const int64_t t_begin = (int64_t)split * chunk;
    const int64_t t_end = min(T, t_begin + chunk);
    const int64_t nbh = gridDim.x / n_split;  // B H (b, g) groups
    KVQ_CHECK(n_split >= 1 && n_split <= kMaxSplits && gridDim.x % n_split == 0 && nbh % H == 0 && Hq == G * H &&
              T <= ldt && n_part >= n_split && n_part <= kMaxSplits && t_begin < t_end && bh < nbh);
    KVQ_POISON_LDS(smem, SM::total, tid, kDecThreads);
    KVQ_POISON_LDS(ktab, KLO + SM::NP * KREP, tid, kDecThreads);
    KVQ_POISON_LDS(vtab, 1 << BITS, tid, kDecThreads);
    if (KVQ_DEBUG_ON) __syncthreads();
    // The prologue holds no block barrier once loads are in flight: a barrier
    // would hold every wave until the last one had issued its record loads,
    // i.e. until the memory system had accepted the whole block's tiles.
    // Wave h < G rotates query head h and publishes it in LDS with a count;
    // the other waves issue their loads and then wait for the count.  The
    // count is cleared behind the one barrier at the start, which also puts
    // the block's query loads ahead of all of its record loads (lane l loads
    // coordinates 2l, 2l+1 of head wv).
    unsigned *ready = reinterpret_cast<unsigned *>(smem + SM::flag) + 1;
    uint32_t qv = 0u;
    f2_t qs = f2_t{0.0f, 0.0f};
    if (wv < G) {
        qv = reinterpret_cast<const uint32_t *>(q + ((int64_t)b * Hq + (int64_t)g * G + wv) * kD)[lane];
        qs = reinterpret_cast<const f2_t *>(signs_k + g * kD)[lane];
    }
    if (tid == 0) *ready = 0u;
    // The pair tables, all copies, before the barrier (the centroids are
    // kernel arguments at constant offsets: scalar loads; a lane picks its
    // two with selects rather than an indexed copy of the argument).
    for (int i = tid; i < SM::NP * KREP; i += kDecThreads) {
        const int e = i / KREP;
        float ca = cb.c[0], cb2 = cb.c[0];
#pragma unroll
        for (int k = 1; k < (1 << BITS); ++k) {
            ca = (e & (int)cm) == k ? cb.c[k] : ca;
            cb2 = (e >> BITS) == k ? cb.c[k] : cb2;
        }
        _Float16 ha, la, hb, lb;
        split_f16(ca, ha, la);
        split_f16(cb2, hb, lb);
        ktab[i] = pack_h2(ha, hb);
        ktab[KLO + i] = pack_h2(la, lb);
    }
    __syncthreads();
    // The records of the wave's next tile are held in registers.  For the
    // first tile the keys of its first two 16-token groups (and the key
    // norms) are loaded before the prologue, the other keys and the values
    // once the queries are published: the launch's first burst of loads is
    // then a quarter as large, and the query loads queued behind it return
    // sooner (18.9 us per launch on the 8 x 32768-token layer, against 19.8
    // with every record loaded first, 19.1 with all keys first and 19.2 with
    // one group first).  For the other
    // tiles, the keys once the current logits are formed and the values once
    // the current value products are issued, so that only one of the two is
    // in flight during each phase.  Every lane loads (tokens past the end re-read the last one
    // of the range), so the loads carry no lane-dependent branch.  Keys: the
    // lane's window (BITS dwords) of the records of tokens 16 rg + n, and
    // rho_K of token `lane`; values and rho_V: token `lane`.
    uint32_t Kw[4][BITS], Vw[W];
    float rk = 0.0f, rv = 0.0f;
    // Addresses: a wave-uniform 64-bit base for the tile plus a 32-bit lane
    // offset (scalar-base loads).
    // t0 < t_end; `last` = min(63, t_end - 1 - t0), the tile's last valid
    // token (32-bit scalar arithmetic: the scalar unit has no 64-bit compare).
    auto tile_last = [&](int64_t t0) { return (uint32_t)min((int)(t_end - t0) - 1, 63); };
    // keys of the 16-token groups rg0 .. rg1 - 1 (and, with norm, rho_K)
    auto fetch_k = [&](int64_t t0, uint32_t last, int rg0 = 0, int rg1 = 4, bool norm = true) {
        KVQ_CHECK(t0 >= t_begin && t0 + (int64_t)last < t_end && last < 64);
        const int64_t v0 = bh * ldt + t0;
        const uint32_t l = min((uint32_t)lane, last);
        const char *kb = reinterpret_cast<const char *>(kc) + v0 * (16 * BITS);
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            if (rg < rg0 || rg >= rg1) continue;
            const uint32_t t = min((uint32_t)(16 * rg + n), last);
            // opaque, so that the lane part stays out of the (scalar) base
            uint32_t off = t * (16u * BITS) + 4u * BITS * kg;
            asm volatile("" : "+v"(off));
            const uint32_t *src = reinterpret_cast<const uint32_t *>(kb + off);
#pragma unroll
            for (int i = 0; i < BITS; ++i) Kw[rg][i] = src[i];
        }
        if (norm) rk = *reinterpret_cast<const float *>(reinterpret_cast<const char *>(kn + v0) + 4 * l);
    };
    auto fetch_v = [&](int64_t t0, uint32_t last) {
        KVQ_CHECK(t0 >= t_begin && t0 + (int64_t)last < t_end && last < 64);
        const int64_t v0 = bh * ldt + t0;
        const uint32_t l = min((uint32_t)lane, last);
        const u4_t *vs = reinterpret_cast<const u4_t *>(reinterpret_cast<const char *>(vc) + v0 * (16 * BITS) +
                                                          l * (16u * BITS));
#pragma unroll
        for (int k = 0; k < BITS; ++k) {
            const u4_t y = vs[k];
            Vw[4 * k] = y.x;
            Vw[4 * k + 1] = y.y;
            Vw[4 * k + 2] = y.z;
            Vw[4 * k + 3] = y.w;
        }
        rv = *reinterpret_cast<const float *>(reinterpret_cast<const char *>(vn + v0) + 4 * l);
    };
    constexpr int64_t kStride = (int64_t)kDecWaves * 64;
    __builtin_amdgcn_sched_barrier(0);  // keep the prologue's loads ahead of the records
    {
        // a wave without a tile loads the range's last token
        const int64_t t0 = t_begin + min(wv * 64, (int)(t_end - t_begin) - 1);
        fetch_k(t0, tile_last(t0), 0, 2, true);
    }

    float *ctab = smem + SM::ctab;
    float *qf = smem + SM::qf;
    _Float16 *qh = reinterpret_cast<_Float16 *>(smem + SM::qh);
    // value table: every wave writes the same values and reads back its own
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < (1 << BITS); ++k) ctab[k] = cb.c[k];
    }
    // rows of the weight operand that no head writes stay zero
    for (int i = lane; i < 8 * SM::PS; i += 64) stg[SM::PT + i] = 0u;
    if (wv == 0) reinterpret_cast<uint32_t *>(qh + 2 * G * SM::QS)[lane] = 0u;  // the zero query row
    wave_lds_sync();
    if (lane < (1 << BITS)) {
        _Float16 h, l;
        split_f16(ctab[lane], h, l);
        vtab[lane] = pack_h2(h, l);
    }
    if (wv < G) {
        // q'_h = H (D_K .* q_h), scaled by a power of two that puts its
        // largest entry in [2^14, 2^15): inside the fp16 range, with full
        // precision for the high and low parts (rows 2h and 2h + 1 of qh).
        // The logit factor undoes the scale.
        float x0 = (float)__builtin_bit_cast(h2_t, qv).x;
        float x1 = (float)__builtin_bit_cast(h2_t, qv).y;
        if (qrot) {
            const f2_t r = reinterpret_cast<const f2_t *>(qrot + ((int64_t)b * Hq + (int64_t)g * G + wv) * kD)[lane];
            x0 = r.x;
            x1 = r.y;
        } else {
            x0 *= qs.x;
            x1 *= qs.y;
            wave_fwht(x0, x1, lane);
        }
        const float amax = wave_max(fmaxf(__builtin_fabsf(x0), __builtin_fabsf(x1)));
        const int e = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) : 0;
        const float sc = __builtin_ldexpf(1.0f, 15 - e);
        _Float16 h0, l0, h1, l1;
        split_f16(x0 * sc, h0, l0);
        split_f16(x1 * sc, h1, l1);
        reinterpret_cast<uint32_t *>(qh + (2 * wv) * SM::QS)[lane] = pack_h2(h0, h1);
        reinterpret_cast<uint32_t *>(qh + (2 * wv + 1) * SM::QS)[lane] = pack_h2(l0, l1);
        if (lane == 0) qf[wv] = scale_log2 / ((float)kD * sc);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        if (lane == 0) __hip_atomic_fetch_add(ready, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    // wait until the G heads are published (the zero row was written by wave
    // 0 before its own count, or is this wave's own write)
    while (__hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < (unsigned)G)
        __builtin_amdgcn_s_sleep(1);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    {
        const int64_t t0 = t_begin + min(wv * 64, (int)(t_end - t_begin) - 1);
        fetch_k(t0, tile_last(t0), 2, 4, false);
        fetch_v(t0, tile_last(t0));
    }
    // A operand of the logits: row n is part (n & 3) of head n >> 2 (0: high,
    // 1: low, 2 and 3: zero), coordinates 32 kg + 8 cb + j.
    h8_t aq[4];
    {
        const int ah = n >> 2, ap = n & 3;
        const int row = ah < G && ap < 2 ? 2 * ah + ap : 2 * G;
        const h8_t *src = reinterpret_cast<const h8_t *>(qh + row * SM::QS + 32 * kg);
#pragma unroll
        for (int c = 0; c < 4; ++c) aq[c] = src[c];
    }
    const float fq = kg < G ? qf[kg] : 0.0f;

    float m_run = -INFINITY, l_run = 0.0f, mv_run = -INFINITY;
    f4_t acc[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[nb] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int obit = 8 * BITS * n, ow = obit >> 5, osh = obit & 31;

    // token positions relative to the range start, in 32-bit scalar registers
    const int span = (int)(t_end - t_begin);
    for (int rel = wv * 64; rel < span; rel += (int)kStride) {
        const int nt = min(64, span - rel);
        const bool more = rel + (int)kStride < span;
        // start of the next tile, opaque so that the whole of it stays in the
        // scalar base of the loads rather than in the lane offsets
        int64_t tn = t_begin + rel + kStride;
        asm volatile("" : "+s"(tn));
        const uint32_t lastn = (uint32_t)min(span - rel - (int)kStride - 1, 63);
        // logits of tokens 16 rg + n for head kg (rows 4 kg, 4 kg + 1)
        float s[4];
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const f4_t d = logit_group<BITS, KREP>(Kw[rg], khi, klo, aq);
            s[rg] = d[0] + d[1];
        }
        float rkb[4], lvb[4];
        row_broadcast(rk, rkb);
        row_broadcast(__builtin_amdgcn_logf(rv), lvb);  // log2 rho_V; -inf for a zero vector
        if (more) fetch_k(tn, lastn);  // this tile's keys are consumed
        // stage the V records transposed: dword w of token `lane` at [w][lane]
#pragma unroll
        for (int w = 0; w < W; ++w) stg[SM::VS * w + lane] = Vw[w];
        // online softmax of head kg over the 16 lanes of its row
        float sv[4], mt = -INFINITY, mvt = -INFINITY;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            s[rg] = 16 * rg + n < nt ? s[rg] * (fq * rkb[rg]) : -INFINITY;
            sv[rg] = s[rg] + lvb[rg];
            mt = fmaxf(mt, s[rg]);
            mvt = fmaxf(mvt, sv[rg]);
        }
        const float mn = fmaxf(m_run, row_max(mt));  // finite: token 0 of the tile is valid
        const float mvn = fmaxf(mv_run, row_max(mvt));
        const float mvs = mvn == -INFINITY ? 0.0f : mvn;  // all numerators zero so far
        const float alpha = __builtin_amdgcn_exp2f(m_run - mn);    // 0 on the first tile
        const float beta = __builtin_amdgcn_exp2f(mv_run - mvs);
        float ps = 0.0f;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            ps += __builtin_amdgcn_exp2f(s[rg] - mn);
            const float pv = __builtin_amdgcn_exp2f(sv[rg] - mvs);  // in [0, 1]
            _Float16 hi, lo;
            split_f16(pv, hi, lo);
            pT[(4 * kg) * SM::PS + 16 * rg + n] = hi;
            pT[(4 * kg + 1) * SM::PS + 16 * rg + n] = lo;
        }
        l_run = l_run * alpha + row_sum(ps);
        m_run = mn;
        mv_run = mvn;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
            acc[nb][0] *= beta;
            acc[nb][1] *= beta;
        }
        wave_lds_sync();
        // values: acc += P' V over the tile's four 16-token groups
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
            const int tb = 16 * kq + 4 * kg;
            const u2_t pp = *reinterpret_cast<const u2_t *>(pT + n * SM::PS + tb);
            const u4_t a = u4_t{__builtin_amdgcn_perm(pp.x, pp.x, 0x01000100u), __builtin_amdgcn_perm(pp.x, pp.x, 0x03020302u),
                                __builtin_amdgcn_perm(pp.y, pp.y, 0x01000100u), __builtin_amdgcn_perm(pp.y, pp.y, 0x03020302u)};
            const u4_t x = *reinterpret_cast<const u4_t *>(stg + SM::VS * ow + tb);
            uint32_t oc[4];
            if constexpr (BITS == 3) {  // octets straddle dwords
                const u4_t y = *reinterpret_cast<const u4_t *>(stg + SM::VS * (ow + 1) + tb);
                oc[0] = __builtin_amdgcn_alignbit(y.x, x.x, (uint32_t)osh);
                oc[1] = __builtin_amdgcn_alignbit(y.y, x.y, (uint32_t)osh);
                oc[2] = __builtin_amdgcn_alignbit(y.z, x.z, (uint32_t)osh);
                oc[3] = __builtin_amdgcn_alignbit(y.w, x.w, (uint32_t)osh);
            } else {
                oc[0] = x.x >> osh;
                oc[1] = x.y >> osh;
                oc[2] = x.z >> osh;
                oc[3] = x.w >> osh;
            }
            // each product's operand is looked up while the previous one runs
            const h8_t ah = __builtin_bit_cast(h8_t, a);
            u4_t b0 = value_operand<BITS, 0>(oc, vtab), b1;
#define KVQ_VSTEP(NB, CUR, NXT)                                                              \
    if constexpr (NB < 7) NXT = value_operand<BITS, (NB < 7 ? NB + 1 : 7)>(oc, vtab);       \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    acc[NB] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, __builtin_bit_cast(h8_t, CUR), acc[NB], 0, 0, 0);
            KVQ_VSTEP(0, b0, b1)
            KVQ_VSTEP(1, b1, b0)
            KVQ_VSTEP(2, b0, b1)
            KVQ_VSTEP(3, b1, b0)
            KVQ_VSTEP(4, b0, b1)
            KVQ_VSTEP(5, b1, b0)
            KVQ_VSTEP(6, b0, b1)
            KVQ_VSTEP(7, b1, b0)
#undef KVQ_VSTEP
        }
        if (more) fetch_v(tn, lastn);
        wave_lds_sync();  // the staging area is rewritten by the next tile
    }

    // Block merge of the waves: the wave's accumulator in the 2^(s - m)
    // scale, then M = max_w m_w, acc = sum_w 2^(m_w - M) acc_w, same for l.
    float *wacc = smem + SM::stage;  // reuse: [waves][G][128]
    float *wm = smem + SM::wm;
    float *wl = smem + SM::wl;
    const float fv = mv_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mv_run - m_run);
    __syncthreads();  // all waves done with their staging areas
    if (kg < G) {
        float r[8];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) r[nb] = (acc[nb][0] + acc[nb][1]) * fv;
        f4_t *dst = reinterpret_cast<f4_t *>(wacc + (wv * G + kg) * kD + 8 * n);
        dst[0] = f4_t{r[0], r[1], r[2], r[3]};
        dst[1] = f4_t{r[4], r[5], r[6], r[7]};
        if (n == 0) {
            wm[wv * G + kg] = m_run;
            wl[wv * G + kg] = l_run;
        }
    }
    __syncthreads();
    // Hand-over of the split partials to the last block of (b, g): every
    // thread's partial stores happen before the block barrier, the barrier
    // before wave 0's arrival count, which releases them at device scope;
    // the count's read in the last block is followed by a device-scope
    // acquire fence, and that block's other waves follow it through a
    // barrier.  The partials themselves are device-scope stores and loads
    // (written through to the coherence point).
    auto st_dev = [](float *p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    float *my = part + ((bh * n_part + split) * G) * (kD + 2);
    KVQ_CHECK(split < n_split && (bh * n_part + split) < nbh * n_part);
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
        st_dev(my + h * (kD + 2) + 2 + i, A);
        if (i == 0) {
            st_dev(my + h * (kD + 2), M);
            st_dev(my + h * (kD + 2) + 1, L);
        }
    }

    // Arrival: the last split of (b, g) to finish merges.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's partial stores are complete
    __syncthreads();
    unsigned &last = *reinterpret_cast<unsigned *>(smem + SM::flag);
    if (wv == 0) {
        unsigned prev = 0;
        if (lane == 0) prev = __hip_atomic_fetch_add(counters + bh, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned is_last = __builtin_amdgcn_readfirstlane(prev) == (unsigned)(n_split - 1);
        // only the last block acquires (a device-scope acquire invalidates
        // the caches, which would cost every other block its cached records)
        if (is_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (lane == 0) last = is_last;
    }
    __syncthreads();
    if (!last) return;
    GemvSlice<kDecThreads> qts;  // dense rotation: Q^T's slices in flight during the merge
    if (Qtm) gemv_load<kDecThreads>(Qtm, tid, qts);

    // Merge of the splits: f_s = 2^(m_s - M) / (d L) with M = max_s m_s,
    // L = sum_s l_s 2^(m_s - M), acc = sum_s f_s acc_s, then the inverse
    // rotation out = D_V .* H acc.  The kDecWaves / G waves of head h = w % G
    // each take every (kDecWaves / G)-th split (lane l: coordinates 2l, 2l+1)
    // and one of them sums their partial sums and rotates.
    auto ld_dev = [](const float *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    auto ld_dev2 = [](const float *p) {  // two floats at an 8-byte aligned address
        return __builtin_bit_cast(f2_t, __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT));
    };
    constexpr int WPH = kDecWaves / G;                   // waves per head
    constexpr int kPerLane = kMaxSplits / 64;
    const int mh = wv % G, mj = wv / G;
    float *fh = smem + SM::stage + wv * kMaxSplits;       // reuse: this wave's merge weights [n_split]
    float *pacc = smem + SM::stage + kDecWaves * kMaxSplits;  // [waves][128] partial sums
    const float *ah = part + (bh * n_part) * G * (kD + 2) + mh * (kD + 2);
    const int64_t sst = (int64_t)G * (kD + 2);  // split stride
    {
        float mv[kPerLane], lv[kPerLane];
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            const int sp = lane + 64 * k;
            mv[k] = sp < n_part ? ld_dev(ah + sp * sst) : -INFINITY;
            lv[k] = sp < n_part ? ld_dev(ah + sp * sst + 1) : 0.0f;
            M = fmaxf(M, mv[k]);
        }
        M = wave_max(M);
        float L = 0.0f;
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) L = fmaf(lv[k], __builtin_amdgcn_exp2f(mv[k] - M), L);
        L = wave_sum(L);
        const float inv = 1.0f / (L * kD);
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            const int sp = lane + 64 * k;
            if (sp < n_part) fh[sp] = __builtin_amdgcn_exp2f(mv[k] - M) * inv;
        }
        wave_lds_sync();
        const float *col = ah + 2 + 2 * lane;
        float a0 = 0.0f, a1 = 0.0f;
        int sp = mj;
        for (; sp + 7 * WPH < n_part; sp += 8 * WPH) {  // 8 independent loads in flight
            f2_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = ld_dev2(col + (sp + u * WPH) * sst);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                a0 = fmaf(fh[sp + u * WPH], v[u].x, a0);
                a1 = fmaf(fh[sp + u * WPH], v[u].y, a1);
            }
        }
        for (; sp < n_part; sp += WPH) {
            const f2_t v = ld_dev2(col + sp * sst);
            a0 = fmaf(fh[sp], v.x, a0);
            a1 = fmaf(fh[sp], v.y, a1);
        }
        reinterpret_cast<f2_t *>(pacc + wv * kD)[lane] = f2_t{a0, a1};
    }
    __syncthreads();
    if (mj == 0) {
        float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int j = 0; j < WPH; ++j) {
            const f2_t v = reinterpret_cast<const f2_t *>(pacc + (j * G + mh) * kD)[lane];
            a0 += v.x;
            a1 += v.y;
        }
        if (Qtm) {  // acc of head mh into slot mh (wave mh = this wave), rotated below
            reinterpret_cast<f2_t *>(pacc + wv * kD)[lane] = f2_t{a0, a1};
        } else {
            wave_fwht(a0, a1, lane);
            const f2_t sv = reinterpret_cast<const f2_t *>(signs_v + g * kD)[lane];
            reinterpret_cast<f2_t *>(out + ((b * Hq) + (int64_t)g * G + mh) * kD)[lane] = f2_t{a0 * sv.x, a1 * sv.y};
        }
    }
    if (Qtm) {  // out = sqrt(d) Q^T acc for the G heads, by the whole block
        __syncthreads();
        const float y = block_gemv<G, kDecThreads>(qts, pacc, pacc + G * kD, tid);
        if (tid < G * kD) out[((b * Hq) + (int64_t)g * G + (tid >> 7)) * kD + (tid & 127)] = y * 11.313708498984761f;
    }
    if (tid == 0)  // leave the counter ready for the next call
        __hip_atomic_store(counters + bh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Large dynamic LDS must be allowed per kernel and device, once: a bit per
// device (the current one) records that it was done.  Concurrent first calls
// may both set it, which is harmless.
inline bool need_attr(const std::atomic<uint64_t> &mask)
{
    int dev = 0;
    (void)hipGetDevice(&dev);
    return dev >= 64 || !(mask.load(std::memory_order_acquire) & (1ull << dev));
}

inline void mark_attr(std::atomic<uint64_t> &mask)
{
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev < 64) mask.fetch_or(1ull << dev, std::memory_order_release);
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
    constexpr int LA = FD::NF * FD::E > kLgThreads ? FD::NF * FD::E : kLgThreads;  // tables or rotation sums
    const size_t shm = sizeof(float) * (G * kD + LA * G + (QJL ? 32 * 16 * G + G * kD : 0) + 16);
    static std::atomic<uint64_t> attr_set{0};  // one bit per device that has the attribute
    if (need_attr(attr_set)) {
        (void)hipFuncSetAttribute((const void *)k_logits<BITS, G, QJL>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        mark_attr(attr_set);
    }
    hipLaunchKernelGGL((k_logits<BITS, G, QJL>), dim3((unsigned)(bhs * blocks_per_bh)), dim3(kLgThreads), shm,
                       s, (const half_t *)q, codes, norms, (const uint32_t *)qjl_signs, qjl_gamma,
                       ctx->d_signs, ctx->d_S, ctx->cb, logits, T, ctx->H, (int)Hq, tpb, blocks_per_bh,
                       ctx->rotation == KVQ_ROTATION_DENSE ? ctx->d_Q : nullptr);
    return hipGetLastError();
}

// Residual window of a streaming cache: the partial (m, l, acc) of its R
// full-precision tokens for the G query heads of (b, g), in the convention of
// the decode partials (base-2 scores s = scale_log2 <q, k>, acc in the
// rotated domain: H (D_V .* sum_t 2^(s_t - m) v_t)), written to slot n_split
// of the (b, g) partials; with no quantised tokens (direct) it writes the
// output itself, sum_t 2^(s_t - m) v_t / l.  One wave per query head.
template <int G>
__global__ __launch_bounds__(64 * G) void k_tail(const half_t *__restrict__ q, const half_t *__restrict__ kt,
                                                 const half_t *__restrict__ vt, const float *__restrict__ signs_v,
                                                 float scale_log2, float *__restrict__ part, float *__restrict__ out,
                                                 int64_t R, int64_t R_cap, int H, int Hq, int n_part, int n_split,
                                                 bool direct)
{
    __shared__ __align__(16) float qf[G][kD];
    const int lane = threadIdx.x & 63, h = threadIdx.x >> 6;
    const int64_t bh = blockIdx.x, b = bh / H;
    const int g = (int)(bh - b * H);
    const int64_t qrow = b * Hq + (int64_t)g * G + h;
    const WindowPartial w = window_partial(qf[h], kt + bh * R_cap * kD, vt + bh * R_cap * kD, R, scale_log2, lane, [&] {
        const h2_t pr = reinterpret_cast<const h2_t *>(q + qrow * kD)[lane];
        reinterpret_cast<f2_t *>(qf[h])[lane] = f2_t{(float)pr.x, (float)pr.y};
    });
    if (direct) {
        const float inv = 1.0f / w.l;
        reinterpret_cast<f2_t *>(out + qrow * kD)[lane] = f2_t{w.a0 * inv, w.a1 * inv};
        return;
    }
    const f2_t sv = reinterpret_cast<const f2_t *>(signs_v + g * kD)[lane];
    float x0 = w.a0 * sv.x, x1 = w.a1 * sv.y;
    wave_fwht(x0, x1, lane);
    float *dst = part + ((bh * n_part + n_split) * G + h) * (kD + 2);
    reinterpret_cast<f2_t *>(dst + 2)[lane] = f2_t{x0, x1};
    if (lane == 0) {
        dst[0] = w.m;
        dst[1] = w.l;
    }
}

constexpr int kRotWaves = 8, kRotHeads = 1;

// Rotated queries of the dense rotation, sqrt(d) Q q for each of `heads`
// fp16 query vectors, kRotHeads per block (Q read once per block, every
// thread's share of it in flight at once).
__global__ __launch_bounds__(64 * kRotWaves) void k_rotate_dense(const half_t *__restrict__ q,
                                                                 const float *__restrict__ Qm,
                                                                 float *__restrict__ qrot, int64_t heads)
{
    __shared__ __align__(16) float qv[kRotHeads][kD];
    __shared__ __align__(16) float part[64 * kRotWaves / kD][kRotHeads][kD];
    const int tid = threadIdx.x;
    const int64_t h0 = (int64_t)blockIdx.x * kRotHeads;
    GemvSlice<64 * kRotWaves> qs;
    gemv_load<64 * kRotWaves>(Qm, tid, qs);  // in flight while the queries are staged
    for (int i = tid; i < kRotHeads * kD; i += 64 * kRotWaves) {
        const int64_t h = h0 + i / kD;
        qv[i / kD][i % kD] = h < heads ? (float)q[h * kD + i % kD] : 0.0f;
    }
    __syncthreads();
    const float y = block_gemv<kRotHeads, 64 * kRotWaves>(qs, &qv[0][0], &part[0][0][0], tid);
    const int64_t h = h0 + tid / kD;
    if (tid < kRotHeads * kD && h < heads) qrot[h * kD + tid % kD] = y * 11.313708498984761f;
}

// ws: arrival counters (cbytes), then the split partials of `slots` slots per
// (batch, query head), then (dense rotation) the rotated queries.
template <int BITS, int G>
hipError_t run_decode(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T, int64_t ldt,
                      const uint8_t *kc, const float *kn, const uint8_t *vc, const float *vn, const DecodeTail *tail,
                      float sm_scale, float *out, void *ws, int n_split, int64_t slots, size_t cbytes, hipStream_t s)
{
    using SM = DecSmem<BITS, G>;
    const int64_t bhs = B * ctx->H;
    const float scale_log2 = sm_scale * 1.4426950408889634f;
    unsigned *counters = (unsigned *)ws;
    float *part = (float *)((char *)ws + cbytes);
    int n_part = 0;
    int64_t chunk = 0;
    if (T > 0) {
        chunk = (T + n_split - 1) / n_split;
        n_split = (int)((T + chunk - 1) / chunk);  // no empty split
        n_part = n_split + (tail ? 1 : 0);
    }
    if (tail) {
        hipLaunchKernelGGL((k_tail<G>), dim3((unsigned)bhs), dim3(64 * G), 0, s, (const half_t *)q,
                           (const half_t *)tail->k, (const half_t *)tail->v, ctx->d_signs + ctx->H * kD, scale_log2,
                           part, out, tail->R, tail->R_cap, ctx->H, (int)Hq, n_part, n_split, T == 0);
        if (T == 0) return hipGetLastError();
    }
    const size_t shm = sizeof(float) * SM::total;
    static std::atomic<uint64_t> attr_set{0};  // one bit per device that has the attribute
    if (need_attr(attr_set)) {
        (void)hipFuncSetAttribute((const void *)k_decode<BITS, G>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)shm);
        mark_attr(attr_set);
    }
    const bool dense = ctx->rotation == KVQ_ROTATION_DENSE;
    float *qrot = nullptr;
    if (dense) {  // after the partials
        qrot = part + (size_t)(B * Hq) * (size_t)slots * (kD + 2);
        const int64_t heads = B * Hq;
        hipLaunchKernelGGL(k_rotate_dense, dim3((unsigned)((heads + kRotHeads - 1) / kRotHeads)),
                           dim3(64 * kRotWaves), 0, s, (const half_t *)q, ctx->d_Q, qrot, heads);
    }
    hipLaunchKernelGGL((k_decode<BITS, G>), dim3((unsigned)(bhs * n_split)), dim3(kDecThreads), shm, s,
                       (const half_t *)q, kc, kn, vc, vn, ctx->d_signs, ctx->d_signs + ctx->H * kD, ctx->cb,
                       scale_log2, out, part, counters, T, ldt, ctx->H, (int)Hq, n_split, n_part, chunk, qrot,
                       dense ? ctx->d_Qt : nullptr);
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
hipError_t dispatch_decode(const kvq_ctx *ctx, int G, const void *q, int64_t B, int64_t Hq, int64_t T, int64_t ldt,
                           const uint8_t *kc, const float *kn, const uint8_t *vc, const float *vn,
                           const DecodeTail *tail, float sm, float *out, void *ws, int ns, int64_t slots,
                           size_t cb, hipStream_t s)
{
    switch (G) {
    case 1: return run_decode<BITS, 1>(ctx, q, B, Hq, T, ldt, kc, kn, vc, vn, tail, sm, out, ws, ns, slots, cb, s);
    case 2: return run_decode<BITS, 2>(ctx, q, B, Hq, T, ldt, kc, kn, vc, vn, tail, sm, out, ws, ns, slots, cb, s);
    case 4: return run_decode<BITS, 4>(ctx, q, B, Hq, T, ldt, kc, kn, vc, vn, tail, sm, out, ws, ns, slots, cb, s);
    }
    return hipErrorNotSupported;
}

__global__ void k_zero_u32(uint32_t *p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// Device addresses of `scratch`, one per device, found once.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];

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

namespace {
hipError_t decode_bits(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T, int64_t ldt,
                       const uint8_t *kc, const float *kn, const uint8_t *vc, const float *vn, const DecodeTail *tail,
                       float sm, float *out, void *ws, int ns, int64_t slots, size_t cb, hipStream_t s)
{
    const int G = (int)(Hq / ctx->H);
    switch (ctx->bits) {
    case 1: return dispatch_decode<1>(ctx, G, q, B, Hq, T, ldt, kc, kn, vc, vn, tail, sm, out, ws, ns, slots, cb, s);
    case 2: return dispatch_decode<2>(ctx, G, q, B, Hq, T, ldt, kc, kn, vc, vn, tail, sm, out, ws, ns, slots, cb, s);
    case 3: return dispatch_decode<3>(ctx, G, q, B, Hq, T, ldt, kc, kn, vc, vn, tail, sm, out, ws, ns, slots, cb, s);
    case 4: return dispatch_decode<4>(ctx, G, q, B, Hq, T, ldt, kc, kn, vc, vn, tail, sm, out, ws, ns, slots, cb, s);
    }
    return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_decode(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                         const uint8_t *kc, const float *kn, const uint8_t *vc, const float *vn,
                         float sm_scale, float *out, void *ws, int n_split, hipStream_t s)
{
    return decode_bits(ctx, q, B, Hq, T, T, kc, kn, vc, vn, nullptr, sm_scale, out, ws, n_split,
                       decode_max_splits(T), decode_count_bytes(B * ctx->H), s);
}

hipError_t launch_decode_stream(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T, int64_t ldt,
                                const uint8_t *kc, const float *kn, const uint8_t *vc, const float *vn,
                                const DecodeTail *tail, float sm_scale, float *out, void *ws, int n_split,
                                hipStream_t s)
{
    // no dense rotation here, so nothing follows the partials
    return decode_bits(ctx, q, B, Hq, T, ldt, kc, kn, vc, vn, tail, sm_scale, out, ws, n_split, 0,
                       decode_count_bytes(B * ctx->H), s);
}

hipError_t noalloc_setup(int device)
{
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[device]) return hipSuccess;
    void *p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // the arrival counters start at zero (every completed call leaves them so)
    hipLaunchKernelGGL(k_zero_u32, dim3(256), dim3(256), 0, nullptr, (uint32_t *)p,
                       (int64_t)(kNoAllocScratchBytes / sizeof(uint32_t)));
    e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
    if (e != hipSuccess) return e;
    g_scratch[device] = p;
    return hipSuccess;
}

hipError_t launch_decode_noalloc(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                                 const uint8_t *kc, const float *kn, const uint8_t *vc, const float *vn,
                                 float sm_scale, float *out, int n_split, hipStream_t s)
{
    void *p = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (ctx->device >= 0 && ctx->device < kMaxDevices) p = g_scratch[ctx->device];
    }
    if (!p) return hipErrorNotInitialized;  // kvq_create sets it up
    return decode_bits(ctx, q, B, Hq, T, T, kc, kn, vc, vn, nullptr, sm_scale, out, p, n_split, n_split,
                       kNoAllocCountBytes, s);
}

}  // namespace kvq
