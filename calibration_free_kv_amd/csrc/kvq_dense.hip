// Quantisation with a dense orthogonal rotation ("O Que E TurboQuant?", Como
// Funciona, Estagio 1: a random orthogonal transformation from the QR
// decomposition of a Gaussian matrix, then Lloyd-Max buckets per coordinate).
// The rotation is scaled like the Hadamard path so that coordinates have unit
// variance: y = sqrt(d) Q x / ||x||, index = #{thresholds < y}, codes packed
// LSB-first, rho = ||x|| kept.  One Q serves every head, so the B H T vectors
// of a call form one list.
//
// The rotation is a dense contraction and runs on the matrix cores:
// v_mfma_f32_16x16x32_f16 with A = 16 rows of Q (as its fp16 high and low
// parts: two products, so Q enters to about 2^-22) and B = 32 inputs x 16
// vectors (the fp16 inputs themselves, exact), fp32 accumulation.  A wave
// takes 64 vectors at a time (four B tiles share every A tile read from
// LDS, where Q's rows are padded to 272 bytes so that the 16 rows one read
// touches fall in distinct banks).  Q's rows sit in LDS in an order chosen
// so that the accumulator registers of a lane hold 8 consecutive output
// coordinates of one vector, 32 j + 8 kg .. + 7 for j = 0..3 (kg = lane / 16):
// their indices form one 8 b-bit piece of the record, assembled in registers
// and written to the vector's LDS row at byte b (4 j + kg).  The norm comes
// from the B registers (packed fp16 dot products and two lane swaps) and is
// folded into the thresholds (t rho / sqrt(d) against Q x); the bucket is the
// antisymmetric binary search over the positive thresholds.  Records leave
// with lane = vector as 16-byte stores.  Eight waves share one copy of Q.
#include "kvq_internal.h"
#include "kvq_wave.h"

namespace kvq {
KVQ_DEBUG_UNIT(dense, 5)
namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

constexpr int kDenseWaves = 8;
constexpr int kQRow = kD + 8;   // padded row of Q in LDS, in halves

struct PosThresholds {
    float p[8];  // t_{L/2} .. t_{L-2}: the positive thresholds of the antisymmetric table
};

// idx = #{j : t_j < y} for the antisymmetric table (t_{L/2-1} = 0): with
// a = |y| and h = #{k : a > p_k}, idx = L/2 + h if y > 0, else L/2 - 1 - h
// (an exact tie at a negative threshold lands one cell up; such a coordinate
// lies inside any decision band).
template <int BITS>
__device__ __forceinline__ uint32_t bucket_idx(float y, const float *p)
{
    constexpr uint32_t half = 1u << (BITS - 1);
    const float a = __builtin_fabsf(y);
    uint32_t h = 0;
    if constexpr (BITS == 2) {
        h = a > p[0];
    } else if constexpr (BITS == 3) {
        const bool c1 = a > p[1];
        const bool c2 = a > (c1 ? p[2] : p[0]);
        h = 2u * c1 + c2;
    } else if constexpr (BITS == 4) {
        const bool c1 = a > p[3];
        const bool c2 = a > (c1 ? p[5] : p[1]);
        const bool c3 = a > (c1 ? (c2 ? p[6] : p[4]) : (c2 ? p[2] : p[0]));
        h = 4u * c1 + 2u * c2 + c3;
    }
    return y > 0.0f ? half + h : half - 1u - h;
}

template <int BITS>
__global__ __launch_bounds__(64 * kDenseWaves) void k_quantize_dense(
    const _Float16 *__restrict__ xk, const _Float16 *__restrict__ xv, const u4_t *__restrict__ q16,
    PosThresholds P, uint32_t *__restrict__ ck, float *__restrict__ nk, uint32_t *__restrict__ cv,
    float *__restrict__ nv, int64_t N, int64_t Ntot, int64_t n_groups)
{
    constexpr int RW = 4 * BITS;  // dwords per record
    constexpr int SR = RW + 1;    // stage row stride in dwords (odd: a dword read of 64 rows is conflict-free)
    constexpr int NP = (1 << (BITS - 1)) - 1;  // positive thresholds
    __shared__ __align__(16) _Float16 qs[2][kD * kQRow];  // Q high, low parts, rows permuted
    __shared__ __align__(16) uint32_t stage[kDenseWaves][64 * SR];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    KVQ_CHECK(N >= 0 && Ntot >= N && n_groups * 64 >= Ntot);
    KVQ_POISON_LDS(qs, 2 * kD * kQRow / 2, tid, 64 * kDenseWaves);
    KVQ_POISON_LDS(stage, kDenseWaves * 64 * SR, tid, 64 * kDenseWaves);
    if (KVQ_DEBUG_ON) __syncthreads();
    // LDS row 16 nb + a holds Q row 32 (nb / 2) + 8 (a / 4) + 4 (nb % 2) + a % 4:
    // accumulator r of tile nb in lane group kg is then output 32 (nb / 2) + 8 kg + 4 (nb % 2) + r
    for (int i = tid; i < 2 * kD * 16; i += 64 * kDenseWaves) {
        const int part = i >> 11, row = (i >> 4) & (kD - 1), ch = i & 15;
        const int nb = row >> 4, a = row & 15;
        const int src = 32 * (nb >> 1) + 8 * (a >> 2) + 4 * (nb & 1) + (a & 3);
        *reinterpret_cast<u4_t *>(&qs[part][row * kQRow + 8 * ch]) = q16[(part * kD + src) * 16 + ch];
    }
    __syncthreads();
    const int m16 = lane & 15, kg = lane >> 4;
    const float kInvSqrtD = 0.08838834764831845f;
    uint8_t *srow_base = reinterpret_cast<uint8_t *>(&stage[wv][0]);
    // vectors 64 grp .. 64 grp + 63 of the list: K (0 .. N-1), then V (N .. Ntot-1);
    // vector 16 sg + m16 of a group is column m16 of B tile sg
    h8_t X[4][4];
    auto load_x = [&](int64_t grp) {
#pragma unroll
        for (int sg = 0; sg < 4; ++sg) {
            int64_t v = 64 * grp + 16 * sg + m16;
            if (v >= Ntot) v = Ntot - 1;
            const _Float16 *src = v < N ? xk + v * kD : xv + (v - N) * kD;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) X[sg][ks] = *reinterpret_cast<const h8_t *>(src + 32 * ks + 8 * kg);
        }
    };
    const int64_t gstride = (int64_t)gridDim.x * kDenseWaves;
    int64_t grp = (int64_t)blockIdx.x * kDenseWaves + wv;
    if (grp < n_groups) load_x(grp);
    for (; grp < n_groups; grp += gstride) {
        const int64_t g0 = 64 * grp;
        float ps[4][NP > 0 ? NP : 1];  // thresholds scaled by rho / sqrt(d), per vector
#pragma unroll
        for (int sg = 0; sg < 4; ++sg) {
            float ss = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                // squares of fp16 values are exact in fp32; pairs summed by the packed dot product
                const h8_t a = X[sg][ks];
                ss = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 0, 1), __builtin_shufflevector(a, a, 0, 1), ss, false);
                ss = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 2, 3), __builtin_shufflevector(a, a, 2, 3), ss, false);
                ss = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 4, 5), __builtin_shufflevector(a, a, 4, 5), ss, false);
                ss = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 6, 7), __builtin_shufflevector(a, a, 6, 7), ss, false);
            }
            // the four lanes of a vector (kg = 0..3) hold a quarter each
            float2 p = swap16(ss);
            const float s1 = p.x + p.y;
            p = swap32(s1);
            const float rho = __builtin_sqrtf(p.x + p.y);
            const float sc = rho * kInvSqrtD;
#pragma unroll
            for (int k = 0; k < NP; ++k) ps[sg][k] = P.p[k] * sc;
            const int64_t vn = g0 + 16 * sg + m16;
            if (kg == 0 && vn < Ntot) (vn < N ? nk[vn] : nv[vn - N]) = rho;
        }
        // Q x for the 64 vectors, 16 (permuted) outputs per tile nb
        f4_t D[4][8];
#pragma unroll
        for (int sg = 0; sg < 4; ++sg)
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) D[sg][nb] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int off = (16 * nb + m16) * kQRow + 32 * ks + 8 * kg;
                const h8_t ah = *reinterpret_cast<const h8_t *>(&qs[0][off]);
                const h8_t al = *reinterpret_cast<const h8_t *>(&qs[1][off]);
#pragma unroll
                for (int sg = 0; sg < 4; ++sg) {
                    D[sg][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, X[sg][ks], D[sg][nb], 0, 0, 0);
                    D[sg][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, X[sg][ks], D[sg][nb], 0, 0, 0);
                }
            }
        }
        // the inputs are consumed: the next group's loads overlap the bucketing below
        if (grp + gstride < n_groups) load_x(grp + gstride);
        // indices of outputs 32 j + 8 kg + u (u = 4 (nb % 2) + r, nb = 2 j + nb % 2) -> bits b u of piece j
#pragma unroll
        for (int sg = 0; sg < 4; ++sg) {
            uint8_t *row = srow_base + (16 * sg + m16) * (4 * SR);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t pc = 0u;
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    pc |= bucket_idx<BITS>(D[sg][2 * j + (u >> 2)][u & 3], ps[sg]) << (BITS * u);
                const int off = BITS * (4 * j + kg);  // byte offset of the piece in the record
                if constexpr (BITS == 4) {
                    *reinterpret_cast<uint32_t *>(row + off) = pc;
                } else if constexpr (BITS == 2) {
                    *reinterpret_cast<uint16_t *>(row + off) = (uint16_t)pc;
                } else if constexpr (BITS == 1) {
                    row[off] = (uint8_t)pc;
                } else {
                    row[off] = (uint8_t)pc;
                    row[off + 1] = (uint8_t)(pc >> 8);
                    row[off + 2] = (uint8_t)(pc >> 16);
                }
            }
        }
        wave_lds_sync();
        // lane = vector 64 grp + lane
        {
            const uint32_t *row = &stage[wv][lane * SR];
            uint32_t W[RW];
#pragma unroll
            for (int w = 0; w < RW; ++w) W[w] = row[w];
            const int64_t v = g0 + lane;
            if (v < Ntot) {
                u4_t *dst = reinterpret_cast<u4_t *>(v < N ? ck + v * RW : cv + (v - N) * RW);
#pragma unroll
                for (int k = 0; k < BITS; ++k) dst[k] = u4_t{W[4 * k], W[4 * k + 1], W[4 * k + 2], W[4 * k + 3]};
            }
        }
        wave_lds_sync();  // the stage is free for the next group
    }
}

// ---------------------------------------------------------------------------
// Dense rotation followed by the 1-bit QJL residual ("O Que E TurboQuant?",
// Como Funciona, Estagio 1 + Estagio 2): the MSE codes of y = sqrt(d) Q x /
// ||x|| as above, then in the rotated space the residual e = y - c[idx]
// (r = e / sqrt(d), gamma = ||e|| / sqrt(d)) and the sign bits of its
// Gaussian projection S e.  Keys only (one list of N vectors).
//
// A wave takes 64 keys and works through them 16 at a time (the B tile sg):
// rotation of the 16 keys (the products of the MSE kernel), codes written to
// the stage rows, e formed in place of the accumulators, then the projection
// z = S e as 16x16x32 products: A = 16 rows of S (fp16, from LDS), B = e of
// the 16 keys as exact fp16 high and low parts.  The rotation's accumulator
// layout is already the B layout of the projection: lane (m16, kg) holds
// e[32 j + 8 kg .. + 7] of key m16 in the registers of K step j.  The result
// gives lane (m16, kg) outputs 16 ot + 4 kg + r of key m16; its sign bits are
// gathered into the key's four 32-bit words with two lane exchanges.  With an
// S that is not exactly fp16, a third pass adds e_hi . S_lo (S_lo from global
// memory).
template <int BITS>
__device__ __forceinline__ float bucket_centroid(float a, float y, const float *p, const float *mag)
{
    // the centroid c[idx] of the antisymmetric table, by the comparisons of bucket_idx
    float m = mag[0];
    if constexpr (BITS == 2) {
        m = a > p[0] ? mag[1] : mag[0];
    } else if constexpr (BITS == 3) {
        const bool c1 = a > p[1];
        const bool c2 = a > (c1 ? p[2] : p[0]);
        m = c1 ? (c2 ? mag[3] : mag[2]) : (c2 ? mag[1] : mag[0]);
    } else if constexpr (BITS == 4) {
        const bool c1 = a > p[3];
        const bool c2 = a > (c1 ? p[5] : p[1]);
        const bool c3 = a > (c1 ? (c2 ? p[6] : p[4]) : (c2 ? p[2] : p[0]));
        const int h = 4 * c1 + 2 * c2 + c3;
#pragma unroll
        for (int k = 1; k < 8; ++k) m = h == k ? mag[k] : m;
    }
    return y > 0.0f ? m : -m;
}

// (v0, v1) = hi + lo as packed fp16 pairs: hi = v truncated to fp16 by one
// round-toward-zero conversion (v - hi is then exact in fp32), lo = v - hi
// rounded once to fp16 by two mixed-precision FMAs that read the packed hi
// itself, so the hi subtracted is the hi stored.  |hi + lo - v| <= 2^-21 |v|
// (2^-25 absolute below the fp16 normal range); three instructions per pair.
struct SplitPair {
    uint32_t hi, lo;
};
__device__ __forceinline__ SplitPair split_pair(float v0, float v1)
{
    const uint32_t hp = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(v0, v1));
    uint32_t lp;
    asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel:[0,0,0] op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %0, %1, -1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=&v"(lp) : "v"(hp), "v"(v0), "v"(v1));
    return SplitPair{hp, lp};
}

struct DenseMags {
    float m[8];  // positive centroids c_{L/2} .. c_{L-1}
};

template <int BITS, bool S_LO>
__global__ __launch_bounds__(64 * kDenseWaves) void k_quantize_dense_qjl(
    const _Float16 *__restrict__ xk, const u4_t *__restrict__ q16, const u4_t *__restrict__ s16,
    PosThresholds P, DenseMags Mg, uint32_t *__restrict__ ck, float *__restrict__ nk, u4_t *__restrict__ sg_out,
    float *__restrict__ gamma, int64_t N, int64_t n_groups)
{
    constexpr int RW = 4 * BITS;  // dwords per record
    constexpr int SR = RW + 1;    // stage row stride in dwords
    constexpr int NP = (1 << (BITS - 1)) - 1;
    __shared__ __align__(16) _Float16 qs[2][kD * kQRow];  // Q high, low parts, rows permuted
    __shared__ __align__(16) _Float16 ss_[kD * kQRow];    // S high part, rows in order
    __shared__ __align__(16) uint32_t stage[kDenseWaves][64 * SR];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int i = tid; i < 2 * kD * 16; i += 64 * kDenseWaves) {
        const int part = i >> 11, row = (i >> 4) & (kD - 1), ch = i & 15;
        const int nb = row >> 4, a = row & 15;
        const int src = 32 * (nb >> 1) + 8 * (a >> 2) + 4 * (nb & 1) + (a & 3);
        *reinterpret_cast<u4_t *>(&qs[part][row * kQRow + 8 * ch]) = q16[(part * kD + src) * 16 + ch];
    }
    for (int i = tid; i < kD * 16; i += 64 * kDenseWaves) {
        const int row = i >> 4, ch = i & 15;
        *reinterpret_cast<u4_t *>(&ss_[row * kQRow + 8 * ch]) = s16[row * 16 + ch];
    }
    __syncthreads();
    const int m16 = lane & 15, kg = lane >> 4;
    const float kInvSqrtD = 0.08838834764831845f;
    uint8_t *srow_base = reinterpret_cast<uint8_t *>(&stage[wv][0]);
    h8_t X[4][4];
    auto load_x = [&](int64_t grp, int sg) {
        int64_t v = 64 * grp + 16 * sg + m16;
        if (v >= N) v = N - 1;
        const _Float16 *src = xk + v * kD;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) X[sg][ks] = *reinterpret_cast<const h8_t *>(src + 32 * ks + 8 * kg);
    };
    const int64_t gstride = (int64_t)gridDim.x * kDenseWaves;
    int64_t grp = (int64_t)blockIdx.x * kDenseWaves + wv;
    if (grp < n_groups)
#pragma unroll
        for (int sg = 0; sg < 4; ++sg) load_x(grp, sg);
    for (; grp < n_groups; grp += gstride) {
        const int64_t g0 = 64 * grp;
        const bool more = grp + gstride < n_groups;
#pragma unroll
        for (int sg = 0; sg < 4; ++sg) {
            // one key tile at a time: no scheduling across tiles (their
            // registers would be live together)
            __builtin_amdgcn_sched_barrier(0);
            // norm of key 16 sg + m16 (the four lanes kg hold a quarter each)
            float ssum = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const h8_t a = X[sg][ks];
                ssum = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 0, 1), __builtin_shufflevector(a, a, 0, 1), ssum, false);
                ssum = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 2, 3), __builtin_shufflevector(a, a, 2, 3), ssum, false);
                ssum = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 4, 5), __builtin_shufflevector(a, a, 4, 5), ssum, false);
                ssum = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 6, 7), __builtin_shufflevector(a, a, 6, 7), ssum, false);
            }
            float2 pr = swap16(ssum);
            const float s1 = pr.x + pr.y;
            pr = swap32(s1);
            const float rho = __builtin_sqrtf(pr.x + pr.y);
            const float sc = rho * kInvSqrtD;
            const float inv = rho > 0.0f ? 11.313708498984761f / rho : 0.0f;  // sqrt(d) / rho
            float ps[NP > 0 ? NP : 1];
#pragma unroll
            for (int k = 0; k < NP; ++k) ps[k] = P.p[k] * sc;
            const int64_t vn = g0 + 16 * sg + m16;
            if (kg == 0 && vn < N) nk[vn] = rho;
            // Q x of the 16 keys
            f4_t D[8];
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) D[nb] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int off = (16 * nb + m16) * kQRow + 32 * ks + 8 * kg;
                    const h8_t ah = *reinterpret_cast<const h8_t *>(&qs[0][off]);
                    const h8_t al = *reinterpret_cast<const h8_t *>(&qs[1][off]);
                    D[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, X[sg][ks], D[nb], 0, 0, 0);
                    D[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, X[sg][ks], D[nb], 0, 0, 0);
                }
            }
            if (more) load_x(grp + gstride, sg);  // this key tile's inputs are consumed
            // codes (pieces of 8 consecutive outputs 32 j + 8 kg + u) and the
            // residual e = y - c[idx] in place, split into exact fp16 parts
            uint8_t *row = srow_base + (16 * sg + m16) * (4 * SR);
            u4_t eh[4], el[4];
            float e2 = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t pc = 0u;
                float ev[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float y = D[2 * j + (u >> 2)][u & 3];
                    pc |= bucket_idx<BITS>(y, ps) << (BITS * u);
                    ev[u] = y * inv - bucket_centroid<BITS>(__builtin_fabsf(y), y, ps, Mg.m);
                    e2 = fmaf(ev[u], ev[u], e2);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const SplitPair sp = split_pair(ev[2 * u], ev[2 * u + 1]);
                    eh[j][u] = sp.hi;
                    el[j][u] = sp.lo;
                }
                const int off = BITS * (4 * j + kg);
                if constexpr (BITS == 4) {
                    *reinterpret_cast<uint32_t *>(row + off) = pc;
                } else if constexpr (BITS == 2) {
                    *reinterpret_cast<uint16_t *>(row + off) = (uint16_t)pc;
                } else if constexpr (BITS == 1) {
                    row[off] = (uint8_t)pc;
                } else {
                    row[off] = (uint8_t)pc;
                    row[off + 1] = (uint8_t)(pc >> 8);
                    row[off + 2] = (uint8_t)(pc >> 16);
                }
            }
            pr = swap16(e2);
            const float e2a = pr.x + pr.y;
            pr = swap32(e2a);
            if (kg == 0 && vn < N) gamma[vn] = __builtin_sqrtf(pr.x + pr.y) * kInvSqrtD;
            // z = S e: output tile ot (outputs 16 ot .. + 15), K steps j
            uint32_t wsg[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int ot = 0; ot < 8; ++ot) {
                f4_t z = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const h8_t sa = *reinterpret_cast<const h8_t *>(&ss_[(16 * ot + m16) * kQRow + 32 * j + 8 * kg]);
                    z = __builtin_amdgcn_mfma_f32_16x16x32_f16(sa, __builtin_bit_cast(h8_t, eh[j]), z, 0, 0, 0);
                    z = __builtin_amdgcn_mfma_f32_16x16x32_f16(sa, __builtin_bit_cast(h8_t, el[j]), z, 0, 0, 0);
                    if constexpr (S_LO) {
                        const h8_t sl = __builtin_bit_cast(h8_t, s16[(kD + 16 * ot + m16) * 16 + 4 * j + kg]);
                        z = __builtin_amdgcn_mfma_f32_16x16x32_f16(sl, __builtin_bit_cast(h8_t, eh[j]), z, 0, 0, 0);
                    }
                }
                // outputs 16 ot + 4 kg + r: bit 16 (ot & 1) + 4 kg + r of word ot / 2
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (z[r] >= 0.0f) wsg[ot >> 1] |= 1u << (16 * (ot & 1) + 4 * kg + r);
            }
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                wsg[w] |= (uint32_t)__shfl_xor((int)wsg[w], 16);
                wsg[w] |= (uint32_t)__shfl_xor((int)wsg[w], 32);
            }
            if (kg == 0 && vn < N) sg_out[vn] = u4_t{wsg[0], wsg[1], wsg[2], wsg[3]};
        }
        wave_lds_sync();
        {
            const uint32_t *row = &stage[wv][lane * SR];
            uint32_t W[RW];
#pragma unroll
            for (int w = 0; w < RW; ++w) W[w] = row[w];
            const int64_t v = g0 + lane;
            if (v < N) {
                u4_t *dst = reinterpret_cast<u4_t *>(ck + v * RW);
#pragma unroll
                for (int k = 0; k < BITS; ++k) dst[k] = u4_t{W[4 * k], W[4 * k + 1], W[4 * k + 2], W[4 * k + 3]};
            }
        }
        wave_lds_sync();  // the stage is free for the next group
    }
}

template <int BITS>
hipError_t dense_qjl_b(const kvq_ctx *ctx, const void *xk, int64_t N, uint8_t *ck, float *nk, uint8_t *signs,
                       float *gamma, hipStream_t s)
{
    constexpr int L = 1 << BITS;
    PosThresholds P{};
    for (int k = 0; k < L / 2 - 1; ++k) P.p[k] = ctx->cb.t[L / 2 + k];
    DenseMags M{};
    for (int k = 0; k < L / 2; ++k) M.m[k] = ctx->cb.c[L / 2 + k];
    const int64_t n_groups = (N + 63) / 64;
    int64_t blocks = (n_groups + kDenseWaves - 1) / kDenseWaves;
    if (blocks > ctx->n_cu) blocks = ctx->n_cu;
    if (ctx->S_exact_f16)
        hipLaunchKernelGGL((k_quantize_dense_qjl<BITS, false>), dim3((unsigned)blocks), dim3(64 * kDenseWaves), 0, s,
                           (const _Float16 *)xk, (const u4_t *)ctx->d_Q16, (const u4_t *)ctx->d_S16, P, M,
                           (uint32_t *)ck, nk, (u4_t *)signs, gamma, N, n_groups);
    else
        hipLaunchKernelGGL((k_quantize_dense_qjl<BITS, true>), dim3((unsigned)blocks), dim3(64 * kDenseWaves), 0, s,
                           (const _Float16 *)xk, (const u4_t *)ctx->d_Q16, (const u4_t *)ctx->d_S16, P, M,
                           (uint32_t *)ck, nk, (u4_t *)signs, gamma, N, n_groups);
    return hipGetLastError();
}

template <int BITS>
hipError_t dense_b(const kvq_ctx *ctx, const void *xk, const void *xv, int64_t N, uint8_t *ck, float *nk,
                   uint8_t *cv, float *nv, hipStream_t s)
{
    constexpr int L = 1 << BITS;
    PosThresholds P{};
    for (int k = 0; k < L / 2 - 1; ++k) P.p[k] = ctx->cb.t[L / 2 + k];
    const int64_t total = xv ? 2 * N : N;
    const int64_t n_groups = (total + 63) / 64;
    int64_t blocks = (n_groups + kDenseWaves - 1) / kDenseWaves;
    const int64_t cap = ctx->n_cu;  // one block fits a CU's LDS: persistent blocks
    if (blocks > cap) blocks = cap;
    // with no V list the index space ends at N
    hipLaunchKernelGGL(k_quantize_dense<BITS>, dim3((unsigned)blocks), dim3(64 * kDenseWaves), 0, s,
                       (const _Float16 *)xk, (const _Float16 *)(xv ? xv : xk), (const u4_t *)ctx->d_Q16, P,
                       (uint32_t *)ck, nk, (uint32_t *)(cv ? cv : ck), nv ? nv : nk, N, total, n_groups);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_dense_qjl(const kvq_ctx *ctx, const void *xk, int64_t N, uint8_t *ck, float *nk,
                                     uint8_t *signs, float *gamma, hipStream_t s)
{
    switch (ctx->bits) {
    case 1: return dense_qjl_b<1>(ctx, xk, N, ck, nk, signs, gamma, s);
    case 2: return dense_qjl_b<2>(ctx, xk, N, ck, nk, signs, gamma, s);
    case 3: return dense_qjl_b<3>(ctx, xk, N, ck, nk, signs, gamma, s);
    case 4: return dense_qjl_b<4>(ctx, xk, N, ck, nk, signs, gamma, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_quantize_dense(const kvq_ctx *ctx, const void *xk, const void *xv, int64_t N, uint8_t *ck,
                                 float *nk, uint8_t *cv, float *nv, hipStream_t s)
{
    switch (ctx->bits) {
    case 1: return dense_b<1>(ctx, xk, xv, N, ck, nk, cv, nv, s);
    case 2: return dense_b<2>(ctx, xk, xv, N, ck, nk, cv, nv, s);
    case 3: return dense_b<3>(ctx, xk, xv, N, ck, nk, cv, nv, s);
    case 4: return dense_b<4>(ctx, xk, xv, N, ck, nk, cv, nv, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace kvq
