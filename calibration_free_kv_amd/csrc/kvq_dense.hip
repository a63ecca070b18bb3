// Quantisation with a dense orthogonal rotation ("O Que E TurboQuant?", Como
// Funciona, Estagio 1: a random orthogonal transformation from the QR
// decomposition of a Gaussian matrix, then Lloyd-Max buckets per coordinate).
// The rotation is scaled like the Hadamard path so that coordinates have unit
// variance: y = sqrt(d) Q x / ||x||, index = #{thresholds < y}, codes packed
// LSB-first, rho = ||x|| kept.  One Q serves every head, so the B H T vectors
// of a call form one list.
//
// The rotation is a dense contraction and runs on the matrix cores:
// v_mfma_f32_16x16x32_f16 with A = 16 vectors x 32 inputs (the fp16 inputs
// themselves, exact) and B = 32 inputs x 16 outputs of Q, as its fp16 high
// and low parts (two products, so Q enters to about 2^-22), fp32
// accumulation.  A wave takes 64 vectors at a time (four A tiles share every
// B tile read from LDS, where Q's rows are padded to 272 bytes so that the 16
// rows one read touches fall in distinct banks).  The norm comes from the A
// registers; the scaled outputs are bucketed with the antisymmetric binary
// search over the positive thresholds, staged in LDS as bytes, and packed
// with lane = vector.  A lane's D registers hold, for one vector, the outputs
// m, m + 16, ..., m + 112: the stage keeps a row in that order (byte 8 m + j
// holds output 16 j + m), so that they leave as one 8-byte write, and the
// packing loop, whose positions are all compile-time, reads them back in the
// same order.  Eight waves share one copy of Q (two per SIMD).
#include "kvq_internal.h"
#include "kvq_wave.h"

namespace kvq {
namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

constexpr int kDenseWaves = 8;
constexpr int kQRow = kD + 8;   // padded row of Q in LDS, in halves
constexpr int kSRow = kD + 16;  // padded row of the index stage, in bytes (36 dwords: a 16-lane
                                // read of 16-byte pieces of 16 rows touches 64 distinct banks)

struct PosThresholds {
    float p[8];  // t_{L/2} .. t_{L-2}: the positive thresholds of the antisymmetric table
};

// idx = #{j : t_j < y} for the antisymmetric table (t_{L/2-1} = 0): with
// a = |y| and h = #{k : a > p_k}, idx = L/2 + h if y > 0, else L/2 - 1 - h
// (an exact tie at a negative threshold lands one cell up; such a coordinate
// lies inside any decision band).
template <int BITS>
__device__ __forceinline__ uint32_t bucket_idx(float y, const PosThresholds &P)
{
    constexpr uint32_t half = 1u << (BITS - 1);
    const float a = __builtin_fabsf(y);
    uint32_t h = 0;
    if constexpr (BITS == 2) {
        h = a > P.p[0];
    } else if constexpr (BITS == 3) {
        const bool c1 = a > P.p[1];
        const bool c2 = a > (c1 ? P.p[2] : P.p[0]);
        h = 2u * c1 + c2;
    } else if constexpr (BITS == 4) {
        const bool c1 = a > P.p[3];
        const bool c2 = a > (c1 ? P.p[5] : P.p[1]);
        const bool c3 = a > (c1 ? (c2 ? P.p[6] : P.p[4]) : (c2 ? P.p[2] : P.p[0]));
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
    __shared__ __align__(16) _Float16 qs[2][kD * kQRow];  // Q high, low parts; row = output
    __shared__ __align__(16) uint8_t stage[kDenseWaves][64 * kSRow];
    __shared__ __align__(16) float scl[kDenseWaves][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Q parts into LDS: 2 x 128 rows x 16 chunks of 8 halves
    for (int i = tid; i < 2 * kD * 16; i += 64 * kDenseWaves) {
        const int part = i >> 11, row = (i >> 4) & (kD - 1), ch = i & 15;
        *reinterpret_cast<u4_t *>(&qs[part][row * kQRow + 8 * ch]) = q16[i];
    }
    __syncthreads();
    const int m16 = lane & 15, kg = lane >> 4;
    const float kSqrtD = 11.313708498984761f;
    for (int64_t grp = (int64_t)blockIdx.x * kDenseWaves + wv; grp < n_groups;
         grp += (int64_t)gridDim.x * kDenseWaves) {
        // vectors 64 grp .. 64 grp + 63 of the list: K (0 .. N-1), then V (N .. Ntot-1)
        const int64_t g0 = 64 * grp;
        h8_t A[4][4];
        float ss[4];
#pragma unroll
        for (int sg = 0; sg < 4; ++sg) {
            int64_t v = g0 + 16 * sg + m16;
            if (v >= Ntot) v = Ntot - 1;
            const _Float16 *src = v < N ? xk + v * kD : xv + (v - N) * kD;
            float s = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                A[sg][ks] = *reinterpret_cast<const h8_t *>(src + 32 * ks + 8 * kg);
                // squares of fp16 values are exact in fp32; pairs summed by the packed dot product
                const h8_t a = A[sg][ks];
                s = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 0, 1), __builtin_shufflevector(a, a, 0, 1), s, false);
                s = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 2, 3), __builtin_shufflevector(a, a, 2, 3), s, false);
                s = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 4, 5), __builtin_shufflevector(a, a, 4, 5), s, false);
                s = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 6, 7), __builtin_shufflevector(a, a, 6, 7), s, false);
            }
            ss[sg] = s;
        }
        // norms: the four lanes of a vector (kg = 0..3) hold a quarter each
#pragma unroll
        for (int sg = 0; sg < 4; ++sg) {
            float2 p = swap16(ss[sg]);
            const float s1 = p.x + p.y;
            p = swap32(s1);
            const float tot = p.x + p.y;
            const float rho = __builtin_sqrtf(tot);
            const int64_t v = g0 + 16 * sg + m16;
            if (kg == 0) {
                scl[wv][16 * sg + m16] = rho > 0.0f ? kSqrtD / rho : 0.0f;
                if (v < Ntot) (v < N ? nk[v] : nv[v - N]) = rho;
            }
        }
        // y' = Q x for the 64 vectors, 16 outputs (nb) at a time
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
                const h8_t bh = *reinterpret_cast<const h8_t *>(&qs[0][off]);
                const h8_t bl = *reinterpret_cast<const h8_t *>(&qs[1][off]);
#pragma unroll
                for (int sg = 0; sg < 4; ++sg) {
                    D[sg][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[sg][ks], bh, D[sg][nb], 0, 0, 0);
                    D[sg][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[sg][ks], bl, D[sg][nb], 0, 0, 0);
                }
            }
        }
        wave_lds_sync();  // the scales are in LDS
        // D[sg][nb][r]: vector 16 sg + 4 kg + r, output 16 nb + m16 -> stage byte 8 m16 + nb
#pragma unroll
        for (int sg = 0; sg < 4; ++sg) {
            const f4_t s4 = *reinterpret_cast<const f4_t *>(&scl[wv][16 * sg + 4 * kg]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    w0 |= bucket_idx<BITS>(D[sg][nb][r] * s4[r], P) << (8 * nb);
                    w1 |= bucket_idx<BITS>(D[sg][nb + 4][r] * s4[r], P) << (8 * nb);
                }
                *reinterpret_cast<uint2 *>(&stage[wv][(16 * sg + 4 * kg + r) * kSRow + 8 * m16]) = uint2{w0, w1};
            }
        }
        wave_lds_sync();
        // pack: lane = vector 64 grp + lane
        {
            const u4_t *row = reinterpret_cast<const u4_t *>(&stage[wv][lane * kSRow]);
            uint32_t W[RW];
#pragma unroll
            for (int w = 0; w < RW; ++w) W[w] = 0u;
#pragma unroll
            for (int c = 0; c < kD / 16; ++c) {
                const u4_t b16 = row[c];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const uint32_t ix = (b16[e >> 2] >> (8 * (e & 3))) & 0xFFu;
                    const int pos = 16 * c + e, i = 16 * (pos & 7) + (pos >> 3);  // output index
                    const int p = BITS * i, w = p >> 5, sh = p & 31;
                    W[w] |= ix << sh;
                    if (sh + BITS > 32) W[w + 1] |= ix >> (32 - sh);
                }
            }
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
