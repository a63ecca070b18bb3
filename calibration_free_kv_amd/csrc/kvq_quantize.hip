// kvq_quantize: per-vector norm, random-sign Walsh-Hadamard rotation, Gaussian
// Lloyd-Max bucketing and LSB-first bit packing of fp16 K/V vectors
// ("PolarQuant", Technical summary sec. 2; "TurboQuant", Como Funciona,
// Estagio 1).
//
// Mapping on gfx950: one wave quantises a tile of 64 consecutive vectors of
// one (batch, KV head), one vector per lane.  The tile (16 KiB of fp16) is
// read with fully coalesced 16-byte loads (each load instruction covers 1 KiB
// of contiguous memory), staged through a padded LDS tile and read back one
// row per lane.  Each lane then holds its whole vector in VGPRs, so the 7
// butterfly stages of the transform (896 add/sub) need no cross-lane traffic.
// The random signs D of the head are wave-uniform and applied as an XOR on
// the fp16 sign bits; the norm is a chain of packed fp16 dot products with
// fp32 accumulation.  Instead of dividing the 128 coordinates by the norm,
// the rotated coordinates of x itself are compared with the thresholds
// scaled by ||x|| (same decisions up to fp32 rounding, 128 fewer multiplies).
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;     // vectors per wave
constexpr int kWaves = 4;     // waves per block

struct HalfThresholds {
    float p[8];  // positive thresholds t_{L/2}, ..., t_{L-2} (L/2 - 1 of them)
};

// fp16 pair -> fp32 (lo + hi) and (lo - hi) in one mixed-precision FMA each:
// the first butterfly stage fused with the widening.
__device__ __forceinline__ float pair_sum(uint32_t p)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(p));
    return r;
}
__device__ __forceinline__ float pair_diff(uint32_t p)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, 1.0, -%1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(p));
    return r;
}

// acc = 2 * acc + (bit of this lane in the wave mask m): appends one bit to a
// dword that is filled most-significant bit first.
__device__ __forceinline__ uint32_t append_bit(uint32_t acc, uint64_t m)
{
    uint32_t r;
    uint64_t carry;
    asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry) : "v"(acc), "s"(m));
    return r;
}

// Two or three appends in one statement (bits of one coordinate that land in
// the same dword), most significant first.
__device__ __forceinline__ uint32_t append_bits(uint32_t acc, uint64_t m1, uint64_t m0)
{
    uint64_t carry;
    asm("v_addc_co_u32_e64 %0, %1, %0, %0, %2\n\t"
        "v_addc_co_u32_e64 %0, %1, %0, %0, %3"
        : "+v"(acc), "=&s"(carry) : "s"(m1), "s"(m0));
    return acc;
}
__device__ __forceinline__ uint32_t append_bits(uint32_t acc, uint64_t m2, uint64_t m1, uint64_t m0)
{
    uint64_t carry;
    asm("v_addc_co_u32_e64 %0, %1, %0, %0, %2\n\t"
        "v_addc_co_u32_e64 %0, %1, %0, %0, %3\n\t"
        "v_addc_co_u32_e64 %0, %1, %0, %0, %4"
        : "+v"(acc), "=&s"(carry) : "s"(m2), "s"(m1), "s"(m0));
    return acc;
}

// Bits of the index of coordinate y (unnormalised) as wave lane masks,
// M[k] = bit k.  idx = #{j : t_j < y} for the antisymmetric table: with
// a = |y| and h = #{k : a > p_k} (p = positive thresholds scaled by ||x||),
// idx = L/2 + h if y > 0 else L/2 - 1 - h; so the top bit is [y > 0] and the
// low bits are the bits of h, inverted when y <= 0.  h comes from a binary
// search over the positive thresholds.
template <int BITS>
__device__ __forceinline__ void index_bits(float y, const float *P, uint64_t *M)
{
    const float a = __builtin_fabsf(y);
    const uint64_t s = __builtin_amdgcn_ballot_w64(y > 0.0f);
    M[BITS - 1] = s;
    if constexpr (BITS == 2) {
        M[0] = ~(__builtin_amdgcn_ballot_w64(a > P[0]) ^ s);
    } else if constexpr (BITS == 3) {
        const bool c1 = a > P[1];
        const bool c2 = a > (c1 ? P[2] : P[0]);
        M[1] = ~(__builtin_amdgcn_ballot_w64(c1) ^ s);
        M[0] = ~(__builtin_amdgcn_ballot_w64(c2) ^ s);
    } else if constexpr (BITS == 4) {
        const bool c1 = a > P[3];
        const float t2 = c1 ? P[5] : P[1];
        const float tA = c1 ? P[6] : P[2];
        const float tB = c1 ? P[4] : P[0];
        const bool c2 = a > t2;
        const bool c3 = a > (c2 ? tA : tB);
        M[2] = ~(__builtin_amdgcn_ballot_w64(c1) ^ s);
        M[1] = ~(__builtin_amdgcn_ballot_w64(c2) ^ s);
        M[0] = ~(__builtin_amdgcn_ballot_w64(c3) ^ s);
    }
}

// Direct global -> LDS copy of one tile (no VGPR staging).  Load instruction j
// writes LDS bytes [1024 j, 1024 j + 1024) of the wave's buffer, lane l at
// offset 16 l, i.e. vector v = 4 j + l/16, slot s = l % 16.  The lane fetches
// 16-byte chunk c = (s - v) mod 16 of that vector, so chunk c of vector v ends
// up in slot (c + v) mod 16: a skewed layout in which the later per-lane row
// reads (lane v, chunk c) fall into distinct LDS banks.  Each instruction
// still reads one contiguous KiB of HBM.
__device__ __forceinline__ void tile_to_lds(const u4_t *src, int nv, u4_t *L, int lane)
{
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int v = 4 * j + (lane >> 4);
        const int c = ((lane & 15) - v) & 15;
        if (v < nv)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(src + v * 16 + c),
                (__attribute__((address_space(3))) void *)(L + j * 64), 16, 0, 0);
    }
}

__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07F); } // lgkmcnt(0)

struct TileGeom {
    int64_t v0;  // first vector of the tile
    int nv;      // vectors in the tile (ragged at the end of a head)
    int h;       // KV head
};

__device__ __forceinline__ TileGeom geom(int64_t tile, int64_t T, int H, int64_t tiles_per_bh)
{
    TileGeom g;
    const int64_t bh = tile / tiles_per_bh;
    const int64_t t0 = (tile - bh * tiles_per_bh) * kTile;
    g.v0 = bh * T + t0;
    g.nv = (int)min((int64_t)kTile, T - t0);
    g.h = (int)(bh % H);
    return g;
}

// Persistent waves: wave w processes tiles w, w + W, w + 2W, ... (W = waves in
// the grid).  The next tile's loads are issued as soon as the current tile
// has been read from LDS into registers, so they overlap the transform.
// One launch may cover two tensors of the same shape (K and V): tiles
// [0, n_tiles) belong to tensor 0 and [n_tiles, 2 n_tiles) to tensor 1.
struct QArgs {
    const u4_t *x[2];
    u4_t *codes[2];
    float *norms[2];
    const uint32_t *sgnmask[2];
};

template <int BITS>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_quantize(QArgs a, HalfThresholds ht, int64_t T, int H,
                                                          int64_t tiles_per_bh, int64_t n_tiles,
                                                          int n_tensors)
{
    __shared__ u4_t lds[kWaves][kTile * 16];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    u4_t *L = lds[wv];
    const int64_t total = n_tiles * n_tensors;
    const int64_t stride = (int64_t)gridDim.x * kWaves;
    int64_t tile = (int64_t)blockIdx.x * kWaves + wv;
    if (tile < total) {
        const int k = tile >= n_tiles;
        const TileGeom g = geom(tile - k * n_tiles, T, H, tiles_per_bh);
        tile_to_lds(a.x[k] + g.v0 * 16, g.nv, L, lane);
    }
    for (; tile < total; tile += stride) {
        const int kt = tile >= n_tiles;
        const TileGeom g = geom(tile - kt * n_tiles, T, H, tiles_per_bh);
        wait_vm();
        uint32_t w[64];
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const u4_t v = L[lane * 16 + ((c + lane) & 15)];
            w[4 * c + 0] = v.x;
            w[4 * c + 1] = v.y;
            w[4 * c + 2] = v.z;
            w[4 * c + 3] = v.w;
        }
        wait_lgkm();
        const int64_t next = tile + stride;
        if (next < total) {
            const int kn = next >= n_tiles;
            const TileGeom gn = geom(next - kn * n_tiles, T, H, tiles_per_bh);
            tile_to_lds(a.x[kn] + gn.v0 * 16, gn.nv, L, lane);
        }
        if (lane >= g.nv) continue;

        const uint32_t *sg = a.sgnmask[kt] + g.h * 64;
        // ||x||^2 with fp16 products (exact in fp32) accumulated in fp32, and D.
        float ss = 0.0f;
#pragma unroll
        for (int k = 0; k < 64; ++k) {
            const h2_t p = __builtin_bit_cast(h2_t, w[k]);
            ss = __builtin_amdgcn_fdot2(p, p, ss, false);
            w[k] ^= sg[k];
        }
        // First butterfly stage fused with the fp16 -> fp32 widening.
        float y[128];
#pragma unroll
        for (int k = 0; k < 64; ++k) {
            y[2 * k] = pair_sum(w[k]);
            y[2 * k + 1] = pair_diff(w[k]);
        }
#pragma unroll
        for (int s = 2; s < 128; s <<= 1) {
#pragma unroll
            for (int i = 0; i < 128; i += 2 * s) {
#pragma unroll
                for (int j = i; j < i + s; ++j) {
                    const float a = y[j], b = y[j + s];
                    y[j] = a + b;
                    y[j + s] = a - b;
                }
            }
        }

        const float rho = __builtin_sqrtf(ss);
        const float r = rho > 0.0f ? rho : 1.0f;  // zero vector: y = 0 -> index L/2 - 1
        float P[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) P[k] = ht.p[k] * r;

        // Emit the LSB-first stream from its last bit backwards: bit p = BITS*i + k
        // goes to dword p/32, which is filled most-significant bit first.
        uint32_t out[4 * BITS];
#pragma unroll
        for (int k = 0; k < 4 * BITS; ++k) out[k] = 0u;
#pragma unroll
        for (int i = 127; i >= 0; --i) {
            uint64_t M[BITS];
            index_bits<BITS>(y[i], P, M);
            const int lo = (BITS * i) >> 5, hi = (BITS * i + BITS - 1) >> 5;
            if constexpr (BITS == 1) {
                out[lo] = append_bit(out[lo], M[0]);
            } else if (lo == hi) {
                if constexpr (BITS == 2) out[lo] = append_bits(out[lo], M[1], M[0]);
                if constexpr (BITS == 3) out[lo] = append_bits(out[lo], M[2], M[1], M[0]);
                if constexpr (BITS == 4) {
                    out[lo] = append_bits(out[lo], M[3], M[2]);
                    out[lo] = append_bits(out[lo], M[1], M[0]);
                }
            } else {
#pragma unroll
                for (int k = BITS - 1; k >= 0; --k) {
                    const int wd = (BITS * i + k) >> 5;
                    out[wd] = append_bit(out[wd], M[k]);
                }
            }
        }

        const int64_t v = g.v0 + lane;
        u4_t *dst = a.codes[kt] + v * BITS;
#pragma unroll
        for (int q = 0; q < BITS; ++q) {
            u4_t o = {out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]};
            dst[q] = o;
        }
        a.norms[kt][v] = rho;
    }
}

template <int BITS>
hipError_t run(const kvq_ctx *ctx, const QArgs &a, int n_tensors, int64_t B, int64_t T, hipStream_t s)
{
    HalfThresholds ht{};
    const int L = 1 << BITS;
    for (int k = 0; k < L / 2 - 1; ++k) ht.p[k] = ctx->cb.t[L / 2 + k];
    const int64_t tiles_per_bh = (T + kTile - 1) / kTile;
    const int64_t n_tiles = tiles_per_bh * B * ctx->H;
    int64_t blocks = (n_tiles * n_tensors + kWaves - 1) / kWaves;
    if (blocks > 2 * (int64_t)ctx->n_cu) blocks = 2 * (int64_t)ctx->n_cu;  // 8 resident waves per CU
    hipLaunchKernelGGL(k_quantize<BITS>, dim3((unsigned)blocks), dim3(kWaves * 64), 0, s, a, ht, T, ctx->H,
                       tiles_per_bh, n_tiles, n_tensors);
    return hipGetLastError();
}

hipError_t dispatch(const kvq_ctx *ctx, const QArgs &a, int n, int64_t B, int64_t T, hipStream_t s)
{
    switch (ctx->bits) {
    case 1: return run<1>(ctx, a, n, B, T, s);
    case 2: return run<2>(ctx, a, n, B, T, s);
    case 3: return run<3>(ctx, a, n, B, T, s);
    case 4: return run<4>(ctx, a, n, B, T, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_quantize(const kvq_ctx *ctx, int kind, const void *x, int64_t B, int64_t T,
                           uint8_t *codes, float *norms, uint8_t *qjl_signs, float *qjl_gamma,
                           hipStream_t s)
{
    if (qjl_signs || qjl_gamma) return hipErrorNotSupported;
    QArgs a{};
    a.x[0] = a.x[1] = (const u4_t *)x;
    a.codes[0] = a.codes[1] = (u4_t *)codes;
    a.norms[0] = a.norms[1] = norms;
    a.sgnmask[0] = a.sgnmask[1] = ctx->d_sgnmask + (size_t)kind * ctx->H * 64;
    return dispatch(ctx, a, 1, B, T, s);
}

hipError_t launch_quantize_kv(const kvq_ctx *ctx, const void *k, const void *v, int64_t B, int64_t T,
                              uint8_t *k_codes, float *k_norms, uint8_t *v_codes, float *v_norms,
                              hipStream_t s)
{
    QArgs a{};
    a.x[0] = (const u4_t *)k;
    a.x[1] = (const u4_t *)v;
    a.codes[0] = (u4_t *)k_codes;
    a.codes[1] = (u4_t *)v_codes;
    a.norms[0] = k_norms;
    a.norms[1] = v_norms;
    a.sgnmask[0] = ctx->d_sgnmask;
    a.sgnmask[1] = ctx->d_sgnmask + (size_t)ctx->H * 64;
    return dispatch(ctx, a, 2, B, T, s);
}

}  // namespace kvq
