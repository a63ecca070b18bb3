// Flush of a streaming cache's residual window ("NSNQuant", Detalhes de
// Implementacao: following KIVI the cache is a quantised part plus a
// full-precision residual that is quantised and appended when it fills).
// The R tokens of each (batch, KV head) window are encoded exactly as
// kvq_quantize encodes a vector ("PolarQuant" sec. 2 normalisation and
// rotation; "TurboQuant" Estagio 1 Lloyd-Max buckets): rho = ||x||,
// y = H (D .* x / rho), index = #{thresholds < y_i}, LSB-first packing, and
// written at positions T0 .. T0 + R - 1 of packed arrays holding T_cap
// tokens per (batch, KV head).  A window holds at most a few hundred tokens,
// so one wave per vector (lane l: coordinates 2l, 2l+1) suffices.
#include "kvq_internal.h"
#include "kvq_wave.h"

namespace kvq {
KVQ_DEBUG_UNIT(stream, 6)
namespace {

typedef _Float16 half_t;
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef float f2_t __attribute__((ext_vector_type(2)));

constexpr int kFlushWaves = 4;

template <int BITS>
__global__ __launch_bounds__(64 * kFlushWaves) void k_flush(const half_t *__restrict__ kt, const half_t *__restrict__ vt,
                                                           const float *__restrict__ signs, Codebook cb,
                                                           uint32_t *__restrict__ kc, float *__restrict__ kn,
                                                           uint32_t *__restrict__ vc, float *__restrict__ vn,
                                                           int64_t BH, int H, int64_t R, int64_t R_cap, int64_t T0,
                                                           int64_t T_cap)
{
    constexpr int L = 1 << BITS, RW = 4 * BITS;  // levels, dwords per record
    __shared__ uint32_t pk[kFlushWaves][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t v = (int64_t)blockIdx.x * kFlushWaves + wv;
    if (v >= 2 * BH * R) return;  // wave-uniform
    const int kind = v >= BH * R;
    const int64_t rem = v - kind * BH * R, bh = rem / R, t = rem - bh * R;
    const int g = (int)(bh % H);
    KVQ_CHECK(R <= R_cap && T0 >= 0 && T0 + R <= T_cap && bh < BH && t < R);
    const h2_t x = reinterpret_cast<const h2_t *>((kind ? vt : kt) + (bh * R_cap + t) * kD)[lane];
    const float x0 = (float)x.x, x1 = (float)x.y;
    const float rho = __builtin_sqrtf(wave_sum(fmaf(x1, x1, x0 * x0)));
    const float inv = rho > 0.0f ? 1.0f / rho : 0.0f;
    const f2_t d = reinterpret_cast<const f2_t *>(signs + ((int64_t)kind * H + g) * kD)[lane];
    float y0 = x0 * inv * d.x, y1 = x1 * inv * d.y;
    wave_fwht(y0, y1, lane);
    uint32_t i0 = 0, i1 = 0;
#pragma unroll
    for (int j = 0; j < L - 1; ++j) {
        i0 += cb.t[j] < y0;
        i1 += cb.t[j] < y1;
    }
    pk[wv][lane] = i0 | (i1 << BITS);  // bits [2 BITS lane, 2 BITS lane + 2 BITS) of the record
    wave_lds_sync();
    const int64_t dst = bh * T_cap + T0 + t;
    if (lane < RW) {
        const int b0 = 32 * lane;
        uint32_t w = 0;
        for (int l = b0 / (2 * BITS); l <= (b0 + 31) / (2 * BITS); ++l) {
            const int o = 2 * BITS * l - b0;
            const uint32_t val = pk[wv][l];
            w |= o >= 0 ? val << o : val >> (-o);
        }
        (kind ? vc : kc)[dst * RW + lane] = w;
    }
    if (lane == 0) (kind ? vn : kn)[dst] = rho;
}

template <int BITS>
hipError_t flush_b(const kvq_ctx *ctx, const void *kt, const void *vt, int64_t B, int64_t R, int64_t R_cap,
                   uint8_t *kc, float *kn, uint8_t *vc, float *vn, int64_t T0, int64_t T_cap, hipStream_t s)
{
    const int64_t BH = B * ctx->H;
    const int64_t blocks = (2 * BH * R + kFlushWaves - 1) / kFlushWaves;
    hipLaunchKernelGGL(k_flush<BITS>, dim3((unsigned)blocks), dim3(64 * kFlushWaves), 0, s, (const half_t *)kt,
                       (const half_t *)vt, ctx->d_signs, ctx->cb, (uint32_t *)kc, kn, (uint32_t *)vc, vn, BH, ctx->H,
                       R, R_cap, T0, T_cap);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_flush(const kvq_ctx *ctx, const void *kt, const void *vt, int64_t B, int64_t R, int64_t R_cap,
                        uint8_t *kc, float *kn, uint8_t *vc, float *vn, int64_t T0, int64_t T_cap, hipStream_t s)
{
    switch (ctx->bits) {
    case 1: return flush_b<1>(ctx, kt, vt, B, R, R_cap, kc, kn, vc, vn, T0, T_cap, s);
    case 2: return flush_b<2>(ctx, kt, vt, B, R, R_cap, kc, kn, vc, vn, T0, T_cap, s);
    case 3: return flush_b<3>(ctx, kt, vt, B, R, R_cap, kc, kn, vc, vn, T0, T_cap, s);
    case 4: return flush_b<4>(ctx, kt, vt, B, R, R_cap, kc, kn, vc, vn, T0, T_cap, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace kvq
