// Wave-level helpers shared by the score kernels (gfx950, 64-lane waves).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kvq {
namespace {

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

// Reductions inside each row of 16 lanes (four DPP steps), and over the wave
// (then the exchanges across rows and halves); result in every lane.
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_max(float x)
{
    x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
    return fmaxf(x, dpp<0x140>(x));  // row_mirror
}
__device__ __forceinline__ float row_sum(float x)
{
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    return x + dpp<0x140>(x);
}
__device__ __forceinline__ float wave_max(float x)
{
    x = row_max(x);
    float2 p = swap16(x);
    x = fmaxf(p.x, p.y);
    p = swap32(x);
    return fmaxf(p.x, p.y);
}
__device__ __forceinline__ float wave_sum(float x)
{
    x = row_sum(x);
    float2 p = swap16(x);
    x = p.x + p.y;
    p = swap32(x);
    return p.x + p.y;
}
// LDS written by some lanes of a wave is read by other lanes of the same wave.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Block-wide y[h][r] = sum_c M[r][c] x[h][c] for NH vectors x (LDS,
// [NH][128]) and a 128 x 128 row-major fp32 matrix M in global memory, by
// all NT threads of the block: thread t takes row t % 128 and the
// 128 / (NT / 128) columns of slice t / 128.  gemv_load issues the thread's
// part of M (all of it in flight at once, the block reading M once), so
// that it can overlap other work; block_gemv then forms the partial sums in
// part[NT / 128][NH][128] (LDS) and, after a barrier that every thread of
// the block must reach, returns y[t / 128][t % 128] to threads t < 128 NH.
// `part` may be reused after a further barrier.
template <int NT>
struct GemvSlice {
    typedef float f4v __attribute__((ext_vector_type(4)));
    static constexpr int P = NT / 128, CW = 128 / P;
    static_assert(NT % 128 == 0 && CW % 4 == 0, "whole rows and f4 pieces");
    f4v m[CW / 4];
};

template <int NT>
__device__ __forceinline__ void gemv_load(const float *__restrict__ M, int tid, GemvSlice<NT> &g)
{
    using S = GemvSlice<NT>;
    const typename S::f4v *m = reinterpret_cast<const typename S::f4v *>(M + (tid & 127) * 128 + (tid >> 7) * S::CW);
#pragma unroll
    for (int u = 0; u < S::CW / 4; ++u) g.m[u] = m[u];
}

template <int NH, int NT>
__device__ __forceinline__ float block_gemv(const GemvSlice<NT> &g, const float *x, float *part, int tid)
{
    using S = GemvSlice<NT>;
    const int r = tid & 127, sl = tid >> 7;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const typename S::f4v *xv = reinterpret_cast<const typename S::f4v *>(x + h * 128 + sl * S::CW);
        float a = 0.0f;
#pragma unroll
        for (int u = 0; u < S::CW / 4; ++u) {
            const typename S::f4v xx = xv[u];
            a = fmaf(g.m[u].x, xx.x, a);
            a = fmaf(g.m[u].y, xx.y, a);
            a = fmaf(g.m[u].z, xx.z, a);
            a = fmaf(g.m[u].w, xx.w, a);
        }
        part[(sl * NH + h) * 128 + r] = a;
    }
    __syncthreads();
    float y = 0.0f;
    if (tid < NH * 128) {
        const int h = tid >> 7;
#pragma unroll
        for (int k = 0; k < S::P; ++k) y += part[(k * NH + h) * 128 + r];
    }
    return y;
}

// Softmax partial of one query head over R full-precision tokens (fp16 rows
// of 128 at kb, vb), by one wave.  Per 64-token chunk the lanes score one
// token each against the fp32 query qf (LDS, staged by stage_query while
// the first chunk's loads are in flight), then act as coordinate pairs
// (2 lane, 2 lane + 1) summing the values.  Scores are base 2,
// scale_log2 <q, k>; the result is the maximum m, the sum l of 2^(s_t - m)
// (every lane) and the lane's pair of sum_t 2^(s_t - m) v_t.
struct WindowPartial {
    float m, l, a0, a1;
};
template <class StageQuery>
__device__ __forceinline__ WindowPartial window_partial(const float *qf, const _Float16 *__restrict__ kb,
                                                        const _Float16 *__restrict__ vb, int64_t R,
                                                        float scale_log2, int lane, StageQuery stage_query)
{
    typedef _Float16 h8v __attribute__((ext_vector_type(8)));
    typedef _Float16 h2v __attribute__((ext_vector_type(2)));
    typedef float f4v __attribute__((ext_vector_type(4)));
    // one 64-token chunk: the lane's key row and the chunk's value pairs
    h8v krow[128 / 8];
    h2v vrow[64];
    auto load_chunk = [&](int64_t c) {
        const int64_t t = c + lane < R ? c + lane : c;
#pragma unroll
        for (int i = 0; i < 128 / 8; ++i) krow[i] = reinterpret_cast<const h8v *>(kb + t * 128)[i];
#pragma unroll
        for (int u = 0; u < 64; ++u)
            vrow[u] = reinterpret_cast<const h2v *>(vb + (c + u < R ? c + u : c) * 128)[lane];
    };
    load_chunk(0);
    stage_query();
    wave_lds_sync();
    float m = -__builtin_inff(), l = 0.0f, a0 = 0.0f, a1 = 0.0f;
    for (int64_t c = 0; c < R; c += 64) {
        if (c > 0) load_chunk(c);
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 128 / 8; ++i) {
            const h8v kv = krow[i];
            const f4v q0 = reinterpret_cast<const f4v *>(qf)[2 * i];
            const f4v q1 = reinterpret_cast<const f4v *>(qf)[2 * i + 1];
            acc = fmaf(q0.x, (float)kv[0], acc);
            acc = fmaf(q0.y, (float)kv[1], acc);
            acc = fmaf(q0.z, (float)kv[2], acc);
            acc = fmaf(q0.w, (float)kv[3], acc);
            acc = fmaf(q1.x, (float)kv[4], acc);
            acc = fmaf(q1.y, (float)kv[5], acc);
            acc = fmaf(q1.z, (float)kv[6], acc);
            acc = fmaf(q1.w, (float)kv[7], acc);
        }
        const float sc = c + lane < R ? acc * scale_log2 : -__builtin_inff();
        const float mn = fmaxf(m, wave_max(sc));
        const float al = __builtin_amdgcn_exp2f(m - mn);
        const float p = __builtin_amdgcn_exp2f(sc - mn);
        m = mn;
        l = fmaf(l, al, p);
        a0 *= al;
        a1 *= al;
        // tokens past the end re-read the chunk's first one, with weight 0
#pragma unroll
        for (int u = 0; u < 64; ++u) {
            const float pj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), u));
            a0 = fmaf(pj, (float)vrow[u].x, a0);
            a1 = fmaf(pj, (float)vrow[u].y, a1);
        }
    }
    return WindowPartial{m, wave_sum(l), a0, a1};
}

}  // namespace
}  // namespace kvq
