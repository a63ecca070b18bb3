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

// o0 = sum_j M[2 lane][j] v[j], o1 = sum_j M[2 lane + 1][j] v[j]: a 128 x 128
// row-major fp32 matrix in global memory times a 128-vector in LDS (16-byte
// aligned), eight row pieces of each row in flight at a time.
__device__ __forceinline__ void gemv_rows2(const float *__restrict__ M, const float *v, int lane, float &o0,
                                           float &o1)
{
    typedef float f4v __attribute__((ext_vector_type(4)));
    const f4v *r0 = reinterpret_cast<const f4v *>(M + 256 * lane);
    const f4v *r1 = r0 + 32;
    const f4v *x = reinterpret_cast<const f4v *>(v);
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int c0 = 0; c0 < 32; c0 += 8) {
        f4v m0[8], m1[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            m0[u] = r0[c0 + u];
            m1[u] = r1[c0 + u];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const f4v xv = x[c0 + u];
            a0 = fmaf(m0[u].x, xv.x, a0);
            a0 = fmaf(m0[u].y, xv.y, a0);
            a0 = fmaf(m0[u].z, xv.z, a0);
            a0 = fmaf(m0[u].w, xv.w, a0);
            a1 = fmaf(m1[u].x, xv.x, a1);
            a1 = fmaf(m1[u].y, xv.y, a1);
            a1 = fmaf(m1[u].z, xv.z, a1);
            a1 = fmaf(m1[u].w, xv.w, a1);
        }
    }
    o0 = a0;
    o1 = a1;
}

}  // namespace
}  // namespace kvq
