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

#include <type_traits>

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
// The chunk a lane fetches depends on j only through j mod 4, so the address
// is a wave-uniform base (src + 256 (j/4), in 16-byte units) plus one of four
// per-lane offsets: 4 VGPRs instead of 16 64-bit addresses held across the
// persistent loop.  Every call issues exactly 16 load instructions with all
// lanes active (waits count them); rows past a ragged tail re-read the last
// valid row, and are never stored.
__device__ __forceinline__ void tile_to_lds(const u4_t *src, int nv, u4_t *L, int lane)
{
    // lane is made opaque so that the offsets are recomputed here (a few
    // VALU ops) rather than hoisted out of the persistent loop and spilled
    asm volatile("" : "+v"(lane));
    if (nv == kTile) {
        uint32_t off[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int v = 4 * r + (lane >> 4);
            off[r] = (uint32_t)(v * 16 + (((lane & 15) - v) & 15));
        }
#pragma unroll
        for (int j = 0; j < 16; ++j)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(src + 256 * (j >> 2) + off[j & 3]),
                (__attribute__((address_space(3))) void *)(L + j * 64), 16, 0, 0);
    } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int v = 4 * j + (lane >> 4);
            const int c = ((lane & 15) - v) & 15;
            const int row = v < nv ? v : nv - 1;
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(src + row * 16 + c),
                (__attribute__((address_space(3))) void *)(L + j * 64), 16, 0, 0);
        }
    }
}

__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)
// vmcnt(N): all but the N most recently issued vector memory operations have
// completed (they complete in issue order); lgkmcnt and expcnt not waited on.
template <int N>
__device__ __forceinline__ void wait_vm_n()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07F); } // lgkmcnt(0)

// Wait for the wave's tile copy and read row `lane` (its vector) into w.
template <int N>
__device__ __forceinline__ void take_rows(const u4_t *L, int lane, uint32_t *w)
{
    // the row reads stay after the preceding arithmetic: moved up into it
    // they would hold 64 more VGPRs live through the transform
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" : "+v"(lane));  // addresses recomputed per tile, not hoisted and spilled
    wait_vm_n<N>();
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const u4_t v = L[lane * 16 + ((c + lane) & 15)];
        w[4 * c + 0] = v.x;
        w[4 * c + 1] = v.y;
        w[4 * c + 2] = v.z;
        w[4 * c + 3] = v.w;
    }
    wait_lgkm();
    __builtin_amdgcn_wave_barrier();
}

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

// Persistent waves, two per SIMD: wave w processes tiles w, w + W, w + 2W, ...
// (W = waves in the grid).  The next tile's copy into the wave's LDS buffer
// is issued before this tile is encoded; after encoding, the wave waits for
// it (vmcnt(0): it had the whole encode to complete), reads it into
// registers, issues the copy of the tile after it and only then stores this
// tile's codes, so that no wait sits right behind the wave's own stores (vmcnt
// counts stores too).  One launch may cover two tensors of the same shape (K
// and V): tiles [0, n_tiles) belong to tensor 0 and [n_tiles, 2 n_tiles) to
// tensor 1.
struct QArgs {
    const u4_t *x[2];
    u4_t *codes[2];
    float *norms[2];
    int kind[2];  // K (0) or V (1): selects the random signs of each tensor
};

// sgn: sign masks [2][H][64] of D_K and D_V; a separate read-only, non-aliased
// argument so that (with a wave-uniform index) the masks are scalar loads.
template <int BITS>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_quantize(
    QArgs a, const uint32_t *__restrict__ sgn, HalfThresholds ht, int64_t T, int H, int64_t tiles_per_bh,
    int64_t n_tiles, int n_tensors)
{
    __shared__ u4_t lds[kWaves][kTile * 16];  // 64 KiB
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    u4_t *L = lds[wv];
    const int64_t total = n_tiles * n_tensors;
    const int64_t stride = (int64_t)gridDim.x * kWaves;
    int64_t tile = (int64_t)blockIdx.x * kWaves + wv;
    if (tile >= total) return;  // wave-uniform
    auto issue = [&](int64_t t) {
        const int k = t >= n_tiles;
        const TileGeom gg = geom(t - k * n_tiles, T, H, tiles_per_bh);
        tile_to_lds(a.x[k] + gg.v0 * 16, gg.nv, L, lane);
    };
    uint32_t w[64];
    issue(tile);
    take_rows<0>(L, lane, w);
    if (tile + stride < total) issue(tile + stride);
    for (;;) {
        const int kt = tile >= n_tiles;
        const TileGeom g = geom(tile - kt * n_tiles, T, H, tiles_per_bh);

        // wave-uniform head: the masks come through the scalar cache (lgkmcnt),
        // so waiting for them does not wait for the next tile's copy (vmcnt)
        const uint32_t *sg = sgn + __builtin_amdgcn_readfirstlane((a.kind[kt] * H + g.h) * 64);
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

        // The next tile's rows, then the copy of the tile after it, then this
        // tile's stores: the only wait comes right after the encode.
        const int64_t next = tile + stride;
        const bool has_next = next < total;
        if (has_next) {
            take_rows<0>(L, lane, w);
            if (next + stride < total) issue(next + stride);
        }
        if (lane < g.nv) {  // lanes past a ragged tail encoded stale rows
            const int64_t v = g.v0 + lane;
            u4_t *dst = a.codes[kt] + v * BITS;
#pragma unroll
            for (int q = 0; q < BITS; ++q) {
                u4_t o = {out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]};
                dst[q] = o;
            }
            a.norms[kt][v] = rho;
        }
        if (!has_next) break;
        tile = next;
    }
}

// ---------------------------------------------------------------------------
// Quantise with the 1-bit QJL residual ("TurboQuant", Como Funciona,
// Estagio 2).  Per key, besides the MSE codes: the residual in the orthonormal
// rotated space r = (y/rho - c[idx]) / sqrt(d), its norm gamma = ||r|| and
// the 128 sign bits [(S r)_j >= 0] of its Gaussian projection.  Only the signs
// are stored, and they do not depend on the positive factor 1/sqrt(d), so the
// kernel projects e = y/rho - c[idx].
//
// The projection is a dense 64 x 128 x 128 contraction per tile and runs on
// the matrix cores (v_mfma_f32_16x16x32_f16).  The sign decisions need the
// product to about 1e-6 of ||e||, so e is split into fp16 hi + lo parts and
// accumulated in fp32 over two passes (a third pass adds e_hi * S_lo when S
// is not exactly representable in fp16).  e of the 64 keys is staged in LDS
// as fp16 hi and lo rows (16-byte chunks XOR-swizzled by row so that the
// operand reads are conflict-free) and read back in the operand layout: lane
// l holds row l%16, k = 8 (l/16) .. +7.  The
// 16 x 16 result blocks (lane l: rows 4 (l/16) .. +3, column l%16) are turned
// into sign bits with wave ballots; each key's 16-bit chunks are gathered on
// the scalar unit and written into its own lane with v_writelane.
// ---------------------------------------------------------------------------
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

struct QjlArgs {
    const u4_t *x;
    u4_t *codes;
    float *norms;
    u4_t *signs;        // [n][16 bytes]
    float *gamma;       // [n]
    const u4_t *S_hi;   // [128][128] fp16, row-major (row j = output j)
    const u4_t *S_lo;   // same, or nullptr when S is exactly fp16
    float mags[8];      // positive centroids c_{L/2}, ..., c_{L-1}
};

// Magnitude |c[idx]| of coordinate y from the same binary search as the codes.
template <int BITS>
__device__ __forceinline__ float centroid_mag(float a, const float *P, const float *Mg)
{
    if constexpr (BITS == 1) {
        return Mg[0];
    } else if constexpr (BITS == 2) {
        return a > P[0] ? Mg[1] : Mg[0];
    } else if constexpr (BITS == 3) {
        const bool c1 = a > P[1];
        const bool c2 = a > (c1 ? P[2] : P[0]);
        const float lo = c2 ? Mg[1] : Mg[0], hi = c2 ? Mg[3] : Mg[2];
        return c1 ? hi : lo;
    } else {
        const bool c1 = a > P[3];
        const float t2 = c1 ? P[5] : P[1];
        const float tA = c1 ? P[6] : P[2];
        const float tB = c1 ? P[4] : P[0];
        const bool c2 = a > t2;
        const bool c3 = a > (c2 ? tA : tB);
        const int h = (c1 ? 4 : 0) + (c2 ? 2 : 0) + (c3 ? 1 : 0);
        float m = Mg[0];
#pragma unroll
        for (int k = 1; k < 8; ++k) m = h == k ? Mg[k] : m;
        return m;
    }
}

// v = hi + lo (hi returned) with hi exactly representable in fp16: hi keeps the 11 leading
// significant bits of v (values below the fp16 normal range go wholly to lo),
// so its conversion is exact under any rounding and v - hi is exact in fp32;
// only lo is rounded (|error| <= 2^-21 |v|).  Rounding hi to nearest instead
// lets the compiler emit two different conversions for it (one for the stored
// hi, one for the hi subtracted to form lo) that break exact ties differently,
// leaving an error of one fp16 ulp.
__device__ __forceinline__ _Float16 split_f16(float v, _Float16 &lo)
{
    float h = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) & 0xFFFFE000u);
    h = __builtin_fabsf(v) < 0x1p-14f ? 0.0f : h;
    lo = (_Float16)(v - h);
    return (_Float16)h;
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * 16 + (chunk ^ (row & 15)); }

// Write a wave-uniform value into lane KEY of v (other lanes unchanged).
template <int KEY>
__device__ __forceinline__ uint32_t write_lane(uint32_t v, uint32_t val)
{
    asm("v_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(val), "n"(KEY));
    return v;
}

template <int K0, int N>
struct StaticFor {
    template <class F>
    __device__ __forceinline__ static void run(F &&f)
    {
        if constexpr (N > 0) {
            f(std::integral_constant<int, K0>{});
            StaticFor<K0 + 1, N - 1>::run(f);
        }
    }
};

template <int BITS>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_quantize_qjl(
    QjlArgs a, const uint32_t *__restrict__ sgn, HalfThresholds ht, int64_t T, int H, int64_t tiles_per_bh,
    int64_t n_tiles)
{
    __shared__ u4_t Ehi[kWaves][kTile * 16];  // fp16 hi rows of e (16-byte chunks swizzled)
    __shared__ u4_t Elo[kWaves][kTile * 16];  // fp16 lo rows of e
    __shared__ u4_t Ss[kD * 16];              // S_hi, row j chunk c at slot j*16 + (c ^ (j & 15))
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int i = threadIdx.x; i < kD * 16; i += kWaves * 64) Ss[swz(i >> 4, i & 15)] = a.S_hi[i];
    __syncthreads();
    u4_t *Lhi = Ehi[wv], *Llo = Elo[wv];
    const int64_t stride = (int64_t)gridDim.x * kWaves;
    int64_t tile = (int64_t)blockIdx.x * kWaves + wv;
    // Each lane loads its key's row straight into registers; the next tile's
    // rows are requested before the current tile's projection.
    u4_t xr[16];
    auto load_rows = [&](int64_t t) {
        const TileGeom gq = geom(t, T, H, tiles_per_bh);
        const u4_t *src = a.x + (gq.v0 + min(lane, gq.nv - 1)) * 16;  // rows past a tail: last valid row
#pragma unroll
        for (int c = 0; c < 16; ++c) xr[c] = __builtin_nontemporal_load(src + c);
    };
    if (tile < n_tiles) load_rows(tile);
    for (; tile < n_tiles; tile += stride) {
        const TileGeom g = geom(tile, T, H, tiles_per_bh);
        uint32_t w[64];
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            w[4 * c + 0] = xr[c].x;
            w[4 * c + 1] = xr[c].y;
            w[4 * c + 2] = xr[c].z;
            w[4 * c + 3] = xr[c].w;
        }
        const bool active = lane < g.nv;
        const uint32_t *sg = sgn + __builtin_amdgcn_readfirstlane(g.h * 64);
        float ss = 0.0f;
#pragma unroll
        for (int k = 0; k < 64; ++k) {
            const h2_t p = __builtin_bit_cast(h2_t, w[k]);
            ss = __builtin_amdgcn_fdot2(p, p, ss, false);
            w[k] ^= sg[k];
        }
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
                    const float p0 = y[j], p1 = y[j + s];
                    y[j] = p0 + p1;
                    y[j + s] = p0 - p1;
                }
            }
        }
        const float rho = __builtin_sqrtf(ss);
        const float r = rho > 0.0f ? rho : 1.0f;
        const float inv = rho > 0.0f ? 1.0f / rho : 0.0f;
        float P[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) P[k] = ht.p[k] * r;

        uint32_t out[4 * BITS];
#pragma unroll
        for (int k = 0; k < 4 * BITS; ++k) out[k] = 0u;
#pragma unroll
        for (int i = 127; i >= 0; --i) {
            uint64_t M[BITS];
            index_bits<BITS>(y[i], P, M);
#pragma unroll
            for (int k = BITS - 1; k >= 0; --k) {
                const int wd = (BITS * i + k) >> 5;
                out[wd] = append_bit(out[wd], M[k]);
            }
        }
        // residual e = y / rho - c[idx] (the sign of c[idx] is [y > 0]), and gamma
        float g2 = 0.0f;
#pragma unroll
        for (int i = 0; i < 128; ++i) {
            const float mg = centroid_mag<BITS>(__builtin_fabsf(y[i]), P, a.mags);
            const float e = fmaf(y[i], inv, y[i] > 0.0f ? -mg : mg);
            y[i] = e;
            g2 = fmaf(e, e, g2);
        }

        // Stage e of all 64 keys as fp16 hi / lo rows (16-byte chunks swizzled).
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            h8_t hv, lv;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                _Float16 lo;
                hv[j] = split_f16(y[8 * c + j], lo);
                lv[j] = lo;
            }
            Lhi[swz(lane, c)] = __builtin_bit_cast(u4_t, hv);
            Llo[swz(lane, c)] = __builtin_bit_cast(u4_t, lv);
        }
        wait_lgkm();
        __builtin_amdgcn_wave_barrier();
        if (tile + stride < n_tiles) load_rows(tile + stride);

        // Projection of 16 keys at a time against all 128 rows of S: eight
        // independent 16 x 16 accumulators (output blocks nb) per key block.
        uint32_t sgnw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            f4_t z[8];
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) z[nb] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int row = 16 * mb + (lane & 15), chunk = 4 * kb + (lane >> 4);
                const h8_t Ah = __builtin_bit_cast(h8_t, Lhi[swz(row, chunk)]);
                const h8_t Al = __builtin_bit_cast(h8_t, Llo[swz(row, chunk)]);
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) {
                    const int srow = 16 * nb + (lane & 15);
                    const h8_t Bh = __builtin_bit_cast(h8_t, Ss[swz(srow, chunk)]);
                    z[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Bh, z[nb], 0, 0, 0);
                    z[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, Bh, z[nb], 0, 0, 0);
                    if (a.S_lo) {
                        const h8_t Bl = __builtin_bit_cast(h8_t, a.S_lo[srow * 16 + chunk]);
                        z[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Bl, z[nb], 0, 0, 0);
                    }
                }
            }
            // Output block nb, row 4 q + rr of the 16 x 16 result (lane: q = lane/16, column
            // lane%16 = output j - 16 nb): ballot bit 16 q + c is the sign of output
            // 16 nb + c of key 16 mb + 4 q + rr.  Dword np of a key holds outputs
            // 32 np .. 32 np + 31: blocks 2 np (low half) and 2 np + 1 (high half).
#pragma unroll
            for (int np = 0; np < 4; ++np) {
                uint64_t m[2][4];
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) m[t2][rr] = __builtin_amdgcn_ballot_w64(z[2 * np + t2][rr] >= 0.0f);
                uint32_t acc_np = sgnw[np];
                StaticFor<0, 16>::run([&](auto kk) {
                    constexpr int k = decltype(kk)::value;
                    constexpr int q = k / 4, rr = k % 4;
                    const uint32_t lo16 = (uint32_t)(m[0][rr] >> (16 * q)) & 0xFFFFu;
                    const uint32_t hi16 = (uint32_t)(m[1][rr] >> (16 * q)) & 0xFFFFu;
                    const uint32_t val = __builtin_amdgcn_readfirstlane(lo16 | (hi16 << 16));
                    if (mb == 0) acc_np = write_lane<k>(acc_np, val);
                    if (mb == 1) acc_np = write_lane<16 + k>(acc_np, val);
                    if (mb == 2) acc_np = write_lane<32 + k>(acc_np, val);
                    if (mb == 3) acc_np = write_lane<48 + k>(acc_np, val);
                });
                sgnw[np] = acc_np;
            }
        }
        __builtin_amdgcn_wave_barrier();
        if (active) {
            const int64_t v = g.v0 + lane;
            u4_t *dst = a.codes + v * BITS;
#pragma unroll
            for (int q = 0; q < BITS; ++q) {
                u4_t o = {out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]};
                dst[q] = o;
            }
            a.norms[v] = rho;
            u4_t so = {sgnw[0], sgnw[1], sgnw[2], sgnw[3]};
            a.signs[v] = so;
            a.gamma[v] = __builtin_sqrtf(g2) * 0.08838834764831845f;  // ||e|| / sqrt(d)
        }
    }
}

template <int BITS>
hipError_t run_qjl(const kvq_ctx *ctx, const void *x, int64_t B, int64_t T, uint8_t *codes, float *norms,
                   uint8_t *signs, float *gamma, hipStream_t s)
{
    HalfThresholds ht{};
    const int L = 1 << BITS;
    for (int k = 0; k < L / 2 - 1; ++k) ht.p[k] = ctx->cb.t[L / 2 + k];
    QjlArgs a{};
    a.x = (const u4_t *)x;
    a.codes = (u4_t *)codes;
    a.norms = norms;
    a.signs = (u4_t *)signs;
    a.gamma = gamma;
    a.S_hi = (const u4_t *)ctx->d_S16;
    a.S_lo = ctx->S_exact_f16 ? nullptr : (const u4_t *)(ctx->d_S16 + kD * kD);
    for (int k = 0; k < L / 2; ++k) a.mags[k] = ctx->cb.c[L / 2 + k];
    const int64_t tiles_per_bh = (T + kTile - 1) / kTile;
    const int64_t n_tiles = tiles_per_bh * B * ctx->H;
    int64_t blocks = (n_tiles + kWaves - 1) / kWaves;
    if (blocks > (int64_t)ctx->n_cu) blocks = ctx->n_cu;  // one wave per SIMD (512 registers each)
    hipLaunchKernelGGL(k_quantize_qjl<BITS>, dim3((unsigned)blocks), dim3(kWaves * 64), 0, s, a,
                       (const uint32_t *)ctx->d_sgnmask, ht, T, ctx->H, tiles_per_bh, n_tiles);
    return hipGetLastError();
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
    hipLaunchKernelGGL(k_quantize<BITS>, dim3((unsigned)blocks), dim3(kWaves * 64), 0, s, a,
                       (const uint32_t *)ctx->d_sgnmask, ht, T, ctx->H, tiles_per_bh, n_tiles, n_tensors);
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
    if (qjl_signs) {
        switch (ctx->bits) {
        case 1: return run_qjl<1>(ctx, x, B, T, codes, norms, qjl_signs, qjl_gamma, s);
        case 2: return run_qjl<2>(ctx, x, B, T, codes, norms, qjl_signs, qjl_gamma, s);
        case 3: return run_qjl<3>(ctx, x, B, T, codes, norms, qjl_signs, qjl_gamma, s);
        case 4: return run_qjl<4>(ctx, x, B, T, codes, norms, qjl_signs, qjl_gamma, s);
        }
        return hipErrorInvalidValue;
    }
    QArgs a{};
    a.x[0] = a.x[1] = (const u4_t *)x;
    a.codes[0] = a.codes[1] = (u4_t *)codes;
    a.norms[0] = a.norms[1] = norms;
    a.kind[0] = a.kind[1] = kind;
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
    a.kind[0] = 0;
    a.kind[1] = 1;
    return dispatch(ctx, a, 2, B, T, s);
}

}  // namespace kvq
