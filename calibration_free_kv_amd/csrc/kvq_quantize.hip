// kvq_quantize: per-vector norm, random-sign Walsh-Hadamard rotation, Gaussian
// Lloyd-Max bucketing and LSB-first bit packing of fp16 K/V vectors
// ("PolarQuant", Technical summary sec. 2; "TurboQuant", Como Funciona,
// Estagio 1).
//
// Mapping on gfx950: a wave quantises a tile of 32 consecutive vectors of one
// (batch, KV head) with two lanes per vector: lane 2v + h holds coordinates
// [64 h, 64 h + 64) of vector v, so a wave needs about 100 VGPRs and four
// waves share each SIMD.  The tile (8 KiB of fp16) is copied from HBM straight
// into LDS (each copy instruction reads one contiguous KiB) and read back as
// half rows.  Six of the seven butterfly stages of the transform run inside
// the lane; the stage that pairs coordinate i with i + 64 is one DPP lane swap
// fused into an FMA.  The random signs D of the head travel with the tile and
// are applied as an XOR on the fp16 sign bits; the norm is a chain of packed
// fp16 dot products with fp32 accumulation, completed across the lane pair.
// Instead of dividing the coordinates by the norm, the rotated coordinates of
// x itself are compared with the thresholds scaled by ||x|| (same decisions up
// to fp32 rounding, no per-coordinate multiply).
#include "kvq_internal.h"

#include <type_traits>

namespace kvq {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;     // vectors per wave tile, one per lane (QJL kernel)
constexpr int kTileH = 32;    // vectors per wave tile, two lanes each (MSE kernel)
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

struct TileGeom {
    int64_t v0;  // first vector of the tile
    int nv;      // vectors in the tile (ragged at the end of a head)
    int h;       // KV head
};

// floor(n / d) for 0 <= n < 2^31 and 1 <= d < 2^31 as (umulhi(n, m) + n) >> l,
// with l = ceil(log2 d) and m = ceil(2^(32+l) / d) - 2^32 (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994):
// a few scalar instructions instead of a 64-bit division sequence.
struct FastDiv {
    uint32_t m, l;
};
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) { return (__umulhi(n, f.m) + n) >> f.l; }

// Tile index -> (batch, head) row block: tiles_per_bh tiles of TILE vectors
// per (batch, head), T vectors each, H heads.
struct TileMap {
    int64_t T;
    uint32_t tiles_per_bh, H;
    FastDiv by_tiles, by_H;
};

// Host side: the map of a launch.
FastDiv make_fastdiv(uint32_t d)
{
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    const uint64_t m = ((1ull << (32 + l)) - 1) / d + 1;  // ceil(2^(32+l) / d), l <= 31
    return FastDiv{(uint32_t)(m - (1ull << 32)), l};
}

TileMap make_map(int64_t T, int H, int64_t tiles_per_bh)
{
    return TileMap{T, (uint32_t)tiles_per_bh, (uint32_t)H, make_fastdiv((uint32_t)tiles_per_bh),
                   make_fastdiv((uint32_t)H)};
}

template <int TILE = kTile>
__device__ __forceinline__ TileGeom geom(uint32_t tile, const TileMap &mp)
{
    TileGeom g;
    const uint32_t bh = fdiv(tile, mp.by_tiles);
    const uint32_t t0 = (tile - bh * mp.tiles_per_bh) * TILE;
    g.v0 = (int64_t)bh * mp.T + t0;
    g.nv = (int)min((int64_t)TILE, mp.T - t0);
    g.h = (int)(bh - fdiv(bh, mp.by_H) * mp.H);
    return g;
}

// LDS image of one wave tile: 32 rows of 16 chunks (16 bytes = 8 coordinates
// each), then the 64 sign-mask dwords of the tile's head.  Half h of row v
// (chunks 8h .. 8h+7) sits in slots [16 v + 8 h, 16 v + 8 h + 8), chunk
// 8h + k at slot 16 v + 8 h + (k ^ m) with m = (v mod 8) ^ 4h.  At each of its
// eight reads, lane 2v + h asks for slot k ^ m of its half row; over any 8 (or
// 16) consecutive lanes these fall into distinct 16-byte bank groups, so the
// half-row reads are free of bank conflicts.
constexpr int kRowsH = kTileH * 16;   // 16-byte chunks of rows per tile
constexpr int kBufH = kRowsH + 16;    // + 256 bytes of sign masks

// Direct global -> LDS copy of one tile and its head's sign masks (no VGPR
// staging).  Row-copy instruction j writes slots [64 j, 64 j + 64) of the
// buffer, lane l at slot 64 j + l: vector v = 4 j + l/16, slot q = l % 16 of
// its row, i.e. half h = q/8 and chunk 8h + ((q mod 8) ^ m).  Each such
// instruction reads one contiguous KiB (four whole rows).  The chunk depends
// on j only through j mod 2, so the address is a wave-uniform base plus one
// of two per-lane offsets.  A ninth instruction copies the 64 mask dwords.
// Every call issues exactly 9 load instructions with all lanes active (waits
// count them); rows past a ragged tail re-read the last valid row, and are
// never stored.
__device__ __forceinline__ int half_chunk(int v, int q)
{
    const int h = q >> 3;
    return 8 * h + ((q & 7) ^ ((v & 7) ^ (4 * h)));
}

__device__ __forceinline__ void tile_to_lds(const u4_t *src, int nv, const uint32_t *msk, u4_t *L, int lane)
{
    // lane is made opaque so that the offsets are recomputed here (a few
    // VALU ops) rather than hoisted out of the persistent loop and spilled
    asm volatile("" : "+v"(lane));
    if (nv == kTileH) {
        uint32_t off[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int v = 4 * p + (lane >> 4);
            off[p] = (uint32_t)((lane >> 4) * 16 + half_chunk(v, lane & 15));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(src + 64 * j + off[j & 1]),
                (__attribute__((address_space(3))) void *)(L + j * 64), 16, 0, 0);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int v = 4 * j + (lane >> 4);
            const int row = v < nv ? v : nv - 1;
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(src + row * 16 + half_chunk(v, lane & 15)),
                (__attribute__((address_space(3))) void *)(L + j * 64), 16, 0, 0);
        }
    }
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(msk + lane),
                                     (__attribute__((address_space(3))) void *)(L + kRowsH), 4, 0, 0);
}

// Wait for the wave's tile copy, read half row h of vector v into w (lane
// 2v + h) and apply the signs of D.  Also draws the wave's next ticket from
// the workgroup's LDS counter: the atomic goes out with the row reads, after
// the copy has landed (the compiler makes any LDS access wait for all copies
// into LDS that are still in flight).
template <int N>
__device__ __forceinline__ int take_rows(const u4_t *L, int lane, uint32_t *w, int *counter)
{
    // the row reads stay after the preceding arithmetic: moved up into it
    // they would hold 32 more VGPRs live through the transform
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" : "+v"(lane));  // addresses recomputed per tile, not hoisted and spilled
    wait_vm_n<N>();
    const int v = lane >> 1, h = lane & 1;
    const int b = 16 * v + 8 * h + ((v & 7) ^ (4 * h));  // slot of chunk k: b ^ k
    const u4_t *M = L + kRowsH + 8 * h;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const u4_t x = L[b ^ k];
        const u4_t m = M[k];
        w[4 * k + 0] = x.x ^ m.x;
        w[4 * k + 1] = x.y ^ m.y;
        w[4 * k + 2] = x.z ^ m.z;
        w[4 * k + 3] = x.w ^ m.w;
    }
    int t = 0;
    if (lane == 0) t = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    wait_lgkm();
    __builtin_amdgcn_wave_barrier();
    return __builtin_amdgcn_readfirstlane(t);
}

// The value of x in the other lane of the pair (lanes 2v, 2v + 1).
__device__ __forceinline__ float pair_swap(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
}

// y[i] += c * (y[i] of the other lane of the pair), i = 0..7, as one
// v_fmac_f32 with a DPP source each (the compiler keeps the lane swap as a
// separate move).  Every read of y[i] in the block happens before any lane
// writes it, and each instruction reads a register no earlier instruction of
// the block wrote; the leading s_nop 4 provides the wait states a DPP source
// needs after a VALU write of that register (2) or a write of EXEC (5) by the
// code before the block.
__device__ __forceinline__ void pair_fmac8(float *y, float c)
{
    asm volatile(
        "s_nop 4\n\t"
        "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
        : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3]), "+v"(y[4]), "+v"(y[5]), "+v"(y[6]), "+v"(y[7])
        : "v"(c));
}

// One workgroup of 16 waves per CU (four per SIMD) owns every G-th tile (G =
// workgroups in the grid).  Each wave starts on one of them; after that the
// waves take the remaining ones in order from a counter in LDS, so a wave whose first
// copy arrives late (every wave requests one at the same moment, and the last
// ones arrive several microseconds after the first) simply processes fewer
// tiles.  The next tile's copy into the wave's LDS buffer is issued before
// this tile is encoded; after encoding, the wave waits for it (vmcnt(0): it
// had the whole encode to complete), reads it into registers, issues the copy
// of the tile after it and only then stores this tile's codes, so that no
// wait sits right behind the wave's own stores (vmcnt counts stores too).  The
// ticket for the tile after next is drawn along with the row reads.  One launch may
// cover two tensors of the same shape (K and V): tiles [0, n_tiles) belong to
// tensor 0 and [n_tiles, 2 n_tiles) to tensor 1.
constexpr int kWavesQ = 16;  // waves per workgroup of the MSE kernel

struct QArgs {
    const u4_t *x[2];
    u4_t *codes[2];
    float *norms[2];
    int kind[2];  // K (0) or V (1): selects the random signs of each tensor
};

// sgnh: sign masks [2][H][64] of D_K and D_V as fp16-pair XOR masks, with the
// masks of coordinates 64..127 also flipping every sign: the upper lane of a
// pair transforms -x[64..127], which lets one FMA form both outputs of the
// cross-lane butterfly stage (lower lane: a - (-b), upper lane: -b + a).
template <int BITS>
__global__ __launch_bounds__(kWavesQ * 64) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_quantize(
    QArgs a, const uint32_t *__restrict__ sgnh, HalfThresholds ht, TileMap mp,
    int64_t n_tiles, int n_tensors)
{
    __shared__ u4_t lds[kWavesQ][kBufH];  // 132 KiB
    __shared__ int next_tile;             // next unclaimed tile of the range, relative to its start
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    u4_t *L = lds[wv];
    const int64_t total = n_tiles * n_tensors;
    // ticket k of this workgroup is tile blockIdx.x + k * gridDim.x: at any
    // moment the workgroups read one window of consecutive tiles
    const int64_t G = gridDim.x;
    if (threadIdx.x == 0) next_tile = kWavesQ;
    __syncthreads();
    int64_t tile = blockIdx.x + wv * G;
    if (tile >= total) return;  // wave-uniform
    auto issue = [&](int64_t t) {
        const int k = t >= n_tiles;
        const TileGeom gg = geom<kTileH>((uint32_t)(t - k * n_tiles), mp);
        tile_to_lds(a.x[k] + gg.v0 * 16, gg.nv, sgnh + (a.kind[k] * (int)mp.H + gg.h) * 64, L, lane);
    };
    // cross-lane stage: lower lane a - (-b) = a + b, upper lane -b + a = a - b
    const float cross = (lane & 1) ? 1.0f : -1.0f;
    uint32_t w[32];
    issue(tile);
    int64_t next = blockIdx.x + take_rows<0>(L, lane, w, &next_tile) * G;
    if (next < total) issue(next);
    constexpr bool kMidIssue = BITS <= 3;
    int64_t pending = total;  // a drawn tile whose copy is not yet issued
    for (;;) {
        const int kt = tile >= n_tiles;
        const TileGeom g = geom<kTileH>((uint32_t)(tile - kt * n_tiles), mp);

        // ||x||^2 of the half row with fp16 products (exact in fp32)
        // accumulated in fp32; D is already applied (signs do not change it).
        float ss = 0.0f;
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            const h2_t p = __builtin_bit_cast(h2_t, w[k]);
            ss = __builtin_amdgcn_fdot2(p, p, ss, false);
        }
        // First butterfly stage fused with the fp16 -> fp32 widening, then the
        // other in-lane stages (strides 2 .. 32).
        float y[64];
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            y[2 * k] = pair_sum(w[k]);
            y[2 * k + 1] = pair_diff(w[k]);
        }
#pragma unroll
        for (int s = 2; s < 64; s <<= 1) {
#pragma unroll
            for (int i = 0; i < 64; i += 2 * s) {
#pragma unroll
                for (int j = i; j < i + s; ++j) {
                    const float p = y[j], q = y[j + s];
                    y[j] = p + q;
                    y[j + s] = p - q;
                }
            }
        }
        // Stride-64 stage across the lane pair.
#pragma unroll
        for (int i = 0; i < 64; i += 8) pair_fmac8(y + i, cross);
        // Both lanes form the same sum (fp32 addition commutes).
        ss += pair_swap(ss);
        // The copy of the tile after next goes out here, half an encode
        // before its wait: issued a whole encode ahead, the copies of all
        // waves kept about twice the data in flight that the memory system
        // needs to stay busy, and every request waited correspondingly longer
        // in its queues (which shows at the start and at the end of the grid).
        // At b = 4 the register held for it over the transform costs spills,
        // and the copy goes out right after the row reads instead.
        if constexpr (kMidIssue) {
            if (pending < total) issue(pending);
            pending = total;
        }

        const float rho = __builtin_sqrtf(ss);
        const float r = rho > 0.0f ? rho : 1.0f;  // zero vector: y = 0 -> index L/2 - 1
        float P[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) P[k] = ht.p[k] * r;

        // Emit this lane's 64 BITS-bit indices (bits [64 BITS h, 64 BITS (h+1))
        // of the vector's LSB-first stream) from the last bit backwards: local
        // bit p = BITS*i + k goes to dword p/32, filled most-significant first.
        uint32_t out[2 * BITS];
#pragma unroll
        for (int k = 0; k < 2 * BITS; ++k) out[k] = 0u;
#pragma unroll
        for (int i = 63; i >= 0; --i) {
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
        const bool has_next = next < total;
        int64_t after = total;
        if (has_next) {
            after = blockIdx.x + take_rows<0>(L, lane, w, &next_tile) * G;
            if constexpr (kMidIssue)
                pending = after;
            else if (after < total)
                issue(after);
        }
        if ((lane >> 1) < g.nv) {  // lanes past a ragged tail encoded stale rows
            // the lanes of the tile write 64 * 8 BITS contiguous bytes
            uint2 *dst = (uint2 *)(a.codes[kt] + g.v0 * BITS) + lane * BITS;
#pragma unroll
            for (int q = 0; q < BITS; ++q) dst[q] = make_uint2(out[2 * q], out[2 * q + 1]);
            if (!(lane & 1)) a.norms[kt][g.v0 + (lane >> 1)] = rho;
        }
        if (!has_next) break;
        tile = next;
        next = after;
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
typedef float f16_t __attribute__((ext_vector_type(16)));

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

// Write the low and high halves of a lane mask into lanes KLO and KHI of v.
// The leading s_nop 4 gives the wait states a read of an SGPR pair needs right
// after a VALU instruction (the compare that made the mask) wrote it: the
// compiler cannot see into the asm, and without them the first read returned
// the previous value.
template <int KLO, int KHI>
__device__ __forceinline__ uint32_t write_lane_pair(uint32_t v, uint64_t m)
{
    asm("s_nop 4\n\t"
        "v_writelane_b32 %0, %1, %3\n\t"
        "v_writelane_b32 %0, %2, %4"
        : "+v"(v) : "s"((uint32_t)m), "s"((uint32_t)(m >> 32)), "n"(KLO), "n"(KHI));
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

// Tile of 32 keys for the QJL kernel, two lanes per key: lane 32h + v holds
// coordinates [64 h, 64 h + 64) of key v (so that the residual can feed the
// matrix cores straight from registers, see below).  Chunk c of row v sits at
// LDS slot 16 v + ((c + v) mod 16): the 16 lanes of one half that read chunk
// 8h + k of 16 consecutive rows hit 16 different bank groups.  Copy
// instruction j writes slots [64 j, 64 j + 64) (rows 4j .. 4j+3, one
// contiguous KiB of HBM); the chunk a lane fetches depends on j only through
// j mod 4.  A ninth instruction copies the head's 64 sign-mask dwords.
__device__ __forceinline__ void qjl_tile_to_lds(const u4_t *src, int nv, const uint32_t *msk, u4_t *L, int lane)
{
    asm volatile("" : "+v"(lane));
    if (nv == kTileH) {
        uint32_t off[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int v = 4 * r + (lane >> 4);
            off[r] = (uint32_t)((lane >> 4) * 16 + (((lane & 15) - v) & 15));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(src + 64 * j + off[j & 3]),
                (__attribute__((address_space(3))) void *)(L + j * 64), 16, 0, 0);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int v = 4 * j + (lane >> 4);
            const int row = v < nv ? v : nv - 1;
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(src + row * 16 + (((lane & 15) - v) & 15)),
                (__attribute__((address_space(3))) void *)(L + j * 64), 16, 0, 0);
        }
    }
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(msk + lane),
                                     (__attribute__((address_space(3))) void *)(L + kRowsH), 4, 0, 0);
}

// Wait for the tile copy, read half row h of key v into w (lane 32h + v),
// apply D, and draw the wave's next ticket from the LDS counter (see
// take_rows).
__device__ __forceinline__ int qjl_take_rows(const u4_t *L, int lane, uint32_t *w, int *counter)
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" : "+v"(lane));
    wait_vm_n<0>();
    const int v = lane & 31, h = lane >> 5;
    const u4_t *M = L + kRowsH + 8 * h;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const u4_t x = L[16 * v + ((8 * h + k + v) & 15)];
        const u4_t m = M[k];
        w[4 * k + 0] = x.x ^ m.x;
        w[4 * k + 1] = x.y ^ m.y;
        w[4 * k + 2] = x.z ^ m.z;
        w[4 * k + 3] = x.w ^ m.w;
    }
    int t = 0;
    if (lane == 0) t = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    wait_lgkm();
    __builtin_amdgcn_wave_barrier();
    return __builtin_amdgcn_readfirstlane(t);
}

// Swap of lanes 32..63 of x with lanes 0..31 of y (gfx950): returns
// (x', y') with x' = [x_lo | y_lo] and y' = [x_hi | y_hi].
__device__ __forceinline__ void swap_halves(float &x, float &y)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y),
                                                    false, false);
    x = __builtin_bit_cast(float, (unsigned)r[0]);
    y = __builtin_bit_cast(float, (unsigned)r[1]);
}

// Append the BITS-bit indices of 32 coordinates y[0..31] (LSB-first stream of
// 32 BITS bits) to out[0 .. BITS), from the last bit backwards, and replace
// each y[i] by its residual y[i] / rho - c[idx] (inv = 1 / rho; the sign of
// c[idx] is [y > 0]).
template <int BITS>
__device__ __forceinline__ void encode32(float *y, const float *P, const float *Mg, float inv, uint32_t *out)
{
#pragma unroll
    for (int i = 31; i >= 0; --i) {
        uint64_t M[BITS];
        index_bits<BITS>(y[i], P, M);
        const float mg = centroid_mag<BITS>(__builtin_fabsf(y[i]), P, Mg);
        y[i] = fmaf(y[i], inv, y[i] > 0.0f ? -mg : mg);
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
}

// Quantise with the 1-bit QJL residual, one workgroup of 12 waves per CU
// (three per SIMD), tiles of 32 keys claimed as in k_quantize.
//  - MSE part as in k_quantize, except that the stride-64 butterfly pairs
//    lanes l and l ^ 32: one gfx950 half swap of registers (i, i + 32) and an
//    add and a subtract give coordinates i, i + 64 (lanes 0-31) and 32 + i,
//    96 + i (lanes 32-63).  So register r of half h holds coordinate
//    C(h, r) = 32 h + r for r < 32 and 64 + 32 h + (r - 32) for r >= 32, and
//    each half packs two runs of 32 coordinates.
//  - e = y / rho - c[idx] per coordinate (the factor 1/sqrt(d) of r does not
//    change a sign), gamma = ||e|| / sqrt(d); e is split exactly into fp16
//    hi + lo (hi by round-toward-zero conversion, i.e. its 11 leading
//    significant bits; lo = e - hi exactly, then rounded once).
//  - The projection S e of the 32 keys runs on v_mfma_f32_32x32x16_f16 with
//    the A operand straight from registers: the contraction may visit the
//    coordinates in any order as long as both operands agree, so k-step s
//    takes, in lane half h, registers 8s .. 8s+7 (coordinates C(h, 8s) ..
//    +7, contiguous), and the B operand reads the same coordinates of the
//    rows of S staged in LDS.  Each accumulator register of a 32 x 32 block
//    (rows = keys, columns = outputs) gives, with one ballot, two keys' 32
//    sign bits of the block, which are written into the key's lane.
constexpr int kWavesJ = 12;  // waves per workgroup of the QJL kernel

template <int BITS, bool S_LO>
__global__ __launch_bounds__(kWavesJ * 64) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_quantize_qjl(
    QjlArgs a, const uint32_t *__restrict__ sgn, HalfThresholds ht, TileMap mp,
    int64_t n_tiles)
{
    __shared__ u4_t Ss[kD * 16];              // S_hi, row n chunk c at slot n*16 + (c ^ (n & 15))
    __shared__ u4_t lds[kWavesJ][kBufH];      // tiles of the waves
    __shared__ int next_tile;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int i = threadIdx.x; i < kD * 16; i += kWavesJ * 64) Ss[swz(i >> 4, i & 15)] = a.S_hi[i];
    if (threadIdx.x == 0) next_tile = kWavesJ;
    __syncthreads();
    u4_t *L = lds[wv];
    const int64_t G = gridDim.x;
    int64_t tile = blockIdx.x + wv * G;
    if (tile >= n_tiles) return;  // wave-uniform
    auto issue = [&](int64_t t) {
        const TileGeom gg = geom<kTileH>((uint32_t)(t), mp);
        qjl_tile_to_lds(a.x + gg.v0 * 16, gg.nv, sgn + gg.h * 64, L, lane);
    };
    const int v = lane & 31, h = lane >> 5;
    float Mg[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) Mg[k] = a.mags[k];
    uint32_t w[32];
    issue(tile);
    int64_t next = blockIdx.x + qjl_take_rows(L, lane, w, &next_tile) * G;
    if (next < n_tiles) issue(next);
    for (;;) {
        const TileGeom g = geom<kTileH>((uint32_t)(tile), mp);
        float ss = 0.0f;
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            const h2_t p = __builtin_bit_cast(h2_t, w[k]);
            ss = __builtin_amdgcn_fdot2(p, p, ss, false);
        }
        float y[64];
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            y[2 * k] = pair_sum(w[k]);
            y[2 * k + 1] = pair_diff(w[k]);
        }
#pragma unroll
        for (int s = 2; s < 64; s <<= 1) {
#pragma unroll
            for (int i = 0; i < 64; i += 2 * s) {
#pragma unroll
                for (int j = i; j < i + s; ++j) {
                    const float p = y[j], q = y[j + s];
                    y[j] = p + q;
                    y[j + s] = p - q;
                }
            }
        }
        // stride-64 stage across the halves
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            float p = y[i], q = y[i + 32];
            swap_halves(p, q);
            y[i] = p + q;
            y[i + 32] = p - q;
        }
        {
            float p = ss, q = ss;
            swap_halves(p, q);
            ss = p + q;  // the same sum in both halves
        }
        const float rho = __builtin_sqrtf(ss);
        const float r = rho > 0.0f ? rho : 1.0f;
        const float inv = rho > 0.0f ? 1.0f / rho : 0.0f;
        float P[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) P[k] = ht.p[k] * r;

        // codes: run 0 = coordinates 32h .. 32h+31, run 1 = 64+32h .. 64+32h+31
        uint32_t out[2 * BITS];
#pragma unroll
        for (int k = 0; k < 2 * BITS; ++k) out[k] = 0u;
        encode32<BITS>(y, P, Mg, inv, out);
        encode32<BITS>(y + 32, P, Mg, inv, out + BITS);

        // y now holds the residual e: gamma and the exact fp16 split
        float g2 = 0.0f;
        uint32_t eh[32], el[32];
#pragma unroll
        for (int m = 0; m < 32; ++m) {
            const float e0 = y[2 * m], e1 = y[2 * m + 1];
            g2 = fmaf(e0, e0, g2);
            g2 = fmaf(e1, e1, g2);
            const h2_t hp = __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(e0, e1));
            const h2_t lp = h2_t{(_Float16)(e0 - (float)hp.x), (_Float16)(e1 - (float)hp.y)};
            eh[m] = __builtin_bit_cast(uint32_t, hp);
            el[m] = __builtin_bit_cast(uint32_t, lp);
        }
        {
            float p = g2, q = g2;
            swap_halves(p, q);
            g2 = p + q;
        }

        uint32_t sgnw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            f16_t z = {};
            const int n = 32 * nb + v;  // output row of S read by this lane
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int ch = (s < 4 ? s : s + 4) + 4 * h;  // 16-byte chunk of the coordinates C(h, 8s..8s+7)
                const h8_t B = __builtin_bit_cast(h8_t, Ss[swz(n, ch)]);
                const h8_t Ah = __builtin_bit_cast(h8_t, u4_t{eh[4 * s], eh[4 * s + 1], eh[4 * s + 2], eh[4 * s + 3]});
                const h8_t Al = __builtin_bit_cast(h8_t, u4_t{el[4 * s], el[4 * s + 1], el[4 * s + 2], el[4 * s + 3]});
                z = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ah, B, z, 0, 0, 0);
                z = __builtin_amdgcn_mfma_f32_32x32x16_f16(Al, B, z, 0, 0, 0);
                if constexpr (S_LO) {  // S not exactly fp16: third pass with its lo part
                    const h8_t Bl = __builtin_bit_cast(h8_t, a.S_lo[n * 16 + ch]);
                    z = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ah, Bl, z, 0, 0, 0);
                }
            }
            // register rr: lanes 0-31 hold key 8(rr/4) + rr%4, lanes 32-63 key
            // 8(rr/4) + 4 + rr%4, columns = outputs 32 nb + (lane % 32)
            uint32_t acc = sgnw[nb];
            StaticFor<0, 16>::run([&](auto kk) {
                constexpr int rr = decltype(kk)::value;
                constexpr int k0 = 8 * (rr / 4) + rr % 4;
                const uint64_t m = __builtin_amdgcn_ballot_w64(z[rr] >= 0.0f);
                acc = write_lane_pair<k0, k0 + 4>(acc, m);
            });
            sgnw[nb] = acc;
        }
        // The next tile's rows, then the copy of the tile after it, then this
        // tile's stores (as in k_quantize).  The rows are read only now: held
        // through the projection they would not fit in the registers.
        const bool has_next = next < n_tiles;
        int64_t after = n_tiles;
        if (has_next) {
            after = blockIdx.x + qjl_take_rows(L, lane, w, &next_tile) * G;
            if (after < n_tiles) issue(after);
        }
        if (v < g.nv) {  // lanes of keys past a ragged tail encoded stale rows
            const int64_t key = g.v0 + v;
            uint32_t *dst = reinterpret_cast<uint32_t *>(a.codes + key * BITS);
#pragma unroll
            for (int k = 0; k < BITS; ++k) {
                dst[h * BITS + k] = out[k];
                dst[(2 + h) * BITS + k] = out[BITS + k];
            }
            if (h == 0) {
                a.norms[key] = rho;
                a.signs[key] = u4_t{sgnw[0], sgnw[1], sgnw[2], sgnw[3]};
                a.gamma[key] = __builtin_sqrtf(g2) * 0.08838834764831845f;  // ||e|| / sqrt(d)
            }
        }
        if (!has_next) break;
        tile = next;
        next = after;
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
    const int64_t tiles_per_bh = (T + kTileH - 1) / kTileH;
    const int64_t n_tiles = tiles_per_bh * B * ctx->H;
    // one workgroup per CU, each with at least one tile
    int64_t blocks = n_tiles;
    if (blocks > (int64_t)ctx->n_cu) blocks = ctx->n_cu;
    if (n_tiles >= (int64_t)1 << 31) return hipErrorInvalidValue;  // 32-bit tile indices
    const TileMap mp = make_map(T, ctx->H, tiles_per_bh);
    if (a.S_lo)
        hipLaunchKernelGGL((k_quantize_qjl<BITS, true>), dim3((unsigned)blocks), dim3(kWavesJ * 64), 0, s, a,
                           (const uint32_t *)ctx->d_sgnmask, ht, mp, n_tiles);
    else
        hipLaunchKernelGGL((k_quantize_qjl<BITS, false>), dim3((unsigned)blocks), dim3(kWavesJ * 64), 0, s, a,
                           (const uint32_t *)ctx->d_sgnmask, ht, mp, n_tiles);
    return hipGetLastError();
}

template <int BITS>
hipError_t run(const kvq_ctx *ctx, const QArgs &a, int n_tensors, int64_t B, int64_t T, hipStream_t s)
{
    HalfThresholds ht{};
    const int L = 1 << BITS;
    for (int k = 0; k < L / 2 - 1; ++k) ht.p[k] = ctx->cb.t[L / 2 + k];
    const int64_t tiles_per_bh = (T + kTileH - 1) / kTileH;
    const int64_t n_tiles = tiles_per_bh * B * ctx->H;
    // one workgroup per CU, each with at least one tile
    int64_t blocks = n_tiles * n_tensors;
    if (blocks > (int64_t)ctx->n_cu) blocks = ctx->n_cu;
    if (n_tiles * n_tensors >= (int64_t)1 << 31) return hipErrorInvalidValue;  // 32-bit tile indices
    hipLaunchKernelGGL(k_quantize<BITS>, dim3((unsigned)blocks), dim3(kWavesQ * 64), 0, s, a,
                       (const uint32_t *)ctx->d_sgnmask_h, ht, make_map(T, ctx->H, tiles_per_bh), n_tiles,
                       n_tensors);
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
