// NSN vector quantisation ("NSNQuant", Metodologia sec. 1-3): per head over
// the tokens of one call
//   a_t = sqrt(d) x_t / ||x_t||,  s1_t = ||x_t|| / sqrt(d)     (normalise)
//   o   = mean_t a_t                                          (shift)
//   b_t = a_t - o,  s2_t = ||b_t|| / sqrt(d)                  (normalise)
//   z_t = H (b_t / s2_t) / sqrt(d) = H b_t / ||b_t||          (Hadamard)
// and every 8-dim sub-vector of z_t is replaced by the index of the nearest
// entry of a 256 x 8 codebook (squared Euclidean distance, lowest index on
// ties).
//
// Three launches: (1) partial channel sums of a_t per (head, token chunk),
// (2) o per head from those partials in a fixed order (deterministic), (3)
// the per-token transform and the search.  The search is a contraction of
// the 16 sub-vectors of 32 tokens with the codebook: score_j = <z_s, C_j> -
// ||C_j||^2 / 2 (the nearest entry has the largest score), on the matrix
// cores, codewords as rows and tokens as columns, the bias preloaded in the
// accumulator (details at k_nsn_vq).  The scores must be exact to about 1e-6,
// so z and the codebook are split into fp16 hi + lo parts.
#include "kvq_internal.h"

namespace kvq {
KVQ_DEBUG_UNIT(nsn, 3)
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef float f16v_t __attribute__((ext_vector_type(16)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;
constexpr int kChunk = kNsnChunk;  // tokens per stats block
constexpr float kSqrtD = 11.313708498984761f;

__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Skewed direct-to-LDS tile copy (chunk c of vector v lands in slot (c + v) % 16).
// Always 16 copy instructions with every lane active (rows past nv re-read
// the last row), so that a wait can count them.
__device__ __forceinline__ void tile_to_lds(const u4_t *src, int nv, u4_t *L, int lane)
{
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

__device__ __forceinline__ void read_row(const u4_t *L, int lane, uint32_t *w)
{
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const u4_t v = L[lane * 16 + ((c + lane) & 15)];
        w[4 * c + 0] = v.x;
        w[4 * c + 1] = v.y;
        w[4 * c + 2] = v.z;
        w[4 * c + 3] = v.w;
    }
}

// ||x||^2 of a row as two chains over its halves, then their sum: the search
// kernel holds the halves in two lanes and must obtain the same value (a_t is
// rounded identically in both passes).
__device__ __forceinline__ float norm2_f16(const uint32_t *w)
{
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
        const h2_t p = __builtin_bit_cast(h2_t, w[k]), q = __builtin_bit_cast(h2_t, w[32 + k]);
        s0 = __builtin_amdgcn_fdot2(p, p, s0, false);
        s1 = __builtin_amdgcn_fdot2(q, q, s1, false);
    }
    return s0 + s1;
}

// (1) partial sums over token chunks of a_t = sqrt(d) x_t / ||x_t||.
// Block (h, chunk), kStatWaves waves with one 16 KiB tile buffer each.  A wave
// waits for its tile, reads it into registers twice (lane = token: the whole
// row for the norm; lane = channel pair: dword `lane` of every row), sends the
// copy of its next tile into the freed buffer, and only then does the
// arithmetic, so its next copy is in flight meanwhile.  Rows past the end of
// the chunk hold a copy of the last row and get the factor 0.
constexpr int kStatWaves = 8;
__global__ __launch_bounds__(64 * kStatWaves) void k_nsn_stats(const u4_t *__restrict__ x,
                                                               float *__restrict__ part, int64_t T, int n_chunks,
                                                               int64_t ldx)
{
    __shared__ u4_t lds[kStatWaves][kTile * 16];  // 128 KiB
    __shared__ float red[kStatWaves][kD];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = blockIdx.x / n_chunks, chunk = blockIdx.x % n_chunks;
    const int64_t c0 = (int64_t)chunk * kChunk, c1 = min(T, c0 + kChunk);
    KVQ_CHECK(c0 < c1 && T <= ldx);
    KVQ_POISON_LDS(lds, kStatWaves * kTile * 16 * 4, threadIdx.x, 64 * kStatWaves);
    KVQ_POISON_LDS(red, kStatWaves * kD, threadIdx.x, 64 * kStatWaves);
    if (KVQ_DEBUG_ON) __syncthreads();
    const u4_t *xh = x + (int64_t)h * ldx * 16;  // the head's tokens (ldx apart per head)
    u4_t *L = lds[wv];
    const uint32_t *Ld = (const uint32_t *)L;
    // dword `lane` of row t sits at 64 t + 4 ((lane / 4 + t) mod 16) + lane mod 4
    int cofs[16];
#pragma unroll
    for (int b = 0; b < 16; ++b)
        cofs[b] = 4 * (((lane >> 2) + b) & 15) + (lane & 3);
    float acc0 = 0.0f, acc1 = 0.0f;
    int64_t t0 = c0 + (int64_t)wv * kTile;
    if (t0 < c1)
        tile_to_lds(xh + t0 * 16, (int)min((int64_t)kTile, c1 - t0), L, lane);
    for (; t0 < c1; t0 += kStatWaves * kTile) {
        const int nv = (int)min((int64_t)kTile, c1 - t0);
        wait_vm();
        uint32_t w[64], col[kTile];
        read_row(L, lane, w);
#pragma unroll
        for (int t = 0; t < kTile; ++t)
            col[t] = Ld[64 * t + cofs[t & 15]];
        wait_lgkm();
        __builtin_amdgcn_wave_barrier();
        const int64_t tn = t0 + kStatWaves * kTile;
        if (tn < c1)
            tile_to_lds(xh + tn * 16, (int)min((int64_t)kTile, c1 - tn), L, lane);
        const float ss = norm2_f16(w);
        const float inv = (lane < nv && ss > 0.0f) ? kSqrtD / __builtin_sqrtf(ss) : 0.0f;
#pragma unroll
        for (int t = 0; t < kTile; ++t) {
            const float it = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, inv), t));
            const h2_t p = __builtin_bit_cast(h2_t, col[t]);
            acc0 = fmaf((float)p.x, it, acc0);
            acc1 = fmaf((float)p.y, it, acc1);
        }
    }
    red[wv][2 * lane] = acc0;
    red[wv][2 * lane + 1] = acc1;
    __syncthreads();
    if (threadIdx.x < kD) {
        const int i = threadIdx.x;
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < kStatWaves; ++k)
            s += red[k][i];
        part[((int64_t)h * n_chunks + chunk) * kD + i] = s;
    }
}

// (2) o[h][i] = sum over chunks / T, in a fixed order (deterministic): thread
// group j (of 8) sums chunks j, j + 8, ... with its loads in flight together,
// then the 8 group sums are added in order.
// Double quantisation (oq non-NULL): the head's 128 means become 4-bit codes
// over [lo, lo + 15 step] (lo = min, step = range / 15, nearest level), o
// receives the dequantised means lo + code step that the search shifts by,
// oq the codes (channel i in byte i / 2, low nibble for even i), op (lo, step).
constexpr int kMeanGroups = 8;
__device__ __forceinline__ float lanes_min(float x)
{
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x = fminf(x, __shfl_xor(x, m));
    return x;
}
__device__ __forceinline__ float lanes_max(float x)
{
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}
// 4-bit code of v in [lo, lo + 15 step]: the nearest level (0 when step = 0)
__device__ __forceinline__ int dq4_code(float v, float lo, float step)
{
    if (!(step > 0.0f)) return 0;
    const int c = (int)floorf((v - lo) / step + 0.5f);
    return c < 0 ? 0 : c > 15 ? 15 : c;
}
__global__ __launch_bounds__(kD * kMeanGroups) void k_nsn_mean(const float *__restrict__ part,
                                                              float *__restrict__ o, int64_t T, int n_chunks,
                                                              int64_t ldo, uint8_t *__restrict__ oq,
                                                              float *__restrict__ op)
{
    __shared__ float red[kMeanGroups][kD];
    const int h = blockIdx.x, i = threadIdx.x & (kD - 1), j = threadIdx.x >> 7;
    const float *ph = part + (int64_t)h * n_chunks * kD + i;
    float s = 0.0f;
    int c = j;
    for (; c + 7 * kMeanGroups < n_chunks; c += 8 * kMeanGroups) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = ph[(int64_t)(c + u * kMeanGroups) * kD];
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; c < n_chunks; c += kMeanGroups) s += ph[(int64_t)c * kD];
    red[j][i] = s;
    __syncthreads();
    float ov = 0.0f;
    if (j == 0) {
        float t = 0.0f;
#pragma unroll
        for (int g = 0; g < kMeanGroups; ++g) t += red[g][i];
        ov = t / (float)T;
    }
    if (!oq) {
        if (j == 0) o[h * ldo + i] = ov;
        return;
    }
    __shared__ float ext[2][2];  // per wave of the 128 channels: min, max
    if (j == 0) {
        const float a = lanes_min(ov), b = lanes_max(ov);
        if ((i & 63) == 0) {
            ext[i >> 6][0] = a;
            ext[i >> 6][1] = b;
        }
    }
    __syncthreads();
    if (j == 0) {
        const float lo = fminf(ext[0][0], ext[1][0]), hi = fmaxf(ext[0][1], ext[1][1]);
        const float step = (hi - lo) / 15.0f;
        const int c = dq4_code(ov, lo, step);
        const int c_next = __shfl_xor(c, 1);
        o[h * ldo + i] = fmaf((float)c, step, lo);
        if (!(i & 1)) oq[h * (kD / 2) + i / 2] = (uint8_t)(c | (c_next << 4));
        if (i == 0) {
            op[2 * h] = lo;
            op[2 * h + 1] = step;
        }
    }
}

// (v0, v1) = hi + lo as packed fp16 pairs.  hi is v truncated to fp16
// (v_cvt_pkrtz: the 11 leading significant bits in the fp16 normal range, so
// v - hi is exact in fp32), and lo = v - hi rounded once to fp16, formed by
// mixed-precision FMAs from the packed hi itself: the hi that is subtracted is
// the hi that is stored.  |hi + lo - v| <= 2^-21 |v| (2^-25 absolute below the
// fp16 normal range).  Each pair costs one conversion and two FMAs.
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

// The 16 scores of one accumulator, each with its position r in its low
// four mantissa bits (as 15 - r), reduced to their maximum (v_max3 tree:
// this file is compiled without NaN semantics, the scores being finite sums
// of finite products).
__device__ __forceinline__ float marked(float x, uint32_t r)
{
    return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, x) & ~15u) | (15u - r));
}
__device__ __forceinline__ float max16_marked(const f16v_t &a)
{
    float e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = marked(a[r], (uint32_t)r);
    const float m0 = fmaxf(fmaxf(e[0], e[1]), e[2]), m1 = fmaxf(fmaxf(e[3], e[4]), e[5]);
    const float m2 = fmaxf(fmaxf(e[6], e[7]), e[8]), m3 = fmaxf(fmaxf(e[9], e[10]), e[11]);
    const float m4 = fmaxf(fmaxf(e[12], e[13]), e[14]);
    return fmaxf(fmaxf(fmaxf(fmaxf(m0, m1), m2), fmaxf(m3, m4)), e[15]);
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * 16 + (chunk ^ (row & 15)); }

struct VqArgs {
    const u4_t *x;
    const u4_t *cb_hi;    // [256] entries of 8 fp16 (hi parts)
    const u2_t *cb_lo;    // [256][2] lo parts, dims 4q .. 4q + 3 at index 2 j + q (unused if exactly fp16)
    const float *bias;    // [256] -||C_j||^2 / 2
    u4_t *codes;          // [H][T][16 bytes]
    float *s1, *s2;       // [H][T] (s1 may be NULL with s1q)
    uint8_t *s1q;         // double quantisation: [H][ldq] 4-bit s1 codes (token t in byte t / 2), or NULL
    float *s1p;           // [H][nblk][2] (lo, step) per block of 32 tokens (one tile)
    int64_t ldq, nblk;
};

// (3) per-token transform and nearest-entry search.  Tiles of 32 tokens of
// one head, two lanes per token: lane 32h + v holds coordinates
// [64 h, 64 h + 64) of token v while they are transformed.  One workgroup of
// 8 waves per CU (two per SIMD) claims tiles from an LDS counter as the
// quantize kernels do; each tile is copied straight into LDS together with
// the head's channel means.  The block also stages the codebook.
//
// Transform: a = sqrt(d) x / ||x|| (||x||^2 summed as norm2_f16 does, so that
// a is rounded exactly as in the stats pass), b = a - o, then six butterfly
// stages inside the lane and the stride-64 stage across the halves with
// gfx950 half swaps.  The swap pairs register 8t + k with 8t + 4 + k
// (k < 4), so that afterwards both halves hold sub-vector s in registers
// R(s) = 8 (s mod 8) + 4 (s / 8) .. + 3: half 0 its dims 0..3, half 1 its
// dims 4..7.
//
// Search, per block of 32 codewords (MFMA rows; tokens are the columns): one
// v_mfma_f32_32x32x16_f16 gives C_hi . (z_hi + z_lo) + bias.  Its k slots
// are split between the lane halves exactly as the dims of z are: half h
// supplies dims 4h .. 4h+3 of z_hi (k = 8h .. 8h+3) and of z_lo (k = 8h+4
// .. 8h+7), and the A operand holds dims 4h .. 4h+3 of C_hi twice, so the
// operands come straight from registers.  One v_mfma_f32_32x32x8_f16 adds
// C_lo . z_hi when the codebook is not fp16-exact.  A lane then holds 16
// scores of its token, register r being codeword 32 mb + 8 (r/4) + 4 h + r%4.
// The score's low four mantissa bits are replaced by 15 - r, so that one
// max3 tree over the 16 values yields the best score together with its
// position (on a tie in the other 28 bits the lower codeword wins); the lane
// keeps, per sub-vector, that value and the block mb (strictly larger in
// increasing block order).  The lane holding the other 16 codewords of each
// block does the same, and the better of the two (lower index on ties) is
// the code.  The marking changes a score by at most 15 units in the last
// place, about 4e-6 for the scores here, so it can only reorder entries whose
// bisecting hyperplane lies within that distance of z_s: a decision inside
// the 1e-5 band the parity checks allow.  About 1.7 VALU operations per
// (sub-vector, codeword), and no table reads after the search.
constexpr int kTileN = 32;           // tokens per tile of the search
constexpr int kWavesN = 8;           // waves per workgroup (two per SIMD)
constexpr int kRowsN = kTileN * 16;  // 16-byte chunks of x per tile
static_assert(kTileN == kNsnDqBlock, "a block of double-quantised s1 is one search tile");
constexpr int kBufN = kRowsN + 64;   // + two slots of the head's 128 channel means

// Rows of the tile: chunk c of row v at slot 16 v + ((c + v) mod 16), so the
// 16 lanes of a half that read chunk 8h + k of 16 consecutive rows hit 16
// different bank groups.  Copy instruction j writes slots [64 j, 64 j + 64)
// (rows 4j .. 4j+3, one contiguous KiB); the chunk a lane fetches depends on
// j only through j mod 4.  Two more instructions copy the 128 means.  Every
// call issues exactly 10 load instructions with all lanes active; rows past a
// ragged tail re-read the last valid row and are never stored.  The means go
// to slot Lo: a wave alternates between two slots, so that the copy of the
// tile after next never writes the means the current tile is still reading.
__device__ __forceinline__ void nsn_tile_to_lds(const u4_t *src, int nv, const float *oh, u4_t *L, u4_t *Lo, int lane)
{
    asm volatile("" : "+v"(lane));
    if (nv == kTileN) {
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
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(oh + lane),
                                     (__attribute__((address_space(3))) void *)(Lo), 4, 0, 0);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(oh + 64 + lane),
                                     (__attribute__((address_space(3))) void *)(Lo + 16), 4, 0, 0);
}

// Wait for the tile copy, read half row h of token v into w (lane 32h + v),
// and draw the wave's next ticket (the atomic goes out with the row reads:
// the compiler makes any LDS access wait for all copies into LDS in flight).
__device__ __forceinline__ int nsn_take_rows(const u4_t *L, int lane, uint32_t *w, int *counter)
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" : "+v"(lane));
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    const int v = lane & 31, h = lane >> 5;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const u4_t x = L[16 * v + ((8 * h + k + v) & 15)];
        w[4 * k + 0] = x.x;
        w[4 * k + 1] = x.y;
        w[4 * k + 2] = x.z;
        w[4 * k + 3] = x.w;
    }
    int t = 0;
    if (lane == 0) t = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    wait_lgkm();
    __builtin_amdgcn_wave_barrier();
    return __builtin_amdgcn_readfirstlane(t);
}

// x' = [x_lo | y_lo], y' = [x_hi | y_hi] (gfx950 swap of lanes 32..63 of x
// with lanes 0..31 of y)
__device__ __forceinline__ void swap_halves(float &x, float &y)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y),
                                                    false, false);
    x = __builtin_bit_cast(float, (unsigned)r[0]);
    y = __builtin_bit_cast(float, (unsigned)r[1]);
}
// value of x in lane l ^ 32
__device__ __forceinline__ float other_half(float x, bool upper)
{
    float p = x, q = x;
    swap_halves(p, q);
    return upper ? p : q;
}
__device__ __forceinline__ int other_half_i(int x, bool upper)
{
    return __builtin_bit_cast(int, other_half(__builtin_bit_cast(float, x), upper));
}

// The NSN transform of a tile row held by lane 32 h + v (half h of token v,
// w = its 64 fp16 coordinates as pairs; oL = the same 64 channel means):
// a = sqrt(d) x / ||x|| (||x||^2 summed as norm2_f16 does, so that a is
// rounded exactly as in the statistics pass), b = a - o, then six butterfly
// stages inside the lane and the stride-64 stage across the halves.  Out:
// nx = ||x||, nb = ||b|| and z = H b / ||b||, whose sub-vector s (dims
// 8 s .. 8 s + 7) this half holds as dims 4 h .. 4 h + 3 in zh[s] (fp16 high
// parts) and zl[s] (the fp16 rounding of the rest).
__device__ __forceinline__ void nsn_z(const uint32_t (&w)[32], const f4_t *oL, float &nx, float &nb, u2_t (&zh)[16],
                                      u2_t (&zl)[16])
{
    // ||x||^2: this half's chain, then (half 0) + (half 1) as norm2_f16
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
        const h2_t p = __builtin_bit_cast(h2_t, w[k]);
        ss = __builtin_amdgcn_fdot2(p, p, ss, false);
    }
    {
        float p = ss, q = ss;
        swap_halves(p, q);
        ss = p + q;
    }
    nx = __builtin_sqrtf(ss);
    const float inv = ss > 0.0f ? kSqrtD / nx : 0.0f;
    float y[64];
    {
        // a_t is rounded as in the stats pass before o is subtracted, so
        // a single token (o = a_t) gives b = 0 exactly
#pragma clang fp contract(off)
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const f4_t ov = oL[k];
            const h2_t p0 = __builtin_bit_cast(h2_t, w[2 * k]), p1 = __builtin_bit_cast(h2_t, w[2 * k + 1]);
            y[4 * k] = (float)p0.x * inv - ov.x;
            y[4 * k + 1] = (float)p0.y * inv - ov.y;
            y[4 * k + 2] = (float)p1.x * inv - ov.z;
            y[4 * k + 3] = (float)p1.y * inv - ov.w;
        }
    }
    float nb2 = 0.0f;
#pragma unroll
    for (int k = 0; k < 64; ++k) nb2 = fmaf(y[k], y[k], nb2);
    {
        float p = nb2, q = nb2;
        swap_halves(p, q);
        nb2 = p + q;
    }
#pragma unroll
    for (int st = 1; st < 64; st <<= 1) {
#pragma unroll
        for (int i = 0; i < 64; i += 2 * st) {
#pragma unroll
            for (int j = i; j < i + st; ++j) {
                const float p0 = y[j], p1 = y[j + st];
                y[j] = p0 + p1;
                y[j + st] = p0 - p1;
            }
        }
    }
    // stride-64 stage: register p = 8t + k (k < 4) with q = p + 4
#pragma unroll
    for (int p = 0; p < 64; ++p) {
        if ((p & 4) != 0) continue;
        float x0 = y[p], x1 = y[p + 4];
        swap_halves(x0, x1);
        y[p] = x0 + x1;
        y[p + 4] = x0 - x1;
    }
    nb = __builtin_sqrtf(nb2);
    const float invb = nb2 > 0.0f ? 1.0f / nb : 0.0f;
    // z = H b / ||b||: this half's four dims of each sub-vector as fp16
    // hi + lo pairs
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        const int base = 8 * (s & 7) + 4 * (s >> 3);
        const SplitPair p01 = split_pair(y[base] * invb, y[base + 1] * invb);
        const SplitPair p23 = split_pair(y[base + 2] * invb, y[base + 3] * invb);
        zh[s] = u2_t{p01.hi, p23.hi};
        zl[s] = u2_t{p01.lo, p23.lo};
    }
}

// ADAPT: the adaptive scale (NSNQuant, Metodologia sec. 3, "Ajuste de
// Escala"): s2 is stored as alpha s2 with alpha = ||z||^2 / <z, zq> = d /
// <z, zq> (zq the selected entries; alpha = 1 when <z, zq> <= 0), so that the
// reconstruction s1 (s2 H zq / sqrt(d) + o) preserves the component of the
// token along itself.  <z, zq> is summed from the exact fp16 hi + lo parts of
// z and of the entries once the codes are known.
template <bool CB_LO, bool ADAPT>
// o: channel means [H][128]
__global__ __launch_bounds__(kWavesN * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_nsn_vq(
    VqArgs a, const float *__restrict__ o, int64_t T, int H, int64_t tiles_per_h, int64_t n_tiles, int64_t ldx,
    int64_t ldo, int64_t ldt)
{
    // ldx, ldt: tokens between heads in the input and in the outputs; ldo:
    // floats between the heads' means
    __shared__ u4_t s_cbA[2 * kVqK];  // entry j, half q: dims 4q .. 4q+3 of C_hi, twice
    __shared__ u2_t s_cbl[2 * kVqK];  // lo parts, dims 4q .. 4q+3 at 2 j + q
    __shared__ float s_bias[kVqK];
    __shared__ u4_t lds[kWavesN][kBufN];
    __shared__ int next_tile;
    const int tid = threadIdx.x;
    KVQ_POISON_LDS(s_cbA, 2 * kVqK * 4, tid, kWavesN * 64);
    KVQ_POISON_LDS(s_cbl, 2 * kVqK * 2, tid, kWavesN * 64);
    KVQ_POISON_LDS(s_bias, kVqK, tid, kWavesN * 64);
    KVQ_POISON_LDS(lds, kWavesN * kBufN * 4, tid, kWavesN * 64);
    KVQ_CHECK(n_tiles % tiles_per_h == 0 && tiles_per_h * kTileN >= T && T <= ldx && T <= ldt);
    if (KVQ_DEBUG_ON) __syncthreads();
    for (int j = tid; j < kVqK; j += kWavesN * 64) {
        const u4_t c = a.cb_hi[j];
        s_cbA[2 * j] = u4_t{c.x, c.y, c.x, c.y};
        s_cbA[2 * j + 1] = u4_t{c.z, c.w, c.z, c.w};
        if constexpr (CB_LO) {
            s_cbl[2 * j] = a.cb_lo[2 * j];
            s_cbl[2 * j + 1] = a.cb_lo[2 * j + 1];
        }
        s_bias[j] = a.bias[j];
    }
    if (tid == 0) next_tile = kWavesN;
    __syncthreads();

    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    u4_t *L = lds[wv];
    const int v = lane & 31, h = lane >> 5;
    const bool upper = h != 0;
    const int64_t G = gridDim.x;
    int64_t tile = blockIdx.x + wv * G;
    if (tile >= n_tiles) return;  // wave-uniform
    auto issue = [&](int64_t t, int slot) {
        int64_t tph = tiles_per_h;
        asm volatile("" : "+s"(tph));
        const int64_t hq = t / tph;
        const int64_t tq = (t - hq * tph) * kTileN;
        const int nq = (int)min((int64_t)kTileN, T - tq);
        KVQ_CHECK(t >= 0 && t < n_tiles && nq >= 1 && tq >= 0);
        nsn_tile_to_lds(a.x + (hq * ldx + tq) * 16, nq, o + hq * ldo, L, L + kRowsN + 32 * slot, lane);
    };
    uint32_t w[32];
    int ord = 0;  // ordinal of the current tile among this wave's: its means are in slot ord % 2
    issue(tile, 0);
    int64_t next = blockIdx.x + nsn_take_rows(L, lane, w, &next_tile) * G;
    if (next < n_tiles) issue(next, 1);
    for (;;) {
        int64_t tph = tiles_per_h;
        asm volatile("" : "+s"(tph));
        const int64_t hh = tile / tph;
        const int64_t t0 = (tile - hh * tph) * kTileN;
        const int nv = (int)min((int64_t)kTileN, T - t0);
        const int64_t v0 = hh * ldt + t0;

        // this half's 64 means (the slot the copy of the next tile does not write)
        const f4_t *oL = reinterpret_cast<const f4_t *>(L + kRowsN + 32 * (ord & 1)) + 16 * h;
        float nx, nb;
        u2_t zh[16], zl[16];
        nsn_z(w, oL, nx, nb, zh, zl);

        float bm[16];
        int bg[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            bm[s] = -INFINITY;
            bg[s] = 0;
        }
#pragma unroll 1
        for (int mb = 0; mb < 8; ++mb) {
            const int ent = 32 * mb + v;  // codeword row of this lane's A operand
            const h8_t A16 = __builtin_bit_cast(h8_t, s_cbA[2 * ent + h]);
            h4_t A8 = {};
            if constexpr (CB_LO) A8 = __builtin_bit_cast(h4_t, s_cbl[2 * ent + h]);
            // accumulator rows of this lane: codeword 32 mb + 8 (r/4) + 4 h + r%4
            f16v_t bias;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f4_t bq = reinterpret_cast<const f4_t *>(s_bias)[(32 * mb + 8 * r4 + 4 * h) >> 2];
                bias[4 * r4] = bq.x;
                bias[4 * r4 + 1] = bq.y;
                bias[4 * r4 + 2] = bq.z;
                bias[4 * r4 + 3] = bq.w;
            }
            // four sub-vectors at a time in independent accumulators, so that
            // the matrix cores run while earlier results are scanned
#pragma unroll
            for (int s4 = 0; s4 < 16; s4 += 4) {
                f16v_t acc[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const u2_t zhs = zh[s4 + u], zls = zl[s4 + u];
                    const h8_t B16 = __builtin_bit_cast(h8_t, u4_t{zhs.x, zhs.y, zls.x, zls.y});
                    acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A16, B16, bias, 0, 0, 0);
                }
                if constexpr (CB_LO) {
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        acc[u] = __builtin_amdgcn_mfma_f32_32x32x8f16(A8, __builtin_bit_cast(h4_t, zh[s4 + u]),
                                                                      acc[u], 0, 0, 0);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int s = s4 + u;
                    const float m = max16_marked(acc[u]);
                    const bool better = m > bm[s];
                    bm[s] = better ? m : bm[s];
                    bg[s] = better ? mb : bg[s];
                }
            }
        }
        // the entry of each sub-vector's best marked score, then the better of
        // the two halves (each searched the other 16 codewords of every block)
        uint32_t code[4] = {0u, 0u, 0u, 0u};
        float dot = 0.0f;  // <z, zq> of this half's dims (adaptive scale)
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int r = 15 - (int)(__builtin_bit_cast(uint32_t, bm[s]) & 15u);
            const int bi = 32 * bg[s] + 8 * (r >> 2) + 4 * h + (r & 3);
            const float ob = other_half(bm[s], upper);
            const int oi = other_half_i(bi, upper);
            const int win = (ob > bm[s] || (ob == bm[s] && oi < bi)) ? oi : bi;
            code[s >> 2] |= (uint32_t)win << (8 * (s & 3));
            if constexpr (ADAPT) {
                // (z_hi + z_lo) . (c_hi + c_lo) over dims 4h .. 4h+3 as packed
                // fp16 dot products (exact products, fp32 sums)
                const u4_t ch = s_cbA[2 * win + h];  // dims 4h .. 4h+3 of the entry (twice)
                const u2_t zhs = zh[s], zls = zl[s];
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const h2_t c2 = __builtin_bit_cast(h2_t, p ? ch.y : ch.x);
                    dot = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, p ? zhs.y : zhs.x), c2, dot, false);
                    dot = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, p ? zls.y : zls.x), c2, dot, false);
                }
                if constexpr (CB_LO) {
                    const u2_t cl = s_cbl[2 * win + h];
#pragma unroll
                    for (int p = 0; p < 2; ++p) {
                        const h2_t c2 = __builtin_bit_cast(h2_t, p ? cl.y : cl.x);
                        dot = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, p ? zhs.y : zhs.x), c2, dot, false);
                        dot = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, p ? zls.y : zls.x), c2, dot, false);
                    }
                }
            }
        }
        float s2v = nb / kSqrtD;
        if constexpr (ADAPT) {
            dot += other_half(dot, upper);
            if (dot > 0.0f) s2v *= (float)kD / dot;
        }
        // The next tile's rows, then the copy of the tile after it, then this
        // tile's stores.  The rows are read only now: held through the search
        // they would not fit in the registers.
        const bool has_next = next < n_tiles;
        int64_t after = n_tiles;
        if (has_next) {
            after = blockIdx.x + nsn_take_rows(L, lane, w, &next_tile) * G;
            if (after < n_tiles) issue(after, ord & 1);  // the slot of this tile, no longer read
        }
        const float s1v = nx / kSqrtD;
        if (!upper && v < nv) {  // lanes of tokens past a ragged tail searched stale rows
            const int64_t t = v0 + v;
            KVQ_CHECK(t0 + v < T && hh < n_tiles / tiles_per_h);
            a.codes[t] = u4_t{code[0], code[1], code[2], code[3]};
            if (a.s1) a.s1[t] = s1v;
            a.s2[t] = s2v;
        }
        if (a.s1q) {
            // s1 in 4 bits over the tile's tokens (both halves hold the same values)
            const float lo = lanes_min(v < nv ? s1v : __builtin_inff());
            const float hi = lanes_max(v < nv ? s1v : -__builtin_inff());
            const float step = (hi - lo) / 15.0f;
            const int c = dq4_code(s1v, lo, step);
            const int c_pair = __shfl_xor(c, 1);  // every lane takes part in the exchange
            const int c_next = v + 1 < nv ? c_pair : 0;
            if (!upper && v < nv && !(v & 1)) a.s1q[hh * a.ldq + (t0 + v) / 2] = (uint8_t)(c | (c_next << 4));
            if (lane == 0) {
                float *pp = a.s1p + (hh * a.nblk + t0 / kTileN) * 2;
                pp[0] = lo;
                pp[1] = step;
            }
        }
        if (!has_next) break;
        tile = next;
        next = after;
        ++ord;
    }
}


// ---------------------------------------------------------------------------
// Gain-shape residual quantisation ("GSRQ", q2bstudio: gain-shape k-means
// stages in a residual quantisation pipeline) on the NSN front end: z as for
// NSN-VQ, then per 32-dim sub-vector two stages, each taking the unit shape
// of largest projection onto the running residual (lowest index on ties),
// the gain level by counting thresholds below that projection, and
// subtracting level x shape.  Record of a token: dword 0 = the four stage-1
// shape indices (byte s = sub-vector s), dword 1 = the stage-2 ones, dword 2
// = the four gain bytes c1 | c2 << 4.
//
// The projections are a dense contraction (per stage, 32 tokens x 256 shapes
// x 32 dims for each sub-vector) and run on the matrix cores, in the layout
// of the NSN-VQ search: tiles of 32 tokens, lane 32 h + v holding dims
// 4 h .. 4 h + 3 of every 8-dim chunk of token v's z (nsn_z), the MFMA rows
// being 32 shapes and the columns the tokens.  Per (block of 32 shapes,
// sub-vector S) the four chunks c of S each take one v_mfma_f32_32x32x16_f16,
// S_hi . (z_hi + z_lo) (the A operand holds the lane's four shape dims
// twice), and each pair of chunks one more for S_lo . z_hi (the A operand
// holds the lane's dims of both chunks): the projection to about 2^-22
// relative, as an fp32 dot product.  (A v_mfma_f32_32x32x8_f16 per chunk for
// S_lo . z_hi takes as many cycles as the 32x32x16 form.)  A lane then holds 16 scores
// of its token, register 4 q + e being shape 32 mb + 8 q + 4 h + e.  Each
// group of four (fixed q) is reduced with its position e marked in the two
// low mantissa bits (3 - e, a change of at most 3 units in the last place,
// far inside the 1e-5 decision band), and the groups are compared exactly in
// increasing shape order (strictly greater wins); the two halves' winners are
// compared last (lower index on a tie).  The gain index is a binary search
// over the 15 thresholds; the stage-2 input is r = z - level x shape in fp32,
// split again into fp16 high and low parts.
struct GsrqArgs {
    const u4_t *x;          // [H][T][128] fp16
    const u2_t *shapes16;   // [part hi, lo][stage][cw][256]: u2 word = dims 8 c + 4 h .. + 3 of a shape, cw = 2 c + h
    const float *levels;    // [2][16] gain levels, then [2][15] thresholds
    uint32_t *codes;        // [H][T][3]
    float *s1, *s2;         // [H][T]
};
constexpr int kGsrqM = 32, kGsrqK = 256, kGsrqL = 16;
constexpr int kGsrqShapeU2 = kGsrqK * kGsrqM / 4;  // u2 words (four fp16) per stage table

// One stage for the wave's 32 tokens: zh/zl the sub-vectors (as nsn_z leaves
// them), sh/sl the stage's shape table in LDS (u2 word 256 (2 c + h) + j =
// dims 8 c + 4 h .. + 3 of shape j, so that the 32 lanes of a half read 32
// consecutive words: no bank conflicts).  Out, per sub-vector S: the shape
// index and its (marked) projection, the same in both halves.
__device__ __forceinline__ void gsrq_search(const u2_t *sh, const u2_t *sl, const u2_t (&zh)[16],
                                            const u2_t (&zl)[16], int v, int h, bool upper, int (&jb)[4],
                                            float (&pb)[4])
{
    float bm[4];
    int bg[4];
#pragma unroll
    for (int S = 0; S < 4; ++S) {
        bm[S] = -INFINITY;
        bg[S] = 0;
    }
#pragma unroll 1
    for (int mb = 0; mb < kGsrqK / 32; ++mb) {
        const u2_t *rh = sh + 256 * h + 32 * mb + v, *rl = sl + 256 * h + 32 * mb + v;
        f16v_t acc[4];
#pragma unroll
        for (int S = 0; S < 4; ++S) acc[S] = f16v_t{};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u2_t ah = rh[512 * c];
            const h8_t A16 = __builtin_bit_cast(h8_t, u4_t{ah.x, ah.y, ah.x, ah.y});
#pragma unroll
            for (int S = 0; S < 4; ++S) {
                const int s = 4 * S + c;
                const h8_t B16 = __builtin_bit_cast(h8_t, u4_t{zh[s].x, zh[s].y, zl[s].x, zl[s].y});
                acc[S] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A16, B16, acc[S], 0, 0, 0);
            }
            if (c & 1) {  // S_lo . z_hi for chunks c - 1 and c
                const u2_t l0 = rl[512 * (c - 1)], l1 = rl[512 * c];
                const h8_t AL = __builtin_bit_cast(h8_t, u4_t{l0.x, l0.y, l1.x, l1.y});
#pragma unroll
                for (int S = 0; S < 4; ++S) {
                    const int s = 4 * S + c;
                    const h8_t BL = __builtin_bit_cast(h8_t, u4_t{zh[s - 1].x, zh[s - 1].y, zh[s].x, zh[s].y});
                    acc[S] = __builtin_amdgcn_mfma_f32_32x32x16_f16(AL, BL, acc[S], 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int S = 0; S < 4; ++S) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float e[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    // the element is copied out first: a bit cast applied to
                    // a vector element directly reads element 0
                    const float x = acc[S][4 * q + k];
                    e[k] = __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, x) & ~3u) | (3u - (uint32_t)k));
                }
                const float m = fmaxf(fmaxf(fmaxf(e[0], e[1]), e[2]), e[3]);
                const bool better = m > bm[S];
                bm[S] = better ? m : bm[S];
                bg[S] = better ? 4 * mb + q : bg[S];
            }
        }
    }
#pragma unroll
    for (int S = 0; S < 4; ++S) {
        const int e = 3 - (int)(__builtin_bit_cast(uint32_t, bm[S]) & 3u);
        const int idx = 8 * bg[S] + 4 * h + e;  // 32 mb + 8 q + 4 h + e with bg = 4 mb + q
        const float ob = other_half(bm[S], upper);
        const int oi = other_half_i(idx, upper);
        const bool other = ob > bm[S] || (ob == bm[S] && oi < idx);
        jb[S] = other ? oi : idx;
        pb[S] = other ? ob : bm[S];
    }
}

// Mixed-precision FMAs on fp16 halves held in dwords (SEL: 0 = low half, 1 =
// high half): h2f_sum = fp32 of the two fp16 (hi + lo, exact), and
// fma_h = a * fp16 + c in fp32, each one v_fma_mix_f32.
template <int SEL>
__device__ __forceinline__ float h2f_sum(uint32_t hi, uint32_t lo)
{
    float r;
    if constexpr (SEL == 0)
        asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[0,0,0] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(hi), "v"(lo));
    else
        asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(hi), "v"(lo));
    return r;
}
template <int SEL>
__device__ __forceinline__ float fma_h(float a, uint32_t h, float c)
{
    float r;
    if constexpr (SEL == 0)
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[0,1,0]" : "=v"(r) : "v"(a), "v"(h), "v"(c));
    else
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(r) : "v"(a), "v"(h), "v"(c));
    return r;
}

// number of the 15 ascending thresholds th below p
__device__ __forceinline__ int gsrq_gain(const float *th, float p)
{
    int c = th[7] < p ? 8 : 0;
    c += th[c + 3] < p ? 4 : 0;
    c += th[c + 1] < p ? 2 : 0;
    c += th[c] < p ? 1 : 0;
    return c;
}

// (3) the search, with the tile loop of k_nsn_vq (one workgroup of 8 waves
// per CU claiming 32-token tiles from an LDS counter; tiles copied straight
// into LDS with the head's means).  The block first stages both stages'
// shape tables (fp16 high and low parts, 64 KiB), the levels and thresholds.
__global__ __launch_bounds__(kWavesN * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gsrq_vq(
    GsrqArgs a, const float *__restrict__ o, int64_t T, int64_t tiles_per_h, int64_t n_tiles)
{
    __shared__ u2_t s_sh[2 * 2 * kGsrqShapeU2];  // [part hi, lo][stage][256][8]
    __shared__ float s_tab[2 * kGsrqL + 2 * (kGsrqL - 1)];
    __shared__ u4_t lds[kWavesN][kBufN];
    __shared__ int next_tile;
    const int tid = threadIdx.x;
    KVQ_POISON_LDS(s_sh, 2 * 2 * kGsrqShapeU2 * 2, tid, kWavesN * 64);
    KVQ_POISON_LDS(s_tab, 2 * kGsrqL + 2 * (kGsrqL - 1), tid, kWavesN * 64);
    KVQ_POISON_LDS(lds, kWavesN * kBufN * 4, tid, kWavesN * 64);
    KVQ_CHECK(n_tiles % tiles_per_h == 0 && tiles_per_h * kTileN >= T);
    if (KVQ_DEBUG_ON) __syncthreads();
    {
        const u4_t *src = reinterpret_cast<const u4_t *>(a.shapes16);
        u4_t *dst = reinterpret_cast<u4_t *>(s_sh);
        for (int i = tid; i < 2 * kGsrqShapeU2; i += kWavesN * 64) dst[i] = src[i];
        if (tid < 2 * kGsrqL + 2 * (kGsrqL - 1)) s_tab[tid] = a.levels[tid];
    }
    if (tid == 0) next_tile = kWavesN;
    __syncthreads();

    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    u4_t *L = lds[wv];
    const int v = lane & 31, h = lane >> 5;
    const bool upper = h != 0;
    const int64_t G = gridDim.x;
    int64_t tile = blockIdx.x + wv * G;
    if (tile >= n_tiles) return;  // wave-uniform
    auto issue = [&](int64_t t, int slot) {
        int64_t tph = tiles_per_h;
        asm volatile("" : "+s"(tph));
        const int64_t hq = t / tph;
        const int64_t tq = (t - hq * tph) * kTileN;
        const int nq = (int)min((int64_t)kTileN, T - tq);
        KVQ_CHECK(t >= 0 && t < n_tiles && nq >= 1 && tq >= 0);
        nsn_tile_to_lds(a.x + (hq * T + tq) * 16, nq, o + hq * kD, L, L + kRowsN + 32 * slot, lane);
    };
    const u2_t *sh1 = s_sh, *sh2 = s_sh + kGsrqShapeU2;
    const u2_t *sl1 = s_sh + 2 * kGsrqShapeU2, *sl2 = s_sh + 3 * kGsrqShapeU2;
    const float *lv1 = s_tab, *lv2 = s_tab + kGsrqL;
    const float *th1 = s_tab + 2 * kGsrqL, *th2 = th1 + (kGsrqL - 1);
    uint32_t w[32];
    int ord = 0;  // ordinal of the current tile among this wave's: its means are in slot ord % 2
    issue(tile, 0);
    int64_t next = blockIdx.x + nsn_take_rows(L, lane, w, &next_tile) * G;
    if (next < n_tiles) issue(next, 1);
    for (;;) {
        int64_t tph = tiles_per_h;
        asm volatile("" : "+s"(tph));
        const int64_t hh = tile / tph;
        const int64_t t0 = (tile - hh * tph) * kTileN;
        const int nv = (int)min((int64_t)kTileN, T - t0);

        const f4_t *oL = reinterpret_cast<const f4_t *>(L + kRowsN + 32 * (ord & 1)) + 16 * h;
        float nx, nb;
        u2_t zh[16], zl[16];
        nsn_z(w, oL, nx, nb, zh, zl);

        int j1[4], j2[4], c1[4], c2[4];
        float p[4];
        gsrq_search(sh1, sl1, zh, zl, v, h, upper, j1, p);
        // stage-2 input: r = (z - g S_hi) - g S_lo in fp32 (z from its exact
        // fp16 parts), split again into high and low parts
#pragma unroll
        for (int S = 0; S < 4; ++S) {
            c1[S] = gsrq_gain(th1, p[S]);
            const float ng = -lv1[c1[S]];
            const u2_t *ch = sh1 + 256 * h + j1[S], *cl = sl1 + 256 * h + j1[S];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int s = 4 * S + c;
                const u2_t shw = ch[512 * c], slw = cl[512 * c];
                float r[4];
#pragma unroll
                for (int d = 0; d < 2; ++d) {  // dword d: dims 2 d (low half), 2 d + 1 (high half)
                    const uint32_t zhd = d ? zh[s].y : zh[s].x, zld = d ? zl[s].y : zl[s].x;
                    const uint32_t shd = d ? shw.y : shw.x, sld = d ? slw.y : slw.x;
                    r[2 * d] = fma_h<0>(ng, sld, fma_h<0>(ng, shd, h2f_sum<0>(zhd, zld)));
                    r[2 * d + 1] = fma_h<1>(ng, sld, fma_h<1>(ng, shd, h2f_sum<1>(zhd, zld)));
                }
                const SplitPair p01 = split_pair(r[0], r[1]), p23 = split_pair(r[2], r[3]);
                zh[s] = u2_t{p01.hi, p23.hi};
                zl[s] = u2_t{p01.lo, p23.lo};
            }
        }
        gsrq_search(sh2, sl2, zh, zl, v, h, upper, j2, p);
#pragma unroll
        for (int S = 0; S < 4; ++S) c2[S] = gsrq_gain(th2, p[S]);

        // The next tile's rows, then the copy of the tile after it, then this
        // tile's stores.
        const bool has_next = next < n_tiles;
        int64_t after = n_tiles;
        if (has_next) {
            after = blockIdx.x + nsn_take_rows(L, lane, w, &next_tile) * G;
            if (after < n_tiles) issue(after, ord & 1);  // the slot of this tile, no longer read
        }
        if (!upper && v < nv) {  // lanes of tokens past a ragged tail searched stale rows
            const int64_t t = hh * T + t0 + v;
            KVQ_CHECK(t0 + v < T && hh < n_tiles / tiles_per_h);
            uint32_t d0 = 0, d1 = 0, d2 = 0;
#pragma unroll
            for (int S = 0; S < 4; ++S) {
                d0 |= (uint32_t)j1[S] << (8 * S);
                d1 |= (uint32_t)j2[S] << (8 * S);
                d2 |= (uint32_t)(c1[S] | (c2[S] << 4)) << (8 * S);
            }
            uint32_t *rec = a.codes + t * 3;
            rec[0] = d0;
            rec[1] = d1;
            rec[2] = d2;
            a.s1[t] = nx / kSqrtD;
            a.s2[t] = nb / kSqrtD;
        }
        if (!has_next) break;
        tile = next;
        next = after;
        ++ord;
    }
}

}  // namespace

namespace {
hipError_t nsn_vq_run(const kvq_ctx *ctx, const void *x, int64_t H, int64_t T, int64_t ldx, uint8_t *codes, float *s1,
                      float *s2, int64_t ldt, float *o, int64_t ldo, const NsnDq *dq, void *ws, hipStream_t s);
}  // namespace

hipError_t launch_nsn_vq(const kvq_ctx *ctx, const void *x, int64_t H, int64_t T, uint8_t *codes, float *s1,
                         float *s2, float *o, void *ws, hipStream_t s)
{
    return nsn_vq_run(ctx, x, H, T, T, codes, s1, s2, T, o, kD, nullptr, ws, s);
}

hipError_t launch_nsn_vq_strided(const kvq_ctx *ctx, const void *x, int64_t H, int64_t T, int64_t ldx, uint8_t *codes,
                                 float *s1, float *s2, int64_t ldt, float *o, int64_t ldo, void *ws, hipStream_t s)
{
    return nsn_vq_run(ctx, x, H, T, ldx, codes, s1, s2, ldt, o, ldo, nullptr, ws, s);
}

// Double quantisation: the dequantised means live in the workspace after the
// channel sums.
hipError_t launch_nsn_vq_dq(const kvq_ctx *ctx, const void *x, int64_t H, int64_t T, uint8_t *codes, float *s2,
                            const NsnDq &dq, void *ws, hipStream_t s)
{
    float *ohat = (float *)((char *)ws + nsn_ws_bytes_aligned(H, T));
    return nsn_vq_run(ctx, x, H, T, T, codes, nullptr, s2, T, ohat, kD, &dq, ws, s);
}

namespace {
hipError_t nsn_vq_run(const kvq_ctx *ctx, const void *x, int64_t H, int64_t T, int64_t ldx, uint8_t *codes, float *s1,
                      float *s2, int64_t ldt, float *o, int64_t ldo, const NsnDq *dq, void *ws, hipStream_t s)
{
    const int n_chunks = (int)((T + kChunk - 1) / kChunk);
    float *part = (float *)ws;
    hipLaunchKernelGGL(k_nsn_stats, dim3((unsigned)(H * n_chunks)), dim3(64 * kStatWaves), 0, s, (const u4_t *)x, part, T,
                       n_chunks, ldx);
    hipLaunchKernelGGL(k_nsn_mean, dim3((unsigned)H), dim3(kD * kMeanGroups), 0, s, part, o, T, n_chunks, ldo,
                       dq ? dq->oq : nullptr, dq ? dq->op : nullptr);
    VqArgs a{};
    if (dq) {
        a.s1q = dq->s1q;
        a.s1p = dq->s1p;
        a.ldq = (T + 1) / 2;
        a.nblk = (T + kTileN - 1) / kTileN;
    }
    a.x = (const u4_t *)x;
    a.cb_hi = (const u4_t *)ctx->d_vq16;
    a.cb_lo = (const u2_t *)(ctx->d_vq16 + kVqK * kVqSub);
    a.bias = ctx->d_vqbias;
    a.codes = (u4_t *)codes;
    a.s1 = s1;
    a.s2 = s2;
    const int64_t tiles_per_h = (T + kTileN - 1) / kTileN;
    const int64_t n_tiles = tiles_per_h * H;
    // one workgroup per CU, each with at least one tile
    int64_t blocks = n_tiles;
    if (blocks > ctx->n_cu) blocks = ctx->n_cu;
    const bool adapt = (ctx->nsn_options & KVQ_NSN_ADAPTIVE_SCALE) != 0;
#define KVQ_NSN_LAUNCH(LO, AD)                                                                                     \
    hipLaunchKernelGGL((k_nsn_vq<LO, AD>), dim3((unsigned)blocks), dim3(kWavesN * 64), 0, s, a, (const float *)o, T, \
                       (int)H, tiles_per_h, n_tiles, ldx, ldo, ldt)
    if (ctx->vq_exact_f16) {
        if (adapt) KVQ_NSN_LAUNCH(false, true); else KVQ_NSN_LAUNCH(false, false);
    } else {
        if (adapt) KVQ_NSN_LAUNCH(true, true); else KVQ_NSN_LAUNCH(true, false);
    }
#undef KVQ_NSN_LAUNCH
    return hipGetLastError();
}
}  // namespace

// GSRQ: channel means by the NSN statistics pass, then the search.
hipError_t launch_gsrq(const kvq_ctx *ctx, const void *x, int64_t H, int64_t T, uint8_t *codes, float *s1, float *s2,
                       float *o, void *ws, hipStream_t s)
{
    const int n_chunks = (int)((T + kChunk - 1) / kChunk);
    float *part = (float *)ws;
    hipLaunchKernelGGL(k_nsn_stats, dim3((unsigned)(H * n_chunks)), dim3(64 * kStatWaves), 0, s, (const u4_t *)x, part, T,
                       n_chunks, T);
    hipLaunchKernelGGL(k_nsn_mean, dim3((unsigned)H), dim3(kD * kMeanGroups), 0, s, part, o, T, n_chunks, (int64_t)kD,
                       (uint8_t *)nullptr, (float *)nullptr);
    GsrqArgs a{};
    a.x = (const u4_t *)x;
    a.shapes16 = (const u2_t *)ctx->d_gsrq16;
    a.levels = ctx->d_gsrq + 2 * kGsrqK * kGsrqM;
    a.codes = (uint32_t *)codes;
    a.s1 = s1;
    a.s2 = s2;
    const int64_t tiles_per_h = (T + kTileN - 1) / kTileN;
    const int64_t n_tiles = tiles_per_h * H;
    int64_t blocks = n_tiles;
    if (blocks > ctx->n_cu) blocks = ctx->n_cu;  // one workgroup per CU, each with at least one tile
    hipLaunchKernelGGL(k_gsrq_vq, dim3((unsigned)blocks), dim3(kWavesN * 64), 0, s, a, (const float *)o, T, tiles_per_h,
                       n_tiles);
    return hipGetLastError();
}

}  // namespace kvq
