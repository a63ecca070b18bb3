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
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef float f16v_t __attribute__((ext_vector_type(16)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;
constexpr int kChunk = 1024;  // tokens per stats block
constexpr float kSqrtD = 11.313708498984761f;

__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Skewed direct-to-LDS tile copy (chunk c of vector v lands in slot (c + v) % 16).
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

__device__ __forceinline__ float norm2_f16(const uint32_t *w)
{
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < 64; ++k) {
        const h2_t p = __builtin_bit_cast(h2_t, w[k]);
        ss = __builtin_amdgcn_fdot2(p, p, ss, false);
    }
    return ss;
}

// (1) partial sums over token chunks of a_t = sqrt(d) x_t / ||x_t||.
// Block (h, chunk), 4 waves; lane = token for the norms, then lane = channel
// pair for the sums (rows read back from the staged tile).
__global__ __launch_bounds__(256) void k_nsn_stats(const u4_t *__restrict__ x, float *__restrict__ part,
                                                    int64_t T, int n_chunks)
{
    __shared__ u4_t lds[4][kTile * 16];
    __shared__ float red[4][kD];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = blockIdx.x / n_chunks, chunk = blockIdx.x % n_chunks;
    const int64_t c0 = (int64_t)chunk * kChunk, c1 = min(T, c0 + kChunk);
    u4_t *L = lds[wv];
    float acc0 = 0.0f, acc1 = 0.0f;
    for (int64_t t0 = c0 + (int64_t)wv * kTile; t0 < c1; t0 += 4 * kTile) {
        const int nv = (int)min((int64_t)kTile, c1 - t0);
        tile_to_lds(x + ((int64_t)h * T + t0) * 16, nv, L, lane);
        wait_vm();
        uint32_t w[64];
        read_row(L, lane, w);
        const float ss = norm2_f16(w);
        const float inv = (lane < nv && ss > 0.0f) ? kSqrtD / __builtin_sqrtf(ss) : 0.0f;
        // lane = channel pair (2 lane, 2 lane + 1): dword `lane` of every row
        for (int t = 0; t < nv; ++t) {
            const float it = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, inv), t));
            const u4_t v = L[t * 16 + (((lane >> 2) + t) & 15)];
            const uint32_t d = (lane & 3) == 0 ? v.x : (lane & 3) == 1 ? v.y : (lane & 3) == 2 ? v.z : v.w;
            const h2_t p = __builtin_bit_cast(h2_t, d);
            acc0 = fmaf((float)p.x, it, acc0);
            acc1 = fmaf((float)p.y, it, acc1);
        }
        wait_lgkm();
        __builtin_amdgcn_wave_barrier();
    }
    red[wv][2 * lane] = acc0;
    red[wv][2 * lane + 1] = acc1;
    __syncthreads();
    if (threadIdx.x < kD) {
        const int i = threadIdx.x;
        part[((int64_t)h * n_chunks + chunk) * kD + i] = (red[0][i] + red[1][i]) + (red[2][i] + red[3][i]);
    }
}

// (2) o[h][i] = sum over chunks / T, in a fixed order (deterministic): thread
// group j (of 8) sums chunks j, j + 8, ... with its loads in flight together,
// then the 8 group sums are added in order.
constexpr int kMeanGroups = 8;
__global__ __launch_bounds__(kD * kMeanGroups) void k_nsn_mean(const float *__restrict__ part,
                                                              float *__restrict__ o, int64_t T, int n_chunks)
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
    if (j == 0) {
        float t = 0.0f;
#pragma unroll
        for (int g = 0; g < kMeanGroups; ++g) t += red[g][i];
        o[h * kD + i] = t / (float)T;
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

// max of four scores (v_max3 + v_max: this file is compiled without NaN
// semantics, the scores being finite sums of finite products)
__device__ __forceinline__ float max4(float a, float b, float c, float d)
{
    return fmaxf(fmaxf(fmaxf(a, b), c), d);
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * 16 + (chunk ^ (row & 15)); }

struct VqArgs {
    const u4_t *x;
    const u4_t *cb_hi;    // [256] entries of 8 fp16 (hi parts)
    const u2_t *cb_lo;    // [256][2] lo parts, dims 4q .. 4q + 3 at index 2 j + q (unused if exactly fp16)
    const float *cb;      // [256][8] fp32 codebook
    const float *bias;    // [256] -||C_j||^2 / 2
    u4_t *codes;          // [H][T][16 bytes]
    float *s1, *s2;       // [H][T]
};

// (3) per-token transform and nearest-entry search.  One wave per SIMD:
// 16 KiB of LDS for the x tile (reused for the fp16 hi rows of z) and 16 KiB
// for the lo rows; the block also stages the codebook (hi, lo, fp32, biases).
//
// Search, per block of 32 tokens (MFMA columns) and 32 codewords (rows):
// one v_mfma_f32_32x32x16_f16 gives C_hi . (z_hi + z_lo) + bias (k = 0..7
// pairs the hi parts of z with C_hi, k = 8..15 the lo parts with C_hi again),
// and one v_mfma_f32_32x32x8_f16 adds C_lo . z_hi when the codebook is not
// fp16-exact.  A lane then holds 16 scores of one token: four groups of four
// consecutive codewords.  It keeps, per sub-vector, only the best group (its
// maximum, strictly larger in increasing codeword order), and at the end
// recomputes the group's four scores in fp32 from z = z_hi + z_lo and the
// fp32 codebook to pick the entry; the lane holding the other 16 codewords of
// each block does the same, and the better of the two (lower index on ties)
// is the code.  Keeping groups instead of single entries takes the arg max
// bookkeeping from 3 VALU operations per (sub-vector, codeword) to about 1.3.
template <bool CB_LO>
// o: channel means [H][128], a separate read-only argument so that (read
// with a wave-uniform head) it comes through the scalar cache.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_nsn_vq(
    VqArgs a, const float *__restrict__ o, int64_t T, int H, int64_t tiles_per_h, int64_t n_tiles)
{
    static_assert(kVqK == 256, "one codebook entry per thread when staging");
    __shared__ u4_t lds[4][kTile * 16];
    __shared__ u4_t zlo[4][kTile * 16];
    __shared__ u4_t s_cbh[kVqK];
    __shared__ u2_t s_cbl[2 * kVqK];
    __shared__ f4_t s_cb[2 * kVqK];
    __shared__ float s_bias[kVqK];
    const int tid = threadIdx.x;
    s_cbh[tid] = a.cb_hi[tid];
    if constexpr (CB_LO) {
        s_cbl[2 * tid] = a.cb_lo[2 * tid];
        s_cbl[2 * tid + 1] = a.cb_lo[2 * tid + 1];
    }
    s_cb[2 * tid] = reinterpret_cast<const f4_t *>(a.cb)[2 * tid];
    s_cb[2 * tid + 1] = reinterpret_cast<const f4_t *>(a.cb)[2 * tid + 1];
    s_bias[tid] = a.bias[tid];
    __syncthreads();

    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    u4_t *L = lds[wv];
    u4_t *Llo = zlo[wv];
    const int half = lane >> 5, col = lane & 31;

    // Each lane loads its own token's row straight into registers; the next
    // tile's rows are requested before the current tile's search, which hides
    // their latency (the LDS buffers then only hold the z rows).
    const int64_t stride = (int64_t)gridDim.x * 4;
    int64_t tile = (int64_t)blockIdx.x * 4 + wv;
    u4_t xr[16];
    auto load_rows = [&](int64_t t) {
        const int64_t hq = t / tiles_per_h;
        const int64_t tq = (t - hq * tiles_per_h) * kTile;
        const int nq = (int)min((int64_t)kTile, T - tq);
        const u4_t *src = a.x + (hq * T + tq + min(lane, nq - 1)) * 16;  // rows past a tail: last valid row
#pragma unroll
        for (int c = 0; c < 16; ++c) xr[c] = __builtin_nontemporal_load(src + c);
    };
    if (tile < n_tiles) load_rows(tile);
    for (; tile < n_tiles; tile += stride) {
        const int64_t hh = tile / tiles_per_h;
        const int64_t t0 = (tile - hh * tiles_per_h) * kTile;
        const int nv = (int)min((int64_t)kTile, T - t0);
        const int h = (int)hh;
        const int64_t v0 = hh * T + t0;
        uint32_t w[64];
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            w[4 * c + 0] = xr[c].x;
            w[4 * c + 1] = xr[c].y;
            w[4 * c + 2] = xr[c].z;
            w[4 * c + 3] = xr[c].w;
        }

        const float ss = norm2_f16(w);
        const float nx = __builtin_sqrtf(ss);
        const float inv = ss > 0.0f ? kSqrtD / nx : 0.0f;
        const float *oh = o + __builtin_amdgcn_readfirstlane(h) * kD;
        float y[128];
        float nb2 = 0.0f;
        {
            // a_t is rounded as in the stats pass before o is subtracted, so
            // a single token (o = a_t) gives b = 0 exactly
#pragma clang fp contract(off)
#pragma unroll
            for (int k = 0; k < 64; ++k) {
                const h2_t p = __builtin_bit_cast(h2_t, w[k]);
                y[2 * k] = (float)p.x * inv - oh[2 * k];
                y[2 * k + 1] = (float)p.y * inv - oh[2 * k + 1];
            }
        }
#pragma unroll
        for (int k = 0; k < 128; ++k) nb2 = fmaf(y[k], y[k], nb2);
#pragma unroll
        for (int st = 1; st < 128; st <<= 1) {
#pragma unroll
            for (int i = 0; i < 128; i += 2 * st) {
#pragma unroll
                for (int j = i; j < i + st; ++j) {
                    const float p0 = y[j], p1 = y[j + st];
                    y[j] = p0 + p1;
                    y[j + st] = p0 - p1;
                }
            }
        }
        const float nb = __builtin_sqrtf(nb2);
        const float invb = nb2 > 0.0f ? 1.0f / nb : 0.0f;
        // z = H b / ||b||, staged as fp16 hi / lo rows
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            h8_t hv, lv;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                _Float16 lo;
                hv[j] = split_f16(y[8 * c + j] * invb, lo);
                lv[j] = lo;
            }
            L[swz(lane, c)] = __builtin_bit_cast(u4_t, hv);
            Llo[swz(lane, c)] = __builtin_bit_cast(u4_t, lv);
        }
        wait_lgkm();
        __builtin_amdgcn_wave_barrier();
        if (tile + stride < n_tiles) load_rows(tile + stride);

        uint32_t code[4] = {0u, 0u, 0u, 0u};  // codes of token `lane` (sub-vector s in byte s)
#pragma unroll 1
        for (int tb = 0; tb < 2; ++tb) {
            const int row = 32 * tb + col;  // token of this lane's column
            const u4_t *Lz = half ? Llo : L;  // B of the x16 pass: z_hi (k < 8) or z_lo (k >= 8)
            float bm[16];
            int bg[16];
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                bm[s] = -INFINITY;
                bg[s] = 0;
            }
#pragma unroll 1
            for (int mb = 0; mb < 8; ++mb) {
                const int ent = 32 * mb + col;  // codeword row of this lane's A operand
                const h8_t A16 = __builtin_bit_cast(h8_t, s_cbh[ent]);
                h4_t A8 = {};
                if constexpr (CB_LO) A8 = __builtin_bit_cast(h4_t, s_cbl[2 * ent + half]);
                // accumulator rows of this lane: codeword 32 mb + 8 (r/4) + 4 half + r%4
                f16v_t bias;
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const f4_t bq = reinterpret_cast<const f4_t *>(s_bias)[(32 * mb + 8 * r4 + 4 * half) >> 2];
                    bias[4 * r4] = bq.x;
                    bias[4 * r4 + 1] = bq.y;
                    bias[4 * r4 + 2] = bq.z;
                    bias[4 * r4 + 3] = bq.w;
                }
                // four sub-vectors at a time in independent accumulators, so
                // that the matrix cores run while earlier results are scanned
#pragma unroll
                for (int s4 = 0; s4 < 16; s4 += 4) {
                    f16v_t acc[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const h8_t B16 = __builtin_bit_cast(h8_t, Lz[swz(row, s4 + u)]);
                        acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A16, B16, bias, 0, 0, 0);
                    }
                    if constexpr (CB_LO) {
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const h4_t B8 =
                                __builtin_bit_cast(h4_t, reinterpret_cast<const u2_t *>(L + swz(row, s4 + u))[half]);
                            acc[u] = __builtin_amdgcn_mfma_f32_32x32x8f16(A8, B8, acc[u], 0, 0, 0);
                        }
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int s = s4 + u;
#pragma unroll
                        for (int r4 = 0; r4 < 4; ++r4) {
                            const float m = max4(acc[u][4 * r4], acc[u][4 * r4 + 1], acc[u][4 * r4 + 2], acc[u][4 * r4 + 3]);
                            const bool better = m > bm[s];
                            bm[s] = better ? m : bm[s];
                            bg[s] = better ? 4 * mb + r4 : bg[s];
                        }
                    }
                }
            }
            // resolve the best group of each sub-vector in fp32, then merge with
            // the lane holding the other half of every codeword block
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const h8_t zh = __builtin_bit_cast(h8_t, L[swz(row, s)]);
                const h8_t zl = __builtin_bit_cast(h8_t, Llo[swz(row, s)]);
                float z[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) z[t] = (float)zh[t] + (float)zl[t];
                const int g = bg[s];
                const int j0 = 32 * (g >> 2) + 8 * (g & 3) + 4 * half;
                float best = -INFINITY;
                int bi = j0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = j0 + r;
                    const f4_t c0 = s_cb[2 * j], c1 = s_cb[2 * j + 1];
                    float sc = s_bias[j];
                    sc = fmaf(z[0], c0.x, sc);
                    sc = fmaf(z[1], c0.y, sc);
                    sc = fmaf(z[2], c0.z, sc);
                    sc = fmaf(z[3], c0.w, sc);
                    sc = fmaf(z[4], c1.x, sc);
                    sc = fmaf(z[5], c1.y, sc);
                    sc = fmaf(z[6], c1.z, sc);
                    sc = fmaf(z[7], c1.w, sc);
                    const bool better = sc > best;  // increasing index: strict > keeps the lowest
                    best = better ? sc : best;
                    bi = better ? j : bi;
                }
                const float ob = __shfl_xor(best, 32);
                const int oi = __shfl_xor(bi, 32);
                const int win = (ob > best || (ob == best && oi < bi)) ? oi : bi;
                if (half == tb) code[s >> 2] |= (uint32_t)win << (8 * (s & 3));
            }
        }
        if (lane < nv) {
            const int64_t v = v0 + lane;
            u4_t cv = {code[0], code[1], code[2], code[3]};
            a.codes[v] = cv;
            a.s1[v] = nx / kSqrtD;
            a.s2[v] = nb / kSqrtD;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

}  // namespace

size_t nsn_ws_bytes(int64_t H, int64_t T)
{
    const int64_t n_chunks = (T + kChunk - 1) / kChunk;
    return (size_t)H * n_chunks * kD * sizeof(float);
}

hipError_t launch_nsn_vq(const kvq_ctx *ctx, const void *x, int64_t H, int64_t T, uint8_t *codes, float *s1,
                         float *s2, float *o, void *ws, hipStream_t s)
{
    const int n_chunks = (int)((T + kChunk - 1) / kChunk);
    float *part = (float *)ws;
    hipLaunchKernelGGL(k_nsn_stats, dim3((unsigned)(H * n_chunks)), dim3(256), 0, s, (const u4_t *)x, part, T,
                       n_chunks);
    hipLaunchKernelGGL(k_nsn_mean, dim3((unsigned)H), dim3(kD * kMeanGroups), 0, s, part, o, T, n_chunks);
    VqArgs a{};
    a.x = (const u4_t *)x;
    a.cb_hi = (const u4_t *)ctx->d_vq16;
    a.cb_lo = (const u2_t *)(ctx->d_vq16 + kVqK * kVqSub);
    a.cb = ctx->d_vq;
    a.bias = ctx->d_vqbias;
    a.codes = (u4_t *)codes;
    a.s1 = s1;
    a.s2 = s2;
    const int64_t tiles_per_h = (T + kTile - 1) / kTile;
    const int64_t n_tiles = tiles_per_h * H;
    int64_t blocks = (n_tiles + 3) / 4;
    if (blocks > ctx->n_cu) blocks = ctx->n_cu;
    if (ctx->vq_exact_f16)
        hipLaunchKernelGGL(k_nsn_vq<false>, dim3((unsigned)blocks), dim3(256), 0, s, a, (const float *)o, T, (int)H,
                           tiles_per_h, n_tiles);
    else
        hipLaunchKernelGGL(k_nsn_vq<true>, dim3((unsigned)blocks), dim3(256), 0, s, a, (const float *)o, T, (int)H,
                           tiles_per_h, n_tiles);
    return hipGetLastError();
}

}  // namespace kvq
