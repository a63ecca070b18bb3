// Internal declarations shared by the libkvq host code and its HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "kvq.h"

namespace kvq {

constexpr int kD = 128;       // head dimension
constexpr int kVqSub = 8;     // NSN sub-vector length
constexpr int kVqK = 256;     // NSN codebook entries
constexpr int kMaxGroup = 8;  // query heads per KV head supported by the score kernels
constexpr int kNsnChunk = 2048;            // tokens per NSN statistics block
constexpr int kNsnPartStride = kD + 4;     // floats per NSN decode partial: acc[128], M, L, WO, pad
// Device scratch of the no-allocation decode entry point, per device.
constexpr size_t kNoAllocScratchBytes = size_t(KVQ_NOALLOC_SCRATCH_BYTES);

// Bounds-checked debug build.  Compiled with KVQ_DEBUG defined, a failed
// KVQ_CHECK(cond) in a kernel records the source line of its first failure
// in a device word of the kernel's source file and the kernel carries on (no
// trap); LDS is filled with a NaN pattern before first use, so that a read of
// LDS nothing wrote shows in the results.  debug_take_<file>() reads the
// word of the current device (file id in the high half, line in the low
// half, 0 if no check failed) and clears it.  Without KVQ_DEBUG the checks
// compile to nothing and the take functions return 0.  Each source file with
// kernels expands KVQ_DEBUG_UNIT(name, id) once, inside namespace kvq, before
// its first kernel.
#ifdef KVQ_DEBUG
#define KVQ_CHECK(cond)                                  \
    do {                                                 \
        if (!(cond)) ::kvq::debug_fail((unsigned)__LINE__); \
    } while (0)
#define KVQ_DEBUG_UNIT(NAME, ID)                                                                  \
    namespace {                                                                                   \
    __device__ unsigned g_debug_record;                                                           \
    }                                                                                             \
    __device__ __forceinline__ void debug_fail(unsigned line)                                      \
    {                                                                                             \
        atomicCAS(&g_debug_record, 0u, line & 0xFFFFu);                                           \
    }                                                                                             \
    uint32_t debug_take_##NAME()                                                                  \
    {                                                                                             \
        unsigned v = 0u, z = 0u;                                                                  \
        if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_debug_record), sizeof(v), 0, hipMemcpyDeviceToHost) != hipSuccess) \
            return 0xFFFFFFFFu;                                                                   \
        if (v != 0u && hipMemcpyToSymbol(HIP_SYMBOL(g_debug_record), &z, sizeof(z), 0, hipMemcpyHostToDevice) != hipSuccess) \
            return 0xFFFFFFFFu;                                                                   \
        return v ? ((uint32_t)(ID) << 16) | v : 0u;                                               \
    }
#define KVQ_DEBUG_ON 1
#else
#define KVQ_CHECK(cond) \
    do {                \
    } while (0)
#define KVQ_DEBUG_UNIT(NAME, ID) \
    uint32_t debug_take_##NAME() { return 0u; }
#define KVQ_DEBUG_ON 0
#endif
// the files with kernels: ids 1 .. 6
uint32_t debug_take_quantize();
uint32_t debug_take_score();
uint32_t debug_take_nsn();
uint32_t debug_take_nsn_score();
uint32_t debug_take_dense();
uint32_t debug_take_stream();

// LDS words [0, n) of a block set to a NaN pattern (fp32 and fp16 pairs), by
// its threads, before the block's first barrier (debug build only).
#define KVQ_POISON_LDS(ptr, n_words, tid, n_threads)                                   \
    do {                                                                               \
        if (KVQ_DEBUG_ON) {                                                            \
            for (int i_ = (tid); i_ < (int)(n_words); i_ += (n_threads))               \
                reinterpret_cast<uint32_t *>(ptr)[i_] = 0x7FC07FC0u;                   \
        }                                                                              \
    } while (0)

// Scalar codebook of one bit width, passed to kernels by value.
struct Codebook {
    float c[16];  // centroids c_0 < ... < c_{2^b - 1}
    float t[16];  // thresholds t_0 < ... < t_{2^b - 2}
    int bits;
};

}  // namespace kvq

struct kvq_ctx {
    int d, bits, mode, H, device;
    int n_cu;             // compute units of the device
    kvq::Codebook cb;
    uint32_t *d_sgnmask;  // [2][H][64]: fp16-pair sign masks of D_K, D_V
    float *d_signs;       // [2][H][128]: D_K, D_V as +-1.0f
    int8_t *h_signs;      // host copy [2][H][128] of D_K, D_V (MSE modes)
    float *d_S;           // [128][128] QJL projection transposed, d_S[i][j] = S[j][i] (MSE_QJL)
    _Float16 *d_S16;      // [2][128][128] fp16 hi and lo parts of S (MSE_QJL)
    bool S_exact_f16;     // S_lo == 0
    float *d_vq;          // [256][8] fp32 codebook (NSN_VQ scoring)
    int rotation;         // KVQ_ROTATION_*
    int nsn_options;      // KVQ_NSN_* bits (NSN_VQ)
    float *d_Q;           // [128][128] dense rotation Q, row-major (KVQ_ROTATION_DENSE)
    float *d_Qt;          // its transpose
    _Float16 *d_Q16;      // [2][128][128] fp16 high and low parts of Q
    _Float16 *d_vq16;     // [2][256][8] fp16 hi and lo parts of the codebook
    bool vq_exact_f16;    // codebook lo == 0
    float *d_vqbias;      // [256] -||C_j||^2 / 2
    float *d_gsrq;        // GSRQ tables: shapes [2][256][32], levels [2][16], thresholds [2][15]
    _Float16 *d_gsrq16;   // GSRQ shapes as fp16 high parts [2][256][32], then low parts [2][256][32]
};

namespace kvq {

hipError_t launch_quantize(const kvq_ctx *ctx, int kind, const void *x, int64_t B, int64_t T,
                           uint8_t *codes, float *norms, uint8_t *qjl_signs, float *qjl_gamma,
                           hipStream_t s);

hipError_t launch_quantize_kv(const kvq_ctx *ctx, const void *k, const void *v, int64_t B, int64_t T,
                              uint8_t *k_codes, float *k_norms, uint8_t *v_codes, float *v_norms,
                              hipStream_t s);

hipError_t launch_logits(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                         const uint8_t *codes, const float *norms, const uint8_t *qjl_signs,
                         const float *qjl_gamma, float *logits, hipStream_t s);

constexpr int kMaxSplits = 512;  // token splits per (batch, KV head) in decode
inline int64_t decode_max_splits(int64_t T)
{
    const int64_t m = (T + 63) / 64;
    return m < kMaxSplits ? m : kMaxSplits;
}
size_t decode_ws_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t T);
int decode_auto_splits(int64_t B, int64_t Hkv, int64_t T);
// Arrival counters at the start of a decode workspace: one u32 per (batch,
// KV head), rounded up to 256 bytes.
size_t decode_count_bytes(int64_t B_Hkv);
// The no-allocation scratch reserves a fixed counter region, so that calls of
// different shapes never find earlier partials where their counters lie.
constexpr size_t kNoAllocCountBytes = 65536;

hipError_t launch_decode(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                         const uint8_t *kc, const float *kn, const uint8_t *vc, const float *vn,
                         float sm_scale, float *out, void *ws, int n_split, hipStream_t s);

// No-allocation decode: bytes of the scratch layout (counters, n_split
// partial slots per (batch, query head), rotated queries if dense); the
// one-time per-device set-up (address of the scratch array, counters
// cleared), called by kvq_create with the device current; and the decode
// launch on that scratch.
size_t noalloc_decode_bytes(int64_t B, int64_t Hq, int64_t Hkv, int n_split, bool dense);
hipError_t noalloc_setup(int device);
hipError_t launch_decode_noalloc(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                                 const uint8_t *kc, const float *kn, const uint8_t *vc, const float *vn,
                                 float sm_scale, float *out, int n_split, hipStream_t s);

// Quantise with the dense rotation: N vectors of the list xk (and N of xv
// when xv is not null) into ck/nk (cv/nv).
hipError_t launch_quantize_dense(const kvq_ctx *ctx, const void *xk, const void *xv, int64_t N, uint8_t *ck,
                                 float *nk, uint8_t *cv, float *nv, hipStream_t s);

// Dense rotation plus the QJL residual of N keys: codes, norms, sign bits
// [N][16 bytes] and residual norms gamma.
hipError_t launch_quantize_dense_qjl(const kvq_ctx *ctx, const void *xk, int64_t N, uint8_t *ck, float *nk,
                                     uint8_t *signs, float *gamma, hipStream_t s);

// Residual window of a streaming cache: R full-precision tokens per (batch, KV
// head) in fp16 arrays [B, H_kv, R_cap, 128].
struct DecodeTail {
    const void *k, *v;
    int64_t R, R_cap;
};
// Decode over T quantised tokens (arrays of ldt tokens per (batch, KV head))
// followed by the residual window (tail may be null; T may be 0 with a tail).
hipError_t launch_decode_stream(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T, int64_t ldt,
                                const uint8_t *kc, const float *kn, const uint8_t *vc, const float *vn,
                                const DecodeTail *tail, float sm_scale, float *out, void *ws, int n_split,
                                hipStream_t s);

// Quantise the first R tokens of K and V residual windows ([B, H_kv, R_cap,
// 128] fp16) into positions T0 .. T0 + R - 1 of packed arrays of T_cap tokens
// per (batch, KV head).
hipError_t launch_flush(const kvq_ctx *ctx, const void *kt, const void *vt, int64_t B, int64_t R, int64_t R_cap,
                        uint8_t *kc, float *kn, uint8_t *vc, float *vn, int64_t T0, int64_t T_cap, hipStream_t s);

size_t nsn_ws_bytes(int64_t H, int64_t T);

hipError_t launch_nsn_vq(const kvq_ctx *ctx, const void *x, int64_t H, int64_t T, uint8_t *codes,
                         float *s1, float *s2, float *o, void *ws, hipStream_t s);
// The same over H heads of T tokens held ldx tokens apart (input), written
// ldt tokens apart (codes, s1, s2) with the means ldo floats apart.
hipError_t launch_nsn_vq_strided(const kvq_ctx *ctx, const void *x, int64_t H, int64_t T, int64_t ldx, uint8_t *codes,
                                 float *s1, float *s2, int64_t ldt, float *o, int64_t ldo, void *ws, hipStream_t s);

// Double quantisation of the NSN byproducts: s1 as 4-bit codes with one
// (lo, step) pair per block of kNsnDqBlock tokens, o as 4-bit codes with one
// pair per head.
constexpr int kNsnDqBlock = 32;
struct NsnDq {
    uint8_t *s1q;  // [H][ceil(T / 2)]
    float *s1p;    // [H][ceil(T / 32)][2]
    uint8_t *oq;   // [H][64]
    float *op;     // [H][2]
};
size_t nsn_ws_bytes_aligned(int64_t H, int64_t T);  // nsn_ws_bytes rounded up to 256 bytes
size_t nsn_dq_ws_bytes(int64_t H, int64_t T);       // + the dequantised means [H][128]
hipError_t launch_nsn_vq_dq(const kvq_ctx *ctx, const void *x, int64_t H, int64_t T, uint8_t *codes, float *s2,
                            const NsnDq &dq, void *ws, hipStream_t s);

// Gain-shape residual quantisation on the NSN front end: codes [H][T][12]
// (three dwords per token), s1, s2 [H][T], means o [H][128]; ws as the NSN
// statistics (nsn_ws_bytes).
constexpr int kGsrqRec = 12;  // record bytes per token
hipError_t launch_gsrq(const kvq_ctx *ctx, const void *x, int64_t H, int64_t T, uint8_t *codes, float *s1, float *s2,
                       float *o, void *ws, hipStream_t s);
hipError_t launch_gsrq_logits(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                              const uint8_t *codes, const float *s1, const float *s2, const float *o, float *logits,
                              hipStream_t s);

// NSN-VQ encoded keys and values of one decode call (outputs of
// kvq_nsn_vq_quantize, or of kvq_nsn_vq_quantize_dq: then s1 and o are read
// from the 4-bit forms in kdq / vdq and ks1, ko, vs1, vo are unused).
struct NsnDqIn {
    const uint8_t *s1q;
    const float *s1p;
    const uint8_t *oq;
    const float *op;
};
struct NsnKV {
    const uint8_t *kc;
    const float *ks1, *ks2, *ko;
    const uint8_t *vc;
    const float *vs1, *vs2, *vo;
    bool dq;
    NsnDqIn kdq, vdq;
};

hipError_t launch_nsn_logits(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                             const uint8_t *codes, const float *s1, const float *s2, const float *o, float *logits,
                             hipStream_t s);
hipError_t launch_nsn_logits_dq(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                                const uint8_t *codes, const NsnDqIn &dq, const float *s2, float *logits,
                                hipStream_t s);

int64_t nsn_decode_chunk(int64_t T, int n_split);
int nsn_decode_auto_splits(const kvq_ctx *ctx, int64_t B, int64_t T);
size_t nsn_decode_ws_bytes(int64_t B, int64_t Hq, int64_t T);
hipError_t launch_nsn_decode(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T, const NsnKV &kv,
                             float sm_scale, float *out, void *ws, int n_split, hipStream_t s);
// Decode over GSRQ records (kc, vc: [B Hkv][T][12]) with the NSN byproducts;
// workspace as the NSN-VQ decode.
hipError_t launch_gsrq_decode(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T, const NsnKV &kv,
                              float sm_scale, float *out, void *ws, int n_split, hipStream_t s);

// Streaming NSN-VQ cache: packed rows of T_cap tokens flushed in groups of Gs
// tokens, each group with its own K and V means ([B Hkv][T_cap / Gs][128]
// fp32, in NsnKV's ko and vo), and a window of R (of R_cap) fp16 tokens.
struct NsnStream {
    int64_t T_cap, Gs;
    const void *kt, *vt;
    int64_t R, R_cap;
};
constexpr int kNsnMaxGroupsBlk = 32;  // flush groups one decode block covers at most
// tokens per split: a multiple of Gs (itself a multiple of 64), at most
// kNsnMaxGroupsBlk groups; 0 if T needs more than kMaxSplits - 1 such splits
int64_t nsn_stream_chunk(int64_t T, int n_split, int64_t Gs);
size_t nsn_stream_ws_bytes(int64_t B, int64_t Hq, int64_t T_cap);
hipError_t launch_nsn_decode_stream(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                                    const NsnKV &kv, const NsnStream &st, float sm_scale, float *out, void *ws,
                                    int n_split, hipStream_t s);

}  // namespace kvq
