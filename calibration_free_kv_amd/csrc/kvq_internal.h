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
    uint32_t *d_sgnmask_h;  // same, masks of coordinates 64..127 also flipping every sign
    float *d_signs;       // [2][H][128]: D_K, D_V as +-1.0f
    int8_t *h_signs;      // host copy [2][H][128] of D_K, D_V (MSE modes)
    float *d_S;           // [128][128] QJL projection transposed, d_S[i][j] = S[j][i] (MSE_QJL)
    _Float16 *d_S16;      // [2][128][128] fp16 hi and lo parts of S (MSE_QJL)
    bool S_exact_f16;     // S_lo == 0
    float *d_vq;          // [256][8] fp32 codebook (NSN_VQ scoring)
    int rotation;         // KVQ_ROTATION_*
    float *d_Q;           // [128][128] dense rotation Q, row-major (KVQ_ROTATION_DENSE)
    float *d_Qt;          // its transpose
    _Float16 *d_Q16;      // [2][128][128] fp16 high and low parts of Q
    _Float16 *d_vq16;     // [2][256][8] fp16 hi and lo parts of the codebook
    bool vq_exact_f16;    // codebook lo == 0
    float *d_vqbias;      // [256] -||C_j||^2 / 2
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

hipError_t launch_decode(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                         const uint8_t *kc, const float *kn, const uint8_t *vc, const float *vn,
                         float sm_scale, float *out, void *ws, int n_split, hipStream_t s);

// Quantise with the dense rotation: N vectors of the list xk (and N of xv
// when xv is not null) into ck/nk (cv/nv).
hipError_t launch_quantize_dense(const kvq_ctx *ctx, const void *xk, const void *xv, int64_t N, uint8_t *ck,
                                 float *nk, uint8_t *cv, float *nv, hipStream_t s);

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

// NSN-VQ encoded keys and values of one decode call (outputs of kvq_nsn_vq_quantize).
struct NsnKV {
    const uint8_t *kc;
    const float *ks1, *ks2, *ko;
    const uint8_t *vc;
    const float *vs1, *vs2, *vo;
};

hipError_t launch_nsn_logits(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T,
                             const uint8_t *codes, const float *s1, const float *s2, const float *o, float *logits,
                             hipStream_t s);

int64_t nsn_decode_chunk(int64_t T, int n_split);
int nsn_decode_auto_splits(const kvq_ctx *ctx, int64_t B, int64_t T);
size_t nsn_decode_ws_bytes(int64_t B, int64_t Hq, int64_t T);
hipError_t launch_nsn_decode(const kvq_ctx *ctx, const void *q, int64_t B, int64_t Hq, int64_t T, const NsnKV &kv,
                             float sm_scale, float *out, void *ws, int n_split, hipStream_t s);

}  // namespace kvq
