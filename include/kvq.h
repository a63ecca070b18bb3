/*
 * kvq.h -- C ABI of libkvq: calibration-free rotate-then-quantize compression
 * of LLM KV-cache vectors, and attention read directly from the packed codes,
 * on AMD Instinct MI355X (gfx950).
 *
 * The operations follow these pages:
 *  [PQ]  "PolarQuant: Optimal Gaussian Weight Quantization via Hadamard
 *        Rotation" (gist.science 2603.29078), Technical summary sec. 2
 *        Methodology: per-block L2 norm kept, Walsh-Hadamard rotation, scale
 *        to unit variance, Gaussian Lloyd-Max centroids; dequantisation is
 *        centroid lookup, inverse (self-inverse) Hadamard, norm restore.
 *  [TQ]  "O Que E TurboQuant?" (a2a-mcp.org), Como Funciona: Estagio 1
 *        (random rotation, per-coordinate Lloyd-Max code), Estagio 2 (1-bit
 *        QJL sign residual for unbiased inner products, attention logits
 *        computed from the compressed indices); Como Implementar (codebooks
 *        precomputed per dimension and bit width, query rotated once).
 *  [NSN] "NSNQuant: A Double Normalization Approach for Calibration-Free
 *        Low-Bit Vector Quantization of KV Cache" (gist.science 2505.18231),
 *        Metodologia sec. 1 (Normalize-Shift-Normalize, byproducts s1, o,
 *        s2), sec. 2 (Hadamard), sec. 3 (one global N(0,1) vector codebook).
 *  [GSRQ] "GSRQ: Quantitzacio Residual de Forma-Guanys per a Cau KV de Menys
 *        d'1 Bit" (q2bstudio.com): gain-shape k-means (norm kept apart from
 *        direction) in a residual quantisation pipeline, below 1 bit per
 *        element.
 *
 * Conventions for every call
 *  - d = 128 (head dimension).  Vectors are fp16, row-major, tokens
 *    contiguous: a K or V tensor is [B, H_kv, T, d].
 *  - Rotation of a vector u: y = H (D .* u) with the +-1 Sylvester Hadamard
 *    matrix H_ij = (-1)^popcount(i & j) and the random-sign diagonal D of the
 *    tensor (K or V) and KV head; for a unit vector u this gives coordinates
 *    of unit variance.
 *  - b-bit MSE codes: index i of a coordinate y_i is #{j : t_j < y_i} over the
 *    2^b - 1 thresholds t_j (midpoints of the N(0,1) Lloyd-Max centroids
 *    c_j, both stored as fp32).  A vector's record is 16*b bytes holding its
 *    128 indices as an LSB-first bit stream: coordinate i occupies bits
 *    [b*i, b*i + b).  Records are [B, H_kv, T, 16*b] bytes; the norms
 *    rho = ||x||_2 are fp32 [B, H_kv, T].  A zero vector has rho = 0 and all
 *    indices 2^(b-1) - 1.
 *  - Grouped-query attention: query head h reads KV head h / (H_q / H_kv).
 *  - All tensor arguments are DEVICE pointers on the context's device,
 *    16-byte aligned, contiguous, owned by the caller.  `stream` is a
 *    hipStream_t (NULL = the null stream); every compute call only enqueues
 *    work on it and returns without synchronising.
 *  - Errors: arguments are validated on the host before anything is
 *    launched; a rejected call launches nothing and leaves outputs untouched.
 *    Launch failures are reported as KVQ_E_DEVICE.  Faults during kernel
 *    execution surface at the caller's next synchronisation of the stream.
 *  - A context is immutable after kvq_create: calls on different streams may
 *    run concurrently as long as their output buffers do not overlap.
 */
#ifndef KVQ_H_
#define KVQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvq_ctx kvq_ctx;

typedef enum {
    KVQ_OK = 0,
    KVQ_E_INVAL = 1,       /* bad pointer, size, shape or combination      */
    KVQ_E_UNSUPPORTED = 2, /* valid request the library does not implement */
    KVQ_E_DEVICE = 3,      /* no usable GPU, or a HIP runtime/launch error   */
    KVQ_E_NOMEM = 4,       /* host or device allocation failed              */
    KVQ_E_WORKSPACE = 5    /* caller workspace smaller than required        */
} kvq_status;

/* KVQ_MODE_GSRQ: gain-shape residual quantisation ([GSRQ]) on the NSN front
 * end; see kvq_gsrq_quantize. */
enum { KVQ_MODE_MSE = 0, KVQ_MODE_MSE_QJL = 1, KVQ_MODE_NSN_VQ = 2, KVQ_MODE_GSRQ = 3 };
enum { KVQ_KIND_K = 0, KVQ_KIND_V = 1 };
/* Scalar codebook of the MSE modes: Lloyd-Max for N(0,1) ([PQ] sec. 2), or
 * Lloyd-Max for the exact law of a rotated unit vector's coordinate at
 * d = 128, Beta((d-1)/2, (d-1)/2) on [-1, 1] scaled by sqrt(d) ([TQ] Como
 * Funciona, Estagio 1). */
enum { KVQ_CODEBOOK_GAUSS = 0, KVQ_CODEBOOK_BETA = 1 };
/* Rotation of the MSE modes: the randomized Hadamard transform y = H (D .* u)
 * ([PQ] sec. 2; [NSN] sec. 2), or a dense orthogonal Q given by the caller,
 * y = sqrt(d) Q u ([TQ] Como Funciona, Estagio 1: QR of a Gaussian matrix),
 * the same Q for K, V and every head (KVQ_MODE_MSE, and KVQ_MODE_MSE_QJL
 * where the QJL residual lives in the rotated space: [TQ] Estagio 1 +
 * Estagio 2; not with the NSN_VQ mode or the streaming-cache calls). */
enum { KVQ_ROTATION_HADAMARD = 0, KVQ_ROTATION_DENSE = 1 };
/* Options of the NSN_VQ mode (bits of kvq_config.nsn_options).
 * KVQ_NSN_ADAPTIVE_SCALE ([NSN] Metodologia sec. 3, adaptive scale): the
 * selected entries zq of a token are scaled by alpha = ||z||^2 / <z, zq>
 * (1 when <z, zq> <= 0), which keeps the component of the reconstruction
 * along the token exact; alpha is folded into the stored s2 (s2 <- alpha s2),
 * so the scoring calls use it unchanged. */
/* KVQ_NSN_DQ_CODEBOOK ([NSN] Metodologia sec. 3, double quantisation): the
 * codebook's entries are stored with 4 bits: the 2048 values as one block,
 * lo = min, step = (max - lo) / 15, each replaced by lo + c step with c the
 * nearest of the 16 levels (decided in double precision at kvq_create); the
 * context then encodes and scores with these values. */
enum { KVQ_NSN_ADAPTIVE_SCALE = 1, KVQ_NSN_DQ_CODEBOOK = 2 };

/* Configuration of a context.  Host arrays are copied by kvq_create.
 *
 * The random-sign diagonal D of the rotation ([PQ] sec. 2, randomized
 * Hadamard transform: a random +-1 diagonal before H) is chosen per tensor
 * (K, V) and per KV head.  In the MSE modes a non-NULL signs_k / signs_v gives
 * it explicitly; a NULL one is generated from `seed` with SplitMix64 (Steele,
 * Lea and Flood, "Fast splittable pseudorandom number generators", 2014):
 * output n of the generator is mix64(seed + (n + 1) * 0x9E3779B97F4A7C15)
 * with mix64(z) = z' ^ (z' >> 31), z' the result of
 * z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27; z *= 0x94D049BB133111EB
 * (all arithmetic mod 2^64), and coordinate i of head h of tensor kind
 * (KVQ_KIND_K = 0, KVQ_KIND_V = 1) takes sign -1 when the top bit of output
 * n = kind * 2^32 + h * d + i is set, else +1.  kvq_get_tables returns the
 * signs a context uses. */
typedef struct {
    int32_t d;                 /* head dimension; must be 128                         */
    int32_t bits;              /* MSE code width b in {1,2,3,4} (MSE, MSE_QJL modes)  */
    int32_t mode;              /* KVQ_MODE_*                                          */
    int32_t n_kv_heads;        /* H_kv >= 1                                           */
    uint64_t seed;             /* seed of D where signs_k or signs_v is NULL         */
    const int8_t *signs_k;     /* host [n_kv_heads, d], entries +1/-1: D of K, or NULL */
    const int8_t *signs_v;     /* host [n_kv_heads, d], entries +1/-1: D of V, or NULL */
    const float *qjl_S;        /* host [d, d] row-major Gaussian projection (MSE_QJL) */
    const float *vq_codebook;  /* host [256, 8] fp32 codebook (NSN_VQ)                */
    int32_t device;            /* HIP device ordinal                                  */
    int32_t codebook;          /* KVQ_CODEBOOK_* (MSE modes; 0 = N(0,1))              */
    int32_t rotation;          /* KVQ_ROTATION_* (0 = randomized Hadamard)            */
    const float *rot_Q;        /* host [d, d] row-major orthogonal Q (ROTATION_DENSE)  */
    int32_t nsn_options;       /* KVQ_NSN_* bits (NSN_VQ mode; 0 = none)              */
    const float *gsrq_tables;  /* host GSRQ tables (GSRQ mode): stage 1 shapes [256, 32],
                                  its 16 gain levels, stage 2 shapes [256, 32], its 16
                                  levels, fp32, levels strictly increasing             */
} kvq_config;

/* Create a context: validates the configuration, builds the b-bit Lloyd-Max
 * tables ([PQ] sec. 2, [TQ] Como Implementar: codebooks precomputed per bit
 * width; N(0,1) or the exact-d law) and uploads them with D, S, the VQ
 * codebook and the dense rotation Q (with its transpose and fp16 high/low
 * parts) to the device.  *out receives the context (NULL on failure).
 * Errors: KVQ_E_INVAL (NULL pointers, d != 128, bits outside 1..4, a sign
 * entry not +-1, missing table for the mode, unknown codebook or rotation,
 * rot_Q NULL, with an entry not finite or above 1 in magnitude, or not
 * orthogonal to within 1e-3 in every entry of Q Q^T - I),
 * KVQ_E_UNSUPPORTED (dense rotation in KVQ_MODE_NSN_VQ), KVQ_E_DEVICE (no
 * such device), KVQ_E_NOMEM. */
kvq_status kvq_create(const kvq_config *cfg, kvq_ctx **out);

/* Release a context and its device tables.  NULL is accepted (no-op).
 * The caller must not destroy a context while its work is in flight. */
kvq_status kvq_destroy(kvq_ctx *ctx);

/* Copy the context's tables to host memory: the fp32 Lloyd-Max centroids
 * [2^b] and thresholds [2^b - 1] ([PQ] sec. 2), and the int8 +-1 diagonals
 * of D for K and V, [n_kv_heads, d] each ([PQ] sec. 2, randomized Hadamard
 * transform), whether given or generated from the seed.  Any output pointer
 * may be NULL.  Errors: KVQ_E_INVAL for a NULL context, or a sign output in
 * the NSN_VQ mode (which has no D). */
kvq_status kvq_get_tables(const kvq_ctx *ctx, float *centroids, float *thresholds, int8_t *signs_k,
                          int8_t *signs_v);

/* The fp32 tables of a bit width without a context or a device: centroids
 * [2^b] and thresholds [2^b - 1] of the N(0,1) Lloyd-Max quantiser, exactly
 * as kvq_create stores them ([PQ] sec. 2; [TQ] Como Implementar).
 * Errors: KVQ_E_INVAL for bits outside 1..4 or NULL outputs. */
kvq_status kvq_codebook(int32_t bits, float *centroids, float *thresholds);

/* Bytes of one packed record (16*b for MSE modes, 16 for NSN_VQ); 0 if ctx
 * is NULL. */
int64_t kvq_code_bytes_per_vec(const kvq_ctx *ctx);

/* Static description of a status code (never NULL). */
const char *kvq_strerror(kvq_status s);

/* Bounds-checked debug build (libkvq compiled with KVQ_DEBUG defined; the
 * build script writes it as libkvq_debug.so beside libkvq.so).  Its kernels
 * check the ranges of the token, record, tile and split indices they form
 * against the shapes of the launch; a failed check does not stop the kernel
 * but records, per kernel source file and device, the source line of the
 * first failure.  The kernels also fill their LDS with a NaN pattern before
 * first use, so a read of LDS that nothing wrote shows in the results.
 * kvq_debug_build() is 1 in that build, 0 otherwise.
 * kvq_debug_take() returns the first failure recorded on the current device
 * since the last call (source file id 1..6 in bits 16..31, line in bits
 * 0..15; 0 if none, 0xFFFFFFFF if the record could not be read) and clears
 * the records; call it once the work it should cover has completed (after a
 * device synchronisation).  In other builds it returns 0 and touches no
 * device. */
int32_t kvq_debug_build(void);
uint32_t kvq_debug_take(void);

/* Quantise T tokens of K or V ([PQ] sec. 2 and [TQ] Estagio 1; QJL residual:
 * [TQ] Estagio 2).
 *   kind        KVQ_KIND_K or KVQ_KIND_V (selects D)
 *   x_f16       [B, H_kv, T, d] fp16, H_kv == cfg.n_kv_heads
 *   codes       out [B, H_kv, T, 16*b] bytes
 *   norms       out [B, H_kv, T] fp32, rho = ||x||
 *   qjl_signs   out [B, H_kv, T, 16] bytes, or NULL.  Required for kind K in
 *               MSE_QJL mode, must be NULL otherwise.  Bit j (LSB-first) is
 *               [z_j >= 0], z = S r, r = (y - c[idx]) / sqrt(d).
 *   qjl_gamma   out [B, H_kv, T] fp32 residual norms ||r||, with qjl_signs.
 * T == 0 or B == 0 is a valid empty call. */
kvq_status kvq_quantize(kvq_ctx *ctx, int32_t kind, const void *x_f16, int64_t B,
                        int64_t H_kv, int64_t T, uint8_t *codes, float *norms,
                        uint8_t *qjl_signs, float *qjl_gamma, void *stream);

/* kvq_quantize of K (with D_K) and of V (with D_V) of the same shape in one
 * launch, e.g. the K and V of the tokens just produced by a layer (MSE mode
 * only).  Arguments and outputs as in kvq_quantize; the results are
 * identical to two kvq_quantize calls. */
kvq_status kvq_quantize_kv(kvq_ctx *ctx, const void *k_f16, const void *v_f16, int64_t B, int64_t H_kv,
                           int64_t T, uint8_t *k_codes, float *k_norms, uint8_t *v_codes, float *v_norms,
                           void *stream);

/* Attention logits from the packed codes ([TQ] Estagio 2 and Como
 * Implementar: the query is rotated once, q' = H (D_K .* q), and each key is
 * scored from its indices without dequantising it):
 *   logits[b,h,t] = rho_t / d * sum_i q'_i c[idx_t,i]
 *                 (+ rho_t gamma_t sqrt(pi/2)/d * sum_j (2 sgn_t,j - 1) (S q')_j / sqrt(d)
 *                    in MSE_QJL mode)
 *   q_f16       [B, H_q, d] fp16 queries; H_q a multiple of H_kv (else
 *               KVQ_E_INVAL) with H_q/H_kv in {1, 2, 4, 8} (other ratios:
 *               KVQ_E_UNSUPPORTED)
 *   codes, norms, qjl_signs, qjl_gamma   the K outputs of kvq_quantize
 *               (qjl_* required in MSE_QJL mode, NULL otherwise)
 *   logits      out [B, H_q, T] fp32 (raw inner products, no softmax scale) */
kvq_status kvq_logits(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                      const uint8_t *codes, const float *norms, const uint8_t *qjl_signs,
                      const float *qjl_gamma, float *logits, void *stream);

/* Workspace bytes kvq_attn_decode needs for these sizes (split-K partials
 * and per-(batch, KV head) arrival counters). */
size_t kvq_attn_decode_ws_bytes(const kvq_ctx *ctx, int64_t B, int64_t H_q, int64_t T);

/* One decode step of attention over the quantised cache (MSE mode): logits
 * from the K codes as in kvq_logits, softmax with scale sm_scale (0 means
 * 1/sqrt(d)), and the V codes dequantised and accumulated:
 *   out[b,h] = sum_t softmax_t * v_hat_t,  v_hat = rho_V D_V .* (H c[idx_V]) / d
 * ([PQ] sec. 2 dequantisation; [NSN] Resultados: decode is memory-bound).
 *   q_f16       [B, H_q, d] fp16; H_q a multiple of H_kv (else KVQ_E_INVAL)
 *               with H_q/H_kv in {1, 2, 4} (other ratios, e.g. 8 query heads
 *               per KV head: KVQ_E_UNSUPPORTED)
 *   k_codes/k_norms, v_codes/v_norms   outputs of kvq_quantize for K and V
 *   out         [B, H_q, d] fp32
 *   ws          device workspace of at least kvq_attn_decode_ws_bytes() bytes.
 *               Its counter words must be zero before the first call that
 *               uses it (e.g. allocate it zero-filled), and again before a
 *               call with a larger B * H_kv (its counters then reach into
 *               the partials of the calls before); every completed call
 *               leaves them zero.  Calls that share a workspace must be
 *               ordered on one stream.
 * T must be >= 1.  Errors: KVQ_E_WORKSPACE if ws_bytes is too small. */
kvq_status kvq_attn_decode(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                           const uint8_t *k_codes, const float *k_norms,
                           const uint8_t *v_codes, const float *v_norms, float sm_scale,
                           float *out, void *ws, size_t ws_bytes, void *stream);

/* As kvq_attn_decode with an explicit number of token splits per (batch, KV
 * head) (0 = automatic).  The result does not depend on n_split beyond fp32
 * rounding.  n_split is clamped to [1, min(512, ceil(T / 64))].
 * The automatic count (here and in every decode entry point) is about one
 * block per compute unit, or the value of the environment variable
 * KVQ_SPLITS when it holds a positive integer (read once per process). */
kvq_status kvq_attn_decode_splits(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q,
                                  int64_t T, const uint8_t *k_codes, const float *k_norms,
                                  const uint8_t *v_codes, const float *v_norms, float sm_scale,
                                  float *out, void *ws, size_t ws_bytes, int32_t n_split,
                                  void *stream);

/* Bytes of device scratch the library keeps per device for
 * kvq_attn_decode_noalloc (held from the first kvq_create on that device
 * until the process ends). */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

/* kvq_attn_decode for callers that cannot allocate device memory or pass a
 * workspace: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid allocation.  It takes no workspace; its split
 * partials and arrival counters live in a fixed scratch array of
 * KVQ_NOALLOC_SCRATCH_BYTES on the context's device, shared by every call on
 * that device (set up, counters cleared, by kvq_create).  The call allocates
 * nothing and makes no synchronising call.  Arguments, layouts and results
 * are those of kvq_attn_decode (equal to it up to fp32 rounding of a
 * different split count).
 * Limit: the scratch holds a fixed 64 KiB of counters (B H_kv up to 16384),
 * plus 520 bytes per (batch, query head) and token split, plus (dense
 * rotation) 512 bytes per (batch, query head).  The split count of
 * kvq_attn_decode is lowered until that fits; if even one split does not
 * (B * H_q above about 16000, about 8000 with the dense rotation) the call
 * returns KVQ_E_WORKSPACE and launches nothing.
 * Concurrency: all calls on one device share the scratch, which keeps the
 * last call's contents, so calls that may overlap in time on one device (on
 * different streams, or from different host threads) race and give wrong
 * results; order them on one stream.  Other errors as kvq_attn_decode. */
kvq_status kvq_attn_decode_noalloc(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                                   const uint8_t *k_codes, const float *k_norms, const uint8_t *v_codes,
                                   const float *v_norms, float sm_scale, float *out, void *stream);

/* Workspace bytes kvq_nsn_vq_quantize needs for H heads of T tokens. */
size_t kvq_nsn_vq_ws_bytes(const kvq_ctx *ctx, int64_t H, int64_t T);

/* NSN vector quantisation ([NSN] Metodologia 1-3), per head over the T
 * tokens of the call:
 *   a_t = sqrt(d) x_t/||x_t||, s1_t = ||x_t||/sqrt(d);  o = mean_t a_t;
 *   b_t = a_t - o, s2_t = ||b_t||/sqrt(d);  z_t = H (b_t / s2_t) / sqrt(d);
 *   each 8-dim sub-vector of z_t -> index of the nearest codebook entry
 *   (squared Euclidean distance; lowest index on ties).
 *   x_f16   [H, T, d] fp16
 *   codes   out [H, T, 16] bytes (one per sub-vector)
 *   s1, s2  out [H, T] fp32;  o  out [H, d] fp32
 *   ws      device workspace, kvq_nsn_vq_ws_bytes() bytes (no init needed).
 * Degenerate tokens: ||x_t|| = 0 gives a_t = 0; s2_t = 0 gives z_t = 0.
 * T must be >= 1.  Requires a context in KVQ_MODE_NSN_VQ. */
kvq_status kvq_nsn_vq_quantize(kvq_ctx *ctx, const void *x_f16, int64_t H, int64_t T,
                               uint8_t *codes, float *s1, float *s2, float *o, void *ws,
                               size_t ws_bytes, void *stream);

/* Streaming cache ([NSN] Detalhes de Implementacao: following KIVI, the KV
 * cache is a quantised part plus a full-precision residual window that is
 * quantised and appended when it fills).  Per (batch, KV head) the packed
 * arrays hold T_cap tokens ([B, H_kv, T_cap, 16 b] codes, [B, H_kv, T_cap]
 * norms) of which the first T are valid, and the window arrays hold R_cap
 * fp16 tokens ([B, H_kv, R_cap, d]) of which the first R are valid.
 *
 * Workspace bytes kvq_attn_decode_stream needs for caches of T_cap tokens. */
size_t kvq_attn_decode_stream_ws_bytes(const kvq_ctx *ctx, int64_t B, int64_t H_q, int64_t T_cap);

/* One decode step over such a cache (MSE mode): attention of each query over
 * the T quantised tokens followed by the R window tokens, one softmax over
 * all T + R (scale sm_scale, 0 means 1/sqrt(d)); the quantised tokens are
 * scored and dequantised as in kvq_attn_decode, the window tokens used as
 * they are.  H_q / H_kv in {1, 2, 4}; 0 <= T <= T_cap, 0 <= R <= R_cap,
 * T + R >= 1 (either part may be empty; its pointers may then be NULL).
 *   out  [B, H_q, d] fp32
 *   ws   at least kvq_attn_decode_stream_ws_bytes() bytes, 256-byte aligned,
 *        its counter words zero before the first call (every completed call
 *        leaves them zero); calls sharing it must be ordered on one stream.
 * Errors: KVQ_E_WORKSPACE if ws_bytes is too small; KVQ_E_UNSUPPORTED for a
 * context with the dense rotation. */
kvq_status kvq_attn_decode_stream(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                                  int64_t T_cap, const uint8_t *k_codes, const float *k_norms,
                                  const uint8_t *v_codes, const float *v_norms, int64_t R, int64_t R_cap,
                                  const void *k_tail_f16, const void *v_tail_f16, float sm_scale,
                                  float *out, void *ws, size_t ws_bytes, void *stream);

/* Flush of the window: the first R tokens of the K and V windows of every
 * (batch, KV head) are quantised exactly as kvq_quantize quantises a vector
 * and written to positions T0 .. T0 + R - 1 of the packed arrays (layouts as
 * above, H_kv = the context's n_kv_heads; MSE mode).  Other positions are not
 * touched.  Requires T0 + R <= T_cap.  R == 0 or B == 0 is a no-op.
 * Errors: KVQ_E_INVAL (sizes), KVQ_E_UNSUPPORTED (dense rotation). */
kvq_status kvq_flush(kvq_ctx *ctx, const void *k_tail_f16, const void *v_tail_f16, int64_t B, int64_t H_kv,
                     int64_t R, int64_t R_cap, uint8_t *k_codes, float *k_norms, uint8_t *v_codes,
                     float *v_norms, int64_t T0, int64_t T_cap, void *stream);

/* Attention logits from NSN-VQ codes ([NSN] Detalhes de Implementacao: the
 * score takes the byproducts s1, s2, o directly).  A key reconstructs as
 * x_hat = s1 (s2 H zq / sqrt(d) + o), zq the 16 codebook entries its codes
 * name (the inverse of [NSN] Metodologia 1-2), so with q' = H q / sqrt(d)
 *   logits[b,h,t] = s1_t (s2_t sum_s <q'_s, C[code_t,s]> + <q_h, o_g>),
 *   g = h / (H_q / H_kv), H_kv = the context's n_kv_heads.
 *   q_f16    [B, H_q, d] fp16; H_q / H_kv in {1, 2, 4, 8}
 *   codes    [B, H_kv, T, 16] bytes; s1, s2 [B, H_kv, T] fp32; o [B, H_kv, d]
 *            fp32 (16-byte aligned): kvq_nsn_vq_quantize's outputs with its
 *            heads = the B * H_kv (batch, KV head) pairs
 *   logits   out [B, H_q, T] fp32 (raw inner products, no softmax scale)
 * Requires a context in KVQ_MODE_NSN_VQ (its codebook is the one used).
 * B * H_kv <= 65535.  B == 0 or T == 0 is a no-op. */
kvq_status kvq_nsn_logits(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                          const uint8_t *codes, const float *s1, const float *s2, const float *o,
                          float *logits, void *stream);

/* Workspace bytes kvq_nsn_attn_decode needs for these sizes (per-split partial
 * sums). */
size_t kvq_nsn_attn_decode_ws_bytes(const kvq_ctx *ctx, int64_t B, int64_t H_q, int64_t T);

/* One decode step of attention over NSN-VQ encoded keys and values: logits as
 * in kvq_nsn_logits, softmax with scale sm_scale (0 means 1/sqrt(d)), and
 *   out[b,h] = sum_t softmax_t x_hat^V_t
 *            = (H (sum_t w_t s1_t s2_t zq_t) / sqrt(d) + (sum_t w_t s1_t) o_V) / sum_t w_t.
 *   k_*, v_*  kvq_nsn_vq_quantize's outputs for K and V (layouts as in
 *             kvq_nsn_logits)
 *   out       [B, H_q, d] fp32
 *   ws        device workspace of at least kvq_nsn_attn_decode_ws_bytes()
 *             bytes, 256-byte aligned; no initialisation needed.  Calls that
 *             share a workspace must be ordered on one stream.
 * T must be >= 1.  Errors: KVQ_E_WORKSPACE if ws_bytes is too small. */
kvq_status kvq_nsn_attn_decode(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                               const uint8_t *k_codes, const float *k_s1, const float *k_s2,
                               const float *k_o, const uint8_t *v_codes, const float *v_s1,
                               const float *v_s2, const float *v_o, float sm_scale, float *out,
                               void *ws, size_t ws_bytes, void *stream);

/* As kvq_nsn_attn_decode with an explicit number of token splits per (batch,
 * KV head) (0 = automatic); the result does not depend on it beyond fp32
 * rounding.  n_split is clamped to [1, min(512, ceil(T / 64))]. */
kvq_status kvq_nsn_attn_decode_splits(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q,
                                      int64_t T, const uint8_t *k_codes, const float *k_s1,
                                      const float *k_s2, const float *k_o, const uint8_t *v_codes,
                                      const float *v_s1, const float *v_s2, const float *v_o,
                                      float sm_scale, float *out, void *ws, size_t ws_bytes,
                                      int32_t n_split, void *stream);

/* Double quantisation of the NSN byproducts ([NSN] Metodologia sec. 3: the
 * parameters o and s1 are stored with 4 bits).  The page gives no scheme;
 * here a block of values v is stored as 4-bit codes c with one fp32 pair
 * (lo, step): lo = min v, step = (max v - lo) / 15, c the nearest level of
 * (v - lo) / step (0 when step = 0), value lo + c step.  Blocks: the 128
 * means of a head; s1 in blocks of 32 consecutive tokens of a head (the last
 * one shorter).  Packing: code i of a row in byte i / 2, low nibble for even
 * i.  Per token 16 code bytes + 0.5 (s1) + 0.25 (block pair) + 4 (s2).
 *
 * Workspace bytes kvq_nsn_vq_quantize_dq needs. */
size_t kvq_nsn_vq_dq_ws_bytes(const kvq_ctx *ctx, int64_t H, int64_t T);

/* NSN-VQ as kvq_nsn_vq_quantize, with the double-quantised byproducts: the
 * mean o of each head is quantised first and the shift b_t = a_t - o_hat
 * uses the stored (dequantised) means, so that
 * x_hat = s1_hat (s2 H zq / sqrt(d) + o_hat) inverts the encoding; s1 is
 * quantised per block of 32 tokens.
 *   codes  out [H, T, 16] bytes;  s2 out [H, T] fp32
 *   s1q    out [H, ceil(T / 2)] bytes;  s1p out [H, ceil(T / 32), 2] fp32 (lo, step)
 *   oq     out [H, 64] bytes;  op out [H, 2] fp32 (lo, step)
 *   ws     kvq_nsn_vq_dq_ws_bytes() bytes, 256-byte aligned, no initialisation.
 * s1p and op 8-byte aligned.  T >= 1.  Requires a context in KVQ_MODE_NSN_VQ. */
kvq_status kvq_nsn_vq_quantize_dq(kvq_ctx *ctx, const void *x_f16, int64_t H, int64_t T, uint8_t *codes,
                                  uint8_t *s1q, float *s1p, float *s2, uint8_t *oq, float *op, void *ws,
                                  size_t ws_bytes, void *stream);

/* kvq_nsn_logits over double-quantised byproducts (layouts of
 * kvq_nsn_vq_quantize_dq with its heads = the B * H_kv pairs): s1 and o are
 * read as lo + c step.  Other arguments and errors as kvq_nsn_logits. */
kvq_status kvq_nsn_logits_dq(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                             const uint8_t *codes, const uint8_t *s1q, const float *s1p, const float *s2,
                             const uint8_t *oq, const float *op, float *logits, void *stream);

/* kvq_nsn_attn_decode_splits over double-quantised keys and values (layouts
 * of kvq_nsn_vq_quantize_dq); workspace kvq_nsn_attn_decode_ws_bytes().
 * Other arguments and errors as kvq_nsn_attn_decode_splits. */
kvq_status kvq_nsn_attn_decode_dq(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                                  const uint8_t *k_codes, const uint8_t *k_s1q, const float *k_s1p,
                                  const float *k_s2, const uint8_t *k_oq, const float *k_op,
                                  const uint8_t *v_codes, const uint8_t *v_s1q, const float *v_s1p,
                                  const float *v_s2, const uint8_t *v_oq, const float *v_op, float sm_scale,
                                  float *out, void *ws, size_t ws_bytes, int32_t n_split, void *stream);

/* Gain-shape residual quantisation ([GSRQ]: gain-shape k-means, which keeps
 * a reproduction's norm apart from its direction, in a residual quantisation
 * pipeline, below 1 bit per element).  The page gives no dimensions or front
 * end; here the NSN front end ([NSN] Metodologia 1-2: s1, o, s2 and
 * z = H (b / s2) / sqrt(d), as kvq_nsn_vq_quantize) feeds 4 sub-vectors of
 * 32 dimensions, each encoded in two stages k = 1, 2 on the running residual
 * r (r = z_s first): j = the shape of largest projection <r, S_k[j]> (lowest
 * j on ties), c = the number of thresholds (midpoints of adjacent levels)
 * below that projection, r -= G_k[c] S_k[j].  The context's tables
 * (kvq_config.gsrq_tables) are the codebook.  Record of a token, 12 bytes:
 * the 4 stage-1 shape indices, the 4 stage-2 ones, then c1 | c2 << 4 per
 * sub-vector (24 bits per 32 elements: 0.75 bit per element, plus s1, s2).
 *
 * Workspace bytes kvq_gsrq_quantize needs for H heads of T tokens. */
size_t kvq_gsrq_ws_bytes(const kvq_ctx *ctx, int64_t H, int64_t T);

/* GSRQ of x_f16 [H, T, d] fp16, per head over the T tokens of the call:
 *   codes  out [H, T, 12] bytes (4-byte aligned); s1, s2 out [H, T] fp32;
 *   o      out [H, d] fp32 (16-byte aligned)
 *   ws     kvq_gsrq_ws_bytes() bytes, 256-byte aligned, no initialisation.
 * T >= 1.  Requires a context in KVQ_MODE_GSRQ. */
kvq_status kvq_gsrq_quantize(kvq_ctx *ctx, const void *x_f16, int64_t H, int64_t T, uint8_t *codes, float *s1,
                             float *s2, float *o, void *ws, size_t ws_bytes, void *stream);

/* Logits from GSRQ records: x_hat = s1 (s2 H zq / sqrt(d) + o) with
 * zq_s = G1[c1] S1[j1] + G2[c2] S2[j2], so with q' = H q / sqrt(d)
 *   logits[b,h,t] = s1 (s2 sum_s (G1[c1] <q'_s, S1[j1]> + G2[c2] <q'_s, S2[j2]>) + <q_h, o_g>).
 * Layouts as kvq_nsn_logits with 12-byte records; H_q / H_kv in {1, 2, 4, 8}. */
kvq_status kvq_gsrq_logits(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T, const uint8_t *codes,
                           const float *s1, const float *s2, const float *o, float *logits, void *stream);

/* One decode step over GSRQ keys and values, as kvq_nsn_attn_decode_splits
 * (workspace kvq_nsn_attn_decode_ws_bytes(), no initialisation);
 * H_q / H_kv in {1, 2, 4}. */
kvq_status kvq_gsrq_attn_decode(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                                const uint8_t *k_codes, const float *k_s1, const float *k_s2, const float *k_o,
                                const uint8_t *v_codes, const float *v_s1, const float *v_s2, const float *v_o,
                                float sm_scale, float *out, void *ws, size_t ws_bytes, int32_t n_split,
                                void *stream);

/* Streaming NSN-VQ cache ([NSN] Detalhes de Implementacao: recent tokens
 * stay in a full-precision window that is quantised when it fills, as in
 * KIVI).  The pages do not say which tokens the channel mean o of
 * [NSN] Metodologia 2 runs over in this setting; here every flush of Gs
 * window tokens is encoded as one call of kvq_nsn_vq_quantize would encode
 * them, with its own K and V means, so packed tokens never change once
 * written.  Per (batch, KV head) the packed arrays hold T_cap tokens
 * ([B, H_kv, T_cap, 16] codes, [B, H_kv, T_cap] s1 and s2 fp32) of which the
 * first T are valid, the means [B, H_kv, T_cap / Gs, d] fp32 (mean g belongs
 * to tokens g Gs .. g Gs + Gs - 1), and the windows [B, H_kv, R_cap, d] fp16
 * of which the first R are valid.  Gs is a multiple of 64.
 *
 * Workspace bytes kvq_nsn_flush needs. */
size_t kvq_nsn_flush_ws_bytes(const kvq_ctx *ctx, int64_t B, int64_t Gs);

/* Flush: the first Gs tokens of the K and V windows of every (batch, KV
 * head) are encoded as kvq_nsn_vq_quantize encodes Gs tokens of one head,
 * and written to positions T0 .. T0 + Gs - 1 of the packed arrays and to
 * mean T0 / Gs.  Other positions are not touched.  H_kv must be the
 * context's n_kv_heads; Gs <= R_cap; T0 and T_cap multiples of Gs;
 * T0 + Gs <= T_cap.  ws: kvq_nsn_flush_ws_bytes() bytes, 256-byte aligned,
 * no initialisation needed.  B == 0 is a no-op.  Requires a context in
 * KVQ_MODE_NSN_VQ.  Errors: KVQ_E_INVAL (sizes, alignment), KVQ_E_WORKSPACE. */
kvq_status kvq_nsn_flush(kvq_ctx *ctx, const void *k_tail_f16, const void *v_tail_f16, int64_t B, int64_t H_kv,
                         int64_t Gs, int64_t R_cap, uint8_t *k_codes, float *k_s1, float *k_s2, float *k_o,
                         uint8_t *v_codes, float *v_s1, float *v_s2, float *v_o, int64_t T0, int64_t T_cap,
                         void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes kvq_nsn_attn_decode_stream needs for caches of T_cap tokens. */
size_t kvq_nsn_attn_decode_stream_ws_bytes(const kvq_ctx *ctx, int64_t B, int64_t H_q, int64_t T_cap);

/* One decode step over such a cache: one softmax (scale sm_scale, 0 means
 * 1/sqrt(d)) over the T packed tokens, each reconstructed with the means of
 * its flush group as x_hat = s1 (s2 H zq / sqrt(d) + o_g), followed by the
 * R window tokens as they are.  H_q / H_kv in {1, 2, 4}; 0 <= T <= T_cap,
 * T a multiple of Gs, 0 <= R <= R_cap, T + R >= 1 (an empty part's pointers
 * may be NULL); T <= 511 * 32 * Gs.  n_split: token splits per (batch, KV
 * head), 0 = automatic; a split holds whole flush groups, at most 32 of
 * them, so the count used may differ; the result depends on it only through
 * fp32 rounding.
 *   out  [B, H_q, d] fp32
 *   ws   at least kvq_nsn_attn_decode_stream_ws_bytes() bytes, 256-byte
 *        aligned, no initialisation needed; calls sharing it must be ordered
 *        on one stream.
 * B * H_kv <= 65535.  Errors: KVQ_E_INVAL, KVQ_E_WORKSPACE. */
kvq_status kvq_nsn_attn_decode_stream(kvq_ctx *ctx, const void *q_f16, int64_t B, int64_t H_q, int64_t T,
                                      int64_t T_cap, int64_t Gs, const uint8_t *k_codes, const float *k_s1,
                                      const float *k_s2, const float *k_o, const uint8_t *v_codes,
                                      const float *v_s1, const float *v_s2, const float *v_o, int64_t R,
                                      int64_t R_cap, const void *k_tail_f16, const void *v_tail_f16,
                                      float sm_scale, float *out, void *ws, size_t ws_bytes, int32_t n_split,
                                      void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H_ */
