// Host stand-ins for the HIP runtime calls and kernel launches of libkvq's
// host code, so that its validation, table builders and workspace layouts run
// under the address and undefined-behaviour sanitizers on a machine without a
// GPU.  One fake device with 256 compute units; device memory is host memory.
// Every launch records its call and arguments in `g_last` and succeeds.
#include <cstdlib>
#include <cstring>

#include "kvq_internal.h"
#include "stub_record.h"

StubRecord g_last;

extern "C" {
hipError_t hipGetDeviceCount(int *n) { *n = 1; return hipSuccess; }
hipError_t hipGetDevice(int *d) { *d = 0; return hipSuccess; }
hipError_t hipSetDevice(int d) { return d == 0 ? hipSuccess : hipErrorInvalidDevice; }
hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t a, int d)
{
    (void)d;
    *v = a == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
    return hipSuccess;
}
hipError_t hipMalloc(void **p, size_t n)
{
    *p = std::calloc(n ? n : 1, 1);
    return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void *p) { std::free(p); return hipSuccess; }
hipError_t hipMemcpy(void *dst, const void *src, size_t n, hipMemcpyKind k)
{
    (void)k;
    std::memcpy(dst, src, n);
    return hipSuccess;
}
}

namespace kvq {
static hipError_t rec(const char *what, int64_t a = 0, int64_t b = 0, int64_t c = 0, int n_split = 0)
{
    g_last.calls++;
    g_last.what = what;
    g_last.a = a;
    g_last.b = b;
    g_last.c = c;
    g_last.n_split = n_split;
    return hipSuccess;
}
hipError_t noalloc_setup(int device) { return device == 0 ? hipSuccess : hipErrorInvalidDevice; }
// the kernel files' debug records (a release build: nothing recorded)
uint32_t debug_take_quantize() { return 0u; }
uint32_t debug_take_score() { return 0u; }
uint32_t debug_take_nsn() { return 0u; }
uint32_t debug_take_nsn_score() { return 0u; }
uint32_t debug_take_dense() { return 0u; }
uint32_t debug_take_stream() { return 0u; }
hipError_t launch_quantize(const kvq_ctx *, int kind, const void *, int64_t B, int64_t T, uint8_t *, float *,
                           uint8_t *, float *, hipStream_t)
{ return rec("quantize", kind, B, T); }
hipError_t launch_quantize_kv(const kvq_ctx *, const void *, const void *, int64_t B, int64_t T, uint8_t *, float *,
                              uint8_t *, float *, hipStream_t)
{ return rec("quantize_kv", B, T); }
hipError_t launch_quantize_dense(const kvq_ctx *, const void *, const void *, int64_t N, uint8_t *, float *, uint8_t *,
                                 float *, hipStream_t)
{ return rec("quantize_dense", N); }
hipError_t launch_quantize_dense_qjl(const kvq_ctx *, const void *, int64_t N, uint8_t *, float *, uint8_t *, float *,
                                     hipStream_t)
{ return rec("quantize_dense_qjl", N); }
hipError_t launch_logits(const kvq_ctx *, const void *, int64_t B, int64_t Hq, int64_t T, const uint8_t *,
                         const float *, const uint8_t *, const float *, float *, hipStream_t)
{ return rec("logits", B, Hq, T); }
hipError_t launch_decode(const kvq_ctx *, const void *, int64_t B, int64_t Hq, int64_t T, const uint8_t *,
                         const float *, const uint8_t *, const float *, float, float *, void *, int ns, hipStream_t)
{ return rec("decode", B, Hq, T, ns); }
hipError_t launch_decode_stream(const kvq_ctx *, const void *, int64_t B, int64_t Hq, int64_t T, int64_t,
                                const uint8_t *, const float *, const uint8_t *, const float *, const DecodeTail *,
                                float, float *, void *, int ns, hipStream_t)
{ return rec("decode_stream", B, Hq, T, ns); }
hipError_t launch_decode_noalloc(const kvq_ctx *, const void *, int64_t B, int64_t Hq, int64_t T, const uint8_t *,
                                 const float *, const uint8_t *, const float *, float, float *, int ns, hipStream_t)
{ return rec("decode_noalloc", B, Hq, T, ns); }
hipError_t launch_flush(const kvq_ctx *, const void *, const void *, int64_t B, int64_t R, int64_t, uint8_t *, float *,
                        uint8_t *, float *, int64_t T0, int64_t, hipStream_t)
{ return rec("flush", B, R, T0); }
hipError_t launch_nsn_vq(const kvq_ctx *, const void *, int64_t H, int64_t T, uint8_t *, float *, float *, float *,
                         void *, hipStream_t)
{ return rec("nsn_vq", H, T); }
hipError_t launch_nsn_logits(const kvq_ctx *, const void *, int64_t B, int64_t Hq, int64_t T, const uint8_t *,
                             const float *, const float *, const float *, float *, hipStream_t)
{ return rec("nsn_logits", B, Hq, T); }
hipError_t launch_nsn_decode(const kvq_ctx *, const void *, int64_t B, int64_t Hq, int64_t T, const NsnKV &kv, float,
                             float *, void *, int ns, hipStream_t)
{ return rec(kv.dq ? "nsn_decode_dq" : "nsn_decode", B, Hq, T, ns); }
hipError_t launch_nsn_vq_strided(const kvq_ctx *, const void *, int64_t H, int64_t T, int64_t, uint8_t *, float *,
                                 float *, int64_t ldt, float *, int64_t, void *, hipStream_t)
{ return rec("nsn_vq_strided", H, T, ldt); }
hipError_t launch_nsn_vq_dq(const kvq_ctx *, const void *, int64_t H, int64_t T, uint8_t *, float *, const NsnDq &,
                            void *, hipStream_t)
{ return rec("nsn_vq_dq", H, T); }
hipError_t launch_nsn_logits_dq(const kvq_ctx *, const void *, int64_t B, int64_t Hq, int64_t T, const uint8_t *,
                                const NsnDqIn &, const float *, float *, hipStream_t)
{ return rec("nsn_logits_dq", B, Hq, T); }
hipError_t launch_gsrq(const kvq_ctx *, const void *, int64_t H, int64_t T, uint8_t *, float *, float *, float *,
                       void *, hipStream_t)
{ return rec("gsrq", H, T); }
hipError_t launch_gsrq_logits(const kvq_ctx *, const void *, int64_t B, int64_t Hq, int64_t T, const uint8_t *,
                              const float *, const float *, const float *, float *, hipStream_t)
{ return rec("gsrq_logits", B, Hq, T); }
hipError_t launch_gsrq_decode(const kvq_ctx *, const void *, int64_t B, int64_t Hq, int64_t T, const NsnKV &, float,
                              float *, void *, int ns, hipStream_t)
{ return rec("gsrq_decode", B, Hq, T, ns); }
hipError_t launch_nsn_decode_stream(const kvq_ctx *, const void *, int64_t B, int64_t Hq, int64_t T, const NsnKV &,
                                    const NsnStream &, float, float *, void *, int ns, hipStream_t)
{ return rec("nsn_decode_stream", B, Hq, T, ns); }
}  // namespace kvq
