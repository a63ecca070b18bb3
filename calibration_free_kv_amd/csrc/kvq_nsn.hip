// NSN vector quantisation kernels (placeholder until implemented).
#include "kvq_internal.h"

namespace kvq {

size_t nsn_ws_bytes(int64_t H, int64_t T)
{
    (void)T;
    return (size_t)H * kD * sizeof(float) + 256;
}

hipError_t launch_nsn_vq(const kvq_ctx *, const void *, int64_t, int64_t, uint8_t *, float *, float *,
                         float *, void *, hipStream_t)
{
    return hipErrorNotSupported;
}

}  // namespace kvq
