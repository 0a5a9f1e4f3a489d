// MXFP8 grouped GEMMs: not provided yet.  The entry points report
// MOE_EUNSUPPORTED so callers never receive silently wrong results.
#include "moe_internal.h"

namespace moe {

const bool kMxGemmAvailable = false;

size_t gemm_ws_mxfp8(int E, int64_t n_rows, int d, int f)
{
    (void)E;
    (void)n_rows;
    (void)d;
    (void)f;
    return 256;
}

hipError_t gemm_fwd_mxfp8(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*,
                          const uint8_t*, const uint8_t*, GroupSpec, int, int, uint16_t*,
                          uint16_t*, uint16_t*, void*, hipStream_t)
{
    return hipErrorNotSupported;
}

hipError_t gemm_bwd_mxfp8(const uint16_t*, const uint8_t*, const uint8_t*, const uint16_t*,
                          const uint16_t*, const uint8_t*, const uint8_t*, const uint8_t*,
                          const uint8_t*, GroupSpec, int, int, uint16_t*, uint16_t*, uint16_t*,
                          uint16_t*, void*, hipStream_t)
{
    return hipErrorNotSupported;
}

}  // namespace moe
