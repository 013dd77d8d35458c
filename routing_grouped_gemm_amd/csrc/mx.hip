// MXFP8 path (not built yet): every entry reports hipErrorNotSupported.
#include "mx.h"

namespace moe {
size_t mx_fwd_workspace(long long, int, int, int) { return 0; }
size_t mx_bwd_workspace(long long, int, int, int) { return 0; }
hipError_t launch_mx_dispatch_copy(const void*, const int32_t*, int, int, int, void*, uint8_t*,
                                   hipStream_t) { return hipErrorNotSupported; }
hipError_t mx_ffn_fwd(const void*, const uint8_t*, const int32_t*, int, int, int, int, const void*,
                      const void*, const void*, void*, void*, void*, void*, void*, int,
                      hipStream_t) { return hipErrorNotSupported; }
hipError_t mx_ffn_dgrad(const void*, const void*, const void*, const int32_t*, int, int, int, int,
                        const void*, const void*, const void*, void*, void*, void*, int,
                        hipStream_t) { return hipErrorNotSupported; }
}  // namespace moe
