// Prefill kernels (grouped by expert). Filled in by the grouping, activation
// quantisation and grouped-GEMM kernels.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

bool prefill_supported(int, int, int, int, int) { return false; }
size_t prefill_ws_bytes(int, int, int, int, int, int) { return kCounterBytes; }
hipError_t launch_prefill(int, int, int, int, int, int, const float*, const void* const*, const int32_t*, const float*,
                          void*, int, void*, const PrefillDebug*, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace moe
