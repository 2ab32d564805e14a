// prefill_kernels.hip — causal chunked prefill over the paged cache.
#include "pa_internal.h"

namespace pa {

bool prefill_supported(int32_t, int32_t, int, int, int) { return false; }

hipError_t prefill(const PrefillArgs&) { return hipErrorInvalidValue; }

}  // namespace pa
