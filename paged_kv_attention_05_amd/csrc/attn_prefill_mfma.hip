#include "pa_internal.h"
namespace pa {
bool prefill_mfma_supported(int32_t, int32_t, int32_t) { return false; }
int32_t prefill_tile_tokens(int32_t g) { return 128 / g; }
hipError_t launch_prefill_mfma(const Plan&, const AttnArgs&, void*, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace pa
