#include "pa_internal.h"
namespace pa {
bool small_mfma_supported(int32_t, int32_t) { return false; }
hipError_t launch_small_mfma(const Plan&, const AttnArgs&, void*, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace pa
