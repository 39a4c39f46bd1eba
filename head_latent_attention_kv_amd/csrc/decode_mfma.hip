// bf16 MFMA decode kernel (latent-cache tiles shared by all heads of a sequence).
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

bool decode_mfma_supported(const AttnShape&) { return false; }

void decode_mfma(const AttnShape&, const void*, const void*, const void*, const int64_t*,
                 const int32_t*, int, int, int, float*, float*, float*, hipStream_t) {}

}  // namespace mla
