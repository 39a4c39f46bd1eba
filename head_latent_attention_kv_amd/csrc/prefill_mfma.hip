// bf16 MFMA causal prefill kernel.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

bool prefill_mfma_supported(const AttnShape&) { return false; }

void prefill_mfma(const AttnShape&, const void*, const void*, const void*, const int64_t*, int,
                  int64_t, int, float*, hipStream_t) {}

}  // namespace mla
