// Matrix-core latent-attention decode kernel (placeholder until written).
#include "device_common.h"
#include "mla_internal.h"

namespace mla {
int launch_decode_mfma(const DecodeArgs&, const DecodePlan&, hipStream_t) {
  return int(hipErrorNotSupported);
}
}  // namespace mla
