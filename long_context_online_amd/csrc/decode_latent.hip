// Latent-attention (MLA-shaped) paged decode: placeholder until the kernel lands.
#include "common.hpp"

namespace blasst {
hipError_t launch_decode_latent(const DecodeArgs &, hipStream_t) { return hipErrorNotSupported; }
}  // namespace blasst
