// kda_chunked.hip -- placeholder until the chunked MFMA prefill lands.
#include "kda_internal.h"

namespace kda {
hipError_t launch_chunked(const LayerParams &, int, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace kda
