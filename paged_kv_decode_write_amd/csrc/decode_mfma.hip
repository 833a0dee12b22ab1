// Placeholder until the matrix-core decode kernel lands.
#include "launch.h"

namespace pagedkv {

bool supported_mfma(int, int, int) { return false; }

hipError_t launch_decode_mfma(const DecodeArgs&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace pagedkv
