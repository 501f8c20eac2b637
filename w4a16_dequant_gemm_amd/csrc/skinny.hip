// Skinny-batch MFMA kernel (placeholder until the kernel lands: reports no support).
#include "common.h"
#include "launch.h"

namespace w4a16 {

bool skinny_supports(const LinearArgs&) { return false; }

hipError_t launch_skinny(const LinearArgs&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace w4a16
