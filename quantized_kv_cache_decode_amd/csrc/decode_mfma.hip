// MFMA split-K decode attention (variant 2).  Not built yet: the launcher
// reports "not supported" so the API returns TQ_EHIP for this variant.
#include "tq_device.h"
#include "tq_launch.h"

namespace tq {

hipError_t launch_decode_mfma(const DecodeArgs&, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace tq
