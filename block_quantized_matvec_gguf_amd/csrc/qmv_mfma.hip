// N-token (prefill) kernel family. Not built yet: the planner reports the
// shape as unsupported, so AUTO always takes the streaming GEMV path.
#include "qmv_internal.h"

namespace qmv {

bool plan_mfma(int, int64_t, int64_t, int64_t, int, MfmaPlan *) { return false; }

hipError_t launch_mfma(const MfmaPlan &, const uint8_t *, const float *, float *, int64_t,
                       int64_t, int64_t, int64_t, int64_t, int64_t, int, hipStream_t) {
    return hipErrorInvalidValue;
}

const char *mfma_kernel_name(const MfmaPlan &) { return ""; }

} // namespace qmv
