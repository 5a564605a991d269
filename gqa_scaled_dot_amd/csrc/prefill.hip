// Prefill path of op `attention` (fp32 MFMA flash kernel): not built yet;
// every shape goes to the decode or generic path until it is.
#include "kernels.h"

namespace attn {

bool prefill_supported(int, int) { return false; }

hipError_t launch_prefill(const Problem&, const PrefillPlan&, const Launch&) {
    return hipErrorInvalidValue;
}

}  // namespace attn
