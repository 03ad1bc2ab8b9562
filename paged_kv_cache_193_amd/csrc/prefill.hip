// prefill.hip -- causal paged prefill (MFMA path): not yet implemented.
#include "launch.h"

namespace pkv {

hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pkv
