// sdpa_mfma.hip - split pass, MFMA variant (placeholder until it lands).
#include "common.hpp"
#include "kernels.hpp"

namespace otq {

bool split_mfma_supports(int, int) { return false; }

hipError_t launch_split_mfma(const SplitArgs&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace otq
