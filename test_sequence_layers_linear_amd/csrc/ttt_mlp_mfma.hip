// ttt_mlp_mfma.hip -- TTT-MLP dual-form scan on MFMA (d = 64, m = 256, b = 16).
// Not built yet: every MLP shape runs the generic kernel.
#include "ttt_internal.h"

namespace ttt {

bool mlp_mfma_supports(const MlpArgs&) { return false; }

hipError_t launch_mlp_mfma(const MlpArgs&) { return hipErrorInvalidValue; }

}  // namespace ttt
